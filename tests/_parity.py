"""Helpers shared by the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import sys
import time

import numpy as np

import oracle
from mla_latent_cache_absorbed_amd import inputs

# normwise tolerance: max |gpu - oracle| / max |oracle| over the checked outputs
TOL = {"bf16": 1e-2, "f32": 1e-5}


def log(msg: str) -> None:
    sys.stdout.write("[parity] %s\n" % msg)
    sys.stdout.flush()


def problem(wl) -> oracle.Problem:
    return oracle.Problem(**inputs.oracle_problem_kwargs(wl))


def sample_pairs(wl, heads_per_seq: int, seqs=None, seed: int = 0):
    """(sequence, head) pairs: every listed sequence, a seeded subset of heads."""
    rng = np.random.default_rng(seed + wl.seed)
    seqs = range(wl.batch) if seqs is None else seqs
    pairs = []
    for b in seqs:
        heads = np.sort(rng.choice(wl.h, size=min(heads_per_seq, wl.h), replace=False))
        pairs += [(int(b), int(i)) for i in heads]
    return pairs


def gpu_rows(out_f64: np.ndarray, pairs) -> np.ndarray:
    """GPU output [B, n_q, h, d_h] -> [len(pairs), n_q, d_h]."""
    return np.stack([out_f64[b, :, i, :] for b, i in pairs])


def normwise(got: np.ndarray, ref: np.ndarray) -> float:
    scale = float(np.max(np.abs(ref)))
    return float(np.max(np.abs(got - ref))) / (scale if scale > 0 else 1.0)


def check(got, ref, dtype, what):
    assert np.all(np.isfinite(got)), "%s: non-finite GPU output" % what
    err = normwise(got, ref)
    log("%s: normwise error %.3e (tolerance %.0e)" % (what, err, TOL[dtype]))
    assert err <= TOL[dtype], "%s: normwise error %.3e > %.0e" % (what, err, TOL[dtype])
    return err


class Timer:
    def __enter__(self):
        self.t = time.time()
        return self

    def __exit__(self, *a):
        self.dt = time.time() - self.t
