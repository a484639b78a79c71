"""Seeded synthetic decode workloads.

This module only draws and lays out inputs; it holds none of the method's
arithmetic.  Both the HIP path and the fp64 oracle receive exactly these
arrays (bf16 values travel as their 16-bit patterns, and widen to fp32/fp64
exactly).

Shapes follow DeepSeek-V2's attention (h=128 heads, d_c=512 latent, d_R=64
RoPE, d_h=128 per head; "MLA Explained", section "Memory: the concrete
numbers"; "MLA, dim by dim", section 5.2).  No dataset or trained weight is
involved: every tensor is random with a fixed seed.

Draw order per workload: lengths -> page permutation -> latent pool -> RoPE
pool -> q -> q_R -> W_UK -> W_UV.  Activations are N(0, 1); weights are
N(0, 1/d_c) (variance 1/d_c), which keeps the scaled logits at unit variance.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even) and
    return the 16-bit patterns as uint16."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    # NaN stays NaN (never produced by the generators; kept for completeness)
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class Workload:
    name: str
    dtype: str            # "bf16" or "f32": storage type of every input
    batch: int
    n_q: int
    h: int
    d_c: int
    d_r: int
    d_h: int
    page_size: int
    lens: np.ndarray      # int32 [batch]
    page_table: np.ndarray  # int32 [batch, max_pages]
    num_pages: int
    seed: int
    description: str = ""
    splits: tuple = ()    # split counts the parity tests sweep (0 = library's choice)
    arrays: dict = field(default_factory=dict, repr=False)

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d_h + self.d_r))

    @property
    def max_len(self) -> int:
        return int(self.lens.max())

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def rows(self) -> int:
        return self.batch * self.n_q

    def cache_tokens(self) -> int:
        return int(self.lens.sum())

    def visible_pairs(self) -> int:
        """Number of (query row, cached token) pairs the score step touches."""
        n = 0
        for L in self.lens.tolist():
            for m in range(self.n_q):
                n += L - self.n_q + m + 1
        return n


def _pages(lens, page_size):
    return [(int(L) + page_size - 1) // page_size for L in lens]


def _table(per_seq_pages, perm):
    B = len(per_seq_pages)
    max_pages = max(per_seq_pages)
    table = np.zeros((B, max_pages), dtype=np.int32)
    off = 0
    for b, n in enumerate(per_seq_pages):
        table[b, :n] = perm[off:off + n]
        off += n
    return table


# name -> (description, builder kwargs)
WORKLOADS = {
    "tiny_fp32": dict(
        description="tiny fp32 decode: B=1, one query, h=4, d_c=16, d_R=8, d_h=16, T=64",
        dtype="f32", batch=1, n_q=1, h=4, d_c=16, d_r=8, d_h=16, page_size=16,
        lens=("fixed", 64), shuffled=False, seed=101, splits=(0, 1, 2, 4)),
    "ds2_t4k": dict(
        description="DeepSeek-V2-shaped decode, bf16, B=1, one query, T=4096 contiguous",
        dtype="bf16", batch=1, n_q=1, h=128, d_c=512, d_r=64, d_h=128, page_size=64,
        lens=("fixed", 4096), shuffled=False, seed=102, splits=(0, 1, 16)),
    "ds2_paged_b32": dict(
        description="batched paged decode, bf16, B=32, lengths U{1024..8192}, 64-token "
                    "pages, shuffled page table",
        dtype="bf16", batch=32, n_q=1, h=128, d_c=512, d_r=64, d_h=128, page_size=64,
        lens=("uniform", 1024, 8192), shuffled=True, seed=103, splits=(0,)),
    "ds2_t128k": dict(
        description="long-context split decode, bf16, B=1, T=131072, 64..256 splits",
        dtype="bf16", batch=1, n_q=1, h=128, d_c=512, d_r=64, d_h=128, page_size=64,
        lens=("fixed", 131072), shuffled=False, seed=104, splits=(64, 128, 256)),
    "ds2_mtp_b16": dict(
        description="multi-token decode, bf16, B=16, 4 causal query tokens, T=16384",
        dtype="bf16", batch=16, n_q=4, h=128, d_c=512, d_r=64, d_h=128, page_size=64,
        lens=("fixed", 16384), shuffled=False, seed=105, splits=(0,)),
    "ds2_t32k": dict(
        description="single-sequence decode, bf16, B=1, T=32768 contiguous",
        dtype="bf16", batch=1, n_q=1, h=128, d_c=512, d_r=64, d_h=128, page_size=64,
        lens=("fixed", 32768), shuffled=False, seed=106, splits=(0,)),
}

# the five parity configurations, in order
CONFIG_ORDER = ["tiny_fp32", "ds2_t4k", "ds2_paged_b32", "ds2_t128k", "ds2_mtp_b16"]


def make(name: str = None, *, materialize: bool = True, **override) -> Workload:
    """Build a named workload (or a custom one from keyword arguments) and,
    unless ``materialize`` is False, draw its tensors."""
    spec = dict(WORKLOADS[name]) if name is not None else {}
    spec.update(override)
    rng = np.random.default_rng(spec["seed"])
    B = spec["batch"]
    kind = spec["lens"]
    if kind[0] == "fixed":
        lens = np.full(B, kind[1], dtype=np.int32)
    elif kind[0] == "uniform":
        lens = rng.integers(kind[1], kind[2], size=B, endpoint=True).astype(np.int32)
    elif kind[0] == "list":
        lens = np.asarray(kind[1], dtype=np.int32)
        if lens.shape != (B,):
            raise ValueError("one length per sequence")
    else:
        raise ValueError(kind)
    ps = spec["page_size"]
    per_seq = _pages(lens, ps)
    total = int(sum(per_seq))
    perm = rng.permutation(total).astype(np.int32) if spec.get("shuffled") else np.arange(total, dtype=np.int32)
    wl = Workload(name=name or spec.get("name", "custom"), dtype=spec["dtype"], batch=B,
                  n_q=spec["n_q"], h=spec["h"], d_c=spec["d_c"], d_r=spec["d_r"],
                  d_h=spec["d_h"], page_size=ps, lens=lens, page_table=_table(per_seq, perm),
                  num_pages=total, seed=spec["seed"], description=spec.get("description", ""),
                  splits=tuple(spec.get("splits", (0,))))
    if materialize:
        _draw(wl, rng)
    return wl


def _draw(wl: Workload, rng) -> None:
    f32 = np.float32
    shapes = [
        ("latent_pool", (wl.num_pages, wl.page_size, wl.d_c), 1.0),
        ("rope_pool", (wl.num_pages, wl.page_size, wl.d_r), 1.0),
        ("q", (wl.batch, wl.n_q, wl.h, wl.d_h), 1.0),
        ("q_r", (wl.batch, wl.n_q, wl.h, wl.d_r), 1.0),
        ("w_uk", (wl.h, wl.d_h, wl.d_c), float(np.sqrt(1.0 / wl.d_c))),
        ("w_uv", (wl.h, wl.d_h, wl.d_c), float(np.sqrt(1.0 / wl.d_c))),
    ]
    for key, shape, std in shapes:
        x = rng.standard_normal(shape, dtype=f32)
        if std != 1.0:
            x *= f32(std)
        wl.arrays[key] = bf16_bits(x) if wl.dtype == "bf16" else x


def as_f32(wl: Workload, key: str) -> np.ndarray:
    """The stored values of one input as float32 (exact)."""
    a = wl.arrays[key]
    return bf16_to_f32(a) if wl.dtype == "bf16" else a


def as_f64(wl: Workload, key: str) -> np.ndarray:
    return as_f32(wl, key).astype(np.float64)


def digest(wl: Workload) -> dict:
    """SHA-256 of every generated tensor's bytes (reproducibility log)."""
    out = {k: hashlib.sha256(np.ascontiguousarray(v).tobytes()).hexdigest()[:16]
           for k, v in sorted(wl.arrays.items())}
    out["lens"] = hashlib.sha256(wl.lens.tobytes()).hexdigest()[:16]
    out["page_table"] = hashlib.sha256(wl.page_table.tobytes()).hexdigest()[:16]
    return out


def oracle_problem_kwargs(wl: Workload) -> dict:
    """Keyword arguments for the oracle's problem description (fp64 views of
    the same stored values)."""
    return dict(q=as_f64(wl, "q"), q_r=as_f64(wl, "q_r"),
                latent_pool=as_f64(wl, "latent_pool"), rope_pool=as_f64(wl, "rope_pool"),
                page_table=wl.page_table, context_lens=wl.lens,
                w_uk=as_f64(wl, "w_uk"), w_uv=as_f64(wl, "w_uv"), scale=wl.scale)


# --------------------------------------------------------------------------
# The output projection that follows the decode step
# --------------------------------------------------------------------------
# DeepSeek-V2's model width ("MLA Explained", section "Memory: the concrete
# numbers").
D_MODEL = 5120


def make_oproj(rows: int, h: int = 128, d_h: int = 128, d_model: int = D_MODEL, dtype: str = "bf16",
               seed: int = 300) -> dict:
    """Head outputs o [rows][h][d_h] ~ N(0, 1), then W^O in the pages'
    orientation, k x d_model with k = h d_h, ~ N(0, 1/k) (variance 1/k, as
    the other weights: variance 1 / fan-in); drawn in that order.  bf16
    values travel as their 16-bit patterns, fp32 values as float32."""
    rng = np.random.default_rng(seed)
    k = h * d_h
    o = rng.standard_normal((rows, h, d_h), dtype=np.float32)
    w = (rng.standard_normal((k, d_model), dtype=np.float32) / np.float32(np.sqrt(k))).astype(np.float32)
    if dtype == "bf16":
        return dict(o=bf16_bits(o), w_o=bf16_bits(w), dtype=dtype, rows=rows, k=k, d=d_model)
    return dict(o=o, w_o=w, dtype=dtype, rows=rows, k=k, d=d_model)


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """bf16 patterns or fp32 values -> float64 (exact)."""
    return bf16_to_f32(a).astype(np.float64) if dtype == "bf16" else np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# The current token's projections (cache append and query side)
# --------------------------------------------------------------------------
# DeepSeek-V2's query latent width d_c' ("MLA Explained", section "Query
# compression: an optional bonus").
D_QC = 1536


def make_projections(rows: int, d_model: int = D_MODEL, d_c: int = 512, d_r: int = 64, d_qc: int = D_QC,
                     h: int = 128, d_h: int = 128, dtype: str = "bf16", seed: int = 400) -> dict:
    """Hidden states x [rows][d_model] ~ N(0, 1), then W_DKV [d_c][d_model],
    W_KR [d_r][d_model], W_DQ [d_qc][d_model] ~ N(0, 1/d_model) and
    W_UQ [h][d_h][d_qc], W_QR [h][d_r][d_qc] ~ N(0, 1/d_qc) (variance
    1/fan-in), drawn in that order, bf16 patterns or float32."""
    rng = np.random.default_rng(seed)

    def draw(shape, fan_in):
        a = rng.standard_normal(shape, dtype=np.float32)
        return a if fan_in is None else (a / np.float32(np.sqrt(fan_in))).astype(np.float32)

    out = dict(x=draw((rows, d_model), None), w_dkv=draw((d_c, d_model), d_model), w_kr=draw((d_r, d_model), d_model),
               w_dq=draw((d_qc, d_model), d_model), w_uq=draw((h, d_h, d_qc), d_qc), w_qr=draw((h, d_r, d_qc), d_qc))
    if dtype == "bf16":
        out = {k: bf16_bits(v) for k, v in out.items()}
    out.update(dtype=dtype, rows=rows, d_model=d_model, d_c=d_c, d_r=d_r, d_qc=d_qc, h=h, d_h=d_h)
    return out


# --------------------------------------------------------------------------
# Prefill (attention over a whole prompt)
# --------------------------------------------------------------------------
def make_prefill(T: int, h: int = 128, d_c: int = 512, d_r: int = 64, d_h: int = 128, dtype: str = "bf16",
                 seed: int = 500) -> dict:
    """A prompt of T tokens: latents [T][d_c] and rotated RoPE keys [T][d_r]
    ~ N(0, 1), queries [T][h][d_h] and RoPE queries [T][h][d_r] ~ N(0, 1),
    then W_UK, W_UV [h][d_h][d_c] ~ N(0, 1/d_c), drawn in that order (the
    decode workloads' distributions), bf16 patterns or float32."""
    rng = np.random.default_rng(seed)
    out = dict(latent=rng.standard_normal((T, d_c), dtype=np.float32),
               rope=rng.standard_normal((T, d_r), dtype=np.float32),
               q=rng.standard_normal((T, h, d_h), dtype=np.float32),
               q_r=rng.standard_normal((T, h, d_r), dtype=np.float32))
    for k in ("w_uk", "w_uv"):
        out[k] = (rng.standard_normal((h, d_h, d_c), dtype=np.float32) / np.float32(np.sqrt(d_c))).astype(np.float32)
    if dtype == "bf16":
        out = {k: bf16_bits(v) for k, v in out.items()}
    out.update(dtype=dtype, T=T, h=h, d_c=d_c, d_r=d_r, d_h=d_h)
    return out
