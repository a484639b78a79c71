"""fp64 CPU oracle for absorbed-weight MLA decode -- test infrastructure only.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never loads it and it
never loads the HIP library: both sides receive the same seeded inputs and
share nothing else.

The C source (``mla_oracle.c``) holds the arithmetic; this module compiles it
with gcc and marshals numpy arrays through ctypes.  Every function cites the
passage it follows in the C source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mla_oracle.c")
_LIB = os.path.join(_HERE, "libmla_oracle.so")

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)


class _Problem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("n_q", ctypes.c_int32), ("h", ctypes.c_int32),
        ("d_c", ctypes.c_int32), ("d_r", ctypes.c_int32), ("d_h", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("max_pages", ctypes.c_int32),
        ("num_pages", ctypes.c_int32), ("_pad", ctypes.c_int32),
        ("scale", ctypes.c_double),
        ("q", _dp), ("q_r", _dp), ("latent_pool", _dp), ("rope_pool", _dp),
        ("page_table", _ip), ("context_lens", _ip), ("w_uk", _dp), ("w_uv", _dp),
    ]


def build(force: bool = True) -> str:
    """Compile ``mla_oracle.c`` into ``libmla_oracle.so`` (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(
            ["gcc", "-O2", "-fno-fast-math", "-fopenmp", "-fPIC", "-shared", "-std=c11",
             "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"],
            check=True,
        )
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    """Load the oracle library, building it when it is absent or stale."""
    global _lib
    if _lib is None:
        # MLA_ORACLE_LIB lets the mutation tests load a deliberately broken copy
        path = os.environ.get("MLA_ORACLE_LIB")
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build(force=True)
        L = ctypes.CDLL(path)
        L.mla_oracle_matvec.argtypes = [ctypes.c_int, ctypes.c_int, _dp, _dp, _dp]
        L.mla_oracle_matvec_t.argtypes = [ctypes.c_int, ctypes.c_int, _dp, _dp, _dp]
        L.mla_oracle_dot.argtypes = [ctypes.c_int, _dp, _dp]
        L.mla_oracle_dot.restype = ctypes.c_double
        L.mla_oracle_softmax.argtypes = [ctypes.c_int, _dp, _dp]
        L.mla_oracle_absorb_query.argtypes = [ctypes.c_int, ctypes.c_int, _dp, _dp, _dp]
        L.mla_oracle_latent_scores.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_double, _dp, _dp, _dp, _dp, _dp]
        L.mla_oracle_weighted_latent.argtypes = [ctypes.c_int, ctypes.c_int, _dp, _dp, _dp]
        L.mla_oracle_up_project.argtypes = [ctypes.c_int, ctypes.c_int, _dp, _dp, _dp]
        L.mla_oracle_gather.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int, ctypes.c_int,
                                        _dp, _dp]
        L.mla_oracle_decode_explicit.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int,
                                                 _ip, _ip, _dp]
        L.mla_oracle_decode_explicit.restype = ctypes.c_int
        L.mla_oracle_decode_absorbed.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int,
                                                 _ip, _ip, _dp, _dp]
        L.mla_oracle_decode_absorbed.restype = ctypes.c_int
        L.mla_oracle_num_threads.restype = ctypes.c_int
        L.mla_oracle_set_num_threads.argtypes = [ctypes.c_int]
        L.mla_oracle_output_project.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, _dp, _dp, _dp]
        L.mla_oracle_output_project.restype = None
        _i32p = ctypes.POINTER(ctypes.c_int32)
        L.mla_oracle_rope_thetas.argtypes = [ctypes.c_int, ctypes.c_double, _dp]
        L.mla_oracle_rope_thetas.restype = None
        L.mla_oracle_rope.argtypes = [ctypes.c_int, _dp, ctypes.c_double, _dp, _dp]
        L.mla_oracle_rope.restype = None
        L.mla_oracle_cache_append.argtypes = [ctypes.c_int] * 4 + [_dp] * 3 + [_i32p] * 2 + [_dp, _i32p] + \
            [ctypes.c_int] * 3 + [_dp, _dp]
        L.mla_oracle_cache_append.restype = ctypes.c_int
        L.mla_oracle_query_project.argtypes = [ctypes.c_int] * 6 + [_dp] * 4 + [_i32p] + [_dp] * 3
        L.mla_oracle_query_project.restype = None
        L.mla_oracle_set_num_threads.restype = None
        _lib = L
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _p(a: np.ndarray):
    return a.ctypes.data_as(_dp)


# --------------------------------------------------------------------------
# Primitives ("Mathematical Prerequisites for DeepSeek-V2", sections 1, 2, 6)
# --------------------------------------------------------------------------
def matvec(A, x) -> np.ndarray:
    """y = A x (section 1, matrix-vector multiplication)."""
    A = _f64(A); x = _f64(x)
    m, n = A.shape
    if x.shape != (n,):
        raise ValueError("dimension compatibility rule: A has %d columns, x has %d entries" % (n, x.size))
    y = np.empty(m)
    lib().mla_oracle_matvec(m, n, _p(A), _p(x), _p(y))
    return y


def matvec_t(A, x) -> np.ndarray:
    """y = A^T x (section 2, transpose; section 6, moving a matrix across a dot product)."""
    A = _f64(A); x = _f64(x)
    m, n = A.shape
    if x.shape != (m,):
        raise ValueError("dimension compatibility rule: A^T has %d columns, x has %d entries" % (m, x.size))
    y = np.empty(n)
    lib().mla_oracle_matvec_t(m, n, _p(A), _p(x), _p(y))
    return y


def dot(a, b) -> float:
    a = _f64(a); b = _f64(b)
    if a.shape != b.shape or a.ndim != 1:
        raise ValueError("dot needs two vectors of one length")
    return float(lib().mla_oracle_dot(a.size, _p(a), _p(b)))


def softmax(s) -> np.ndarray:
    s = _f64(s)
    p = np.empty_like(s)
    lib().mla_oracle_softmax(s.size, _p(s), _p(p))
    return p


# --------------------------------------------------------------------------
# Absorbed-form steps on one head and one query
# --------------------------------------------------------------------------
def absorb_query(w_uk_i, q) -> np.ndarray:
    """q_abs = W_UK_i^T q."""
    W = _f64(w_uk_i); q = _f64(q)
    d_h, d_c = W.shape
    out = np.empty(d_c)
    lib().mla_oracle_absorb_query(d_h, d_c, _p(W), _p(q), _p(out))
    return out


def latent_scores(q_abs, q_r, C, KR, scale) -> np.ndarray:
    """s_t = scale * (q_abs . C[t] + q_r . KR[t])."""
    qa = _f64(q_abs); C = _f64(C)
    n, d_c = C.shape
    if KR is None or q_r is None:
        d_r = 0
        qr = np.zeros(1); KRa = np.zeros(1)
    else:
        qr = _f64(q_r); KRa = _f64(KR)
        d_r = KRa.shape[1]
    s = np.empty(n)
    lib().mla_oracle_latent_scores(n, d_c, d_r, float(scale), _p(qa), _p(qr), _p(C), _p(KRa), _p(s))
    return s


def weighted_latent(p, C) -> np.ndarray:
    """c_bar = sum_t p_t C[t]."""
    p = _f64(p); C = _f64(C)
    n, d_c = C.shape
    out = np.empty(d_c)
    lib().mla_oracle_weighted_latent(n, d_c, _p(p), _p(C), _p(out))
    return out


def up_project(w_uv_i, c_bar) -> np.ndarray:
    """o = W_UV_i c_bar."""
    W = _f64(w_uv_i); c = _f64(c_bar)
    d_h, d_c = W.shape
    out = np.empty(d_h)
    lib().mla_oracle_up_project(d_h, d_c, _p(W), _p(c), _p(out))
    return out


def output_project(o, w_o) -> np.ndarray:
    """u = [o_1; ...; o_h] W^O per query row.  ``o`` holds head outputs
    [..., h, d_h] (as the decode step returns them); each row's heads are
    concatenated head after head into k = h * d_h values.  ``w_o`` is the
    pages' k x d matrix.  Returns [..., d]."""
    W = _f64(w_o)
    k, d = W.shape
    o = _f64(o)
    if o.ndim < 2 or o.shape[-2] * o.shape[-1] != k:
        raise ValueError("o must be [..., h, d_h] with h * d_h = %d" % k)
    lead = o.shape[:-2]
    rows_arr = np.ascontiguousarray(o.reshape(-1, k))
    out = np.empty((rows_arr.shape[0], d))
    lib().mla_oracle_output_project(rows_arr.shape[0], k, d, _p(rows_arr), _p(W), _p(out))
    return out.reshape(tuple(lead) + (d,))


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def rope_thetas(d: int, base: float = 10000.0) -> np.ndarray:
    """theta_j = base^(-2 j / d), j = 0 .. d/2 - 1."""
    out = np.empty(d // 2)
    lib().mla_oracle_rope_thetas(d, float(base), _p(out))
    return out


def rope(x, t, theta) -> np.ndarray:
    """RoPE of the d-vector x at position t (adjacent pairs)."""
    x = _f64(x); th = _f64(theta)
    assert x.ndim == 1 and x.size % 2 == 0 and th.size == x.size // 2
    y = np.empty_like(x)
    lib().mla_oracle_rope(x.size, _p(x), float(t), _p(th), _p(y))
    return y


def cache_append(x, w_dkv, w_kr, seq, pos, theta, page_table, page_size, latent_pool, rope_pool):
    """Write c = W_DKV x and k_R = RoPE(W_KR x, pos) of each new token into
    the pools (copies of the given pools are returned, the inputs are left
    alone).  x [n][d_model]; w_dkv [d_c][d_model]; w_kr [d_r][d_model];
    seq, pos [n]; pools [num_pages][page_size][d_c | d_r]."""
    x = _f64(x); Wc = _f64(w_dkv); Wr = _f64(w_kr); th = _f64(theta)
    n, d_model = x.shape
    d_c, d_r = Wc.shape[0], Wr.shape[0]
    table = _i32(page_table)
    lat = np.array(latent_pool, dtype=np.float64, order="C", copy=True)
    rp = np.array(rope_pool, dtype=np.float64, order="C", copy=True)
    sq, ps = _i32(seq), _i32(pos)
    rc = lib().mla_oracle_cache_append(n, d_model, d_c, d_r, _p(x), _p(Wc), _p(Wr),
                                       sq.ctypes.data_as(_ip), ps.ctypes.data_as(_ip), _p(th),
                                       table.ctypes.data_as(_ip), table.shape[1], int(page_size), lat.shape[0],
                                       _p(lat), _p(rp))
    if rc != 0:
        raise ValueError("a row's page lies outside the page table or the pool")
    return lat, rp


def query_project(x, w_dq, w_uq, w_qr, pos, theta):
    """q [n][h][d_h] and q_R [n][h][d_r] of n query rows: c_Q = W_DQ x,
    q_i = W_UQ[i] c_Q, q_R,i = RoPE(W_QR[i] c_Q, pos)."""
    x = _f64(x); Wd = _f64(w_dq); Wu = _f64(w_uq); Wr = _f64(w_qr); th = _f64(theta)
    n, d_model = x.shape
    d_qc = Wd.shape[0]
    h, d_h = Wu.shape[:2]
    d_r = Wr.shape[1]
    q = np.empty((n, h, d_h)); q_r = np.empty((n, h, d_r))
    ps = _i32(pos)
    lib().mla_oracle_query_project(n, d_model, d_qc, h, d_h, d_r, _p(x), _p(Wd), _p(Wu), _p(Wr),
                                   ps.ctypes.data_as(_ip), _p(th), _p(q), _p(q_r))
    return q, q_r


# --------------------------------------------------------------------------
# Whole decode step
# --------------------------------------------------------------------------
@dataclass
class Problem:
    """Decode inputs in fp64 (bf16 and fp32 values widen to fp64 exactly).

    Shapes: q [B, n_q, h, d_h]; q_r [B, n_q, h, d_r]; latent_pool
    [P, page_size, d_c]; rope_pool [P, page_size, d_r]; page_table
    [B, max_pages] int32; context_lens [B] int32; w_uk, w_uv [h, d_h, d_c].
    """
    q: np.ndarray
    q_r: np.ndarray
    latent_pool: np.ndarray
    rope_pool: np.ndarray
    page_table: np.ndarray
    context_lens: np.ndarray
    w_uk: np.ndarray
    w_uv: np.ndarray
    scale: float

    def _struct(self):
        self.q = _f64(self.q); self.q_r = _f64(self.q_r)
        self.latent_pool = _f64(self.latent_pool); self.rope_pool = _f64(self.rope_pool)
        self.w_uk = _f64(self.w_uk); self.w_uv = _f64(self.w_uv)
        self.page_table = np.ascontiguousarray(self.page_table, dtype=np.int32)
        self.context_lens = np.ascontiguousarray(self.context_lens, dtype=np.int32)
        B, n_q, h, d_h = self.q.shape
        P, page_size, d_c = self.latent_pool.shape
        d_r = self.q_r.shape[3]
        if self.q_r.shape[:3] != (B, n_q, h):
            raise ValueError("q_r shape")
        if self.rope_pool.shape != (P, page_size, d_r):
            raise ValueError("rope_pool shape")
        if self.w_uk.shape != (h, d_h, d_c) or self.w_uv.shape != (h, d_h, d_c):
            raise ValueError("weight shape")
        if self.page_table.ndim != 2 or self.page_table.shape[0] != B or self.context_lens.shape != (B,):
            raise ValueError("page table / lengths shape")
        # a zero-size rope buffer still needs a valid pointer
        qr = self.q_r if self.q_r.size else np.zeros(1)
        rp = self.rope_pool if self.rope_pool.size else np.zeros(1)
        self._keep = (qr, rp)
        return _Problem(B, n_q, h, d_c, d_r, d_h, page_size, self.page_table.shape[1], P, 0,
                        float(self.scale), _p(self.q), _p(qr), _p(self.latent_pool), _p(rp),
                        self.page_table.ctypes.data_as(_ip), self.context_lens.ctypes.data_as(_ip),
                        _p(self.w_uk), _p(self.w_uv))


def _selection(prob: Problem, pairs):
    B, _, h, _ = np.asarray(prob.q).shape
    if pairs is None:
        pairs = [(b, i) for b in range(B) for i in range(h)]
    pairs = np.asarray(pairs, dtype=np.int32).reshape(-1, 2)
    return (np.ascontiguousarray(pairs[:, 0]), np.ascontiguousarray(pairs[:, 1]), len(pairs))


def decode_explicit(prob: Problem, pairs=None) -> np.ndarray:
    """Explicit-K/V decode.  Returns [B, n_q, h, d_h] when ``pairs`` is None,
    else [len(pairs), n_q, d_h] for the listed (sequence, head) pairs."""
    S = prob._struct()
    sb, sh, n = _selection(prob, pairs)
    B, n_q, h, d_h = prob.q.shape
    out = np.empty((n, n_q, d_h))
    rc = lib().mla_oracle_decode_explicit(ctypes.byref(S), n, sb.ctypes.data_as(_ip),
                                          sh.ctypes.data_as(_ip), _p(out))
    if rc != 0:
        raise ValueError("oracle rejected the problem (code %d)" % rc)
    if pairs is None:
        return out.reshape(B, h, n_q, d_h).transpose(0, 2, 1, 3).copy()
    return out


def decode_absorbed(prob: Problem, pairs=None, return_cbar: bool = False):
    """Absorbed-form decode; same output layout as :func:`decode_explicit`.
    With ``return_cbar`` also returns the softmax-weighted latents."""
    S = prob._struct()
    sb, sh, n = _selection(prob, pairs)
    B, n_q, h, d_h = prob.q.shape
    d_c = prob.latent_pool.shape[2]
    out = np.empty((n, n_q, d_h))
    cb = np.empty((n, n_q, d_c))
    rc = lib().mla_oracle_decode_absorbed(ctypes.byref(S), n, sb.ctypes.data_as(_ip),
                                          sh.ctypes.data_as(_ip), _p(out), _p(cb))
    if rc != 0:
        raise ValueError("oracle rejected the problem (code %d)" % rc)
    if pairs is None:
        out = out.reshape(B, h, n_q, d_h).transpose(0, 2, 1, 3).copy()
        cb = cb.reshape(B, h, n_q, d_c).transpose(0, 2, 1, 3).copy()
    return (out, cb) if return_cbar else out


def prefill(latent, rope, q, q_r, w_uk, w_uv, scale=None, heads=None) -> np.ndarray:
    """Causal attention over a prompt of T tokens in the explicit form (keys
    and values rebuilt per head): the explicit decode with all T tokens as
    new query tokens (query t sees tokens 0 .. t).  latent [T][d_c], rope
    [T][d_r], q [T][h][d_h], q_r [T][h][d_r]; returns [T][h][d_h], or
    [T][len(heads)][d_h] for the listed heads."""
    latent = _f64(latent); rope = _f64(rope); q = _f64(q); q_r = _f64(q_r)
    T, h, d_h = q.shape
    d_r = q_r.shape[2]
    prob = Problem(q=q[None], q_r=q_r[None], latent_pool=latent[None], rope_pool=rope[None],
                   page_table=np.zeros((1, 1), np.int32), context_lens=np.array([T], np.int32),
                   w_uk=w_uk, w_uv=w_uv, scale=(1.0 / np.sqrt(d_h + d_r)) if scale is None else scale)
    if heads is None:
        return decode_explicit(prob)[0]
    out = decode_explicit(prob, [(0, int(i)) for i in heads])  # [len(heads)][T][d_h]
    return np.ascontiguousarray(out.transpose(1, 0, 2))


def gather(prob: Problem, b: int, n: int):
    """Logical cache rows of sequence b: (C [n, d_c], KR [n, d_r])."""
    S = prob._struct()
    d_c = prob.latent_pool.shape[2]
    d_r = prob.rope_pool.shape[2]
    C = np.empty((n, d_c)); KR = np.empty((n, max(d_r, 1)))
    lib().mla_oracle_gather(ctypes.byref(S), b, n, _p(C), _p(KR))
    return C, KR[:, :d_r]


def num_threads() -> int:
    return int(lib().mla_oracle_num_threads())


def set_num_threads(n: int) -> None:
    """OpenMP threads of later oracle calls (timing only; results do not depend on it)."""
    lib().mla_oracle_set_num_threads(int(n))
