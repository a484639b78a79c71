"""ctypes binding of ``libmla_decode.so`` (C ABI in ``include/mla_decode.h``).

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the HIP stream, statuses become exceptions.  Every step of the
decode runs in the library's HIP kernels; there is no fallback of any kind,
and loading fails loudly when the library has not been built.

The functions carry the C names (``mla_decode_create``, ``mla_decode_run``,
...); :class:`MLADecode` is a small convenience wrapper around them.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla_decode.so")

MLA_OK = 0
MLA_ERR_INVALID_ARG = -1
MLA_ERR_UNSUPPORTED = -2
MLA_ERR_WORKSPACE = -3
MLA_ERR_HIP = -4
MLA_ERR_NOMEM = -5

MLA_DTYPE_BF16 = 0
MLA_DTYPE_F32 = 1
_DTYPE = {"bf16": MLA_DTYPE_BF16, "f32": MLA_DTYPE_F32}

EXPORTED = ("mla_decode_create", "mla_decode_workspace_size", "mla_decode_split_plan",
            "mla_decode_run", "mla_decode_run_static", "mla_decode_enable_timing",
            "mla_decode_read_timing", "mla_decode_read_timing_runs", "mla_decode_destroy",
            "mla_decode_last_error", "mla_oproj_workspace_size", "mla_oproj_run",
            "mla_cache_append_workspace_size", "mla_cache_append_run",
            "mla_query_project_workspace_size", "mla_query_project_run",
            "mla_token_project_workspace_size", "mla_token_project_run",
            "mla_prefill_workspace_size", "mla_prefill_run")

KERNELS = ("q_absorb", "split_attn", "combine", "up_project")


class MLAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("mla_decode status %d: %s" % (status, message))
        self.status = status


class Config(ctypes.Structure):
    """Mirror of ``mla_decode_config_t``."""
    _fields_ = [
        ("h", ctypes.c_int32), ("d_c", ctypes.c_int32), ("d_r", ctypes.c_int32),
        ("d_h", ctypes.c_int32), ("dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("max_batch", ctypes.c_int32),
        ("max_q_per_seq", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
        ("num_splits", ctypes.c_int32), ("scale", ctypes.c_float),
    ]


_lib = None


def lib():
    """The loaded library.  Raises when it is missing: build it with
    ``python -m mla_latent_cache_absorbed_amd.build``."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmla_decode.so is not built (%s); run "
                               "`python -m mla_latent_cache_absorbed_amd.build`" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.mla_decode_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(vp)]
        L.mla_decode_create.restype = ctypes.c_int
        L.mla_decode_workspace_size.argtypes = [vp, i32, i32, i32]
        L.mla_decode_workspace_size.restype = sz
        L.mla_decode_split_plan.argtypes = [vp, i32, i32, i32, ctypes.POINTER(i32),
                                            ctypes.POINTER(i32)]
        L.mla_decode_split_plan.restype = ctypes.c_int
        L.mla_decode_run.argtypes = [vp, i32, i32, i32, i32] + [vp] * 10 + [sz, vp]
        L.mla_decode_run.restype = ctypes.c_int
        L.mla_decode_run_static.argtypes = [vp, i32, i32, i32, i32] + [vp] * 9 + [vp]
        L.mla_decode_run_static.restype = ctypes.c_int
        L.mla_decode_enable_timing.argtypes = [vp, i32]
        L.mla_decode_enable_timing.restype = ctypes.c_int
        L.mla_decode_read_timing.argtypes = [vp, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(i32)]
        L.mla_decode_read_timing.restype = ctypes.c_int
        L.mla_decode_read_timing_runs.argtypes = [vp, ctypes.POINTER(ctypes.c_float), i32,
                                                  ctypes.POINTER(i32)]
        L.mla_decode_read_timing_runs.restype = ctypes.c_int
        L.mla_oproj_workspace_size.argtypes = [i32, i32, i32, i32]
        L.mla_oproj_workspace_size.restype = sz
        L.mla_oproj_run.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]
        L.mla_oproj_run.restype = ctypes.c_int
        dbl = ctypes.c_double
        L.mla_cache_append_workspace_size.argtypes = [i32] * 5
        L.mla_cache_append_workspace_size.restype = sz
        L.mla_cache_append_run.argtypes = [i32] * 5 + [vp] * 6 + [i32] * 3 + [vp, vp, vp, dbl, vp, sz, vp]
        L.mla_cache_append_run.restype = ctypes.c_int
        L.mla_query_project_workspace_size.argtypes = [i32] * 7
        L.mla_query_project_workspace_size.restype = sz
        L.mla_query_project_run.argtypes = [i32] * 7 + [vp] * 8 + [dbl, vp, sz, vp]
        L.mla_query_project_run.restype = ctypes.c_int
        L.mla_token_project_workspace_size.argtypes = [i32] * 8
        L.mla_token_project_workspace_size.restype = sz
        L.mla_token_project_run.argtypes = [i32] * 8 + [vp] * 9 + [i32] * 3 + [vp] * 5 + [dbl, vp, sz, vp]
        L.mla_token_project_run.restype = ctypes.c_int
        L.mla_prefill_workspace_size.argtypes = [i32] * 4
        L.mla_prefill_workspace_size.restype = sz
        L.mla_prefill_run.argtypes = [i32] * 7 + [ctypes.c_float] + [vp] * 8 + [sz, vp]
        L.mla_prefill_run.restype = ctypes.c_int
        L.mla_decode_destroy.argtypes = [vp]
        L.mla_decode_destroy.restype = None
        L.mla_decode_last_error.argtypes = []
        L.mla_decode_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def mla_decode_last_error() -> str:
    return lib().mla_decode_last_error().decode()


def _check(status: int) -> int:
    if status != MLA_OK:
        raise MLAError(status, mla_decode_last_error())
    return status


def raise_for_status(status: int) -> int:
    """Raise MLAError (with mla_decode_last_error's text) for a failed status
    returned by a direct call of the library; returns the status otherwise."""
    return _check(status)


def make_config(h, d_c, d_r, d_h, dtype="bf16", out_dtype=None, page_size=64, max_batch=1,
                max_q_per_seq=1, max_pages_per_seq=1, num_splits=0, scale=0.0) -> Config:
    code = {"bf16": MLA_DTYPE_BF16, "f32": MLA_DTYPE_F32}
    return Config(h, d_c, d_r, d_h, code[dtype], -1 if out_dtype is None else code[out_dtype],
                  page_size, max_batch, max_q_per_seq, max_pages_per_seq, num_splits, float(scale))


def mla_decode_create(cfg: Config) -> ctypes.c_void_p:
    plan = ctypes.c_void_p()
    _check(lib().mla_decode_create(ctypes.byref(cfg), ctypes.byref(plan)))
    return plan


def mla_decode_workspace_size(plan, batch: int, n_q: int, max_context_len: int) -> int:
    return int(lib().mla_decode_workspace_size(plan, batch, n_q, max_context_len))


def mla_decode_split_plan(plan, batch: int, n_q: int, max_context_len: int):
    s, c = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().mla_decode_split_plan(plan, batch, n_q, max_context_len, ctypes.byref(s),
                                       ctypes.byref(c)))
    return s.value, c.value


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def mla_decode_run(plan, batch, n_q, max_context_len, num_pages, q, q_r, latent_pool,
                   rope_pool, page_table, context_lens, w_uk, w_uv, out, workspace,
                   workspace_bytes=None, stream=None) -> int:
    """Enqueue one decode step.  Tensor arguments may be torch tensors (their
    ``data_ptr()`` is passed) or raw integer device addresses.  ``stream``
    defaults to torch's current stream on the current device."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    return _check(lib().mla_decode_run(
        plan, batch, n_q, max_context_len, num_pages, _ptr(q), _ptr(q_r), _ptr(latent_pool),
        _ptr(rope_pool), _ptr(page_table), _ptr(context_lens), _ptr(w_uk), _ptr(w_uv),
        _ptr(out), _ptr(workspace), workspace_bytes, stream))


def mla_decode_run_static(plan, batch, n_q, max_context_len, num_pages, q, q_r, latent_pool,
                          rope_pool, page_table, context_lens, w_uk, w_uv, out, stream=None) -> int:
    """Enqueue one decode step with the library's static per-GPU scratch
    instead of a caller workspace (for callers that cannot allocate)."""
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    return _check(lib().mla_decode_run_static(
        plan, batch, n_q, max_context_len, num_pages, _ptr(q), _ptr(q_r), _ptr(latent_pool),
        _ptr(rope_pool), _ptr(page_table), _ptr(context_lens), _ptr(w_uk), _ptr(w_uv),
        _ptr(out), stream))


def mla_decode_enable_timing(plan, max_runs: int) -> None:
    _check(lib().mla_decode_enable_timing(plan, max_runs))


def mla_decode_read_timing(plan):
    """(per-kernel summed milliseconds as a dict, number of recorded runs)."""
    ms = (ctypes.c_float * len(KERNELS))()
    runs = ctypes.c_int32()
    _check(lib().mla_decode_read_timing(plan, ms, ctypes.byref(runs)))
    return dict(zip(KERNELS, [float(x) for x in ms])), runs.value


def mla_decode_read_timing_runs(plan, max_runs: int):
    """Per-run milliseconds of each step: a list of dicts (one per recorded
    run, at most max_runs)."""
    ms = (ctypes.c_float * (len(KERNELS) * max(1, max_runs)))()
    runs = ctypes.c_int32()
    _check(lib().mla_decode_read_timing_runs(plan, ms, max_runs, ctypes.byref(runs)))
    n = len(KERNELS)
    return [dict(zip(KERNELS, [float(x) for x in ms[r * n:(r + 1) * n]])) for r in range(runs.value)]


def mla_oproj_workspace_size(rows: int, k: int, d_model: int, dtype: str = "bf16") -> int:
    return int(lib().mla_oproj_workspace_size(rows, k, d_model, _DTYPE[dtype]))


def mla_oproj_run(rows, k, d_model, o, w_o, u, workspace=None, workspace_bytes=None, dtype="bf16",
                  out_dtype=None, stream=None) -> int:
    """Enqueue the output projection u = [o_1; ...; o_h] W^O of ``rows`` query
    rows (``w_o`` is W^O transposed, [d_model][k]).  Tensors or raw device
    addresses; ``stream`` defaults to torch's current stream."""
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None or isinstance(workspace, int) else \
            workspace.numel() * workspace.element_size()
    if stream is None:
        import torch
        stream = torch.cuda.current_stream().cuda_stream
    elif not isinstance(stream, int):
        stream = stream.cuda_stream
    return _check(lib().mla_oproj_run(rows, k, d_model, _DTYPE[dtype],
                                      -1 if out_dtype is None else _DTYPE[out_dtype], _ptr(o), _ptr(w_o),
                                      _ptr(u), _ptr(workspace), workspace_bytes, stream))


class OutputProjection:
    """u = [o_1; ...; o_h] W^O on torch tensors: checks shapes, dtypes and
    placement, keeps a workspace, and calls mla_oproj_run."""

    def __init__(self, k, d_model, dtype="bf16", out_dtype=None):
        self.k, self.d = int(k), int(d_model)
        self.dtype, self.out_dtype = dtype, out_dtype or dtype
        self._ws = None

    def workspace(self, rows, device="cuda"):
        import torch
        need = mla_oproj_workspace_size(rows, self.k, self.d, self.dtype)
        if need == 0:
            return None
        if self._ws is None or self._ws.numel() < need or self._ws.device != torch.device(device):
            self._ws = torch.empty(need, dtype=torch.uint8, device=device)
        return self._ws

    def run(self, o, w_o, u, stream=None):
        import torch
        tdt = {"bf16": torch.bfloat16, "f32": torch.float32}
        rows = o.numel() // self.k if o.numel() else 0
        for name, t, shape, dt in (("o", o, None, tdt[self.dtype]), ("w_o", w_o, (self.d, self.k), tdt[self.dtype]),
                                   ("u", u, None, tdt[self.out_dtype])):
            if t.dtype != dt or not t.is_cuda or not t.is_contiguous():
                raise ValueError("%s must be a contiguous CUDA tensor of %s" % (name, dt))
            if shape is not None and tuple(t.shape) != shape:
                raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), shape))
        if o.numel() != rows * self.k or u.numel() != rows * self.d:
            raise ValueError("o must hold rows x k and u rows x d_model values")
        ws = self.workspace(rows, o.device)
        return mla_oproj_run(rows, self.k, self.d, o, w_o, u, ws, dtype=self.dtype, out_dtype=self.out_dtype,
                             stream=stream)


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _nbytes(t):
    return 0 if t is None or isinstance(t, int) else t.numel() * t.element_size()


def mla_cache_append_workspace_size(rows, d_model, d_c, d_r, dtype="bf16") -> int:
    return int(lib().mla_cache_append_workspace_size(rows, d_model, d_c, d_r, _DTYPE[dtype]))


def mla_cache_append_run(rows, d_model, d_c, d_r, x, w_dkv, w_kr, seq, pos, page_table, max_pages_per_seq,
                         page_size, num_pages, latent_pool, rope_pool, rope_theta=None, rope_base=10000.0,
                         workspace=None, workspace_bytes=None, dtype="bf16", stream=None) -> int:
    """Write c = W_DKV x and k_R = RoPE(W_KR x, pos) of each new token into
    its pool rows (tensors or raw device addresses)."""
    if workspace_bytes is None:
        workspace_bytes = _nbytes(workspace)
    return _check(lib().mla_cache_append_run(
        rows, d_model, d_c, d_r, _DTYPE[dtype], _ptr(x), _ptr(w_dkv), _ptr(w_kr), _ptr(seq), _ptr(pos),
        _ptr(page_table), max_pages_per_seq, page_size, num_pages, _ptr(latent_pool), _ptr(rope_pool),
        _ptr(rope_theta), float(rope_base), _ptr(workspace), workspace_bytes, _stream(stream)))


def mla_query_project_workspace_size(rows, d_model, d_qc, h, d_h, d_r, dtype="bf16") -> int:
    return int(lib().mla_query_project_workspace_size(rows, d_model, d_qc, h, d_h, d_r, _DTYPE[dtype]))


def mla_query_project_run(rows, d_model, d_qc, h, d_h, d_r, x, w_dq, w_uq, w_qr, pos, q, q_r, rope_theta=None,
                          rope_base=10000.0, workspace=None, workspace_bytes=None, dtype="bf16",
                          stream=None) -> int:
    """q = W_UQ (W_DQ x) per head and q_R = RoPE(W_QR (W_DQ x), pos) of each
    query row (tensors or raw device addresses)."""
    if workspace_bytes is None:
        workspace_bytes = _nbytes(workspace)
    return _check(lib().mla_query_project_run(
        rows, d_model, d_qc, h, d_h, d_r, _DTYPE[dtype], _ptr(x), _ptr(w_dq), _ptr(w_uq), _ptr(w_qr), _ptr(pos),
        _ptr(q), _ptr(q_r), _ptr(rope_theta), float(rope_base), _ptr(workspace), workspace_bytes,
        _stream(stream)))


def mla_token_project_workspace_size(rows, d_model, d_c, d_r, d_qc, h, d_h, dtype="bf16") -> int:
    return int(lib().mla_token_project_workspace_size(rows, d_model, d_c, d_r, d_qc, h, d_h, _DTYPE[dtype]))


def mla_token_project_run(rows, d_model, d_c, d_r, d_qc, h, d_h, x, w_dkv, w_kr, w_dq, w_uq, w_qr, seq, pos,
                          page_table, max_pages_per_seq, page_size, num_pages, latent_pool, rope_pool, q, q_r,
                          rope_theta=None, rope_base=10000.0, workspace=None, workspace_bytes=None, dtype="bf16",
                          stream=None) -> int:
    """The cache append and the query side of the same rows in one call
    (tensors or raw device addresses)."""
    if workspace_bytes is None:
        workspace_bytes = _nbytes(workspace)
    return _check(lib().mla_token_project_run(
        rows, d_model, d_c, d_r, d_qc, h, d_h, _DTYPE[dtype], _ptr(x), _ptr(w_dkv), _ptr(w_kr), _ptr(w_dq),
        _ptr(w_uq), _ptr(w_qr), _ptr(seq), _ptr(pos), _ptr(page_table), max_pages_per_seq, page_size, num_pages,
        _ptr(latent_pool), _ptr(rope_pool), _ptr(q), _ptr(q_r), _ptr(rope_theta), float(rope_base), _ptr(workspace),
        workspace_bytes, _stream(stream)))


def _device_workspace(nbytes, device):
    import torch
    return None if nbytes == 0 else torch.empty(nbytes, dtype=torch.uint8, device=device)


class CacheAppend:
    """The cache append of a step on torch tensors (shape, dtype and
    placement checks, a workspace, then mla_cache_append_run)."""

    def __init__(self, d_model, d_c, d_r, dtype="bf16", rope_base=10000.0, rope_theta=None):
        self.d_model, self.d_c, self.d_r, self.dtype = int(d_model), int(d_c), int(d_r), dtype
        self.rope_base, self.rope_theta = float(rope_base), rope_theta

    def run(self, x, w_dkv, w_kr, seq, pos, page_table, latent_pool, rope_pool, stream=None):
        import torch
        dt = {"bf16": torch.bfloat16, "f32": torch.float32}[self.dtype]
        rows = x.shape[0]
        checks = (("x", x, (rows, self.d_model), dt), ("w_dkv", w_dkv, (self.d_c, self.d_model), dt),
                  ("w_kr", w_kr, (self.d_r, self.d_model), dt), ("seq", seq, (rows,), torch.int32),
                  ("pos", pos, (rows,), torch.int32), ("page_table", page_table, None, torch.int32),
                  ("latent_pool", latent_pool, None, dt), ("rope_pool", rope_pool, None, dt))
        for name, t, shape, want in checks:
            if t.dtype != want or not t.is_cuda or not t.is_contiguous():
                raise ValueError("%s must be a contiguous CUDA tensor of %s" % (name, want))
            if shape is not None and tuple(t.shape) != shape:
                raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), shape))
        num_pages, page_size = latent_pool.shape[0], latent_pool.shape[1]
        if tuple(latent_pool.shape) != (num_pages, page_size, self.d_c) or \
                tuple(rope_pool.shape) != (num_pages, page_size, self.d_r) or page_table.dim() != 2:
            raise ValueError("pools must be [num_pages][page_size][d_c | d_r] and page_table 2-D")
        ws = _device_workspace(mla_cache_append_workspace_size(rows, self.d_model, self.d_c, self.d_r, self.dtype),
                               x.device)
        return mla_cache_append_run(rows, self.d_model, self.d_c, self.d_r, x, w_dkv, w_kr, seq, pos, page_table,
                                    page_table.shape[1], page_size, num_pages, latent_pool, rope_pool,
                                    self.rope_theta, self.rope_base, ws, dtype=self.dtype, stream=stream)


class QueryProjection:
    """The query side of a step on torch tensors (checks, a workspace, then
    mla_query_project_run)."""

    def __init__(self, d_model, d_qc, h, d_h, d_r, dtype="bf16", rope_base=10000.0, rope_theta=None):
        self.d_model, self.d_qc, self.h, self.d_h, self.d_r = int(d_model), int(d_qc), int(h), int(d_h), int(d_r)
        self.dtype, self.rope_base, self.rope_theta = dtype, float(rope_base), rope_theta

    def run(self, x, w_dq, w_uq, w_qr, pos, q, q_r, stream=None):
        import torch
        dt = {"bf16": torch.bfloat16, "f32": torch.float32}[self.dtype]
        rows = x.shape[0]
        checks = (("x", x, (rows, self.d_model), dt), ("w_dq", w_dq, (self.d_qc, self.d_model), dt),
                  ("w_uq", w_uq, (self.h, self.d_h, self.d_qc), dt), ("w_qr", w_qr, (self.h, self.d_r, self.d_qc), dt),
                  ("pos", pos, (rows,), torch.int32), ("q", q, None, dt), ("q_r", q_r, None, dt))
        for name, t, shape, want in checks:
            if t.dtype != want or not t.is_cuda or not t.is_contiguous():
                raise ValueError("%s must be a contiguous CUDA tensor of %s" % (name, want))
            if shape is not None and tuple(t.shape) != shape:
                raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), shape))
        if q.numel() != rows * self.h * self.d_h or q_r.numel() != rows * self.h * self.d_r:
            raise ValueError("q must hold rows x h x d_h and q_r rows x h x d_r values")
        ws = _device_workspace(mla_query_project_workspace_size(rows, self.d_model, self.d_qc, self.h, self.d_h,
                                                                self.d_r, self.dtype), x.device)
        return mla_query_project_run(rows, self.d_model, self.d_qc, self.h, self.d_h, self.d_r, x, w_dq, w_uq, w_qr,
                                     pos, q, q_r, self.rope_theta, self.rope_base, ws, dtype=self.dtype,
                                     stream=stream)


def mla_prefill_workspace_size(T, h, d_h, dtype="bf16") -> int:
    return int(lib().mla_prefill_workspace_size(T, h, d_h, _DTYPE[dtype]))


def mla_prefill_run(T, h, d_c, d_r, d_h, latent, rope, q, q_r, w_uk, w_uv, out, workspace, workspace_bytes=None,
                    dtype="bf16", out_dtype=None, scale=0.0, stream=None) -> int:
    """Causal attention over a prompt of T tokens with K and V rebuilt from
    the latents (tensors or raw device addresses)."""
    if workspace_bytes is None:
        workspace_bytes = _nbytes(workspace)
    return _check(lib().mla_prefill_run(T, h, d_c, d_r, d_h, _DTYPE[dtype],
                                        -1 if out_dtype is None else _DTYPE[out_dtype], float(scale), _ptr(latent),
                                        _ptr(rope), _ptr(q), _ptr(q_r), _ptr(w_uk), _ptr(w_uv), _ptr(out),
                                        _ptr(workspace), workspace_bytes, _stream(stream)))


class Prefill:
    """Prefill attention on torch tensors (checks, a workspace, then
    mla_prefill_run)."""

    def __init__(self, h, d_c, d_r, d_h, dtype="bf16", out_dtype=None, scale=0.0):
        self.h, self.d_c, self.d_r, self.d_h = int(h), int(d_c), int(d_r), int(d_h)
        self.dtype, self.out_dtype, self.scale = dtype, out_dtype or dtype, float(scale)
        self._ws = None

    def run(self, latent, rope, q, q_r, w_uk, w_uv, out, stream=None):
        import torch
        dt = {"bf16": torch.bfloat16, "f32": torch.float32}
        T = latent.shape[0]
        checks = (("latent", latent, (T, self.d_c), dt[self.dtype]), ("rope", rope, (T, self.d_r), dt[self.dtype]),
                  ("q", q, (T, self.h, self.d_h), dt[self.dtype]), ("q_r", q_r, (T, self.h, self.d_r), dt[self.dtype]),
                  ("w_uk", w_uk, (self.h, self.d_h, self.d_c), dt[self.dtype]),
                  ("w_uv", w_uv, (self.h, self.d_h, self.d_c), dt[self.dtype]),
                  ("out", out, (T, self.h, self.d_h), dt[self.out_dtype]))
        for name, t, shape, want in checks:
            if t.dtype != want or not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != shape:
                raise ValueError("%s must be a contiguous CUDA tensor of %s with shape %s" % (name, want, shape))
        need = mla_prefill_workspace_size(T, self.h, self.d_h, self.dtype)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=latent.device)
        return mla_prefill_run(T, self.h, self.d_c, self.d_r, self.d_h, latent, rope, q, q_r, w_uk, w_uv, out,
                               self._ws, dtype=self.dtype, out_dtype=self.out_dtype, scale=self.scale, stream=stream)


def mla_decode_destroy(plan) -> None:
    lib().mla_decode_destroy(plan)


class MLADecode:
    """Owns one plan; checks tensor shapes, dtypes and devices before each run."""

    def __init__(self, h, d_c, d_r, d_h, dtype="bf16", out_dtype=None, page_size=64,
                 max_batch=1, max_q_per_seq=1, max_pages_per_seq=1, num_splits=0, scale=0.0):
        self.cfg = make_config(h, d_c, d_r, d_h, dtype, out_dtype, page_size, max_batch,
                               max_q_per_seq, max_pages_per_seq, num_splits, scale)
        self.dtype = dtype
        self.out_dtype = out_dtype or dtype
        self.plan = mla_decode_create(self.cfg)

    def close(self):
        if self.plan is not None:
            mla_decode_destroy(self.plan)
            self.plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_size(self, batch, n_q, max_context_len) -> int:
        n = mla_decode_workspace_size(self.plan, batch, n_q, max_context_len)
        if n == 0 and batch > 0:
            raise MLAError(MLA_ERR_INVALID_ARG, mla_decode_last_error())
        return n

    def split_plan(self, batch, n_q, max_context_len):
        return mla_decode_split_plan(self.plan, batch, n_q, max_context_len)

    def workspace(self, batch, n_q, max_context_len, device="cuda"):
        import torch
        return torch.empty(max(self.workspace_size(batch, n_q, max_context_len), 256),
                           dtype=torch.uint8, device=device)

    def run(self, q, q_r, latent_pool, rope_pool, page_table, context_lens, w_uk, w_uv, out,
            workspace, max_context_len, stream=None):
        import torch
        c = self.cfg
        tdt = {"bf16": torch.bfloat16, "f32": torch.float32}
        B, n_q, h, d_h = q.shape
        P, ps, d_c = latent_pool.shape
        expect = {
            "q": (q, (B, n_q, c.h, c.d_h), tdt[self.dtype]),
            "q_r": (q_r, (B, n_q, c.h, c.d_r), tdt[self.dtype]),
            "latent_pool": (latent_pool, (P, c.page_size, c.d_c), tdt[self.dtype]),
            "rope_pool": (rope_pool, (P, c.page_size, c.d_r), tdt[self.dtype]),
            "page_table": (page_table, (B, c.max_pages_per_seq), torch.int32),
            "context_lens": (context_lens, (B,), torch.int32),
            "w_uk": (w_uk, (c.h, c.d_h, c.d_c), tdt[self.dtype]),
            "w_uv": (w_uv, (c.h, c.d_h, c.d_c), tdt[self.dtype]),
            "out": (out, (B, n_q, c.h, c.d_h), tdt[self.out_dtype]),
        }
        for name, (t, shape, dt) in expect.items():
            if tuple(t.shape) != shape:
                raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), shape))
            if t.dtype != dt:
                raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dt))
            if not t.is_cuda:
                raise ValueError("%s must be a device tensor" % name)
            if not t.is_contiguous():
                raise ValueError("%s must be contiguous" % name)
        return mla_decode_run(self.plan, B, n_q, max_context_len, P, q, q_r, latent_pool,
                              rope_pool, page_table, context_lens, w_uk, w_uv, out, workspace,
                              stream=stream)
