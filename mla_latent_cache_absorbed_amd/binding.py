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

EXPORTED = ("mla_decode_create", "mla_decode_workspace_size", "mla_decode_split_plan",
            "mla_decode_run", "mla_decode_enable_timing", "mla_decode_read_timing",
            "mla_decode_destroy", "mla_decode_last_error")

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
        L.mla_decode_enable_timing.argtypes = [vp, i32]
        L.mla_decode_enable_timing.restype = ctypes.c_int
        L.mla_decode_read_timing.argtypes = [vp, ctypes.POINTER(ctypes.c_float), ctypes.POINTER(i32)]
        L.mla_decode_read_timing.restype = ctypes.c_int
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


def mla_decode_enable_timing(plan, max_runs: int) -> None:
    _check(lib().mla_decode_enable_timing(plan, max_runs))


def mla_decode_read_timing(plan):
    """(per-kernel summed milliseconds as a dict, number of recorded runs)."""
    ms = (ctypes.c_float * len(KERNELS))()
    runs = ctypes.c_int32()
    _check(lib().mla_decode_read_timing(plan, ms, ctypes.byref(runs)))
    return dict(zip(KERNELS, [float(x) for x in ms])), runs.value


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
