"""Move a seeded workload to the GPU and run the decode through the C ABI.

Marshalling only (numpy -> torch device tensors -> ``binding``); the decode
itself runs in ``libmla_decode.so``.
"""
from __future__ import annotations

import numpy as np

from . import binding
from .inputs import Workload


class DeviceWorkload:
    """Device copies of one workload's tensors plus a plan sized for it."""

    def __init__(self, wl: Workload, device="cuda", num_splits=0, out_dtype=None,
                 max_context_len=None, scale=0.0):
        import torch
        self.wl = wl
        self.device = device
        tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32

        def dev(key):
            a = wl.arrays[key]
            if wl.dtype == "bf16":
                return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
            return torch.from_numpy(a).to(device)

        self.t = {k: dev(k) for k in ("q", "q_r", "latent_pool", "rope_pool", "w_uk", "w_uv")}
        self.t["page_table"] = torch.from_numpy(wl.page_table).to(device)
        self.t["context_lens"] = torch.from_numpy(wl.lens).to(device)
        self.max_len = int(max_context_len or wl.max_len)
        self.out_dtype = out_dtype or wl.dtype
        self.dec = binding.MLADecode(
            wl.h, wl.d_c, wl.d_r, wl.d_h, dtype=wl.dtype, out_dtype=self.out_dtype,
            page_size=wl.page_size, max_batch=max(1, wl.batch), max_q_per_seq=wl.n_q,
            max_pages_per_seq=wl.max_pages, num_splits=num_splits, scale=scale)
        self.ws = self.dec.workspace(wl.batch, wl.n_q, self.max_len, device)
        odt = torch.bfloat16 if self.out_dtype == "bf16" else torch.float32
        self.out = torch.empty((wl.batch, wl.n_q, wl.h, wl.d_h), dtype=odt, device=device)
        self.tdt = tdt

    def split_plan(self):
        return self.dec.split_plan(self.wl.batch, self.wl.n_q, self.max_len)

    def run(self, out=None, stream=None, **override):
        t = dict(self.t)
        t.update(override)
        o = self.out if out is None else out
        self.dec.run(t["q"], t["q_r"], t["latent_pool"], t["rope_pool"], t["page_table"],
                     t["context_lens"], t["w_uk"], t["w_uv"], o, self.ws, self.max_len,
                     stream=stream)
        return o

    def result_f64(self, out=None) -> np.ndarray:
        o = self.out if out is None else out
        return o.float().cpu().numpy().astype(np.float64)
