"""mla_decode_run_static, the entry point for callers that cannot allocate:
the same decode step as mla_decode_run with the library's static per-GPU
scratch in place of a caller workspace.

Two calls in a row on one GPU, the second with a smaller input (the scratch
keeps the first call's contents, which the second must not depend on), each
compared bit for bit with mla_decode_run on the same inputs and with the
fp64 oracle at the bf16 tolerance; and the host-side refusal of a call whose
workspace exceeds the static scratch.
"""
import numpy as np
import pytest

import oracle
from mla_latent_cache_absorbed_amd import binding, inputs
from tests._parity import check, problem


def _run_static(dw, out):
    t = dw.t
    binding.mla_decode_run_static(dw.dec.plan, dw.wl.batch, dw.wl.n_q, dw.max_len, dw.wl.num_pages,
                                  t["q"], t["q_r"], t["latent_pool"], t["rope_pool"], t["page_table"],
                                  t["context_lens"], t["w_uk"], t["w_uv"], out)


@pytest.mark.gpu
def test_static_scratch_matches_the_workspace_entry_point():
    import torch
    from mla_latent_cache_absorbed_amd.runner import DeviceWorkload
    # a ragged paged batch (chunks planned on the device), then a smaller
    # two-sequence call with four causal query tokens
    first = inputs.make("ds2_paged_b32", batch=6, lens=("list", [4000, 333, 2049, 64, 7000, 1]), seed=260)
    second = inputs.make("ds2_mtp_b16", batch=2, lens=("list", [300, 45]), shuffled=True, seed=261)
    for wl in (first, second):
        dw = DeviceWorkload(wl)
        dw.run()
        torch.cuda.synchronize()
        ref = dw.out.clone()
        got = torch.full_like(dw.out, float("nan"))
        _run_static(dw, got)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), "%s: static-scratch call differs from the workspace call" % wl.name
        check(got.float().cpu().numpy().astype(np.float64), oracle.decode_absorbed(problem(wl)), "bf16",
              "static scratch, %s B=%d" % (wl.name, wl.batch))


def test_static_scratch_refuses_a_call_beyond_its_size():
    # 1024 query rows of 128 heads: 128 MiB of absorbed queries alone
    cfg = binding.make_config(h=128, d_c=512, d_r=64, d_h=128, dtype="bf16", page_size=64,
                              max_batch=1024, max_q_per_seq=1, max_pages_per_seq=2)
    plan = binding.mla_decode_create(cfg)
    try:
        assert binding.mla_decode_workspace_size(plan, 1024, 1, 128) > 64 << 20
        with pytest.raises(binding.MLAError) as e:
            binding.mla_decode_run_static(plan, 1024, 1, 128, 1, *([None] * 9), stream=0)
        assert e.value.status == binding.MLA_ERR_WORKSPACE
        assert "static scratch" in binding.mla_decode_last_error()
    finally:
        binding.mla_decode_destroy(plan)
