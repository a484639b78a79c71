"""GPU parity of prefill (attention over a whole prompt, keys and values
rebuilt from the latents, causal) through the C ABI, against the fp64
oracle's explicit form on the same seeded inputs.

- fp32 storage and a small shape on the plain kernels (fp32 tolerance);
- DeepSeek-V2 head shapes (d_c 512, d_r 64, d_h 128) on the MFMA kernels:
  ragged prompt lengths (not multiples of the 32-key or 128-query tiles),
  a head count that is not a multiple of 8, all heads up to T = 1000 and
  sampled heads at T = 4096, bf16 and fp32 outputs.

Tolerance (normwise): 1e-2 for bf16 storage, 1e-5 for fp32."""
import numpy as np
import pytest

import oracle
from mla_latent_cache_absorbed_amd import binding, inputs
from tests._parity import check, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available()
    return t


def _dev(torch, a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _run(torch, case, out_dtype=None):
    dt = case["dtype"]
    out_dtype = out_dtype or dt
    T, h, d_h = case["T"], case["h"], case["d_h"]
    odt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    out = torch.full((T, h, d_h), float("nan"), dtype=odt, device="cuda")
    op = binding.Prefill(h, case["d_c"], case["d_r"], d_h, dt, out_dtype)
    op.run(*(_dev(torch, case[k], dt) for k in ("latent", "rope", "q", "q_r", "w_uk", "w_uv")), out)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def _ref(case, heads=None):
    w = {k: inputs.widen(case[k], case["dtype"]) for k in ("latent", "rope", "q", "q_r", "w_uk", "w_uv")}
    return oracle.prefill(w["latent"], w["rope"], w["q"], w["q_r"], w["w_uk"], w["w_uv"], heads=heads)


def test_fp32_plain_kernels(torch):
    case = inputs.make_prefill(37, h=3, d_c=16, d_r=8, d_h=16, dtype="f32", seed=501)
    check(_run(torch, case), _ref(case), "f32", "prefill fp32 T=37, plain kernels")


@pytest.mark.parametrize("T,h", [(1, 8), (32, 8), (300, 128), (1000, 16), (200, 12)])
def test_mfma_kernels_all_heads(torch, T, h):
    case = inputs.make_prefill(T, h=h, seed=510 + T + h)
    check(_run(torch, case), _ref(case), "bf16", "prefill T=%d h=%d, all heads" % (T, h))


def test_fp32_output(torch):
    case = inputs.make_prefill(257, h=8, seed=520)
    got = _run(torch, case, "f32")
    check(got, _ref(case), "bf16", "prefill T=257 h=8, fp32 output")


def test_long_prompt_sampled_heads(torch):
    case = inputs.make_prefill(4096, h=128, seed=530)
    heads = [0, 77, 127]
    got = _run(torch, case)
    log("prefill T=4096 h=128: checking heads %s" % heads)
    check(got[:, heads], _ref(case, heads), "bf16", "prefill T=4096, heads %s" % heads)


def test_first_token_attends_to_itself_only(torch):
    """Row 0 sees token 0 alone: its output is W_UV[i] c_0 exactly as the
    rebuilt value (a closed form independent of the softmax)."""
    case = inputs.make_prefill(64, h=8, seed=540)
    got = _run(torch, case, "f32")
    lat = inputs.widen(case["latent"], "bf16")
    w_uv = inputs.widen(case["w_uv"], "bf16")
    ref0 = np.stack([w_uv[i] @ lat[0] for i in range(8)])
    check(got[0], ref0, "bf16", "prefill row 0 = W_UV c_0")
