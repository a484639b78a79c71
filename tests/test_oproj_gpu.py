"""GPU parity of the output projection u = [o_1; ...; o_h] W^O (the step
after the decode path) through the C ABI, against the fp64 oracle on the
same seeded inputs: the pages' toy values on the plain fp32 kernel,
DeepSeek-V2 width (k = 16384, d = 5120) on the one-launch few-row kernel
for 1..4 rows and on the MFMA kernels from 5 to 100 rows, an odd shape on the plain bf16 kernel, and the projection of a real
decode step's output.

Tolerance (normwise, as for the decode step): 1e-2 for a bf16 output, 1e-5
for an fp32 output (inputs are exact in fp64, so only the fp32 accumulation
and the output rounding differ)."""
import json
import os

import numpy as np
import pytest

import oracle
from mla_latent_cache_absorbed_amd import binding, inputs
from tests._parity import check, log, problem

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available()
    return t


def _dev(torch, a, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def _project(torch, o, w_pages, dtype, out_dtype, rows, k, d):
    """Run the GPU projection: W^O goes to the device transposed ([d][k])."""
    o_dev = _dev(torch, o.reshape(rows, k), dtype)
    w_dev = _dev(torch, np.ascontiguousarray(w_pages.T), dtype)
    odt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    u = torch.full((rows, d), float("nan"), dtype=odt, device="cuda")
    proj = binding.OutputProjection(k, d, dtype, out_dtype)
    proj.run(o_dev, w_dev, u)
    torch.cuda.synchronize()
    return u, proj, (o_dev, w_dev)


@pytest.mark.parametrize("which", ["with_rope", "content_only"])
def test_p5_toy_output_projection(torch, which):
    """The pages' toy ("From Vanilla Transformers ..." sections 3.h and 3.p):
    W^O is 0/1, so u_4 follows from the printed head outputs exactly."""
    g = json.load(open(os.path.join(ROOT, "tests", "golden", "p5_toy_decode.json")))
    src = g if which == "with_rope" else g["content_only"]
    o = np.asarray(src["o"]["value"], dtype=np.float32)        # [h=2][d_h=2]
    w = np.asarray(g["W_O"]["value"], dtype=np.float32)        # 4 x 5 (k x d)
    u, _, _ = _project(torch, o, w, "f32", "f32", 1, 4, 5)
    got = u.cpu().numpy().astype(np.float64)[0]
    np.testing.assert_allclose(got, src["u4"]["value"], rtol=0, atol=1e-6)


@pytest.mark.parametrize("rows", [1, 2, 3, 4, 5, 32, 64, 100])
@pytest.mark.parametrize("out_dtype", ["bf16", "f32"])
def test_deepseek_v2_width(torch, rows, out_dtype):
    case = inputs.make_oproj(rows, seed=300 + rows)
    k, d = case["k"], case["d"]
    u, _, _ = _project(torch, case["o"], case["w_o"], "bf16", out_dtype, rows, k, d)
    ref = oracle.output_project(inputs.widen(case["o"], "bf16"), inputs.widen(case["w_o"], "bf16"))
    log("oproj rows=%d: %d slices of k" % (rows, binding.mla_oproj_workspace_size(rows, k, d) // max(1, rows * d * 4)))
    check(u.float().cpu().numpy().astype(np.float64), ref, out_dtype, "oproj rows=%d out=%s" % (rows, out_dtype))


@pytest.mark.parametrize("rows,k", [(1, 16384), (1, 32768), (2, 16384), (3, 4096), (4, 4096)])
def test_few_rows_one_launch(torch, rows, k):
    """The one-launch few-row kernel in both of its forms: x read from L2
    (one and two rows) and x staged in LDS (three and four rows of 4096);
    d = 512."""
    case = inputs.make_oproj(rows, h=k // 128, d_h=128, d_model=512, seed=330 + rows + k // 1024)
    assert binding.mla_oproj_workspace_size(rows, k, 512) == 0  # no partials
    for out_dtype in ("bf16", "f32"):
        u, _, _ = _project(torch, case["o"], case["w_o"], "bf16", out_dtype, rows, k, 512)
        ref = oracle.output_project(inputs.widen(case["o"], "bf16"), inputs.widen(case["w_o"], "bf16"))
        check(u.float().cpu().numpy().astype(np.float64), ref, out_dtype,
              "oproj few rows=%d k=%d out=%s" % (rows, k, out_dtype))


def test_odd_shape_takes_the_plain_kernel(torch):
    case = inputs.make_oproj(5, h=5, d_h=40, d_model=70, seed=310)  # k = 200, d = 70
    assert binding.mla_oproj_workspace_size(5, 200, 70) == 0
    u, _, _ = _project(torch, case["o"], case["w_o"], "bf16", "f32", 5, 200, 70)
    ref = oracle.output_project(inputs.widen(case["o"], "bf16"), inputs.widen(case["w_o"], "bf16"))
    check(u.cpu().numpy().astype(np.float64), ref, "f32", "oproj odd shape, plain kernel")


def test_projects_a_decode_step(torch):
    """The decode step's output o [B][n_q][h][d_h] is the projection's input
    as it stands (rows = B n_q)."""
    from mla_latent_cache_absorbed_amd.runner import DeviceWorkload
    wl = inputs.make("ds2_mtp_b16", batch=3, lens=("list", [700, 2049, 64]), seed=311)
    dw = DeviceWorkload(wl)
    dw.run()
    torch.cuda.synchronize()
    rows, k = wl.batch * wl.n_q, wl.h * wl.d_h
    case = inputs.make_oproj(1, seed=312)  # only its W^O is used
    w_pages = case["w_o"]
    proj = binding.OutputProjection(k, case["d"], "bf16", "f32")
    w_dev = _dev(torch, np.ascontiguousarray(w_pages.T), "bf16")
    u = torch.empty((rows, case["d"]), dtype=torch.float32, device="cuda")
    proj.run(dw.out, w_dev, u)
    torch.cuda.synchronize()
    # the oracle projects the GPU's own (bf16) head outputs, and separately the
    # oracle's decode: the first isolates the projection, the second the chain
    o_gpu = dw.result_f64()
    ref_proj = oracle.output_project(o_gpu, inputs.widen(w_pages, "bf16")).reshape(rows, -1)
    check(u.cpu().numpy().astype(np.float64), ref_proj, "f32", "oproj of the GPU decode output")
    ref_chain = oracle.output_project(oracle.decode_absorbed(problem(wl)), inputs.widen(w_pages, "bf16"))
    check(u.cpu().numpy().astype(np.float64), ref_chain.reshape(rows, -1), "bf16", "decode + oproj vs oracle chain")


def test_repeat_runs_are_bitwise_identical(torch):
    case = inputs.make_oproj(64, seed=313)
    u, proj, (o_dev, w_dev) = _project(torch, case["o"], case["w_o"], "bf16", "bf16", 64, case["k"], case["d"])
    first = u.clone()
    for _ in range(3):
        proj.run(o_dev, w_dev, u)
    torch.cuda.synchronize()
    assert torch.equal(first, u)
