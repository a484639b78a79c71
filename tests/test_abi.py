"""The C ABI on the CPU: the library loads, exports every declared symbol,
and rejects bad configurations and calls on the host before any launch."""
import ctypes
import os
import re

import pytest

from mla_latent_cache_absorbed_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla_decode.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        from mla_latent_cache_absorbed_amd import build
        build.build()
    return binding.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_(?:decode|oproj|cache_append|query_project|token_project|prefill)_\w+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert declared_functions() == sorted(binding.EXPORTED)


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_library_loads_without_oracle():
    # the product library must not link anything from oracle/
    import subprocess
    out = subprocess.run(["ldd", binding.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in out


def ds2(**kw):
    base = dict(h=128, d_c=512, d_r=64, d_h=128, dtype="bf16", page_size=64, max_batch=4,
                max_q_per_seq=4, max_pages_per_seq=64)
    base.update(kw)
    return binding.make_config(**base)


def test_create_and_destroy(L):
    plan = binding.mla_decode_create(ds2())
    assert plan.value
    binding.mla_decode_destroy(plan)
    binding.mla_decode_destroy(None)  # NULL is accepted


@pytest.mark.parametrize("bad", [
    dict(h=0), dict(d_c=0), dict(d_h=-1), dict(d_r=-1), dict(page_size=0), dict(max_batch=0),
    dict(max_q_per_seq=0), dict(max_pages_per_seq=0), dict(num_splits=-3), dict(scale=-1.0),
    dict(scale=float("inf")), dict(scale=float("nan")),
])
def test_create_rejects_invalid_config(L, bad):
    with pytest.raises(binding.MLAError) as e:
        binding.mla_decode_create(ds2(**bad))
    assert e.value.status == binding.MLA_ERR_INVALID_ARG
    assert binding.mla_decode_last_error()


def test_create_rejects_unknown_dtype(L):
    cfg = ds2()
    cfg.dtype = 7
    with pytest.raises(binding.MLAError) as e:
        binding.mla_decode_create(cfg)
    assert e.value.status == binding.MLA_ERR_INVALID_ARG
    cfg = ds2()
    cfg.out_dtype = 5
    with pytest.raises(binding.MLAError):
        binding.mla_decode_create(cfg)


def test_create_reports_unsupported_shapes(L):
    with pytest.raises(binding.MLAError) as e:
        binding.mla_decode_create(ds2(d_c=2048, d_r=0))
    assert e.value.status == binding.MLA_ERR_UNSUPPORTED


def test_create_null_arguments(L):
    plan = ctypes.c_void_p()
    assert L.mla_decode_create(None, ctypes.byref(plan)) == binding.MLA_ERR_INVALID_ARG
    assert L.mla_decode_create(ctypes.byref(ds2()), None) == binding.MLA_ERR_INVALID_ARG


def test_workspace_size_and_split_plan(L):
    plan = binding.mla_decode_create(ds2(max_pages_per_seq=2048))
    try:
        for B, n_q, T in [(1, 1, 4096), (1, 1, 131072), (4, 4, 1000), (1, 1, 1), (4, 1, 33)]:
            S, chunk = binding.mla_decode_split_plan(plan, B, n_q, T)
            ws = binding.mla_decode_workspace_size(plan, B, n_q, T)
            R = B * n_q
            target = 256 // (n_q * 2)  # one work-group per CU, two head groups
            if B == 1 or target <= 2 * B:  # one sequence, or few chunks each: fixed
                assert S >= 1 and chunk >= 1
                assert chunk % 32 == 0            # whole LDS tiles on the bf16 path
                assert (S - 1) * chunk < T <= S * chunk
                chunks = B * S
            else:  # several sequences: planned on the device from the lengths
                assert (S, chunk) == (0, 0)
                chunks = max(target, B + -(-B * T // 32768))
            # q_abs (bf16), chunk results (bf16), chunk lse (fp32) per chunk
            # and query token; the fast path merges the chunks straight into
            # the up-projection
            need = R * 128 * 512 * 2 + chunks * n_q * 128 * 512 * 2 + chunks * n_q * 128 * 4
            assert need <= ws <= need + 3 * 256
        assert binding.mla_decode_workspace_size(plan, 0, 1, 10) == 0
        # invalid shapes give 0 and a reason
        assert binding.mla_decode_workspace_size(plan, 5, 1, 10) == 0   # batch > max_batch
        assert "batch" in binding.mla_decode_last_error()
        assert binding.mla_decode_workspace_size(plan, 1, 5, 10) == 0   # n_q > max
        assert binding.mla_decode_workspace_size(plan, 1, 4, 3) == 0    # fewer tokens than queries
        assert binding.mla_decode_workspace_size(plan, 1, 1, 2048 * 64 + 1) == 0  # beyond table
    finally:
        binding.mla_decode_destroy(plan)


def test_forced_split_count(L):
    plan = binding.mla_decode_create(ds2(num_splits=64, max_pages_per_seq=2048))
    try:
        assert binding.mla_decode_split_plan(plan, 1, 1, 131072) == (64, 2048)
        # never more chunks than tiles
        assert binding.mla_decode_split_plan(plan, 1, 1, 40)[0] == 2
    finally:
        binding.mla_decode_destroy(plan)


def test_general_path_split_granularity(L):
    plan = binding.mla_decode_create(binding.make_config(4, 16, 8, 16, dtype="f32",
                                                         page_size=16, max_pages_per_seq=4,
                                                         num_splits=3))
    try:
        assert binding.mla_decode_split_plan(plan, 1, 1, 64) == (3, 22)
    finally:
        binding.mla_decode_destroy(plan)


def test_run_rejects_bad_calls_before_launch(L):
    plan = binding.mla_decode_create(ds2())
    fake = 1 << 20  # any aligned non-null address: never dereferenced on these paths
    args = dict(q=fake, q_r=fake, latent_pool=fake, rope_pool=fake, page_table=fake,
                context_lens=fake, w_uk=fake, w_uv=fake, out=fake, workspace=fake)

    def run(batch=1, n_q=1, T=100, num_pages=2, ws_bytes=1 << 30, **kw):
        a = dict(args)
        a.update(kw)
        return L.mla_decode_run(plan, batch, n_q, T, num_pages, a["q"], a["q_r"],
                                a["latent_pool"], a["rope_pool"], a["page_table"],
                                a["context_lens"], a["w_uk"], a["w_uv"], a["out"],
                                a["workspace"], ws_bytes, None)
    try:
        assert run(batch=0) == binding.MLA_OK  # empty batch: nothing to do
        assert run(batch=-1) == binding.MLA_ERR_INVALID_ARG
        assert run(batch=5) == binding.MLA_ERR_INVALID_ARG
        assert run(n_q=0) == binding.MLA_ERR_INVALID_ARG
        assert run(T=0) == binding.MLA_ERR_INVALID_ARG
        assert run(T=64 * 64 + 1) == binding.MLA_ERR_INVALID_ARG
        assert run(num_pages=0) == binding.MLA_ERR_INVALID_ARG
        for key in args:
            assert run(**{key: None}) == binding.MLA_ERR_INVALID_ARG, key
        assert run(q=fake + 2) == binding.MLA_ERR_INVALID_ARG          # misaligned bf16 tensor
        assert run(workspace=fake + 16) == binding.MLA_ERR_INVALID_ARG  # workspace alignment
        assert run(ws_bytes=1000) == binding.MLA_ERR_WORKSPACE
        assert "workspace" in binding.mla_decode_last_error()
        assert L.mla_decode_run(None, 1, 1, 10, 1, *([fake] * 10), 1 << 30, None) == \
            binding.MLA_ERR_INVALID_ARG
    finally:
        binding.mla_decode_destroy(plan)


def test_last_error_cleared_by_success(L):
    with pytest.raises(binding.MLAError):
        binding.mla_decode_create(ds2(h=0))
    assert binding.mla_decode_last_error() != ""
    plan = binding.mla_decode_create(ds2())
    assert binding.mla_decode_last_error() == ""
    binding.mla_decode_destroy(plan)


def test_output_projection_refuses_bad_calls_on_the_host(L):
    # before any launch: bad sizes, unknown dtype, NULL tensors, missing workspace
    assert binding.mla_oproj_workspace_size(8, 16384, 5120) == 16 * 8 * 5120 * 4  # 16 slices of k
    # one launch, no partials: up to 4 rows whose x fits 40 KB of LDS, or up
    # to 2 rows of any length (x from L2)
    assert binding.mla_oproj_workspace_size(2, 16384, 5120) == 0
    assert binding.mla_oproj_workspace_size(4, 4096, 5120) == 0
    assert binding.mla_oproj_workspace_size(3, 16384, 5120) == 16 * 3 * 5120 * 4  # 96 KB of x: slices
    assert binding.mla_oproj_workspace_size(1, 64, 40, "f32") == 0           # plain kernel, no partials
    with pytest.raises(binding.MLAError) as e:
        binding.mla_oproj_run(1, 0, 5, None, None, None, stream=0)
    assert e.value.status == binding.MLA_ERR_INVALID_ARG
    with pytest.raises(binding.MLAError) as e:
        binding.mla_oproj_run(1, 16384, 5120, None, None, None, stream=0)
    assert e.value.status == binding.MLA_ERR_INVALID_ARG
    with pytest.raises(binding.MLAError) as e:
        binding.mla_oproj_run(8, 16384, 5120, 4096, 4096, 4096, stream=0)
    assert e.value.status == binding.MLA_ERR_WORKSPACE
    assert "2621440 needed" in binding.mla_decode_last_error()
    assert binding.mla_oproj_run(0, 16384, 5120, None, None, None, stream=0) == binding.MLA_OK  # nothing to do


def test_projections_refuse_bad_calls_on_the_host(L):
    # cache append: 9 MFMA blocks of 64 features, k = 5120 in 10 slices;
    # up to 4 rows one launch without partials
    assert binding.mla_cache_append_workspace_size(8, 5120, 512, 64) == 10 * 8 * 576 * 4
    assert binding.mla_cache_append_workspace_size(1, 5120, 512, 64) == 0
    assert binding.mla_cache_append_workspace_size(4, 5, 2, 2, "f32") == 0
    assert binding.mla_cache_append_workspace_size(1, 5120, 512, 63) == 0  # odd d_r
    with pytest.raises(binding.MLAError) as e:
        binding.mla_cache_append_run(1, 5120, 512, 63, *([None] * 6), 4, 64, 8, None, None, stream=0)
    assert e.value.status == binding.MLA_ERR_INVALID_ARG
    with pytest.raises(binding.MLAError) as e:  # NULL tensors
        binding.mla_cache_append_run(1, 5120, 512, 64, *([None] * 6), 4, 64, 8, None, None, stream=0)
    assert e.value.status == binding.MLA_ERR_INVALID_ARG
    with pytest.raises(binding.MLAError) as e:  # no workspace
        binding.mla_cache_append_run(8, 5120, 512, 64, *([4096] * 6), 4, 64, 8, 4096, 4096, stream=0)
    assert e.value.status == binding.MLA_ERR_WORKSPACE
    with pytest.raises(binding.MLAError) as e:  # no frequencies and a base <= 1
        binding.mla_cache_append_run(1, 5120, 512, 64, *([4096] * 6), 4, 64, 8, 4096, 4096, rope_base=1.0,
                                     stream=0)
    assert e.value.status == binding.MLA_ERR_INVALID_ARG
    # query side: c_Q (256-aligned) plus the larger of the two stages' partials
    need = binding.mla_query_project_workspace_size(8, 5120, 1536, 128, 128, 64)
    assert need == 8 * 3072 + max(10 * 8 * 1536 * 4, 3 * 8 * 128 * 192 * 4)
    assert binding.mla_query_project_workspace_size(1, 5120, 1536, 128, 128, 64) == 3072  # c_Q only
    with pytest.raises(binding.MLAError) as e:
        binding.mla_query_project_run(8, 5120, 1536, 128, 128, 64, *([4096] * 7), workspace=4096,
                                      workspace_bytes=need - 1, stream=0)
    assert e.value.status == binding.MLA_ERR_WORKSPACE
    assert binding.mla_query_project_run(0, 5120, 1536, 128, 128, 64, *([None] * 7), stream=0) == binding.MLA_OK
    # both in one call: c_Q only when the first stages share a launch (up to
    # four rows), else what the two calls in turn need
    assert binding.mla_token_project_workspace_size(1, 5120, 512, 64, 1536, 128, 128) == 3072
    assert binding.mla_token_project_workspace_size(8, 5120, 512, 64, 1536, 128, 128) == max(
        binding.mla_cache_append_workspace_size(8, 5120, 512, 64),
        binding.mla_query_project_workspace_size(8, 5120, 1536, 128, 128, 64))
    assert binding.mla_token_project_workspace_size(1, 5120, 512, 63, 1536, 128, 128) == 0  # odd d_r
    shape = (1, 5120, 512, 64, 1536, 128, 128)
    with pytest.raises(binding.MLAError) as e:  # NULL tensors
        binding.mla_token_project_run(*shape, *([None] * 9), 4, 64, 8, *([None] * 4), stream=0)
    assert e.value.status == binding.MLA_ERR_INVALID_ARG
    with pytest.raises(binding.MLAError) as e:  # workspace too small
        binding.mla_token_project_run(*shape, *([4096] * 9), 4, 64, 8, *([4096] * 4), workspace=4096,
                                      workspace_bytes=3071, stream=0)
    assert e.value.status == binding.MLA_ERR_WORKSPACE
    with pytest.raises(binding.MLAError) as e:  # no pools for the pages
        binding.mla_token_project_run(*shape, *([4096] * 9), 4, 64, 0, *([4096] * 4), workspace=4096,
                                      workspace_bytes=3072, stream=0)
    assert e.value.status == binding.MLA_ERR_INVALID_ARG
    assert binding.mla_token_project_run(0, *shape[1:], *([None] * 9), 4, 64, 8, *([None] * 4),
                                         stream=0) == binding.MLA_OK


def test_prefill_refuses_bad_calls_on_the_host(L):
    assert binding.mla_prefill_workspace_size(4096, 128, 128) == 2 * 4096 * 128 * 128 * 2
    with pytest.raises(binding.MLAError) as e:
        binding.mla_prefill_run(16, 0, 512, 64, 128, *([None] * 8), stream=0)
    assert e.value.status == binding.MLA_ERR_INVALID_ARG
    with pytest.raises(binding.MLAError) as e:
        binding.mla_prefill_run(16, 2, 512, 64, 128, *([4096] * 7), 4096, workspace_bytes=16, stream=0)
    assert e.value.status == binding.MLA_ERR_WORKSPACE
    assert binding.mla_prefill_run(0, 2, 512, 64, 128, *([None] * 8), stream=0) == binding.MLA_OK
