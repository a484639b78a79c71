"""The benchmark's algorithmic counts, pinned to figures derived by hand.

Per visible (query row, cached token) pair the absorbed decode costs
4 h d_c + 2 h d_R + h FLOPs ("MLA, dim by dim", FLOP count of section
5.2: 278,656 at DeepSeek-V2's h=128, d_c=512, d_R=64) and reads the token's
d_c + d_R cached values once (1,152 bytes in bf16); each projection streams
h d_h d_c weights (16,777,216 bytes in bf16) and costs 2 h d_h d_c FLOPs per
query row.  These tests check bench.py's bookkeeping against those numbers
written out for each workload, so that the reported TFLOP/s, GB/s and
roofline fractions rest on the stated definitions.  CPU only.
"""
import bench
from mla_latent_cache_absorbed_amd import inputs

PER_PAIR = 278_656
PER_TOKEN = 1_152
W_BYTES = 16_777_216


def _counts(name, chunks=1, **kw):
    wl = inputs.make(name, materialize=False, **kw)
    return wl, bench.counts(wl, chunks)


def test_single_query_4k():
    wl, c = _counts("ds2_t4k", chunks=32)
    assert c["split_attn"]["bytes"] == 4096 * PER_TOKEN == 4_718_592
    assert c["split_attn"]["flops"] == 4096 * PER_PAIR
    assert c["step"]["bytes"] == 4_718_592 + 2 * W_BYTES == 38_273_024
    assert c["q_absorb"]["flops"] == c["finish"]["flops"] == 2 * 128 * 128 * 512
    # 32 chunk results of 128 heads: bf16 latent rows and fp32 lse
    assert c["split_attn"]["partial_bytes"] == 32 * 128 * (512 * 2 + 4)
    # arithmetic intensity of the cache stream at one query row
    assert abs(c["split_attn"]["flops"] / c["split_attn"]["bytes"] - 241.89) < 0.01


def test_single_query_32k_and_128k():
    _, c = _counts("ds2_t32k")
    assert c["split_attn"]["bytes"] == 37_748_736
    assert c["split_attn"]["flops"] == 32768 * PER_PAIR  # 9.131 GFLOP
    _, c = _counts("ds2_t128k")
    assert c["split_attn"]["bytes"] == 150_994_944


def test_multi_token_counts_causal_pairs():
    # 16 sequences of 16,384 cached tokens; query m sees 16,381 + m of them
    wl, c = _counts("ds2_mtp_b16")
    pairs = 16 * (16381 + 16382 + 16383 + 16384)
    assert wl.visible_pairs() == pairs
    assert c["split_attn"]["flops"] == pairs * PER_PAIR  # 292.17 GFLOP
    assert c["split_attn"]["bytes"] == 16 * 16384 * PER_TOKEN == 301_989_888  # read once, whatever n_q
    assert c["q_absorb"]["flops"] == 2 * 64 * 128 * 128 * 512


def test_tiny_fp32_counts():
    _, c = _counts("tiny_fp32")
    assert c["split_attn"]["bytes"] == 64 * (16 + 8) * 4 == 6_144
    assert c["split_attn"]["flops"] == 64 * (4 * 4 * 16 + 2 * 4 * 8 + 4) == 20_736


def test_paged_counts_follow_the_drawn_lengths():
    wl, c = _counts("ds2_paged_b32")
    tokens = int(wl.lens.sum())
    assert c["split_attn"]["bytes"] == tokens * PER_TOKEN
    assert c["split_attn"]["flops"] == tokens * PER_PAIR


def test_planned_chunk_count_stays_near_the_target():
    wl = inputs.make("ds2_paged_b32", materialize=False)
    n = bench.chunk_count(wl, 0, 0, 256)
    target = 256 // (wl.n_q * (wl.h // 64))
    assert wl.batch <= n <= target + wl.batch


def test_kernel_roofline_bound_and_fraction():
    _, c = _counts("ds2_t32k")
    r = bench.kernel_roofline("split_attn", c["split_attn"], 10e-6, "bf16")
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["achieved"] - 37_748_736 / 10e-6 / 1e9) < 1e-6
    assert abs(r["frac"] - r["achieved"] / 8000.0) < 1e-12
    # four query rows per token push the cache stream past the MFMA ridge
    _, c = _counts("ds2_mtp_b16")
    r = bench.kernel_roofline("split_attn", c["split_attn"], 100e-6, "bf16")
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"


def test_measured_traffic_needs_a_matching_entry():
    assert bench.measured_traffic("split_attn", "no_such_workload") is None
    assert bench.measured_traffic("no_such_kernel", "ds2_t4k") is None
