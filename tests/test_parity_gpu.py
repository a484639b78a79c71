"""GPU parity: the HIP path through the C ABI against the fp64 oracle, on the
same seeded inputs, for the five configurations and their edge cases.

Tolerance (normwise, max |gpu - oracle| / max |oracle|): 1e-2 for bf16
storage with fp32 accumulation, 1e-5 for the fp32 mode.  Every
configuration is checked on all its heads with the absorbed fp64 form
(itself pinned equal to the explicit K/V form), plus a few (sequence, head)
pairs with the explicit form.  Two constructions make the GPU result exact,
so that they are compared bit for bit: split-count invariance (zero queries
and block-constant integer latents) and the causal rows of a multi-token
step against single-token decodes at the matching lengths.
"""
import numpy as np
import pytest

import oracle
from mla_latent_cache_absorbed_amd import inputs
from tests._parity import check, gpu_rows, log, problem, sample_pairs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as t
    assert t.cuda.is_available()
    return t


def _run(wl, torch, **kw):
    from mla_latent_cache_absorbed_amd.runner import DeviceWorkload
    dw = DeviceWorkload(wl, **kw)
    log("%s: splits/chunk = %s" % (wl.name, dw.split_plan()))
    dw.run()
    torch.cuda.synchronize()
    return dw


# --------------------------------------------------------------------------
# configuration 1: tiny fp32 (general path), whole output, every split count
# --------------------------------------------------------------------------
@pytest.mark.parametrize("splits", [0, 1, 2, 4])
@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_tiny_fp32(torch, splits, out_dtype):
    wl = inputs.make("tiny_fp32")
    dw = _run(wl, torch, num_splits=splits, out_dtype=out_dtype)
    ref = oracle.decode_explicit(problem(wl))
    got = dw.result_f64()
    assert got.shape == ref.shape == (1, 1, 4, 16)
    check(got, ref, "f32" if out_dtype == "f32" else "bf16", "tiny_fp32 S=%d out=%s" % (splits, out_dtype))


# --------------------------------------------------------------------------
# configuration 2: T = 4096, all heads (absorbed oracle) + explicit sample
# --------------------------------------------------------------------------
@pytest.mark.parametrize("splits", [0, 1, 16])
def test_ds2_t4k(torch, splits):
    wl = inputs.make("ds2_t4k")
    dw = _run(wl, torch, num_splits=splits)
    got = dw.result_f64()
    prob = problem(wl)
    ref = oracle.decode_absorbed(prob)
    check(got, ref, "bf16", "ds2_t4k S=%d all heads" % splits)
    if splits == 0:
        pairs = sample_pairs(wl, 4)
        check(gpu_rows(got, pairs), oracle.decode_explicit(prob, pairs), "bf16",
              "ds2_t4k explicit sample")


def test_ds2_t4k_fp32_output_matches_bf16_output(torch):
    wl = inputs.make("ds2_t4k")
    a = _run(wl, torch, out_dtype="f32").result_f64()
    b = _run(wl, torch, out_dtype="bf16").result_f64()
    ref = oracle.decode_absorbed(problem(wl))
    check(a, ref, "bf16", "ds2_t4k fp32 output")
    # the bf16 output is the fp32 one rounded to nearest
    assert np.max(np.abs(a - b)) <= np.max(np.abs(a)) * 2.0 ** -8


# --------------------------------------------------------------------------
# configuration 3: batched, paged, shuffled, variable lengths
# --------------------------------------------------------------------------
def test_ds2_paged_b32(torch):
    wl = inputs.make("ds2_paged_b32")
    log("lengths %s" % wl.lens.tolist())
    dw = _run(wl, torch)
    got = dw.result_f64()
    prob = problem(wl)
    check(got, oracle.decode_absorbed(prob), "bf16", "ds2_paged_b32 absorbed, all heads")
    pairs = sample_pairs(wl, 4)
    few = pairs[::32][:4]
    check(gpu_rows(got, few), oracle.decode_explicit(prob, few), "bf16",
          "ds2_paged_b32 explicit sample")


def test_paging_permutation_is_bitwise_invisible(torch):
    """The same logical cache under another page permutation gives the same bits."""
    wl = inputs.make("ds2_paged_b32")
    dw = _run(wl, torch)
    first = dw.out.clone()
    rng = np.random.default_rng(77)
    perm = rng.permutation(wl.num_pages)  # new pool position of each old page
    inv = np.argsort(perm)
    lat = dw.t["latent_pool"][torch.from_numpy(inv).cuda()].contiguous()
    rope = dw.t["rope_pool"][torch.from_numpy(inv).cuda()].contiguous()
    table = torch.from_numpy(perm[wl.page_table].astype(np.int32)).cuda()
    dw.run(latent_pool=lat, rope_pool=rope, page_table=table)
    torch.cuda.synchronize()
    assert torch.equal(first, dw.out)


# --------------------------------------------------------------------------
# configuration 4: T = 131072, forced chunk counts 64 / 128 / 256
# --------------------------------------------------------------------------
@pytest.fixture(scope="module")
def t128k_ref():
    wl = inputs.make("ds2_t128k")
    prob = problem(wl)
    return wl, oracle.decode_absorbed(prob), prob


@pytest.mark.parametrize("splits", [64, 128, 256])
def test_ds2_t128k(torch, t128k_ref, splits):
    wl, ref, prob = t128k_ref
    dw = _run(wl, torch, num_splits=splits)
    assert dw.split_plan() == (splits, 131072 // splits)
    got = dw.result_f64()
    check(got, ref, "bf16", "ds2_t128k S=%d, all heads" % splits)
    if splits == 128:
        one = sample_pairs(wl, 1)
        check(gpu_rows(got, one), oracle.decode_explicit(prob, one), "bf16",
              "ds2_t128k explicit, 1 head")


# --------------------------------------------------------------------------
# configuration 5: 4 causal query tokens per sequence
# --------------------------------------------------------------------------
def test_ds2_mtp_b16(torch):
    wl = inputs.make("ds2_mtp_b16")
    dw = _run(wl, torch)
    got = dw.result_f64()
    prob = problem(wl)
    check(got, oracle.decode_absorbed(prob), "bf16", "ds2_mtp_b16 absorbed, all heads")
    few = sample_pairs(wl, 1)[:2]
    check(gpu_rows(got, few), oracle.decode_explicit(prob, few), "bf16",
          "ds2_mtp_b16 explicit sample")
    # the four rows differ (the causal mask is applied per query token)
    assert np.max(np.abs(got[0, 0] - got[0, 3])) > 1e-3


def test_ds2_t32k(torch):
    wl = inputs.make("ds2_t32k")
    dw = _run(wl, torch)
    got = dw.result_f64()
    check(got, oracle.decode_absorbed(problem(wl)), "bf16", "ds2_t32k absorbed, all heads")


def test_multi_token_rows_equal_single_token_decodes(torch):
    """Reading C5: query token m of an n_q = 4 step sees tokens 0 .. T-4+m,
    so its row is the single-token decode of the same query at context
    length L = T-3+m.  With the same chunking (forced chunk count, same
    max_context_len) both runs do the same tiles in the same order, so the
    rows must agree bit for bit."""
    wl4 = inputs.make("ds2_mtp_b16")
    T = int(wl4.max_len)
    assert np.all(wl4.lens == T)
    dw4 = _run(wl4, torch, num_splits=2)
    wl1 = inputs.make("ds2_mtp_b16", n_q=1, materialize=False)
    wl1.arrays = dict(wl4.arrays)
    wl1.arrays["q"] = np.ascontiguousarray(wl4.arrays["q"][:, :1])
    wl1.arrays["q_r"] = np.ascontiguousarray(wl4.arrays["q_r"][:, :1])
    from mla_latent_cache_absorbed_amd.runner import DeviceWorkload
    dw1 = DeviceWorkload(wl1, num_splits=2, max_context_len=T)
    dw1.t.update({k: dw4.t[k] for k in ("latent_pool", "rope_pool", "page_table", "w_uk", "w_uv")})
    assert dw1.split_plan() == dw4.split_plan()
    for m in range(4):
        dw1.run(q=dw4.t["q"][:, m:m + 1].contiguous(), q_r=dw4.t["q_r"][:, m:m + 1].contiguous(),
                context_lens=torch.full_like(dw4.t["context_lens"], T - 3 + m))
        torch.cuda.synchronize()
        same = torch.equal(dw1.out[:, 0], dw4.out[:, m])
        log("row m=%d vs single-token decode at L=%d: %s" % (m, T - 3 + m, "bitwise equal" if same else "DIFFER"))
        assert same, "row %d differs from the single-token decode at L=%d" % (m, T - 3 + m)


def _block_constant_zero_query(name, seed):
    """Zero queries (every visible token weighs exactly 1) and latent rows
    constant over aligned 512-token blocks, each block's features drawn from
    {-1, 0, 1}: every chunk sum, weight sum, chunk mean, merge weight and
    merged latent on the GPU path is then exact in its storage type (bf16
    means have at most 8 significant bits for up to 256 blocks), so every
    split count gives the same bits."""
    wl = inputs.make(name, seed=seed)
    wl.arrays["q"] = np.zeros_like(wl.arrays["q"])
    wl.arrays["q_r"] = np.zeros_like(wl.arrays["q_r"])
    rng = np.random.default_rng(seed)
    T = int(wl.max_len)
    blocks = rng.integers(-1, 2, size=(T // 512, wl.d_c)).astype(np.float32)
    per_token = np.repeat(blocks, 512, axis=0)  # logical token t -> its block's row
    lat = wl.arrays["latent_pool"].copy()
    for t in range(0, T, wl.page_size):  # contiguous single sequence: page j holds tokens 64 j ..
        lat[wl.page_table[0, t // wl.page_size]] = inputs.bf16_bits(per_token[t:t + wl.page_size])
    wl.arrays["latent_pool"] = lat
    return wl


@pytest.mark.parametrize("name,splits", [("ds2_t32k", (1, 2, 64, 128, 256)),
                                         ("ds2_t128k", (4, 64, 128, 256))])
def test_split_count_invariance_is_exact(torch, name, splits):
    """The a5 merge pin: on inputs where every step is exact, the output is
    the same bits for every chunk count and equals W_UV (mean latent) to fp32
    rounding."""
    wl = _block_constant_zero_query(name, seed=250)
    ref = oracle.decode_absorbed(problem(wl))
    outs = {}
    for S in splits:
        dw = _run(wl, torch, num_splits=S, out_dtype="f32")
        assert dw.split_plan()[0] == S
        outs[S] = dw.out.clone()
        check(dw.result_f64(), ref, "f32", "%s block-constant zero query S=%d" % (name, S))
        del dw
    first = outs[splits[0]]
    for S in splits[1:]:
        assert torch.equal(outs[S], first), "%s: S=%d differs from S=%d" % (name, S, splits[0])
    log("%s: S=%s give the same bits" % (name, list(splits)))


@pytest.mark.parametrize("name,splits", [("ds2_t32k", (1, 2, 64, 128, 256)),
                                         ("ds2_t128k", (4, 64, 128, 256))])
def test_split_sweep_fp32_output(torch, name, splits):
    """Random inputs, fp32 output, every chunk count against the oracle on
    all heads.  The GPU rounds each weight P and each chunk partial to bf16
    (readings C8, C8a), so different chunk counts differ by rounding noise of
    order 2^-9 relative per token and partial; the normwise bound stays the
    bf16 one and the pairwise spread is reported."""
    wl = inputs.make(name)
    ref = oracle.decode_absorbed(problem(wl))
    outs = {}
    for S in splits:
        dw = _run(wl, torch, num_splits=S, out_dtype="f32")
        assert dw.split_plan()[0] == S
        outs[S] = dw.result_f64()
        check(outs[S], ref, "bf16", "%s fp32 output S=%d, all heads" % (name, S))
        del dw
    base = outs[splits[0]]
    for S in splits[1:]:
        log("%s: S=%d vs S=%d normwise difference %.3e" % (name, S, splits[0],
                                                           float(np.max(np.abs(outs[S] - base)) / np.max(np.abs(ref)))))


# --------------------------------------------------------------------------
# edge cases
# --------------------------------------------------------------------------
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_ragged_lengths_and_tails(torch, splits):
    """Lengths that end inside a tile and inside a page, down to one token."""
    wl = inputs.make("ds2_t4k", batch=6, lens=("list", [1, 31, 33, 97, 300, 2049]),
                     shuffled=True, seed=201)
    dw = _run(wl, torch, num_splits=splits)
    check(dw.result_f64(), oracle.decode_absorbed(problem(wl)), "bf16",
          "ragged lengths S=%d" % splits)


@pytest.mark.parametrize("splits", [5, 12, 20])
def test_chunk_merge_over_row_blocks(torch, splits):
    """20 query rows (a full and a partial block of 16 in the merge) with
    chunk counts that select each merge variant; the short sequences leave
    trailing chunks empty."""
    lens = [1, 2, 40, 64, 65, 100, 127, 128, 129, 200, 255, 256, 300, 333, 400, 480, 511, 512,
            600, 639]
    wl = inputs.make("ds2_t4k", batch=len(lens), lens=("list", lens), shuffled=True, seed=205)
    dw = _run(wl, torch, num_splits=splits)
    check(dw.result_f64(), oracle.decode_absorbed(problem(wl)), "bf16",
          "merge over row blocks S=%d" % splits)


@pytest.mark.parametrize("h,batch", [(64, 100), (128, 130)])
def test_many_sequences(torch, h, batch):
    """More sequences than one scan block of the device chunk plan (100
    sequences with 64 heads: 256 target chunks), and more than half its
    target chunk count (130 with 128 heads: a fixed chunking instead)."""
    rng = np.random.default_rng(206)
    lens = [int(x) for x in rng.integers(1, 400, size=batch)]
    wl = inputs.make("ds2_t4k", h=h, batch=batch, lens=("list", lens), shuffled=True, seed=207)
    dw = _run(wl, torch)
    assert (dw.split_plan() == (0, 0)) == (h == 64)
    check(dw.result_f64(), oracle.decode_absorbed(problem(wl)), "bf16", "%d sequences" % batch)


@pytest.mark.parametrize("splits", [0, 3])
def test_four_head_groups_two_query_tokens(torch, splits):
    """h = 256 (four 64-head groups, each with its own query rows in the
    split kernel's prologue) and two query tokens per sequence, ragged
    paged contexts: every (chunk, token, head group) work-group stages a
    different slice of the absorbed query."""
    wl = inputs.make("ds2_mtp_b16", h=256, n_q=2, batch=3, lens=("list", [70, 333, 190]),
                     shuffled=True, seed=209)
    dw = _run(wl, torch, num_splits=splits)
    check(dw.result_f64(), oracle.decode_absorbed(problem(wl)), "bf16",
          "h=256 n_q=2 S=%d" % splits)


@pytest.mark.parametrize("splits", [0, 4])
def test_three_head_groups_three_query_tokens(torch, splits):
    """h = 192 (an odd number of 64-head groups, so the work-groups of one
    chunk do not fill a multiple of eight) and three query tokens per
    sequence (causal diagonals of three rows, finish row blocks that mix
    sequences), with planned and fixed chunking."""
    wl = inputs.make("ds2_mtp_b16", h=192, n_q=3, batch=5, lens=("list", [3, 95, 1200, 41, 600]),
                     shuffled=True, seed=250)
    dw = _run(wl, torch, num_splits=splits)
    check(dw.result_f64(), oracle.decode_absorbed(problem(wl)), "bf16",
          "h=192 n_q=3 S=%d" % splits)


@pytest.mark.parametrize("page_size,splits", [(32, 0), (32, 5), (256, 0), (256, 3)])
def test_page_sizes(torch, page_size, splits):
    """Pages of one tile (32 tokens) and of eight (256): the fast path's
    tiles never straddle a page, and every page-table lookup (per tile, in
    LDS) lands on the right page of a shuffled pool."""
    wl = inputs.make("ds2_t4k", batch=3, page_size=page_size, lens=("list", [33, 700, 257]),
                     shuffled=True, seed=210 + page_size)
    dw = _run(wl, torch, num_splits=splits)
    check(dw.result_f64(), oracle.decode_absorbed(problem(wl)), "bf16",
          "page size %d S=%d" % (page_size, splits))


def test_skewed_batch_gives_the_long_sequence_most_chunks(torch):
    """One long sequence beside short ones: the device plan gives the long
    one about a hundred chunks (the many-chunk merge of the finish kernel)
    and the short ones one each."""
    wl = inputs.make("ds2_t4k", batch=4, lens=("list", [20000, 100, 37, 3000]), shuffled=True, seed=208)
    dw = _run(wl, torch)
    assert dw.split_plan() == (0, 0)
    check(dw.result_f64(), oracle.decode_absorbed(problem(wl)), "bf16", "skewed batch")


def test_single_token_context_returns_projected_latent(torch):
    wl = inputs.make("ds2_t4k", lens=("fixed", 1), seed=202)
    dw = _run(wl, torch, out_dtype="f32")
    ref = oracle.decode_explicit(problem(wl))
    check(dw.result_f64(), ref, "bf16", "one cached token")


@pytest.mark.parametrize("L", [4, 5, 37, 64])
def test_multi_token_short_contexts(torch, L):
    """n_q = 4 with contexts so short that the causal diagonal spans tiles."""
    wl = inputs.make("ds2_mtp_b16", batch=2, lens=("list", [L, L + 29]), seed=203 + L)
    dw = _run(wl, torch, num_splits=0)
    check(dw.result_f64(), oracle.decode_absorbed(problem(wl)), "bf16", "n_q=4 L=%d" % L)


def test_full_table_capacity(torch):
    """max_context_len equal to the page-table capacity."""
    wl = inputs.make("ds2_t4k", batch=2, lens=("list", [640, 640]), shuffled=True, seed=204)
    assert wl.max_pages * wl.page_size == 640
    dw = _run(wl, torch)
    check(dw.result_f64(), oracle.decode_absorbed(problem(wl)), "bf16", "full table capacity")


def test_repeat_runs_are_bitwise_identical(torch):
    wl = inputs.make("ds2_paged_b32")
    dw = _run(wl, torch)
    first = dw.out.clone()
    for _ in range(3):
        dw.run()
    torch.cuda.synchronize()
    assert torch.equal(first, dw.out)


# --------------------------------------------------------------------------
# score structure: the online softmax's reference maximum moves mid-chunk
# --------------------------------------------------------------------------
def _spike_scores(wl, levels, period, q_r_value=8.0):
    """Rewrite q_R and the RoPE cache so that every head's RoPE logit is 0
    except at offsets o of each `period`-token window, where it is
    levels[o] (in natural-log units); the content logits stay random (unit
    scale).  Every query row and head gets q_R = q_r_value * e_0, and token
    t's RoPE row gets levels[t % period] / (q_r_value * scale) in its
    component 0 (then rounded to the storage type, which the oracle reads
    too)."""
    f32 = np.float32
    q_r = np.zeros((wl.batch, wl.n_q, wl.h, wl.d_r), dtype=f32)
    q_r[..., 0] = q_r_value
    rope = inputs.as_f32(wl, "rope_pool").copy()
    rope[..., 0] = 0.0
    for b in range(wl.batch):
        for t in range(int(wl.lens[b])):
            lvl = levels.get(t % period)
            if lvl is not None:
                page = wl.page_table[b, t // wl.page_size]
                rope[page, t % wl.page_size, 0] = lvl / (q_r_value * wl.scale)
    to_store = inputs.bf16_bits if wl.dtype == "bf16" else (lambda x: x)
    wl.arrays["q_r"] = to_store(q_r)
    wl.arrays["rope_pool"] = to_store(rope)
    return wl


# Rising spikes 10, 20 and 30 natural-log units above the random logits, at
# offsets 40, 80 and 120 of every 128 tokens: each is more than 2^8 above
# the previous maximum, so every chunk that holds a window moves its
# reference maximum three times, across tile boundaries, and what was
# accumulated before each move must be rescaled (a missing or wrong rescale
# weighs it e^10 times too much or too little).
_RISING = {40: 10.0, 80: 20.0, 120: 30.0}


@pytest.mark.parametrize("splits", [0, 1, 7])
def test_rising_scores_rescale_the_accumulator(torch, splits):
    wl = _spike_scores(inputs.make("ds2_t4k", seed=240), _RISING, 128)
    dw = _run(wl, torch, num_splits=splits)
    check(dw.result_f64(), oracle.decode_absorbed(problem(wl)), "bf16", "rising spikes S=%d" % splits)


def test_rising_scores_paged_ragged_batch(torch):
    """Planned chunking over a shuffled page table, lengths that end inside
    a window (some before a spike, some between two)."""
    wl = inputs.make("ds2_paged_b32", batch=5, lens=("list", [3000, 100, 77, 1150, 41]), seed=241)
    _spike_scores(wl, _RISING, 128)
    dw = _run(wl, torch)
    check(dw.result_f64(), oracle.decode_absorbed(problem(wl)), "bf16", "rising spikes, paged")


def test_rising_scores_multi_token(torch):
    """Four causal query tokens; in the second sequence the visible ranges of
    query rows 0 and 1 end on either side of a spike."""
    wl = inputs.make("ds2_mtp_b16", batch=2, lens=("list", [1000, 2178]), seed=242)
    _spike_scores(wl, {40: 10.0, 80: 20.0, 120: 30.0, 127: 40.0}, 128)
    dw = _run(wl, torch, num_splits=0)
    check(dw.result_f64(), oracle.decode_absorbed(problem(wl)), "bf16", "rising spikes, n_q=4")


@pytest.mark.parametrize("splits", [0, 1])
def test_falling_scores_keep_the_first_reference(torch, splits):
    """The highest logits first (40 units above the rest at offset 0 of
    every 128-token window, 30 at offset 1): chunks start on a window, so
    each sets its reference in its first tile and never moves it, and most
    weights are tiny (e^-30 .. e^-40) but not zero."""
    wl = _spike_scores(inputs.make("ds2_t4k", seed=243), {0: 40.0, 1: 30.0}, 128)
    dw = _run(wl, torch, num_splits=splits)
    check(dw.result_f64(), oracle.decode_absorbed(problem(wl)), "bf16", "falling spikes S=%d" % splits)


@pytest.mark.parametrize("splits", [0, 2])
def test_rising_scores_general_path(torch, splits):
    """The fp32 general path's online softmax under the same spikes."""
    wl = _spike_scores(inputs.make("tiny_fp32", lens=("fixed", 300), seed=244), _RISING, 128)
    dw = _run(wl, torch, num_splits=splits)
    check(dw.result_f64(), oracle.decode_explicit(problem(wl)), "f32", "general fp32, rising spikes")


def test_zero_query_averages_the_latents(torch):
    """q = 0 and q_R = 0: every visible token weighs the same, so o_i =
    W_UV[i] (mean of the latents), a closed form independent of the oracle's
    softmax."""
    wl = inputs.make("ds2_t4k", batch=2, lens=("list", [1000, 333]), shuffled=True, seed=245)
    wl.arrays["q"] = np.zeros_like(wl.arrays["q"])
    wl.arrays["q_r"] = np.zeros_like(wl.arrays["q_r"])
    dw = _run(wl, torch, out_dtype="f32")
    lat = inputs.as_f64(wl, "latent_pool")
    w_uv = inputs.as_f64(wl, "w_uv")
    ref = np.empty((wl.batch, wl.n_q, wl.h, wl.d_h))
    for b in range(wl.batch):
        L = int(wl.lens[b])
        rows = [lat[wl.page_table[b, t // wl.page_size], t % wl.page_size] for t in range(L)]
        mean = np.mean(rows, axis=0)
        ref[b, 0] = w_uv @ mean
    check(dw.result_f64(), ref, "bf16", "zero query")


def test_general_path_bf16_odd_shapes(torch):
    """bf16 storage with shapes outside the MFMA kernels (general path)."""
    wl = inputs.make("tiny_fp32", dtype="bf16", h=6, d_c=40, d_r=6, d_h=12, page_size=8,
                     batch=3, n_q=2, lens=("list", [2, 19, 50]), shuffled=True, seed=205)
    dw = _run(wl, torch, num_splits=0)
    check(dw.result_f64(), oracle.decode_explicit(problem(wl)), "bf16", "general bf16")


def test_general_path_fp32_without_rope(torch):
    wl = inputs.make("tiny_fp32", d_r=0, batch=2, lens=("list", [64, 7]), seed=206)
    dw = _run(wl, torch, num_splits=3)
    check(dw.result_f64(), oracle.decode_explicit(problem(wl)), "f32", "general fp32 d_r=0")


def test_empty_batch_is_a_no_op(torch):
    from mla_latent_cache_absorbed_amd import binding
    wl = inputs.make("ds2_t4k", lens=("fixed", 64), seed=207)
    dw = _run(wl, torch)
    before = dw.out.clone()
    t = dw.t
    binding.mla_decode_run(dw.dec.plan, 0, 1, 64, wl.num_pages, t["q"], t["q_r"],
                           t["latent_pool"], t["rope_pool"], t["page_table"],
                           t["context_lens"], t["w_uk"], t["w_uv"], dw.out, dw.ws)
    torch.cuda.synchronize()
    assert torch.equal(before, dw.out)


def test_runs_on_a_side_stream(torch):
    wl = inputs.make("ds2_t4k", lens=("fixed", 512), seed=208)
    dw = _run(wl, torch)
    ref = dw.out.clone()
    dw.out.zero_()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        dw.run()
    s.synchronize()
    assert torch.equal(ref, dw.out)


def test_graph_replays_match_eager_runs(torch):
    """A HIP graph holding two captured decode steps, replayed several times
    with eager work and synchronisations in between, reproduces the eager
    results bit for bit on every replay."""
    from mla_latent_cache_absorbed_amd.runner import DeviceWorkload
    wl_a = inputs.make("ds2_t4k", batch=3, lens=("list", [700, 1500, 64]), seed=231)
    wl_b = inputs.make("ds2_mtp_b16", batch=2, lens=("list", [300, 900]), seed=232)
    dws = [DeviceWorkload(wl_a), DeviceWorkload(wl_b)]
    for dw in dws:
        dw.run()
    torch.cuda.synchronize()
    eager = [dw.out.clone() for dw in dws]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for dw in dws:
            dw.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for dw in dws:
            dw.run()
    for rep in range(4):
        for dw in dws:
            dw.out.fill_(0)
        graph.replay()
        torch.cuda.synchronize()
        for dw, ref in zip(dws, eager):
            assert torch.equal(dw.out, ref), "graph replay %d differs from the eager run" % rep
        dws[rep % 2].run()  # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(dws[rep % 2].out, eager[rep % 2])
