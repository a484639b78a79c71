"""Seeded workload generator: determinism, bf16 rounding, page tables."""
import numpy as np
import pytest

from mla_latent_cache_absorbed_amd import inputs


def test_bf16_round_to_nearest_even():
    one = np.float32(1.0)
    ulp = np.float32(2.0 ** -7)      # bf16 spacing at 1.0
    half = np.float32(2.0 ** -8)     # exactly halfway between 1 and 1 + ulp
    x = np.array([1.0, one + half, one + ulp + half, one + half * 1.001, -2.5, 0.0, 3.0e38],
                 dtype=np.float32)
    got = inputs.bf16_to_f32(inputs.bf16_bits(x))
    assert got[0] == 1.0
    assert got[1] == 1.0                 # tie -> even (1.0)
    assert got[2] == one + 2 * ulp       # tie -> even (1 + 2 ulp)
    assert got[3] == one + ulp           # just above the tie rounds up
    assert got[4] == -2.5 and got[5] == 0.0
    assert np.isfinite(got[6])
    # widening is exact and idempotent
    bits = inputs.bf16_bits(np.random.default_rng(0).standard_normal(1000).astype(np.float32))
    np.testing.assert_array_equal(inputs.bf16_bits(inputs.bf16_to_f32(bits)), bits)


def test_seeded_determinism():
    a = inputs.make("tiny_fp32")
    b = inputs.make("tiny_fp32")
    assert inputs.digest(a) == inputs.digest(b)
    c = inputs.make("tiny_fp32", seed=999)
    assert inputs.digest(a)["q"] != inputs.digest(c)["q"]


def test_shapes_and_dtypes():
    wl = inputs.make("tiny_fp32")
    assert wl.arrays["q"].shape == (1, 1, 4, 16) and wl.arrays["q"].dtype == np.float32
    assert wl.arrays["latent_pool"].shape == (4, 16, 16)
    assert wl.arrays["w_uk"].shape == (4, 16, 16)
    assert wl.scale == pytest.approx(1.0 / np.sqrt(24.0))


def test_paged_workload_structure():
    wl = inputs.make("ds2_paged_b32", materialize=False)
    assert wl.batch == 32
    assert wl.lens.min() >= 1024 and wl.lens.max() <= 8192
    pages = [(int(L) + 63) // 64 for L in wl.lens]
    used = np.concatenate([wl.page_table[b, :n] for b, n in enumerate(pages)])
    # every pool page is used by exactly one (sequence, page) slot
    assert sorted(used.tolist()) == list(range(wl.num_pages))
    assert not np.array_equal(used, np.arange(wl.num_pages))  # shuffled
    contiguous = inputs.make("ds2_t4k", materialize=False)
    np.testing.assert_array_equal(contiguous.page_table[0], np.arange(64))


def test_visible_pairs_counts_causal_rows():
    wl = inputs.make("ds2_mtp_b16", materialize=False)
    per_seq = sum(16384 - 4 + m + 1 for m in range(4))
    assert wl.visible_pairs() == 16 * per_seq
