"""Closed forms, invariants and special cases that pin the fp64 oracle beyond
the pages' worked examples.

- absorption (bilinear) and value-absorption (linearity) identities on random
  inputs ("Mathematical Prerequisites for DeepSeek-V2", sections 6 and 7);
- softmax: rows sum to one, shift invariance, the two-point logistic form;
- the whole step: explicit K/V route == absorbed route ("MLA, dim by dim",
  section 5.2, the cached-decode score and output chains);
- special cases with a plain answer: one cached token, a zero query, and a
  single head with identity weights, which is textbook single-head attention
  (checked against torch's scaled_dot_product_attention in float64 on CPU);
- causality of multi-token decode, paging, and head/sequence selection.
"""
import math

import numpy as np
import pytest

import oracle


def _rand_problem(rng, B=2, n_q=1, h=3, d_c=8, d_r=4, d_h=5, page_size=4, lens=(9, 6),
                  shuffle=True, scale=None):
    lens = np.asarray(lens, dtype=np.int32)
    per = [(int(L) + page_size - 1) // page_size for L in lens]
    total = sum(per)
    perm = rng.permutation(total) if shuffle else np.arange(total)
    table = np.zeros((B, max(per)), dtype=np.int32)
    off = 0
    for b, n in enumerate(per):
        table[b, :n] = perm[off:off + n]
        off += n
    return oracle.Problem(
        q=rng.standard_normal((B, n_q, h, d_h)), q_r=rng.standard_normal((B, n_q, h, d_r)),
        latent_pool=rng.standard_normal((total, page_size, d_c)),
        rope_pool=rng.standard_normal((total, page_size, d_r)),
        page_table=table, context_lens=lens,
        w_uk=rng.standard_normal((h, d_h, d_c)) / math.sqrt(d_c),
        w_uv=rng.standard_normal((h, d_h, d_c)) / math.sqrt(d_c),
        scale=scale if scale is not None else 1.0 / math.sqrt(d_h + d_r))


def test_absorption_identity_random():
    rng = np.random.default_rng(1)
    for _ in range(20):
        d_h, d_c = rng.integers(1, 9, size=2)
        W = rng.standard_normal((d_h, d_c))
        q = rng.standard_normal(d_h)
        c = rng.standard_normal(d_c)
        left = oracle.dot(q, oracle.matvec(W, c))        # q^T (W c)
        right = oracle.dot(oracle.absorb_query(W, q), c)  # (W^T q)^T c
        assert abs(left - right) <= 1e-12 * max(1.0, abs(left))


def test_value_absorption_identity_random():
    rng = np.random.default_rng(2)
    W = rng.standard_normal((5, 7))
    C = rng.standard_normal((11, 7))
    p = oracle.softmax(rng.standard_normal(11))
    left = sum(p[t] * oracle.matvec(W, C[t]) for t in range(11))
    right = oracle.up_project(W, oracle.weighted_latent(p, C))
    np.testing.assert_allclose(left, right, rtol=1e-12, atol=1e-13)


def test_softmax_invariants():
    rng = np.random.default_rng(3)
    for n in (1, 2, 7, 1000):
        s = rng.standard_normal(n) * 10
        p = oracle.softmax(s)
        assert np.all(p >= 0)
        assert abs(p.sum() - 1.0) <= 1e-14 * n
        np.testing.assert_allclose(oracle.softmax(s + 123.25), p, rtol=1e-12, atol=1e-300)
        assert int(np.argmax(p)) == int(np.argmax(s))
    # equal scores -> uniform weights; huge scores do not overflow
    np.testing.assert_allclose(oracle.softmax(np.full(5, 700.0)), np.full(5, 0.2), rtol=1e-15)
    # two points: p_0 = 1 / (1 + e^{-(s_0 - s_1)}) (logistic form)
    for d in (-5.0, -0.3, 0.0, 2.0, 30.0):
        p = oracle.softmax([d, 0.0])
        assert abs(p[0] - 1.0 / (1.0 + math.exp(-d))) <= 1e-15


@pytest.mark.parametrize("n_q", [1, 3])
@pytest.mark.parametrize("d_r", [0, 4])
def test_explicit_equals_absorbed(n_q, d_r):
    rng = np.random.default_rng(4 + n_q + d_r)
    prob = _rand_problem(rng, n_q=n_q, d_r=d_r)
    a = oracle.decode_explicit(prob)
    b = oracle.decode_absorbed(prob)
    assert a.shape == (2, n_q, 3, 5)
    assert np.max(np.abs(a - b)) <= 1e-12 * np.max(np.abs(a))


def test_single_cached_token_returns_projected_latent():
    rng = np.random.default_rng(5)
    prob = _rand_problem(rng, B=1, lens=(1,), shuffle=False)
    o = oracle.decode_explicit(prob)
    c0 = prob.latent_pool[prob.page_table[0, 0], 0]
    expect = np.einsum("iac,c->ia", prob.w_uv, c0)
    np.testing.assert_allclose(o[0, 0], expect, rtol=1e-13, atol=1e-14)


def test_zero_query_gives_mean_latent():
    rng = np.random.default_rng(6)
    prob = _rand_problem(rng, B=1, lens=(10,))
    prob.q[:] = 0.0
    prob.q_r[:] = 0.0
    o = oracle.decode_explicit(prob)
    C, _ = oracle.gather(prob, 0, 10)
    expect = np.einsum("iac,c->ia", prob.w_uv, C.mean(axis=0))
    np.testing.assert_allclose(o[0, 0], expect, rtol=1e-13, atol=1e-14)


def test_identity_head_is_textbook_attention():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    d, d_r, L = 6, 3, 13
    prob = _rand_problem(rng, B=1, h=1, d_c=d, d_h=d, d_r=d_r, lens=(L,), page_size=5)
    prob.w_uk = np.eye(d)[None]
    prob.w_uv = np.eye(d)[None]
    o = oracle.decode_explicit(prob)[0, 0, 0]
    C, KR = oracle.gather(prob, 0, L)
    K = torch.from_numpy(np.concatenate([C, KR], axis=1))[None, None]      # [1,1,L,d+d_r]
    V = torch.from_numpy(C)[None, None]                                     # [1,1,L,d]
    Qt = torch.from_numpy(np.concatenate([prob.q[0, 0, 0], prob.q_r[0, 0, 0]]))[None, None, None]
    ref = torch.nn.functional.scaled_dot_product_attention(Qt, K, V, scale=prob.scale)
    np.testing.assert_allclose(o, ref[0, 0, 0].numpy(), rtol=1e-12, atol=1e-13)


def test_multi_token_rows_are_shorter_single_token_decodes():
    """With n_q new tokens, query m attends to tokens 0 .. L - n_q + m."""
    rng = np.random.default_rng(8)
    n_q, L = 4, 11
    prob = _rand_problem(rng, B=1, n_q=n_q, lens=(L,))
    full = oracle.decode_explicit(prob)
    for m in range(n_q):
        one = oracle.Problem(q=prob.q[:, m:m + 1], q_r=prob.q_r[:, m:m + 1],
                             latent_pool=prob.latent_pool, rope_pool=prob.rope_pool,
                             page_table=prob.page_table,
                             context_lens=np.array([L - n_q + m + 1], np.int32),
                             w_uk=prob.w_uk, w_uv=prob.w_uv, scale=prob.scale)
        np.testing.assert_array_equal(full[:, m], oracle.decode_explicit(one)[:, 0])
    # and the rows differ from each other (the mask is not a no-op)
    assert np.max(np.abs(full[0, 0] - full[0, n_q - 1])) > 1e-6


def test_paging_is_transparent():
    rng = np.random.default_rng(9)
    prob = _rand_problem(rng, B=2, lens=(9, 6), page_size=2, shuffle=True)
    C0, K0 = oracle.gather(prob, 0, 9)
    C1, K1 = oracle.gather(prob, 1, 6)
    # the same logical cache laid out contiguously with one page per sequence
    pool_c = np.zeros((2, 9, prob.latent_pool.shape[2]))
    pool_r = np.zeros((2, 9, prob.rope_pool.shape[2]))
    pool_c[0], pool_r[0] = C0, K0
    pool_c[1, :6], pool_r[1, :6] = C1, K1
    flat = oracle.Problem(q=prob.q, q_r=prob.q_r, latent_pool=pool_c, rope_pool=pool_r,
                          page_table=np.array([[0], [1]], np.int32), context_lens=prob.context_lens,
                          w_uk=prob.w_uk, w_uv=prob.w_uv, scale=prob.scale)
    np.testing.assert_array_equal(oracle.decode_explicit(prob), oracle.decode_explicit(flat))


def test_selection_matches_full_output():
    rng = np.random.default_rng(10)
    prob = _rand_problem(rng, n_q=2)
    full = oracle.decode_explicit(prob)
    pairs = [(1, 2), (0, 0), (1, 0)]
    sub = oracle.decode_explicit(prob, pairs)
    for k, (b, i) in enumerate(pairs):
        np.testing.assert_array_equal(sub[k], full[b, :, i])


def test_rejects_bad_problems():
    rng = np.random.default_rng(11)
    prob = _rand_problem(rng)
    prob.page_table[0, 0] = 10_000  # page outside the pool
    with pytest.raises(ValueError):
        oracle.decode_explicit(prob)
    prob = _rand_problem(rng, n_q=3, lens=(2, 6))  # fewer tokens than new queries
    with pytest.raises(ValueError):
        oracle.decode_explicit(prob)


# --------------------------------------------------------------------------
# Output projection (the step after the decode path)
# --------------------------------------------------------------------------
def test_output_projection_is_a_matrix_product():
    """A special case that reduces to a library routine: the concatenated
    rows times W^O is numpy's matrix product, on random inputs of several
    shapes, one row or several."""
    rng = np.random.default_rng(31)
    for rows, h, d_h, d in ((1, 1, 1, 1), (1, 3, 4, 7), (5, 2, 8, 300), (3, 16, 16, 513)):
        o = rng.standard_normal((rows, h, d_h))
        W = rng.standard_normal((h * d_h, d))
        u = oracle.output_project(o, W)
        assert u.shape == (rows, d)
        np.testing.assert_allclose(u, o.reshape(rows, -1) @ W, rtol=1e-12, atol=1e-12)


def test_output_projection_small_integers_by_hand():
    """Brute force on a tiny integer case worked out by hand: one row of two
    heads with d_h = 2, o_1 = [1, 2] and o_2 = [0, -1], concatenated to
    k = 4 values, and a 4 x 3 W^O."""
    o = np.array([[[1.0, 2.0], [0.0, -1.0]]])  # [row][head][d_h]
    W = np.array([[1.0, 0.0, 2.0],
                  [0.0, 1.0, 1.0],
                  [5.0, 5.0, 5.0],
                  [3.0, -1.0, 0.0]])
    # u_0 = 1*1 + 2*0 + 0*5 + (-1)*3 = -2;  u_1 = 0 + 2 + 0 + 1 = 3;  u_2 = 2 + 2 + 0 + 0 = 4
    np.testing.assert_array_equal(oracle.output_project(o, W), [[-2.0, 3.0, 4.0]])


def test_output_projection_sums_per_head_blocks():
    """u = sum_i o_i W^O_i, where W^O_i is the block of d_h rows of W^O that
    multiplies head i (the per-head form the pages use to merge W^O with
    W_UV): the concatenated product equals the sum of the per-head ones."""
    rng = np.random.default_rng(32)
    h, d_h, d = 5, 6, 11
    o = rng.standard_normal((2, h, d_h))
    W = rng.standard_normal((h * d_h, d))
    whole = oracle.output_project(o, W)
    per_head = sum(oracle.output_project(o[:, i:i + 1, :], W[i * d_h:(i + 1) * d_h]) for i in range(h))
    np.testing.assert_allclose(whole, per_head, rtol=1e-12, atol=1e-12)


def test_output_projection_merges_with_the_value_up_projection():
    """W^O_i merged with W_UV[i] (the pages' W^OUV = W_UV W^O per head, in
    this file's column-vector convention W^OUV_i = W_UV[i]^T W^O_i) applied to
    c_bar gives the same u as the up-projection followed by W^O."""
    rng = np.random.default_rng(33)
    prob = _rand_problem(rng, h=3, d_c=8, d_r=4, d_h=5)
    o, cbar = oracle.decode_absorbed(prob, return_cbar=True)
    h, d_h, d_c = prob.w_uv.shape
    d = 7
    W = rng.standard_normal((h * d_h, d))
    u = oracle.output_project(o, W)  # [B, n_q, d]
    B, n_q = o.shape[:2]
    assert cbar.shape == (B, n_q, h, d_c)
    merged = np.zeros((B, n_q, d))
    for i in range(h):
        w_ouv = prob.w_uv[i].T @ W[i * d_h:(i + 1) * d_h]  # d_c x d
        merged += cbar[:, :, i, :] @ w_ouv
    np.testing.assert_allclose(u, merged, rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------------
# Decoupled RoPE and the current-token projections
# --------------------------------------------------------------------------
def test_rope_frequencies_closed_form():
    """theta_j = b^(-2 (j - 1) / d) ("MLA, dim by dim", RoPE paragraph)."""
    np.testing.assert_allclose(oracle.rope_thetas(4, 10000.0), [1.0, 0.01], rtol=1e-15)
    np.testing.assert_allclose(oracle.rope_thetas(8, 2.0), [1.0, 2 ** -0.25, 2 ** -0.5, 2 ** -0.75], rtol=1e-15)
    np.testing.assert_allclose(oracle.rope_thetas(64, 10000.0)[-1], 10000.0 ** (-62 / 64), rtol=1e-15)


def test_rope_is_a_rotation_per_pair():
    rng = np.random.default_rng(41)
    th = oracle.rope_thetas(16, 10000.0)
    x = rng.standard_normal(16)
    np.testing.assert_allclose(oracle.rope(x, 0, th), x, rtol=0, atol=0)  # position 0: identity
    for t in (1, 7, 100000):
        y = oracle.rope(x, t, th)
        for j in range(8):  # each adjacent pair keeps its length and turns by t theta_j
            a, b = x[2 * j:2 * j + 2], y[2 * j:2 * j + 2]
            assert abs(np.hypot(*a) - np.hypot(*b)) < 1e-12
            ang = math.atan2(b[1], b[0]) - math.atan2(a[1], a[0])
            assert abs(math.remainder(ang - t * th[j], 2 * math.pi)) < 1e-9
        # composition: rotating by a then by b is rotating by a + b
        np.testing.assert_allclose(oracle.rope(oracle.rope(x, t, th), 5, th), oracle.rope(x, t + 5, th),
                                   rtol=1e-10, atol=1e-12)


def test_rope_scores_depend_on_distance_only():
    """("From Vanilla Transformers ..." section 3.n): the score of a query at
    position t and a key at j equals the score of the query turned by t - j
    against the unrotated key."""
    rng = np.random.default_rng(42)
    th = oracle.rope_thetas(64, 10000.0)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for t, j in ((3, 2), (101, 100), (5000, 17)):
        left = oracle.dot(oracle.rope(q, t, th), oracle.rope(k, j, th))
        right = oracle.dot(oracle.rope(q, t - j, th), k)
        assert abs(left - right) <= 1e-10 * max(1.0, abs(left))


def test_cache_append_matches_matrix_products_and_paging():
    rng = np.random.default_rng(43)
    n, d_model, d_c, d_r, ps = 6, 9, 5, 4, 2
    x = rng.standard_normal((n, d_model))
    Wc, Wr = rng.standard_normal((d_c, d_model)), rng.standard_normal((d_r, d_model))
    th = oracle.rope_thetas(d_r, 10000.0)
    seq = np.array([0, 0, 1, 1, 1, 0], np.int32)
    pos = np.array([0, 1, 0, 1, 2, 2], np.int32)
    table = np.array([[3, 0], [1, 2]], np.int32)
    lat, rp = oracle.cache_append(x, Wc, Wr, seq, pos, th, table, ps, np.zeros((4, ps, d_c)), np.zeros((4, ps, d_r)))
    for r in range(n):
        page, row = table[seq[r], pos[r] // ps], pos[r] % ps
        np.testing.assert_allclose(lat[page, row], Wc @ x[r], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(rp[page, row], oracle.rope(Wr @ x[r], pos[r], th), rtol=1e-12, atol=1e-12)
    with pytest.raises(ValueError):  # a position past the page table
        oracle.cache_append(x[:1], Wc, Wr, [0], [4], th, table, ps, np.zeros((4, ps, d_c)), np.zeros((4, ps, d_r)))


def test_query_side_matches_matrix_products():
    rng = np.random.default_rng(44)
    n, d_model, d_qc, h, d_h, d_r = 3, 10, 6, 4, 5, 4
    x = rng.standard_normal((n, d_model))
    Wd = rng.standard_normal((d_qc, d_model))
    Wu, Wr = rng.standard_normal((h, d_h, d_qc)), rng.standard_normal((h, d_r, d_qc))
    pos = np.array([0, 9, 123], np.int32)
    th = oracle.rope_thetas(d_r, 10000.0)
    q, q_r = oracle.query_project(x, Wd, Wu, Wr, pos, th)
    for r in range(n):
        cq = Wd @ x[r]
        for i in range(h):
            np.testing.assert_allclose(q[r, i], Wu[i] @ cq, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(q_r[r, i], oracle.rope(Wr[i] @ cq, pos[r], th), rtol=1e-12, atol=1e-12)



# --------------------------------------------------------------------------
# Prefill: the explicit form with every prompt token as a query
# --------------------------------------------------------------------------
def test_prefill_is_causal_attention_over_rebuilt_keys_and_values():
    """A special case that reduces to a library routine: per head, causal
    scaled-dot-product attention (torch, float64, CPU) over keys
    [W_UK[i] c_t; k_R,t] and values W_UV[i] c_t equals the oracle's prefill
    ("MLA, dim by dim" section 4.1, the rebuilt K and V of prefill)."""
    import torch
    rng = np.random.default_rng(51)
    T, h, d_c, d_r, d_h = 23, 3, 12, 4, 6
    lat = rng.standard_normal((T, d_c)); rope = rng.standard_normal((T, d_r))
    q = rng.standard_normal((T, h, d_h)); q_r = rng.standard_normal((T, h, d_r))
    w_uk = rng.standard_normal((h, d_h, d_c)) / math.sqrt(d_c); w_uv = rng.standard_normal((h, d_h, d_c)) / math.sqrt(d_c)
    got = oracle.prefill(lat, rope, q, q_r, w_uk, w_uv)
    for i in range(h):
        K = np.concatenate([lat @ w_uk[i].T, rope], axis=1)
        V = lat @ w_uv[i].T
        Q = np.concatenate([q[:, i], q_r[:, i]], axis=1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q)[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None], is_causal=True,
            scale=1.0 / math.sqrt(d_h + d_r))[0].numpy()
        np.testing.assert_allclose(got[:, i], ref, rtol=1e-11, atol=1e-12)
    # listed heads only
    np.testing.assert_allclose(oracle.prefill(lat, rope, q, q_r, w_uk, w_uv, heads=[2, 0]), got[:, [2, 0]],
                               rtol=0, atol=0)
