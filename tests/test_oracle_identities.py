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
