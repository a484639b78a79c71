"""Pins of the fp64 oracle against values the pages print.

- "Mathematical Prerequisites for DeepSeek-V2": the worked numerical checks of
  sections 1-9 pin the primitives the oracle is built from.
- "From Vanilla Transformers to Modern LLMs ... Part 3", section 3: a complete
  hand-computable MLA decode step (2 heads, d_h = d_c = d_R = 2, 4 cached
  tokens) pins every step of both oracle forms, with and without the
  decoupled RoPE branch.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


P1 = _load("p1_examples.json")
P5 = _load("p5_toy_decode.json")


def _v(entry):
    return np.asarray(entry["value"] if isinstance(entry, dict) else entry, dtype=np.float64)


def _tol(entry):
    """Half a unit in the last printed decimal (plus a hair for the fp64 side)."""
    d = entry.get("decimals") if isinstance(entry, dict) else None
    return 0.0 if d is None else 0.5 * 10.0 ** (-d) + 1e-12


# --------------------------------------------------------------------------
# "Mathematical Prerequisites for DeepSeek-V2"
# --------------------------------------------------------------------------
def test_p1_matvec():
    np.testing.assert_array_equal(oracle.matvec(P1["A"], P1["x"]), _v(P1["Ax"]))


def test_p1_matvec_rejects_incompatible_shapes():
    with pytest.raises(ValueError):
        oracle.matvec(P1["A"], [1.0, 2.0])


def test_p1_transpose_and_product():
    A = np.asarray(P1["A"], dtype=float)
    # A^T e_j gives row j of A^T's columns: build A^T column by column
    AT = np.stack([oracle.matvec_t(A, e) for e in np.eye(2)], axis=1)
    np.testing.assert_array_equal(AT, _v(P1["AT"]))
    B = np.asarray(P1["B"], dtype=float)
    ATB = np.stack([oracle.matvec_t(A, B[:, j]) for j in range(2)], axis=1)
    np.testing.assert_array_equal(ATB, _v(P1["ATB"]))


def test_p1_associativity():
    A = np.asarray(P1["A"], dtype=float)
    B = np.asarray(P1["B"], dtype=float)
    z = np.asarray(P1["z"], dtype=float)
    Bz = oracle.matvec(B, z)
    np.testing.assert_array_equal(Bz, _v(P1["Bz"]))
    right = oracle.matvec_t(A, Bz)
    ATB = _v(P1["ATB"])
    left = oracle.matvec(ATB, z)
    np.testing.assert_array_equal(left, _v(P1["ATBz"]))
    np.testing.assert_array_equal(right, _v(P1["ATBz"]))


def test_p1_bilinear_identity():
    g = P1["bilinear"]
    Mb = oracle.matvec(g["M"], g["b"])
    np.testing.assert_array_equal(Mb, g["Mb"])
    MTa = oracle.matvec_t(g["M"], g["a"])
    np.testing.assert_array_equal(MTa, g["MTa"])
    assert oracle.dot(g["a"], Mb) == g["value"]
    assert oracle.dot(MTa, g["b"]) == g["value"]


def test_p1_linearity():
    g = P1["linearity"]
    a1, a2 = g["alpha"]
    mix = a1 * np.asarray(g["x1"], float) + a2 * np.asarray(g["x2"], float)
    left = oracle.matvec(g["W"], mix)
    np.testing.assert_allclose(left, g["value"], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(oracle.matvec(g["W"], g["x2"]), g["Wx2"])
    right = a1 * oracle.matvec(g["W"], g["x1"]) + a2 * oracle.matvec(g["W"], g["x2"])
    np.testing.assert_allclose(right, g["value"], rtol=0, atol=1e-12)


def test_p1_low_rank():
    g = P1["low_rank"]
    c = oracle.dot(g["V"], g["x"])
    assert c == g["c"]
    np.testing.assert_array_equal(oracle.matvec(g["W"], g["x"]), g["value"])
    np.testing.assert_array_equal(c * np.asarray(g["U"], float), g["value"])


def test_p1_concat_dot():
    g = P1["concat_dot"]
    assert oracle.dot(g["a"], g["c"]) == g["ac"]
    assert oracle.dot(g["b"], g["d"]) == g["bd"]
    assert oracle.dot(g["a"] + g["b"], g["c"] + g["d"]) == g["value"]


# --------------------------------------------------------------------------
# "From Vanilla Transformers to Modern LLMs ... Part 3", section 3
# --------------------------------------------------------------------------
def _toy_weights(key):
    """Head i's d_h x d_c weight = transpose of the page's column slice."""
    W = _v(P5[key])  # d_c x (h * d_h)
    return np.stack([W[:, 2 * i:2 * i + 2].T for i in range(2)])  # [h][d_h][d_c]


W_UK = _toy_weights("W_UK_page")
W_UV = _toy_weights("W_UV_page")
C = _v(P5["latents"])
KR = _v(P5["rope_keys_rotated"])
Q = _v(P5["q"])
QR = _v(P5["q_rope_rotated"])


def test_p5_naive_keys_and_values():
    for i in range(2):
        for t in range(4):
            np.testing.assert_array_equal(oracle.matvec(W_UK[i], C[t]), _v(P5["keys_naive"])[i, t])
    for t in range(4):
        np.testing.assert_array_equal(oracle.matvec(W_UV[0], C[t]), _v(P5["values_naive_head1"])[t])


def test_p5_absorbed_query():
    for i in range(2):
        np.testing.assert_array_equal(oracle.absorb_query(W_UK[i], Q[i]), _v(P5["q_abs"])[i])


def test_p5_scores_content_rope_and_sum():
    for i in range(2):
        qa = oracle.absorb_query(W_UK[i], Q[i])
        content = oracle.latent_scores(qa, None, C, None, 1.0)
        np.testing.assert_array_equal(content, _v(P5["content_scores"])[i])
        rope = oracle.latent_scores(np.zeros(2), QR[i], np.zeros_like(C), KR, 1.0)
        np.testing.assert_array_equal(rope, _v(P5["rope_scores"])[i])
        summed = oracle.latent_scores(qa, QR[i], C, KR, 1.0)
        np.testing.assert_array_equal(summed, _v(P5["summed_scores"])[i])
        scaled = oracle.latent_scores(qa, QR[i], C, KR, P5["scale"]["value"])
        np.testing.assert_array_equal(scaled, _v(P5["scaled_scores"])[i])


def test_p5_softmax_weighted_latent_and_output():
    for i in range(2):
        qa = oracle.absorb_query(W_UK[i], Q[i])
        s = oracle.latent_scores(qa, QR[i], C, KR, 0.5)
        p = oracle.softmax(s)
        np.testing.assert_allclose(p, _v(P5["softmax"])[i], rtol=0, atol=_tol(P5["softmax"]))
        cb = oracle.weighted_latent(p, C)
        np.testing.assert_allclose(cb, _v(P5["c_bar"])[i], rtol=0, atol=_tol(P5["c_bar"]))
        o = oracle.up_project(W_UV[i], cb)
        np.testing.assert_allclose(o, _v(P5["o"])[i], rtol=0, atol=_tol(P5["o"]))


def _toy_problem(page_size=4, permute=False, scale=0.5, rope=True):
    latent = C.copy()
    rope_rows = KR.copy() if rope else np.zeros_like(KR)
    n_pages = 4 // page_size
    order = np.arange(n_pages)
    if permute:
        order = np.array([2, 0, 3, 1])[:n_pages] if n_pages == 4 else order[::-1]
    pool_c = np.zeros((n_pages, page_size, 2))
    pool_r = np.zeros((n_pages, page_size, 2))
    table = np.zeros((1, n_pages), dtype=np.int32)
    for j in range(n_pages):
        pool_c[order[j]] = latent[j * page_size:(j + 1) * page_size]
        pool_r[order[j]] = rope_rows[j * page_size:(j + 1) * page_size]
        table[0, j] = order[j]
    return oracle.Problem(
        q=Q.reshape(1, 1, 2, 2), q_r=(QR if rope else np.zeros_like(QR)).reshape(1, 1, 2, 2),
        latent_pool=pool_c, rope_pool=pool_r, page_table=table,
        context_lens=np.array([4], np.int32), w_uk=W_UK, w_uv=W_UV, scale=scale)


@pytest.mark.parametrize("page_size,permute", [(4, False), (2, True), (1, True)])
@pytest.mark.parametrize("form", ["explicit", "absorbed"])
def test_p5_whole_decode_with_rope(form, page_size, permute):
    prob = _toy_problem(page_size, permute)
    fn = oracle.decode_explicit if form == "explicit" else oracle.decode_absorbed
    o = fn(prob)[0, 0]
    np.testing.assert_allclose(o, _v(P5["o"]), rtol=0, atol=_tol(P5["o"]))
    # output projection of the next step (u_4 = [o_1; o_2] W^O) -- checks the
    # head order of the output as the page concatenates it
    u4 = oracle.output_project(o, _v(P5["W_O"]))
    np.testing.assert_allclose(u4, _v(P5["u4"]), rtol=0, atol=2 * _tol(P5["u4"]))


@pytest.mark.parametrize("which", ["with_rope", "content_only"])
def test_p5_output_projection_of_the_printed_head_outputs(which):
    """Section 3.h (content only) and 3.p (with RoPE): u_4 = [o_1; o_2] W^O
    from the head outputs as printed.  W^O is 0/1, so the printed u_4 follows
    exactly: its first four entries repeat o_1 and o_2, its fifth is the sum
    of the first and the last."""
    g = P5 if which == "with_rope" else P5["content_only"]
    o = _v(g["o"])  # [[o_1], [o_2]] as printed
    u4 = oracle.output_project(o, _v(P5["W_O"]))
    assert u4.shape == (5,)
    np.testing.assert_allclose(u4, _v(g["u4"]), rtol=0, atol=1e-12)


@pytest.mark.parametrize("form", ["explicit", "absorbed"])
def test_p5_whole_decode_content_only(form):
    g = P5["content_only"]
    prob = _toy_problem(4, False, scale=1.0 / math.sqrt(g["scale_sqrt_inverse_of"]), rope=False)
    fn = oracle.decode_explicit if form == "explicit" else oracle.decode_absorbed
    o = fn(prob)[0, 0]
    np.testing.assert_allclose(o, _v(g["o"]), rtol=0, atol=_tol(g["o"]))
    u4 = oracle.output_project(o, _v(P5["W_O"]))
    np.testing.assert_allclose(u4, _v(g["u4"]), rtol=0, atol=2 * _tol(g["u4"]))


def test_p5_content_only_steps():
    g = P5["content_only"]
    scale = 1.0 / math.sqrt(g["scale_sqrt_inverse_of"])
    for i in range(2):
        qa = oracle.absorb_query(W_UK[i], Q[i])
        s = oracle.latent_scores(qa, None, C, None, scale)
        np.testing.assert_allclose(s, _v(g["scaled_scores"])[i], rtol=0, atol=_tol(g["scaled_scores"]))
        p = oracle.softmax(s)
        np.testing.assert_allclose(p, _v(g["softmax"])[i], rtol=0, atol=_tol(g["softmax"]))
        cb = oracle.weighted_latent(p, C)
        np.testing.assert_allclose(cb, _v(g["c_bar"])[i], rtol=0, atol=_tol(g["c_bar"]))


def test_p5_absorbed_returns_cbar():
    prob = _toy_problem()
    _, cb = oracle.decode_absorbed(prob, return_cbar=True)
    np.testing.assert_allclose(cb[0, 0], _v(P5["c_bar"]), rtol=0, atol=_tol(P5["c_bar"]))


# --------------------------------------------------------------------------
# The current-token projections of the toy (the cache rows and the query
# the decode step reads), and the whole chain from the hidden states to u_4
# --------------------------------------------------------------------------
PJ = _load("p5_toy_projections.json")
_HID = _v(PJ["hidden"])
_POS = np.asarray(PJ["positions"]["value"], dtype=np.int32)
_THETA_TOY = np.array([math.pi / 2])  # one pair, 90 degrees per position


def _heads_of(m):
    """A d_model x (h d) page matrix whose head i owns columns d i .. d i + d - 1
    -> [h][d][d_model] (column-vector convention)."""
    m = np.asarray(m, dtype=np.float64)
    return np.stack([m[:, 2 * i:2 * i + 2].T for i in range(m.shape[1] // 2)])


def test_p5_rope_rotations():
    """Sections 3.k, 3.l and 3.i: 90 degrees per position."""
    for t, (k0, k1) in enumerate(zip(_v(PJ["rope_keys_unrotated"]), _v(PJ["rope_keys_rotated"]))):
        np.testing.assert_allclose(oracle.rope(k0, t, _THETA_TOY), k1, rtol=0, atol=1e-12)
    for q0, q1 in zip(_v(PJ["q_rope_unrotated"]), _v(PJ["q_rope_rotated"])):
        np.testing.assert_allclose(oracle.rope(q0, 3, _THETA_TOY), q1, rtol=0, atol=1e-12)
    for steps, q1 in zip((3, 2, 1, 0), _v(PJ["q_head1_rotated_by_distance"])):
        np.testing.assert_allclose(oracle.rope([1, 2], steps, _THETA_TOY), q1, rtol=0, atol=1e-12)


@pytest.mark.parametrize("page_size,permute", [(4, False), (1, True), (2, True)])
def test_p5_cache_append(page_size, permute):
    """Sections 3.b and 3.k: the four tokens' latents and rotated RoPE keys
    land in their pages."""
    pages = 4 // page_size
    order = np.random.default_rng(3).permutation(pages) if permute else np.arange(pages)
    table = order.reshape(1, pages).astype(np.int32)
    lat0 = np.full((pages, page_size, 2), np.nan)
    rp0 = np.full((pages, page_size, 2), np.nan)
    lat, rp = oracle.cache_append(_HID, _v(PJ["W_DKV"]).T, _v(PJ["W_KR"]).T, np.zeros(4, np.int32), _POS,
                                  _THETA_TOY, table, page_size, lat0, rp0)
    for t in range(4):
        page, row = table[0, t // page_size], t % page_size
        np.testing.assert_allclose(lat[page, row], _v(PJ["latents"])[t], rtol=0, atol=1e-12)
        np.testing.assert_allclose(rp[page, row], _v(PJ["rope_keys_rotated"])[t], rtol=0, atol=1e-12)
    assert np.isnan(lat0).all()  # the inputs are left alone


def test_p5_query_side():
    """Sections 3.d and 3.l: the query of token 4 (position 3), with the
    toy's query latent equal to the hidden state."""
    q, q_r = oracle.query_project(_HID[3:4], np.eye(5), _heads_of(PJ["W_Q"]["value"]),
                                  _heads_of(PJ["W_QR"]["value"]), np.array([3], np.int32), _THETA_TOY)
    np.testing.assert_allclose(q[0], _v(PJ["q"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(q_r[0], _v(PJ["q_rope_rotated"]), rtol=0, atol=1e-12)


@pytest.mark.parametrize("form", ["explicit", "absorbed"])
def test_p5_from_hidden_states_to_u4(form):
    """The whole toy step from the hidden states: cache append (3.b, 3.k),
    query side (3.d, 3.l), decode with scale 1/2 (3.o, 3.p) and the output
    projection (3.p): the printed o and u_4."""
    table = np.array([[2, 0, 3, 1]], np.int32)  # one token per page, shuffled
    lat, rp = oracle.cache_append(_HID, _v(PJ["W_DKV"]).T, _v(PJ["W_KR"]).T, np.zeros(4, np.int32), _POS,
                                  _THETA_TOY, table, 1, np.zeros((4, 1, 2)), np.zeros((4, 1, 2)))
    q, q_r = oracle.query_project(_HID[3:4], np.eye(5), _heads_of(PJ["W_Q"]["value"]),
                                  _heads_of(PJ["W_QR"]["value"]), np.array([3], np.int32), _THETA_TOY)
    prob = oracle.Problem(q=q.reshape(1, 1, 2, 2), q_r=q_r.reshape(1, 1, 2, 2), latent_pool=lat, rope_pool=rp,
                          page_table=table, context_lens=np.array([4], np.int32), w_uk=W_UK, w_uv=W_UV, scale=0.5)
    fn = oracle.decode_explicit if form == "explicit" else oracle.decode_absorbed
    o = fn(prob)[0, 0]
    np.testing.assert_allclose(o, _v(P5["o"]), rtol=0, atol=_tol(P5["o"]))
    np.testing.assert_allclose(oracle.output_project(o, _v(P5["W_O"])), _v(P5["u4"]), rtol=0,
                               atol=2 * _tol(P5["u4"]))
