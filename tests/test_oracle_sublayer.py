"""Pins of the sublayer oracle (low-rank queries, grouped output projection) to
facts fixed outside it: the pages' dimension and parameter-count figures
(tests/golden/sublayer_dims.json, with its citation), hand-worked values, and
identities of linear algebra checked through an independent construction
(a block-diagonal matrix built by scipy).  CPU only."""
import json
import os

import numpy as np
import pytest
import scipy.linalg

from oracle import sublayer as osl

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def dims():
    with open(os.path.join(GOLD, "sublayer_dims.json")) as f:
        return json.load(f)["stated"]


def _count(shapes, names):
    return sum(int(np.prod(shapes[n])) for n in names)


@pytest.mark.parametrize("model", ["flash", "pro"])
def test_grouped_projection_parameter_counts(model):
    s = dims()
    m, ix = s[model], s["indexer"]
    shapes = osl.weight_shapes(m["d"], m["d_c"], m["n_h"], m["c"], ix["n_I"], ix["c_I"], m["g"], m["d_g"])
    assert shapes["w_o1"][2] == m["group_width"] and shapes["w_o1"][0] * shapes["w_o1"][2] == m["concat_width"]
    grouped = _count(shapes, ["w_o1", "w_o2"])
    direct = m["concat_width"] * m["d"]
    if model == "flash":
        assert grouped * 2 == direct                                 # exactly half
    else:
        assert round(100 * grouped / direct, 1) == m["grouped_over_direct_percent"]
        assert round(100 - 100 * grouped / direct, 1) == m["reduction_percent"]
        assert abs((direct - grouped) - m["saved_params_approx"]) < 0.5e6


def test_grouped_projection_is_one_rank_limited_direct_projection():
    """No nonlinearity between the two stages: the sublayer equals one direct projection
    by blockdiag(W1_0^T .. W1_{g-1}^T) W2^T, of rank at most g d_g."""
    rng = np.random.default_rng(7)
    g, c, d_g, d, T = 3, 4, 5, 11, 9
    o = rng.standard_normal((T, 8 * g * c))
    w1 = rng.standard_normal((g, d_g, 8 * c))
    w2 = rng.standard_normal((d, g * d_g))
    y = osl.grouped_out_proj(o, w1, w2, act="f64")["y"]
    w_eff = scipy.linalg.block_diag(*[w1[j].T for j in range(g)]) @ w2.T      # [8 g c, d]
    assert np.allclose(y, o @ w_eff, rtol=1e-12, atol=1e-12)
    assert np.linalg.matrix_rank(w_eff) <= g * d_g


def test_identity_group_projections_give_the_direct_projection():
    rng = np.random.default_rng(8)
    g, c, d, T = 2, 3, 7, 5
    o = rng.standard_normal((T, 8 * g * c))
    w1 = np.stack([np.eye(8 * c)] * g)                               # d_g = 8 c, identity
    w2 = rng.standard_normal((d, g * 8 * c))
    r = osl.grouped_out_proj(o, w1, w2, act="f64")
    assert np.array_equal(r["u"], o)
    assert np.allclose(r["y"], np.einsum("tk,dk->td", o, w2), rtol=1e-12, atol=1e-12)


def test_each_group_reads_its_own_eight_heads():
    """Perturbing the heads of group j moves only u's block j (heads 8j .. 8j+7)."""
    rng = np.random.default_rng(9)
    g, c, d_g, d, T = 4, 2, 3, 5, 3
    o = rng.standard_normal((T, 8 * g * c))
    w1 = rng.standard_normal((g, d_g, 8 * c))
    w2 = rng.standard_normal((d, g * d_g))
    base = osl.grouped_out_proj(o, w1, w2, act="f64")["u"]
    for j in range(g):
        o2 = o.copy()
        o2[:, 8 * c * j:8 * c * (j + 1)] += 1.0
        u2 = osl.grouped_out_proj(o2, w1, w2, act="f64")["u"]
        moved = np.abs(u2 - base).max(0) > 0
        assert moved[j * d_g:(j + 1) * d_g].all() and not np.delete(moved, np.s_[j * d_g:(j + 1) * d_g]).any()


def test_low_rank_query_worked_by_hand():
    """d = 2, d_c = 1: h = (1, 2), W^DQ = [3 4] gives c = 11; W^UQ = (1, -2)^T gives q = (11, -22);
    W^IUQ = (0.5) gives q^I = 5.5; W^w = [[1 0], [0 -1]] gives w = (1, -2)."""
    r = osl.low_rank_query(np.array([[1.0, 2.0]]), np.array([[3.0, 4.0]]), np.array([[1.0], [-2.0]]),
                           np.array([[0.5]]), np.array([[1.0, 0.0], [0.0, -1.0]]), act="f64")
    assert r["c"].tolist() == [[11.0]] and r["q"].tolist() == [[11.0, -22.0]]
    assert r["qI"].tolist() == [[5.5]] and r["w"].tolist() == [[1.0, -2.0]]


def test_both_query_sets_come_from_one_latent_and_w_from_h():
    rng = np.random.default_rng(10)
    T, d, d_c, nq, ni = 40, 16, 6, 24, 3
    h = rng.standard_normal((T, d))
    w_dq, w_uq = rng.standard_normal((d_c, d)), rng.standard_normal((nq, d_c))
    w_w = rng.standard_normal((ni, d))
    r = osl.low_rank_query(h, w_dq, w_uq, w_uq[:10], w_w, act="f64")
    assert np.array_equal(r["qI"], r["q"][:, :10])                   # same latent, same rows -> same queries
    assert np.linalg.matrix_rank(r["q"]) <= d_c < min(T, nq)         # q lives in the latent's span
    r2 = osl.low_rank_query(h, 2.0 * w_dq, w_uq, w_uq[:10], w_w, act="f64")
    assert np.array_equal(r2["w"], r["w"]) and np.allclose(r2["q"], 2.0 * r["q"])
    # basis inputs pick columns: h = e_i gives c = W^DQ[:, i] and w = W^w[:, i]
    e = np.eye(d)
    rb = osl.low_rank_query(e, w_dq, w_uq, w_uq[:10], w_w, act="f64")
    assert np.array_equal(rb["c"], w_dq.T) and np.array_equal(rb["w"], w_w.T)


def test_stored_latent_is_bfloat16_round_to_nearest_even():
    """bf16 keeps 8 significant bits: 1 + 2^-8 is a tie and goes to the even 1.0, 1 + 3 * 2^-8
    goes up to 1 + 2^-6; w^I is stored in fp32."""
    r = osl.low_rank_query(np.array([[1.0]]), np.array([[1.0 + 2.0 ** -8], [1.0 + 3 * 2.0 ** -8]]),
                           np.eye(2), np.eye(2), np.array([[1.0 + 2.0 ** -30]]), act="bf16")
    assert r["c"].tolist() == [[1.0, 1.0 + 2.0 ** -6]]
    assert r["w"].tolist() == [[1.0]]
