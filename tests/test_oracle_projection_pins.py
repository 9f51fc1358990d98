"""Pins for the projection oracle (oracle/projections.py): weights that route
single hidden channels give outputs known exactly by indexing, closed forms
for beta, the rank bound of a low-rank product, and row independence.  Each
is chosen so that a plausible mistake fails it: a transposed or swapped
weight, the wrong [T, H, dk] split of the output, a sign in the sigmoid, a
product that skips the rank-r factor.

Passages: "Kimi K3 Metal Gap Analysis", §2 KDA Attention, rows "Decay
compute" (W_fb W_fa x) and "O projection" (W_o and W_g around the per-head
RMSNorm and gate); "Metal (Apple GPU) backend for Kimi K3", table "What runs
where (per layer)" (fa, fb and bp are fp32 low-rank products).
"""
import math

import numpy as np
import pytest

from oracle.projections import gate_projection, lowrank_gates, output_projection


def _int_rows(rng, T, D):
    # small integers: every product and sum below is exact in fp64
    return rng.integers(-8, 9, size=(T, D)).astype(np.float64)


def _routing(D, r, H, dk, rng):
    """W_fa picks hidden channel pa[j] for rank slot j; W_fb row (h, i) takes
    c[h, i] times rank slot pb[h, i]."""
    pa = rng.permutation(D)[:r]
    pb = rng.integers(0, r, size=(H, dk))
    c = rng.integers(1, 6, size=(H, dk)) * rng.choice([-1, 1], size=(H, dk))
    w_fa = np.zeros((r, D))
    w_fa[np.arange(r), pa] = 1.0
    w_fb = np.zeros((H * dk, r))
    for h in range(H):
        for i in range(dk):
            w_fb[h * dk + i, pb[h, i]] = c[h, i]
    return w_fa, w_fb, pa, pb, c


def test_lowrank_routing_weights_select_hidden_channels():
    rng = np.random.default_rng(11)
    T, D, r, H, dk = 6, 7, 5, 3, 4
    x = _int_rows(rng, T, D)
    w_fa, w_fb, pa, pb, c = _routing(D, r, H, dk, rng)
    f, beta = lowrank_gates(x, w_fa, w_fb, np.zeros((H, D)))
    assert f.shape == (T, H, dk) and beta.shape == (T, H)
    for t in range(T):
        for h in range(H):
            for i in range(dk):
                assert f[t, h, i] == c[h, i] * x[t, pa[pb[h, i]]]
    assert np.all(beta == 0.5)


def test_lowrank_rows_with_two_terms():
    rng = np.random.default_rng(12)
    T, D, r, H, dk = 5, 6, 3, 2, 3
    x = _int_rows(rng, T, D)
    w_fa = np.zeros((r, D))
    w_fa[0, 4] = 1.0
    w_fa[1, 0] = 2.0
    w_fa[2, 5] = -1.0
    w_fb = np.zeros((H * dk, r))
    w_fb[1 * dk + 2, 0] = 2.0          # head 1, channel 2: 2 a0 - 3 a2
    w_fb[1 * dk + 2, 2] = -3.0
    w_fb[0 * dk + 0, 1] = 0.5          # head 0, channel 0: a1 / 2
    f, _ = lowrank_gates(x, w_fa, w_fb, np.zeros((H, D)))
    np.testing.assert_array_equal(f[:, 1, 2], 2.0 * x[:, 4] - 3.0 * (-x[:, 5]))
    np.testing.assert_array_equal(f[:, 0, 0], 0.5 * (2.0 * x[:, 0]))
    mask = np.ones((H, dk), bool)
    mask[1, 2] = mask[0, 0] = False
    assert np.all(f[:, mask] == 0.0)


def test_beta_closed_forms():
    rng = np.random.default_rng(13)
    T, D, H = 7, 5, 3
    x = rng.normal(size=(T, D))
    w_fa, w_fb = np.zeros((2, D)), np.zeros((H * 2, 2))
    j = [3, 0, 4]
    cs = [1.5, -2.0, 0.25]
    w_bp = np.zeros((H, D))
    for h in range(H):
        w_bp[h, j[h]] = cs[h]
    _, beta = lowrank_gates(x, w_fa, w_fb, w_bp)
    for t in range(T):
        for h in range(H):
            z = cs[h] * x[t, j[h]]
            assert beta[t, h] == pytest.approx(1.0 / (1.0 + math.exp(-z)), rel=1e-15)
    # sigmoid(z) + sigmoid(-z) = 1, and beta rises with z
    _, beta_neg = lowrank_gates(-x, w_fa, w_fb, w_bp)
    np.testing.assert_allclose(beta + beta_neg, 1.0, rtol=0, atol=1e-15)
    _, b_hi = lowrank_gates(np.full((1, D), 1.0), w_fa, w_fb, np.full((1, D), 1.0))
    _, b_lo = lowrank_gates(np.full((1, D), 1.0), w_fa, w_fb, np.full((1, D), -1.0))
    assert b_hi[0, 0] > 0.99 and b_lo[0, 0] < 0.01


def test_lowrank_output_has_rank_at_most_r():
    rng = np.random.default_rng(14)
    T, D, r, H, dk = 60, 40, 6, 4, 8
    x = rng.normal(size=(T, D))
    w_fa = rng.normal(size=(r, D))
    w_fb = rng.normal(size=(H * dk, r))
    f, _ = lowrank_gates(x, w_fa, w_fb, np.zeros((H, D)))
    s = np.linalg.svd(f.reshape(T, H * dk), compute_uv=False)
    assert s[r] < 1e-10 * s[0]          # nothing beyond the rank-r factor
    assert s[r - 1] > 1e-3 * s[0]       # and the factor is used in full


def test_gate_projection_routing():
    rng = np.random.default_rng(15)
    T, D, HD = 4, 6, 10
    x = _int_rows(rng, T, D)
    src = rng.integers(0, D, size=HD)
    sc = rng.integers(1, 5, size=HD) * rng.choice([-1, 1], size=HD)
    w_g = np.zeros((HD, D))
    w_g[np.arange(HD), src] = sc
    g = gate_projection(x, w_g)
    assert g.shape == (T, HD)
    for c in range(HD):
        np.testing.assert_array_equal(g[:, c], sc[c] * x[:, src[c]])


def test_output_projection_routing_and_head_order():
    rng = np.random.default_rng(16)
    T, H, dv, D = 3, 2, 4, 5
    y = rng.integers(-8, 9, size=(T, H, dv)).astype(np.float64)
    # out[:, d] takes head hs[d], channel cs[d]: the flattening must be head-major
    hs = [1, 0, 1, 0, 1]
    cs = [3, 0, 0, 2, 1]
    w_o = np.zeros((D, H * dv))
    for d in range(D):
        w_o[d, hs[d] * dv + cs[d]] = d + 1.0
    out = output_projection(y, w_o)
    assert out.shape == (T, D)
    for d in range(D):
        np.testing.assert_array_equal(out[:, d], (d + 1.0) * y[:, hs[d], cs[d]])


@pytest.mark.parametrize("fn", ["lowrank", "gate", "out"])
def test_rows_are_independent(fn):
    # any subset of token rows gives those rows of the full result, bit for bit
    rng = np.random.default_rng(17)
    T, D, r, H, dk = 23, 12, 4, 2, 3
    x = rng.normal(size=(T, D))
    rows = np.array([0, 5, 22, 9])
    if fn == "lowrank":
        ws = (rng.normal(size=(r, D)), rng.normal(size=(H * dk, r)), rng.normal(size=(H, D)))
        full, sub = lowrank_gates(x, *ws), lowrank_gates(x[rows], *ws)
        for a, b in zip(full, sub):
            np.testing.assert_array_equal(a[rows], b)
    elif fn == "gate":
        w = rng.normal(size=(H * dk, D))
        np.testing.assert_array_equal(gate_projection(x, w)[rows], gate_projection(x[rows], w))
    else:
        w = rng.normal(size=(7, D))
        np.testing.assert_array_equal(output_projection(x, w)[rows], output_projection(x[rows], w))


def test_shape_mismatch_is_refused():
    x = np.zeros((2, 6))
    with pytest.raises(AssertionError):
        lowrank_gates(x, np.zeros((6, 3)), np.zeros((4, 3)), np.zeros((2, 6)))   # W_fa transposed
    with pytest.raises(AssertionError):
        gate_projection(x, np.zeros((6, 5)))                                      # W_g transposed
