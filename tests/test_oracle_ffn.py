"""Pins of the oracle's dense forward (z, h, y) to facts fixed independently of its code:
a worked example computed by hand, exact special cases (identity and one-hot weights, a
single active unit), exactness on an integer grid, and the analytic activity rate."""
import math

import numpy as np
import pytest

import synth
from oracle import twell_oracle as orc


def test_worked_example_by_hand():
    # T=2 tokens, d=3, f=4, d_out=2. Every value below was computed by hand:
    #   z[0] = [1*1, .5+1-1-1, -1+2+.5, -1-2] = [1, -0.5, 1.5, -3]
    #   z[1] = [0, -.5+3-1, -1+.5, 3-2]       = [0, 1.5, -0.5, 1]
    #   h    = ReLU(z) with z == 0 inactive
    #   y[0] = 1*[1,-1] + 1.5*[0,4] = [1, 5];  y[1] = 1.5*[2,0] + 1*[-1,1] = [2, 1]
    x = np.array([[1, 2, -1], [0, -1, 3]], float)
    w1t = np.array([[1, 0, 0], [0.5, 0.5, 1], [-1, 1, 0], [0, 0, 1]], float)
    b1 = np.array([0, -1, 0.5, -2], float)
    w2 = np.array([[1, -1], [2, 0], [0, 4], [-1, 1]], float)
    z, h, y = orc.ffn_fwd(x, w1t, b1, w2)
    assert z.tolist() == [[1, -0.5, 1.5, -3], [0, 1.5, -0.5, 1]]
    assert h.tolist() == [[1, 0, 1.5, 0], [0, 1.5, 0, 1]]
    assert y.tolist() == [[1, 5], [2, 1]]


def test_identity_weights_give_x_plus_b():
    rng = np.random.default_rng(5)
    d = 48
    x = rng.standard_normal((7, d))
    b1 = rng.standard_normal(d)
    z = orc.preact(x, np.eye(d), b1)
    assert np.array_equal(z, x + b1[None, :])


def test_one_hot_tokens_select_weight_columns():
    rng = np.random.default_rng(6)
    d, f = 16, 24
    w1t = rng.standard_normal((f, d))
    b1 = rng.standard_normal(f)
    x = np.zeros((d, d))
    x[np.arange(d), np.arange(d)] = 1.0          # token i = e_i
    z = orc.preact(x, w1t, b1)
    for i in range(d):
        # z[i, j] = w1t[j, i] + b1[j]: column i of every unit's weight vector
        assert np.array_equal(z[i], w1t[:, i] + b1)


def test_single_active_unit_is_one_product():
    rng = np.random.default_rng(7)
    f, d = 32, 10
    h = np.zeros((3, f))
    h[0, 5] = 1.75
    h[2, 31] = 0.5
    w2 = rng.standard_normal((f, d))
    y = h @ w2
    assert np.array_equal(y[0], 1.75 * w2[5])
    assert np.array_equal(y[1], np.zeros(d))
    assert np.array_equal(y[2], 0.5 * w2[31])
    assert np.array_equal(orc.gather_rows(h, w2), y)


def test_sparse_rows_equal_dense_product():
    rng = np.random.default_rng(8)
    h = orc.relu(rng.standard_normal((6, 40)) - 1.5)
    w2 = rng.standard_normal((40, 9))
    assert np.allclose(orc.gather_rows(h, w2), h @ w2, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_integer_grid_is_exact(dtype):
    g = synth.integer_grid(T=24, d=256, f=512, seed=11, dtype=dtype)
    x = orc.widen(g["x"], dtype)
    w1t = orc.widen(g["w1t"], dtype)
    w2 = orc.widen(g["w2"], dtype)
    b1 = g["b1"].astype(np.float64)
    z, h, y = orc.ffn_fwd(x, w1t, b1, w2)
    # Exact integer arithmetic: x = xi/4, w = wi/64, b = bi/256  ->  z = (xi.wi + bi)/256.
    xi = np.rint(x * 4).astype(np.int64)
    wi = np.rint(w1t * 64).astype(np.int64)
    bi = np.rint(b1 * 256).astype(np.int64)
    zi = xi @ wi.T + bi[None, :]
    assert np.array_equal(z * 256, zi.astype(np.float64))
    # fp32 evaluation in a different order is exact too (all partial sums on the grid)
    z32 = (x.astype(np.float32)[:, ::-1] @ w1t.astype(np.float32)[:, ::-1].T) + b1.astype(np.float32)
    assert np.array_equal(z32.astype(np.float64), z)
    assert 0.01 < (h > 0).mean() < 0.2
    assert np.array_equal(orc.gather_rows(h, w2), y)


def _density_check(w, T):
    g = synth.generate(w, T=T)
    x = orc.widen(g["x"], w.dtype)
    w1t = orc.widen(g["w1t"], w.dtype)
    b1 = g["b1"].astype(np.float64)
    h = orc.relu(orc.preact(x, w1t, b1))
    p = orc.p_active(b1, w1t)
    # Per-token variance: binomial part + the shared scale |x_t|/sqrt(d) (sd ~ 1/sqrt(2d)),
    # which moves every unit's probability of the token together.
    nrm = np.sqrt((w1t ** 2).sum(1))
    a = -b1 / nrm
    dp_ds = np.exp(-a * a / 2) / math.sqrt(2 * math.pi) * a
    var_tok = (p * (1 - p)).sum() + dp_ds.sum() ** 2 / (2 * w.d)
    sigma = math.sqrt(T * var_tok)
    measured = (h > 0).sum()
    expected = T * p.sum()
    assert abs(measured - expected) < 5 * sigma, (measured, expected, sigma)
    return measured / (T * w.f), p.mean()


def test_density_matches_analytic_c1():
    dens, p = _density_check(synth.C1, synth.C1.T)
    assert abs(p - 0.0101) < 0.001


def test_density_matches_analytic_c2_sample():
    dens, p = _density_check(synth.C2, 256)
    assert abs(p - 0.01003) < 0.0005


def test_density_detects_wrong_bias_sign():
    # A planted mistake (bias sign flipped) must fail the analytic check.
    w = synth.C1
    g = synth.generate(w)
    x = orc.widen(g["x"], w.dtype)
    w1t = orc.widen(g["w1t"], w.dtype)
    b1 = g["b1"].astype(np.float64)
    h_bad = orc.relu(orc.preact(x, w1t, -b1))
    assert (h_bad > 0).mean() > 0.9
    assert orc.p_active(b1, w1t).mean() < 0.02


def test_z_error_bound_holds_for_fp32_evaluation():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((16, 512)).astype(np.float32)
    w1t = (rng.standard_normal((64, 512)) / 16).astype(np.float32)
    b1 = rng.standard_normal(64).astype(np.float32)
    z64 = orc.preact(x.astype(np.float64), w1t.astype(np.float64), b1.astype(np.float64))
    beta = orc.z_error_bound(x.astype(np.float64), w1t.astype(np.float64), b1.astype(np.float64))
    # sequential fp32 accumulation (worst order for error growth)
    acc = np.zeros((16, 64), np.float32)
    for i in range(512):
        acc = acc + x[:, i:i + 1] * w1t[:, i][None, :]
    z32 = (acc + b1).astype(np.float64)
    assert np.all(np.abs(z32 - z64) <= beta)
    assert np.abs(z32 - z64).max() > 0       # the check is not vacuous
