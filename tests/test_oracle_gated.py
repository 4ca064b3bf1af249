"""Pins of the gated feed-forward oracle (CPU only).

"Sparser, Faster, Lighter Transformer Language Models", section "2. Metodologia", blocks
"Formato de Dados TwELL" (the gate activations are the sparse ones) and "Kernels de
Inferência" (per active unit: an up dot product, then the down multiply-add). Each pin
reaches the gated result through a path that does not call ``gated_ffn_fwd``'s formula.
"""
import numpy as np
import pytest

from oracle import twell_oracle as orc


def _layer(rng, T=7, d=12, f=20, bias=-0.3):
    x = rng.standard_normal((T, d))
    wgt = rng.standard_normal((f, d)) / np.sqrt(d)
    wut = rng.standard_normal((f, d)) / np.sqrt(d)
    w2 = rng.standard_normal((f, d)) / np.sqrt(f)
    bg = np.full(f, bias)
    return x, wgt, bg, wut, w2


def test_gate_equal_up_is_squared_relu():
    # Wu = Wg and no gate bias: gate * up = ReLU(z) * z = ReLU(z)^2, an FFN with a squared
    # ReLU, computed here with the plain oracle's pre-activation and ReLU.
    rng = np.random.default_rng(11)
    x, wgt, _, _, w2 = _layer(rng)
    zero = np.zeros(wgt.shape[0])
    y = orc.gated_ffn_fwd(x, wgt, zero, wgt, w2)[4]
    h_sq = orc.relu(orc.preact(x, wgt, zero)) ** 2
    np.testing.assert_allclose(y, h_sq @ w2, rtol=1e-12, atol=1e-12)


def test_unit_up_reduces_to_plain_ffn():
    # A constant-1 input column and up weights that read only that column make u = 1 for
    # every unit, so the gated layer is the plain ReLU layer of the gate weights.
    rng = np.random.default_rng(12)
    x, wgt, bg, _, w2 = _layer(rng)
    x[:, 0] = 1.0
    wut = np.zeros_like(wgt)
    wut[:, 0] = 1.0
    y = orc.gated_ffn_fwd(x, wgt, bg, wut, w2)[4]
    np.testing.assert_allclose(y, orc.ffn_fwd(x, wgt, bg, w2)[2], rtol=1e-12, atol=1e-12)


def test_brute_force_scalar_loops():
    rng = np.random.default_rng(13)
    x, wgt, bg, wut, w2 = _layer(rng, T=3, d=4, f=6, bias=0.1)
    T, d = x.shape
    f = wgt.shape[0]
    y_ref = np.zeros((T, d))
    for t in range(T):
        for j in range(f):
            zg = bg[j]
            u = 0.0
            for i in range(d):
                zg += x[t, i] * wgt[j, i]
                u += x[t, i] * wut[j, i]
            g = zg if zg > 0 else 0.0
            for c in range(d):
                y_ref[t, c] += g * u * w2[j, c]
    np.testing.assert_allclose(orc.gated_ffn_fwd(x, wgt, bg, wut, w2)[4], y_ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("bias", [-2.326, -0.5, 0.0])
def test_active_only_loop_equals_dense(bias):
    rng = np.random.default_rng(14)
    x, wgt, bg, wut, w2 = _layer(rng, T=9, d=16, f=64, bias=bias)
    _, g, _, _, y = orc.gated_ffn_fwd(x, wgt, bg, wut, w2)
    np.testing.assert_allclose(orc.gated_gather(g, x, wut, w2), y, rtol=1e-11, atol=1e-12)
    # and an inactive gate never contributes, whatever the up value
    wut2 = wut.copy()
    wut2[np.all(g == 0, axis=0)] *= 1e6
    np.testing.assert_allclose(orc.gated_ffn_fwd(x, wgt, bg, wut2, w2)[4], y, rtol=1e-11, atol=1e-12)
