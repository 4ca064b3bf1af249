"""Pins of the oracle's analytic helpers (Poisson-binomial tail, expected overflow rows,
activity probability) against textbook special cases and brute force."""
import itertools
import math

import numpy as np
import pytest
from scipy import stats

import synth
from oracle import twell_oracle as orc


def test_poisson_binomial_equal_p_is_binomial():
    for n, p, k in [(128, 0.01, 8), (64, 0.3, 20), (10, 0.5, 4)]:
        assert orc.poisson_binomial_tail(np.full(n, p), k) == pytest.approx(stats.binom.sf(k, n, p), rel=1e-10, abs=1e-300)


def test_poisson_binomial_brute_force():
    p = np.array([0.1, 0.7, 0.25, 0.5, 0.05, 0.9])
    for k in range(7):
        want = 0.0
        for bits in itertools.product([0, 1], repeat=len(p)):
            if sum(bits) > k:
                want += np.prod([pi if b else 1 - pi for pi, b in zip(p, bits)])
        assert orc.poisson_binomial_tail(p, k) == pytest.approx(want, abs=1e-15)


def test_p_active_standard_values():
    # |w| = 1 and b = -2.326 -> Phi(-2.326) ~ 0.01001
    w1t = np.zeros((3, 5)); w1t[:, 0] = 1.0
    p = orc.p_active(np.array([-2.326, 0.0, 1.0]), w1t)
    assert p[0] == pytest.approx(stats.norm.cdf(-2.326), rel=1e-12)
    assert p[1] == pytest.approx(0.5)
    assert p[2] == pytest.approx(stats.norm.cdf(1.0), rel=1e-12)


def test_skewed_bias_recipe():
    # b_j = Phi^-1(p_j) makes a unit-variance pre-activation fire with probability p_j.
    w = synth.C5.with_(T=4, d=64, f=256)
    g = synth.generate(w)
    assert np.allclose(stats.norm.sf(-g["b1"].astype(float)), g["p"], rtol=1e-5)
    assert 0.001 <= g["p"].min() and g["p"].max() <= 0.05


def test_expected_overflow_rows_tiny_brute_force():
    p = np.array([0.2, 0.6, 0.3, 0.9])
    # tiles of 2, one slot: a row overflows iff some tile has both entries active
    want_row = 1 - (1 - 0.2 * 0.6) * (1 - 0.3 * 0.9)
    assert orc.expected_overflow_rows(p, 2, 1, 10) == pytest.approx(10 * want_row)


def test_overflow_rows_measured_vs_expected():
    # Skewed per-unit activity with few slots overflows a predictable number of rows.
    w = synth.C5.with_(T=512, d=256, f=1024, slots=4, tile_w=64)
    g = synth.generate(w)
    x = orc.widen(g["x"], "bf16")
    w1t = orc.widen(g["w1t"], "bf16")
    b1 = g["b1"].astype(np.float64)
    h = orc.relu(orc.preact(x, w1t, b1))
    tw = orc.twell_pack(h, w.tile_w, w.slots, w.T)
    p = orc.p_active(b1, w1t)
    exp = orc.expected_overflow_rows(p, w.tile_w, w.slots, w.T)
    assert exp > 5
    # rows are independent given the weights; allow a wide band for the shared-x correlation
    assert abs(tw["ovf_n"] - exp) < 6 * math.sqrt(exp) + 0.3 * exp, (tw["ovf_n"], exp)


def test_hot_tokens_overflow():
    w = synth.C5.with_(T=256, d=256, f=1024, slots=8, tile_w=128, hot_every=64)
    g = synth.generate(w)
    x = orc.widen(g["x"], "bf16")
    w1t = orc.widen(g["w1t"], "bf16")
    h = orc.relu(orc.preact(x, w1t, g["b1"].astype(np.float64)))
    tw = orc.twell_pack(h, w.tile_w, w.slots, w.T)
    for t in range(0, w.T, 64):
        assert t in set(tw["ovf_rows"].tolist())
