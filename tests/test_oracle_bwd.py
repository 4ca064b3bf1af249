"""Pins of the oracle's backward pass: central finite differences of the loss
<dy, y> + l1 * sum(h) on tiny fp64 problems away from the ReLU kink, and two special cases
with closed forms (dy = 0, and a single active entry)."""
import numpy as np
import pytest

from oracle import twell_oracle as orc


def loss(x, w1t, b1, w2, dy, lam):
    _, h, y = orc.ffn_fwd(x, w1t, b1, w2)
    return float((dy * y).sum() + lam * h.sum())


def problem(seed, T=5, d=7, f=11, e=4):
    rng = np.random.default_rng(seed)
    while True:
        x = rng.standard_normal((T, d))
        w1t = rng.standard_normal((f, d)) / np.sqrt(d)
        b1 = rng.standard_normal(f) * 0.5 - 0.3
        z = orc.preact(x, w1t, b1)
        if np.abs(z).min() > 1e-3:       # keep every entry away from the kink
            break
    w2 = rng.standard_normal((f, e))
    dy = rng.standard_normal((T, e))
    return x, w1t, b1, w2, dy


@pytest.mark.parametrize("lam", [0.0, 2e-5, 0.3])
def test_finite_differences(lam):
    x, w1t, b1, w2, dy = problem(1)
    _, h, _ = orc.ffn_fwd(x, w1t, b1, w2)
    g = orc.ffn_bwd(x, w1t, w2, dy, lam, h)
    eps = 1e-6
    for name, arr, grad in [("x", x, g["dx"]), ("w1t", w1t, g["dw1t"]),
                            ("b1", b1, g["db1"]), ("w2", w2, g["dw2"])]:
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            old = arr[i]
            arr[i] = old + eps
            lp = loss(x, w1t, b1, w2, dy, lam)
            arr[i] = old - eps
            lm = loss(x, w1t, b1, w2, dy, lam)
            arr[i] = old
            num[i] = (lp - lm) / (2 * eps)
        assert np.allclose(num, grad, rtol=1e-6, atol=1e-7), name


def test_zero_upstream_gradient_leaves_only_l1():
    x, w1t, b1, w2, dy = problem(2)
    _, h, _ = orc.ffn_fwd(x, w1t, b1, w2)
    lam = 0.25
    g = orc.ffn_bwd(x, w1t, w2, np.zeros_like(dy), lam, h)
    P = h > 0
    for j in range(w1t.shape[0]):
        want = lam * x[P[:, j]].sum(axis=0)
        assert np.allclose(g["dw1t"][j], want, rtol=0, atol=1e-14)
        assert g["db1"][j] == pytest.approx(lam * P[:, j].sum())
    assert np.array_equal(g["dw2"], np.zeros_like(w2))
    assert np.allclose(g["dx"], lam * (P.astype(float) @ w1t), atol=1e-14)


def test_single_active_entry_rank_one():
    # Only h[2, 3] active and lam = 0: dw2 = h[2,3] * outer(e_3, dy[2]),
    # dw1t = dz[2,3] * outer(e_3, x[2]) with dz[2,3] = dy[2] . w2[3].
    rng = np.random.default_rng(4)
    T, d, f, e = 4, 5, 6, 3
    x = rng.standard_normal((T, d))
    w1t = np.zeros((f, d)); w1t[3] = x[2] / np.dot(x[2], x[2])     # z[2,3] = 1 + b
    b1 = np.full(f, -0.5)
    w2 = rng.standard_normal((f, e))
    dy = rng.standard_normal((T, e))
    z, h, _ = orc.ffn_fwd(x, w1t, b1, w2)
    h = np.where(np.arange(T)[:, None] * f + np.arange(f)[None, :] == 2 * f + 3, h, 0.0)
    assert h[2, 3] > 0 and (h > 0).sum() == 1
    g = orc.ffn_bwd(x, w1t, w2, dy, 0.0, h)
    dz = float(dy[2] @ w2[3])
    want_w2 = np.zeros((f, e)); want_w2[3] = h[2, 3] * dy[2]
    want_w1 = np.zeros((f, d)); want_w1[3] = dz * x[2]
    assert np.allclose(g["dw2"], want_w2, atol=1e-15)
    assert np.allclose(g["dw1t"], want_w1, atol=1e-15)
    want_dx = np.zeros((T, d)); want_dx[2] = dz * w1t[3]
    assert np.allclose(g["dx"], want_dx, atol=1e-15)
