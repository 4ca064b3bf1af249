"""Seeded synthetic FFN layers: the only code that the oracle and the HIP path share.

This module draws random numbers and rounds them to the stored dtypes. It holds none of
the layer's arithmetic (no products, no activation, no packing): both sides receive the
same arrays and compute everything themselves.

Recipe (one fixed order of draws per workload, fp64 standard normals from
``numpy.random.default_rng(seed)``, i.e. PCG64):

  1. x   [T, d]   ~ N(0, 1)
  2. w1t [f, d]   ~ N(0, 1/d)   (row j = input weights of hidden unit j)
  3. p   [f]      log-uniform in [p_lo, p_hi]    (per-unit activity; skewed workload only)
  4. w2  [f, d]   ~ N(0, 1/f)   (row j = output weights of hidden unit j)
  5. dy  [T, d]   ~ N(0, 1)     (training workload only)

fp64 draws are rounded to fp32 (round-to-nearest-even) and, for bf16 workloads, the
fp32 values are rounded again to bf16 (RNE on the bit pattern). The bias b1 is always
fp32: either a constant, or b1_j = Phi^-1(p_j) so that a unit with unit-variance
pre-activation fires with probability p_j. "Hot" tokens (rows t with t % hot_every == 0)
have x scaled by ``hot_scale`` after rounding (a power of two, so exact).

bf16 arrays are returned as ``numpy.uint16`` bit patterns; fp32 arrays as float32.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    f: int
    dtype: str            # "f32" or "bf16": dtype of x, w1t, w2 (and dy)
    seed: int
    tile_w: int = 128
    slots: int = 16
    bias: float | None = -2.326          # constant b1; None -> per-unit log-uniform p
    p_lo: float = 0.001
    p_hi: float = 0.05
    with_dy: bool = False
    l1_coef: float = 0.0
    hot_every: int = 0                   # 0: no hot tokens
    hot_scale: float = 4.0
    nm: tuple = ()                       # ((n, m), ...) pruning patterns

    @property
    def n_tiles(self) -> int:
        return self.f // self.tile_w

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of the activation-sparse FFN study (sizes, scalings, seeds).
C1 = Workload("c1_fp32_T128_d256_f1024", T=128, d=256, f=1024, dtype=F32, seed=0,
              tile_w=64, slots=8)
C2 = Workload("c2_bf16_T4096_d2048_f8192", T=4096, d=2048, f=8192, dtype=BF16, seed=1,
              tile_w=128, slots=16)
C3 = Workload("c3_bf16_T64_d4096_f14336", T=64, d=4096, f=14336, dtype=BF16, seed=2,
              tile_w=128, slots=16)
C4 = Workload("c4_bf16_T4096_d4096_f14336_b0", T=4096, d=4096, f=14336, dtype=BF16, seed=3,
              bias=0.0, nm=((8, 16), (16, 32)))
C5 = Workload("c5_bf16_T16384_d4096_f14336_train", T=16384, d=4096, f=14336, dtype=BF16,
              seed=4, tile_w=128, slots=8, bias=None, with_dy=True, l1_coef=2e-5)

WORKLOADS = {"c1": C1, "c2": C2, "c3": C3, "c4": C4, "c5": C5}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _store(a64: np.ndarray, dtype: str) -> np.ndarray:
    a32 = a64.astype(np.float32)
    return f32_to_bf16_bits(a32) if dtype == BF16 else a32


def _normal(rng, shape, std, dtype):
    # Drawn in row blocks so that the fp64 temporaries of the large workloads stay small.
    rows = shape[0]
    out = np.empty(shape, np.uint16 if dtype == BF16 else np.float32)
    step = max(1, (1 << 24) // max(1, shape[1]))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        out[r0:r1] = _store(rng.standard_normal((r1 - r0, shape[1])) * std, dtype)
    return out


def ndtri(p):
    """Inverse standard normal CDF (scipy's implementation)."""
    from scipy.special import ndtri as _ndtri
    return _ndtri(p)


def generate(w: Workload, T: int | None = None) -> dict:
    """Draw one workload. ``T`` may be smaller than ``w.T``: the first T rows are kept
    (the draw itself always uses ``w.T`` rows so prefixes agree across T)."""
    rng = np.random.default_rng(w.seed)
    x = _normal(rng, (w.T, w.d), 1.0, w.dtype)
    w1t = _normal(rng, (w.f, w.d), 1.0 / math.sqrt(w.d), w.dtype)
    if w.bias is None:
        u = rng.uniform(math.log(w.p_lo), math.log(w.p_hi), size=w.f)
        p = np.exp(u)
        b1 = ndtri(p).astype(np.float32)
    else:
        p = None
        b1 = np.full(w.f, w.bias, np.float32)
    w2 = _normal(rng, (w.f, w.d), 1.0 / math.sqrt(w.f), w.dtype)
    dy = _normal(rng, (w.T, w.d), 1.0, w.dtype) if w.with_dy else None
    if w.hot_every:
        rows = np.arange(0, w.T, w.hot_every)
        if w.dtype == BF16:
            xf = bf16_bits_to_f32(x[rows]) * np.float32(w.hot_scale)
            x[rows] = f32_to_bf16_bits(xf)
        else:
            x[rows] *= np.float32(w.hot_scale)
    if T is not None and T < w.T:
        x = x[:T].copy()
        dy = dy[:T].copy() if dy is not None else None
    return {"x": x, "w1t": w1t, "b1": b1, "w2": w2, "dy": dy, "p": p,
            "dtype": w.dtype, "workload": w}


def up_weights(w: Workload) -> np.ndarray:
    """The up-projection weights of the gated variant of workload ``w``: [f][d] with the same
    scaling as w1t (N(0, 1/d)), from a generator of their own (seed + 1000), so the plain
    workload's draws are unchanged."""
    rng = np.random.default_rng(w.seed + 1000)
    return _normal(rng, (w.f, w.d), 1.0 / math.sqrt(w.d), w.dtype)


def decode_layers(n: int, T: int, densities=(0.005, 0.01, 0.02, 0.03)):
    """``n`` decode-size layers of c3's shape (d=4096, f=14336, bf16) for a multi-layer
    decode loop: layer l draws its weights from seed 2 + 100 (l + 1) (c3's scalings) and has
    the constant bias Phi^-1(p_l) for p_l = densities[l % len(densities)] (per-layer density
    skew). Layers expect unit-RMS inputs; a decode loop normalises each token's output
    before the next layer, as a transformer does between its blocks.
    Returns (x of the first layer [T, d], [per-layer dicts with w1t, b1, w2, p])."""
    layers = []
    x = None
    for l in range(n):
        p = densities[l % len(densities)]
        w = C3.with_(seed=2 + 100 * (l + 1), bias=float(ndtri(np.array([p]))[0]))
        g = generate(w, T=T)
        if x is None:
            x = g["x"]
        layers.append({"w1t": g["w1t"], "b1": g["b1"], "w2": g["w2"], "p": p})
    return x, layers


def integer_grid(T: int, d: int, f: int, seed: int, dtype: str = BF16,
                 active: float = 0.05) -> dict:
    """Inputs on a coarse binary grid: every product and every partial sum is exactly
    representable in fp32, so any summation order gives the same fp32 result.

    x in {-8..8}/4, w1t and w2 in {-8..8}/64, b1 a multiple of 1/256 chosen so that about
    ``active`` of the pre-activations are positive. All values are exact in bf16.
    """
    rng = np.random.default_rng(seed)
    xi = rng.integers(-8, 9, size=(T, d))
    wi = rng.integers(-8, 9, size=(f, d))
    vi = rng.integers(-8, 9, size=(f, d))
    x = xi / 4.0
    w1t = wi / 64.0
    w2 = vi / 64.0
    # Bias: a quantile of a reference draw so that ~active of the units fire (its value is
    # rounded to 1/256; only the grid matters for exactness, not the exact rate).
    sd = math.sqrt(d * (np.mean(xi.astype(float) ** 2) / 16.0) * (np.mean(wi.astype(float) ** 2) / 4096.0))
    b = -float(ndtri(1.0 - active)) * sd
    b1 = (np.round(np.full(f, b) * 256.0) / 256.0).astype(np.float32)
    conv = (lambda a: f32_to_bf16_bits(a.astype(np.float32))) if dtype == BF16 else (lambda a: a.astype(np.float32))
    return {"x": conv(x), "w1t": conv(w1t), "b1": b1, "w2": conv(w2), "dy": conv(rng.integers(-8, 9, size=(T, d)) / 8.0),
            "p": None, "dtype": dtype, "workload": None}


def nm_grid(T: int, d: int, f: int, seed: int, dtype: str = BF16) -> dict:
    """Inputs whose pre-activations are exact in bf16 as well as fp32 (for N:M pruning of
    ReLU(x W1 + b1) stored in bf16): x in {-1, 0, 1}/2, w1t in {-1, 0, 1}/8, b1 in
    {-4..4}/16, so z = k/16 with |k| <= d + 4 <= 256 (d <= 252) in any summation order.
    About half of the pre-activations are positive, and equal magnitudes are frequent.
    """
    assert d <= 252
    rng = np.random.default_rng(seed)
    x = rng.integers(-1, 2, size=(T, d)) / 2.0
    w1t = rng.integers(-1, 2, size=(f, d)) / 8.0
    b1 = (rng.integers(-4, 5, size=f) / 16.0).astype(np.float32)
    conv = (lambda a: f32_to_bf16_bits(a.astype(np.float32))) if dtype == BF16 else (lambda a: a.astype(np.float32))
    return {"x": conv(x), "w1t": conv(w1t), "b1": b1, "dtype": dtype}
