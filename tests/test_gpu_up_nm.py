"""GPU parity of the up projection with N:M pruning in its epilogue (ffn_up_relu_nm).

"Motivating Next-Gen Accelerators with Flexible (N:M) Activation Sparsity ...",
"2. Metodologia" (criterion ACT) applied to h = ReLU(x W1 + b1). Rules:
  - bit-exact against the oracle's nm_prune of the GPU's own dense h (ffn_up_relu_dense in
    the same dtype: same kernel family and accumulation order), on every tile path (256 x 256
    and 64 x 128 bf16 tiles, fp32 tiles, the decode K split) with ragged row and column tails;
  - on the N:M grid (pre-activations exact in bf16 and fp32 in any order) bit-exact against
    the oracle's own z, ReLU and pruning, ties included;
  - at the full c4 size equal to the standalone nm_prune of the dense h, and bit-exact against
    the oracle on sampled rows.
"""
import sys

import numpy as np
import pytest

import synth
from oracle import twell_oracle as orc
from tests.helpers import from_dev, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import activation_sparse_transformer_up_amd as tw  # noqa: E402

PATTERNS = [(2, 4), (4, 8), (8, 16), (16, 32)]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def normal_layer(T, d, f, seed, dt, bias):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d)).astype(np.float32)
    w1t = (rng.standard_normal((f, d)) / np.sqrt(d)).astype(np.float32)
    b1 = np.full(f, bias, np.float32)
    if dt == "bf16":
        x, w1t = synth.f32_to_bf16_bits(x), synth.f32_to_bf16_bits(w1t)
    return to_dev(x, dt), to_dev(w1t, dt), to_dev(b1, "f32")


# (T, d, f, dtype): 256x256 bf16 tiles with a ragged last row tile; 64x128 bf16 tiles with
# ragged rows and a partial column tile; the MFMA W1 stream of 3 to 16 bf16 tokens (d_model a
# multiple of 1024); the decode K split (bf16 and fp32); a K that is not a multiple of the
# decode quarters at a decode token count; fp32 tiles; the v_dot2 W1 stream of 1 or 2 bf16
# tokens (d_model 1024 / 2048 / 4096, a partial 128-unit tile).
SHAPES = [(1000, 256, 2048, "bf16"), (100, 256, 544, "bf16"), (8, 1024, 640, "bf16"), (16, 1024, 512, "bf16"),
          (3, 2048, 384, "bf16"), (8, 512, 640, "bf16"), (64, 256, 384, "bf16"), (8, 264, 256, "bf16"),
          (130, 256, 512, "f32"),
          (8, 256, 256, "f32"), (1, 4096, 256, "bf16"), (2, 1024, 640, "bf16"), (2, 2048, 384, "bf16")]


@pytest.mark.parametrize("n,m", PATTERNS)
@pytest.mark.parametrize("T,d,f,dt", SHAPES)
def test_up_nm_equals_oracle_prune_of_gpu_h(n, m, T, d, f, dt):
    if f % m:
        pytest.skip("d_ff not a multiple of m")
    say("up_nm", n, m, T, d, f, dt)
    x, w1t, b1 = normal_layer(T, d, f, T + d + f + m, dt, 0.0)
    vals, idx = tw.ffn_up_relu_nm(x, w1t, b1, n, m)
    h = tw.ffn_up_relu_dense(x, w1t, b1, x.dtype)
    torch.cuda.synchronize()
    hh = from_dev(h)
    assert 0.4 < (hh > 0).mean() < 0.6
    want_v, want_i = orc.nm_prune(hh, n, m)
    assert np.array_equal(from_dev(idx), want_i)
    gv = from_dev(vals)
    assert np.array_equal(gv, want_v)
    assert not np.any(np.signbit(gv))                 # ReLU output: +0 for inactive units


@pytest.mark.parametrize("n,m", PATTERNS)
@pytest.mark.parametrize("T,f,dt", [(700, 1024, "bf16"), (77, 384, "bf16"), (5, 256, "bf16"), (33, 512, "f32"),
                                    (3, 128, "f32")])
def test_up_nm_grid_exact_against_oracle(n, m, T, f, dt):
    say("up_nm grid", n, m, T, f, dt)
    d = 128
    g = synth.nm_grid(T, d, f, seed=T + f + m, dtype=dt)
    x, w1t, b1 = to_dev(g["x"], dt), to_dev(g["w1t"], dt), to_dev(g["b1"], "f32")
    vals, idx = tw.ffn_up_relu_nm(x, w1t, b1, n, m)
    torch.cuda.synchronize()
    h = orc.relu(orc.preact(orc.widen(g["x"], dt), orc.widen(g["w1t"], dt), g["b1"].astype(np.float64)))
    want_v, want_i = orc.nm_prune(h, n, m)
    assert np.array_equal(from_dev(idx), want_i)
    assert np.array_equal(from_dev(vals), want_v)


def test_up_nm_c4_full():
    """c4: T=4096, d=4096, f=14336, b1=0; 8:16 and 16:32 straight from the up GEMM."""
    w = synth.C4
    g = synth.generate(w)
    x, w1t, b1 = to_dev(g["x"], "bf16"), to_dev(g["w1t"], "bf16"), to_dev(g["b1"], "f32")
    h = tw.ffn_up_relu_dense(x, w1t, b1, torch.bfloat16)
    rows = np.random.default_rng(5).choice(w.T, 48, replace=False)
    rows.sort()
    hs = from_dev(h[torch.from_numpy(rows).cuda()])
    for n, m in w.nm:
        say("up_nm c4", n, m)
        vals, idx = tw.ffn_up_relu_nm(x, w1t, b1, n, m)
        v2, i2 = tw.nm_prune(h, n, m)
        torch.cuda.synchronize()
        assert torch.equal(idx, i2)
        assert torch.equal(vals.view(torch.int16), v2.view(torch.int16))
        want_v, want_i = orc.nm_prune(hs, n, m)
        assert np.array_equal(from_dev(idx)[rows], want_i)
        assert np.array_equal(from_dev(vals)[rows], want_v)


def test_up_nm_repeat_and_empty():
    x, w1t, b1 = normal_layer(40, 256, 512, 3, "bf16", 0.0)
    a = tw.ffn_up_relu_nm(x, w1t, b1, 8, 16)
    b = tw.ffn_up_relu_nm(x, w1t, b1, 8, 16)
    v, i = tw.ffn_up_relu_nm(x[:0], w1t, b1, 8, 16)
    torch.cuda.synchronize()
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])
    assert v.shape == (0, 32, 8) and i.shape == (0, 32, 8)
    with pytest.raises(tw.TwellError):
        tw.ffn_up_relu_nm(x, w1t, b1, 8, 32)
