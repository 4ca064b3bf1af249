"""GPU parity of N:M activation pruning (bit-exact) and of the packed N:M down projection
against the oracle, through the C ABI."""
import sys

import numpy as np
import pytest

import synth
from oracle import twell_oracle as orc
from tests.helpers import from_dev, inputs64, rel_err, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import activation_sparse_transformer_up_amd as tw  # noqa: E402

PATTERNS = [(2, 4), (4, 8), (8, 16), (16, 32)]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rand_h(T, f, seed, dtype, kind):
    rng = np.random.default_rng(seed)
    if kind == "ties":
        h = rng.integers(-3, 4, size=(T, f)).astype(np.float32) * 0.5
        h[rng.random((T, f)) < 0.1] = -0.0
    else:
        h = np.maximum(rng.standard_normal((T, f)), 0).astype(np.float32)
        h[rng.random((T, f)) < 0.05] *= -1
    if dtype == "bf16":
        bits = synth.f32_to_bf16_bits(h)
        return bits, orc.widen(bits, "bf16")
    return h, h.astype(np.float64)


@pytest.mark.parametrize("n,m", PATTERNS)
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("kind", ["ties", "relu"])
def test_nm_prune_bit_exact(n, m, dt, kind):
    T, f = 37, 64 * 9            # groups not a multiple of 64 per wave
    say("nm_prune", n, m, dt, kind)
    store, h64 = rand_h(T, f, n * 100 + m, dt, kind)
    vals, idx = tw.nm_prune(to_dev(store, dt), n, m)
    torch.cuda.synchronize()
    want_v, want_i = orc.nm_prune(h64, n, m)
    assert np.array_equal(from_dev(idx), want_i)
    gv = from_dev(vals)
    assert np.array_equal(gv, want_v)
    assert np.array_equal(np.signbit(gv), np.signbit(want_v))


@pytest.mark.parametrize("n,m", PATTERNS)
@pytest.mark.parametrize("groups", [1, 63, 65, 257])
def test_nm_prune_small_group_counts(n, m, groups):
    """One block, one short wave, one wave plus one block, a ragged last workgroup."""
    say("nm_prune small", n, m, groups)
    store, h64 = rand_h(1, groups * m, groups * 7 + m, "bf16", "ties")
    vals, idx = tw.nm_prune(to_dev(store, "bf16"), n, m)
    torch.cuda.synchronize()
    want_v, want_i = orc.nm_prune(h64, n, m)
    assert np.array_equal(from_dev(idx), want_i)
    gv = from_dev(vals)
    assert np.array_equal(gv, want_v)
    assert np.array_equal(np.signbit(gv), np.signbit(want_v))


@pytest.mark.parametrize("n,m", PATTERNS)
def test_nm_prune_extreme_bf16_patterns(n, m):
    """Infinities, the largest finite value, the smallest subnormal and both zeros, mixed with
    ordinary values: magnitudes compare as sign-cleared bit patterns (monotone for these), and
    the kept set, order and signs equal the oracle's."""
    say("nm_prune extreme", n, m)
    rng = np.random.default_rng(m * 13 + n)
    special = np.array([0x7F80, 0xFF80, 0x7F7F, 0xFF7F, 0x0001, 0x8001, 0x0000, 0x8000, 0x3F80, 0xBF80],
                       dtype=np.uint16)
    bits = rng.choice(special, size=(9, 64 * m)).astype(np.uint16)
    ordinary = synth.f32_to_bf16_bits(rng.standard_normal((9, 64 * m)).astype(np.float32))
    mix = rng.random((9, 64 * m)) < 0.4
    bits = np.where(mix, ordinary, bits).astype(np.uint16)
    h64 = orc.widen(bits, "bf16")
    vals, idx = tw.nm_prune(to_dev(bits, "bf16"), n, m)
    torch.cuda.synchronize()
    want_v, want_i = orc.nm_prune(h64, n, m)
    assert np.array_equal(from_dev(idx), want_i)
    gv = from_dev(vals)
    assert np.array_equal(gv, want_v)
    assert np.array_equal(np.signbit(gv), np.signbit(want_v))


def test_nm_prune_c4_full_bit_exact():
    """c4: h = ReLU(x W1) on the GPU (b1 = 0, about half active), pruned 8:16 and 16:32."""
    say("nm_prune c4 full")
    w = synth.C4
    g = synth.generate(w)
    x, w1t, b1 = to_dev(g["x"], "bf16"), to_dev(g["w1t"], "bf16"), to_dev(g["b1"], "f32")
    h = tw.ffn_up_relu_dense(x, w1t, b1, torch.bfloat16)
    hh = from_dev(h)
    dens = (hh > 0).mean()
    assert abs(dens - 0.5) < 0.01
    for n, m in w.nm:
        vals, idx = tw.nm_prune(h, n, m)
        torch.cuda.synchronize()
        want_v, want_i = orc.nm_prune(hh, n, m)
        assert np.array_equal(from_dev(idx), want_i)
        assert np.array_equal(from_dev(vals), want_v)
        post = (want_v != 0).sum() / hh.size
        assert abs(post - orc.nm_post_density(n, m)) < 0.01


@pytest.mark.parametrize("n,m", [(8, 16), (16, 32)])
@pytest.mark.parametrize("T,d,f", [(64, 256, 512), (300, 320, 1024), (513, 512, 2048), (77, 264, 544)])
def test_nm_down(n, m, T, d, f):
    say("nm_down", n, m, T, d, f)
    rng = np.random.default_rng(T + d)
    hb = synth.f32_to_bf16_bits(np.maximum(rng.standard_normal((T, f)), 0).astype(np.float32))
    w2 = synth.f32_to_bf16_bits((rng.standard_normal((f, d)) / np.sqrt(f)).astype(np.float32))
    vals, idx = tw.nm_prune(to_dev(hb, "bf16"), n, m)
    y = tw.nm_ffn_down(vals, idx, n, m, to_dev(w2, "bf16"))
    torch.cuda.synchronize()
    hv, hi = orc.nm_prune(orc.widen(hb, "bf16"), n, m)
    ref = orc.nm_unpack(hv, hi, m) @ orc.widen(w2, "bf16")
    assert rel_err(from_dev(y), ref) <= 2e-3


def test_nm_down_integer_grid_exact():
    T, d, f = 200, 256, 1024
    rng = np.random.default_rng(9)
    h = rng.integers(0, 9, size=(T, f)) / 4.0
    w2 = rng.integers(-8, 9, size=(f, d)) / 64.0
    hb = synth.f32_to_bf16_bits(h.astype(np.float32))
    w2b = synth.f32_to_bf16_bits(w2.astype(np.float32))
    vals, idx = tw.nm_prune(to_dev(hb, "bf16"), 8, 16)
    y = tw.nm_ffn_down(vals, idx, 8, 16, to_dev(w2b, "bf16"))
    torch.cuda.synchronize()
    hv, hi = orc.nm_prune(h, 8, 16)
    assert np.array_equal(from_dev(y), orc.nm_unpack(hv, hi, 16) @ w2)


def test_nm_rejects():
    h = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tw.TwellError):
        tw.nm_prune(h, 3, 16)
    with pytest.raises(tw.TwellError):
        tw.nm_prune(h[:, :60].contiguous(), 8, 16)
    v, i = tw.nm_prune(h, 2, 4)
    with pytest.raises(tw.TwellError) as e:
        tw.nm_ffn_down(v, i, 2, 4, torch.zeros((64, 16), dtype=torch.bfloat16, device="cuda"))
    assert e.value.status == -7
    v, i = tw.nm_prune(h, 8, 16)
    with pytest.raises(tw.TwellError):  # d_model not a multiple of 8
        tw.nm_ffn_down(v, i, 8, 16, torch.zeros((64, 12), dtype=torch.bfloat16, device="cuda"))


def test_nm_down_c4_full_sampled():
    """c4 at full size as the bench runs it (T=4096, d=4096, f=14336, bf16, b1 = 0): N:M from
    the up GEMM's epilogue, then the packed down projection; 16 sampled rows of y against the
    oracle's product of the unpacked N:M activations with W2 (the pruned entries are checked
    bit-exact against the oracle by the up + N:M tests)."""
    say("nm_down c4 full sampled")
    w = synth.C4
    g = synth.generate(w)
    x, w1t, w2 = (to_dev(g[k], "bf16") for k in ("x", "w1t", "w2"))
    b1 = to_dev(g["b1"], "f32")
    rows = np.sort(np.random.default_rng(11).choice(w.T, 16, replace=False))
    rt = torch.from_numpy(rows).cuda()
    w2r = orc.widen(g["w2"], "bf16")
    for n, m in w.nm:
        vals, idx = tw.ffn_up_relu_nm(x, w1t, b1, n, m)
        y = tw.nm_ffn_down(vals, idx, n, m, w2)
        torch.cuda.synchronize()
        ref = orc.nm_unpack(from_dev(vals[rt]), from_dev(idx[rt]), m) @ w2r
        err = rel_err(from_dev(y[rt]), ref)
        say("nm_down c4", n, m, "err", err)
        assert err <= 2e-3
