"""GPU parity of the fused gated inference path (twell_gated_ffn_infer: the gate GEMM, then one
kernel that walks each token's active gate units, takes the up dot product and multiplies-adds
the down row) against the oracle's gated layer, through the C ABI.

"Sparser, Faster, Lighter Transformer Language Models", section "2. Metodologia", block
"Kernels de Inferência". Tokens with a tile holding more than S active units are recomputed
inside the kernel (dense row), which the low-bias cases exercise.
"""
import ctypes
import sys

import numpy as np
import pytest

import synth
from oracle import twell_oracle as orc
from tests.helpers import from_dev, inputs64, rel_err, to_dev, twell_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import activation_sparse_transformer_up_amd as tw  # noqa: E402

TOL = {"f32": 1e-5, "bf16": 2e-3}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def case(w, T, bias=None):
    g = synth.generate(w, T=T)
    if bias is not None:
        g["b1"] = np.full_like(g["b1"], bias)
    return g, synth.up_weights(w)


def dev(g, wut_bits):
    dt = g["dtype"]
    return (to_dev(g["x"], dt), to_dev(g["w1t"], dt), to_dev(g["b1"], "f32"), to_dev(wut_bits, dt),
            to_dev(g["w2"], dt))


def check_infer(g, wut_bits, W, S, vdt=torch.float32):
    dt = g["dtype"]
    x, wgt, bg, wut, w2 = dev(g, wut_bits)
    T = x.shape[0]
    y, h = tw.twell_gated_ffn_infer(x, wgt, bg, wut, w2, W, S, vdt)
    # the plain forward on the gate weights gives the gate's TwELL: same slots and counts
    _, hp = tw.twell_ffn_fwd(x, wgt, bg, w2, W, S, T, vdt)
    torch.cuda.synchronize()
    got, plain = twell_host(h), twell_host(hp)
    for k in ("counts", "col_idx", "vals"):
        assert np.array_equal(got[k], plain[k]), k
    marked = int((got["counts"].max(axis=1) > S).sum())
    xr, wgr, bgr, w2r, _ = inputs64(g)
    wur = orc.widen(wut_bits, dt)
    y_ref = orc.gated_ffn_fwd(xr, wgr, bgr, wur, w2r)[4]
    yg = from_dev(y)
    if vdt == torch.bfloat16:
        # the gate values are rounded to bf16 as stored: compare with the oracle's product of
        # the GPU gate activations rounded the same way
        gz = from_dev(tw.ffn_up_relu_dense(x, wgt, bg, torch.float32))
        g16 = orc.widen(synth.f32_to_bf16_bits(gz.astype(np.float32)), "bf16")
        y_ref = orc.gated_gather(g16, xr, wur, w2r)
    err = rel_err(yg, y_ref)
    assert err <= TOL[dt], err
    return marked, err, y


@pytest.mark.parametrize("T", [1, 2, 3, 8, 17, 64])
def test_infer_c3_rows(T):
    """c3's d_model (4096) with f = 2048, T from 1 to 64, W = 128, S = 16."""
    say("gated infer", T)
    w = synth.C3.with_(f=2048)
    g, wut = case(w, T)
    marked, err, _ = check_infer(g, wut, 128, 16)
    say("marked", marked, "err", err)


@pytest.mark.parametrize("T", [1, 8, 64])
def test_infer_c3_full(T):
    say("gated infer c3 full", T)
    w = synth.C3
    g, wut = case(w, T)
    marked, err, _ = check_infer(g, wut, w.tile_w, w.slots)
    say("marked", marked, "err", err)


@pytest.mark.parametrize("T,bias,W,S", [(40, -1.0, 128, 16), (9, -0.3, 64, 8), (64, -1.0, 128, 4), (3, 0.5, 64, 2)])
def test_infer_marked_tokens(T, bias, W, S):
    """Low biases make tiles exceed S: those tokens' gate rows are recomputed inside the kernel
    and their products taken from the dense scratch row."""
    say("gated infer marked", T, bias, W, S)
    w = synth.C2.with_(f=2048, d=1024)
    g, wut = case(w, T, bias)
    marked, err, _ = check_infer(g, wut, W, S)
    say("marked", marked, "err", err)
    assert marked > 0


def test_infer_fp32_and_bf16_values():
    """fp32 inputs (c1's scaling, 64 tokens) at 1e-5; bf16 TwELL values against the product of
    the rounded gate."""
    w = synth.C1
    g, wut = case(w, 64)
    marked, err, _ = check_infer(g, wut, w.tile_w, w.slots)
    say("fp32 err", err)
    w = synth.C3.with_(f=2048)
    g, wut = case(w, 24, -1.5)
    marked, err, _ = check_infer(g, wut, 128, 8, torch.bfloat16)
    say("bf16 vals err", err, "marked", marked)


def test_infer_matches_staged_and_is_deterministic():
    """Two calls give the same bits; the staged gated forward (twell_gated_ffn_fwd) agrees within
    the tolerance (the two sum the down products in different orders)."""
    w = synth.C3.with_(f=2048)
    g, wut_bits = case(w, 33)
    x, wgt, bg, wut, w2 = dev(g, wut_bits)
    y1, h = tw.twell_gated_ffn_infer(x, wgt, bg, wut, w2, 128, 16)
    y2, _ = tw.twell_gated_ffn_infer(x, wgt, bg, wut, w2, 128, 16, h=h)
    y3, _ = tw.twell_gated_ffn_fwd(x, wgt, bg, wut, w2, 128, 16, 33)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert rel_err(from_dev(y1), from_dev(y3)) <= 1e-5


def test_infer_sizes_and_errors():
    w = synth.C3.with_(T=65, f=1024, d=512)
    g, wut_bits = case(w, 65)
    x, wgt, bg, wut, w2 = dev(g, wut_bits)
    assert x.shape[0] == 65
    with pytest.raises(tw.TwellError):
        tw.twell_gated_ffn_infer(x, wgt, bg, wut, w2, 128, 16)              # 65 tokens: unsupported
    y, h = tw.twell_gated_ffn_infer(x[:0], wgt, bg, wut, w2, 128, 16)
    torch.cuda.synchronize()
    assert y.shape == (0, 512)
