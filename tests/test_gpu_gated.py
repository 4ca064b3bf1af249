"""GPU parity of the gated forward (gate GEMM + TwELL, up dot products over the active units,
down gather) against the oracle's gated layer, through the C ABI.

"Sparser, Faster, Lighter Transformer Language Models", section "2. Metodologia", blocks
"Formato de Dados TwELL" and "Kernels de Inferência".
"""
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


def gated_case(w, T=None, bias=None):
    g = synth.generate(w, T=T)
    wut = synth.up_weights(w)
    if bias is not None:
        g["b1"] = np.full_like(g["b1"], bias)
    return g, wut


def check_gated(g, wut_bits, W, S, cap):
    dt = g["dtype"]
    x, wgt, bg, w2 = (to_dev(g["x"], dt), to_dev(g["w1t"], dt), to_dev(g["b1"], "f32"), to_dev(g["w2"], dt))
    wut = to_dev(wut_bits, dt)
    y, h = tw.twell_gated_ffn_fwd(x, wgt, bg, wut, w2, W, S, cap)
    # the plain forward on the gate weights: its TwELL must be the same gate pattern
    _, hp = tw.twell_ffn_fwd(x, wgt, bg, w2, W, S, cap)
    torch.cuda.synchronize()
    got, plain = twell_host(h), twell_host(hp)
    for k in ("counts", "col_idx", "vals", "ovf_slot"):
        assert np.array_equal(got[k], plain[k]), k
    xr, wgr, bgr, w2r, _ = inputs64(g)
    wur = orc.widen(wut_bits, dt)
    y_ref = orc.gated_ffn_fwd(xr, wgr, bgr, wur, w2r)[4]
    err = rel_err(from_dev(y), y_ref)
    assert err <= TOL[dt], err
    return got["ovf_n"], err


def test_gated_c1():
    say("gated c1")
    w = synth.C1
    g, wut = gated_case(w)
    n, err = check_gated(g, wut, w.tile_w, w.slots, 8)
    say("c1 ovf", n, "err", err)


@pytest.mark.parametrize("T,bias,W,S,cap", [(300, -1.0, 128, 4, 300), (97, -0.3, 64, 8, 97),
                                            (1, -2.326, 128, 16, 4), (40, -2.326, 128, 16, 8),
                                            (700, -1.0, 128, 4, 700), (517, -2.326, 64, 2, 517)])
def test_gated_c2_shapes(T, bias, W, S, cap):
    # c2's d and f with fewer tokens; low biases make many rows overflow, so the backup
    # rows' up products are exercised as well as the lists'. From 512 tokens on the list
    # products are chunked per XCD through the workspace (517: a partial 16-token block)
    say("gated c2 shapes", T, bias, W, S, cap)
    g, wut = gated_case(synth.C2, T=T, bias=bias)
    n, err = check_gated(g, wut, W, S, cap)
    say("ovf", n, "err", err)
    if bias >= -1.0 or S <= 2:
        assert n > 0


@pytest.mark.parametrize("T,bias,S", [(17, -2.326, 16), (64, -1.0, 4), (200, -2.326, 2)])
def test_gated_wide_rows(T, bias, S):
    # d_model 4096 with 17-200 tokens (the wide-row down gather; f = 2048 keeps the oracle
    # fast); small S sends rows to the backup
    say("gated wide rows", T, bias, S)
    w = synth.C3.with_(f=2048)
    g, wut = gated_case(w, T=T, bias=bias)
    n, err = check_gated(g, wut, 128, S, T)
    say("ovf", n, "err", err)
    if S <= 4:
        assert n > 0


def test_gated_c3_T8():
    say("gated c3 T=8")
    w = synth.C3
    g, wut = gated_case(w, T=8)
    n, err = check_gated(g, wut, w.tile_w, w.slots, 4)
    say("ovf", n, "err", err)


@pytest.mark.parametrize("T", [256, 600])
def test_gated_stages_equal_one_call(T):
    # gate GEMM, finish, up stage and down gather enqueued one by one give the same y bits
    # (600 tokens: the chunked up products, with a workspace given by the caller)
    w = synth.C2
    g, wut_bits = gated_case(w, T=T)
    dt = g["dtype"]
    x, wgt, bg, w2 = (to_dev(g["x"], dt), to_dev(g["w1t"], dt), to_dev(g["b1"], "f32"), to_dev(g["w2"], dt))
    wut = to_dev(wut_bits, dt)
    y1, _ = tw.twell_gated_ffn_fwd(x, wgt, bg, wut, w2, w.tile_w, w.slots, 16)
    h = tw.TwellMatrix(T, w.f, w.tile_w, w.slots, 16, torch.float32, x.device)
    need = tw.twell_gate_up_workspace_bytes(T, w.d, w.f, h)
    assert (need > 0) == (T >= 512)
    ws = torch.full((max(need, 16),), 0xAB, dtype=torch.uint8, device=x.device)
    tw.twell_up_gemm(x, wgt, bg, h)
    tw.twell_up_finish(x, wgt, bg, h)
    tw.twell_gate_up(h, x, wut, workspace=ws)
    y2 = tw.twell_fwd_down(h, w2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


def test_gated_c2_full_sampled():
    """The gated layer at the c2 size as the bench runs it (T=4096, d=2048, f=8192, bf16,
    W=128, S=16, backup capacity 16): the gate's TwELL rows of 16 sampled tokens equal the
    oracle's packing of the GPU's gate activations bit for bit, and y of those rows is within
    tolerance of the oracle's gated layer."""
    say("gated c2 full sampled")
    w = synth.C2
    g, wut_bits = gated_case(w)
    x, wgt, w2 = (to_dev(g[k], "bf16") for k in ("x", "w1t", "w2"))
    bg, wut = to_dev(g["b1"], "f32"), to_dev(wut_bits, "bf16")
    y, h = tw.twell_gated_ffn_fwd(x, wgt, bg, wut, w2, w.tile_w, w.slots, 16)
    hz = tw.ffn_up_relu_dense(x, wgt, bg, torch.float32)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(13).choice(w.T, 16, replace=False))
    rt = torch.from_numpy(rows).cuda()
    hs = from_dev(hz[rt])
    want = orc.twell_pack(hs, w.tile_w, w.slots, len(rows))
    assert np.array_equal(from_dev(h.counts[rt]), want["counts"])
    assert np.array_equal(from_dev(h.col_idx[rt]), want["col_idx"])
    xr = orc.widen(g["x"][rows], "bf16")
    y_ref = orc.gated_ffn_fwd(xr, orc.widen(g["w1t"], "bf16"), g["b1"].astype(np.float64),
                              orc.widen(wut_bits, "bf16"), orc.widen(g["w2"], "bf16"))[4]
    err = rel_err(from_dev(y[rt]), y_ref)
    say("gated c2 full err", err)
    assert err <= TOL["bf16"], err
