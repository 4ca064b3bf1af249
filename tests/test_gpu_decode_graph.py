"""A decode loop over several layers, captured in a HIP graph: every replay equals the
eager chain bit for bit, and the chain follows the oracle's layer-by-layer forward.
Between layers each token is normalised to unit RMS (fp32, then rounded to bf16), the
stand-in for the rest of a transformer block; it is not part of the feed-forward path.

"Sparser, Faster, Lighter Transformer Language Models", section "2. Metodologia", block
"Kernels de Inferência" (the inference path, one FFN layer after another).
"""
import sys

import numpy as np
import pytest

import synth
from oracle import twell_oracle as orc
from tests.helpers import from_dev, rel_err, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import activation_sparse_transformer_up_amd as tw  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def build_chain(T, n_layers, slots=None):
    """slots: per-layer slot counts (default: the workload's S for every layer)."""
    x_bits, layers = synth.decode_layers(n_layers, T)
    w = synth.C3
    slots = slots or [w.slots] * n_layers
    x0 = to_dev(x_bits, "bf16")
    dev_layers = [(to_dev(L["w1t"], "bf16"), to_dev(L["b1"], "f32"), to_dev(L["w2"], "bf16")) for L in layers]
    hs = [tw.TwellMatrix(T, w.f, w.tile_w, S, 4, torch.float32, x0.device) for S in slots]
    ys = [torch.empty((T, w.d), dtype=torch.bfloat16, device=x0.device) for _ in layers]

    xs = [torch.empty((T, w.d), dtype=torch.bfloat16, device=x0.device) for _ in layers]

    def run():
        x = x0
        for l, ((w1t, b1, w2), h, y) in enumerate(zip(dev_layers, hs, ys)):
            tw.twell_ffn_fwd(x, w1t, b1, w2, w.tile_w, h.slots, 4, h=h, y=y, y_dtype=torch.bfloat16)
            yf = y.float()
            xs[l].copy_(yf * torch.rsqrt(yf.square().mean(dim=1, keepdim=True)))
            x = xs[l]
        return ys[-1]
    return x_bits, layers, run, ys, hs


@pytest.mark.parametrize("T", [1, 8])
def test_graph_replays_equal_eager(T):
    say("decode graph", T)
    _, _, run, ys, _ = build_chain(T, 3)
    run()
    torch.cuda.synchronize()
    eager = ys[-1].clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()                                         # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(3):
        ys[-1].zero_()                                # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ys[-1], eager), f"replay {i}"


def test_chain_follows_oracle():
    # Each layer's output is rounded to bf16, normalised per token and rounded to bf16 again
    # before the next layer, on both sides (oracle in fp64). Bound: the roundings of the
    # first layer (output and normalised input, 2^-9 each) carried through the second layer
    # plus the second output's own rounding, under 2^-7.
    T = 4
    x_bits, layers, run, ys, _ = build_chain(T, 2)
    run()
    torch.cuda.synchronize()
    x = orc.widen(x_bits, "bf16")
    refs = []
    for L in layers:
        y = orc.ffn_fwd(x, orc.widen(L["w1t"], "bf16"), L["b1"].astype(np.float64), orc.widen(L["w2"], "bf16"))[2]
        refs.append(y)
        yb = orc.widen(synth.f32_to_bf16_bits(y.astype(np.float32)), "bf16")
        xn = yb / np.sqrt(np.mean(yb * yb, axis=1, keepdims=True))
        x = orc.widen(synth.f32_to_bf16_bits(xn.astype(np.float32)), "bf16")
    e1 = rel_err(from_dev(ys[0]), refs[0])
    e2 = rel_err(from_dev(ys[1]), refs[1])
    say("chain errors", e1, e2)
    assert e1 <= 2 ** -8 and e2 <= 2 ** -7, (e1, e2)


def calibrated_slots(n_layers, T_cal=64, cap=0):
    """Per-layer slot counts from each layer's row-maximum histogram on a calibration batch of
    T_cal tokens: the S with the smallest stash whose overflow rows fit cap."""
    _, _, run, _, hs = build_chain(T_cal, n_layers)
    run()
    torch.cuda.synchronize()
    out = []
    for h in hs:
        hist = tw.twell_row_max_histogram(h).cpu().numpy()
        S, _ = tw.twell_choose_slots(hist, h.tile_w, h.rows, h.cols, cap)
        assert S == orc.choose_slots(hist, h.tile_w, h.rows, h.cols, cap, 4)[0]
        out.append(S)
    return out


@pytest.mark.parametrize("T", [1, 8])
def test_per_layer_slots(T):
    """The layers' densities differ (0.5 / 1 / 2 / 3 %), so the calibrated slot counts differ;
    with no row beyond its S the chain with per-layer S gives the same bits as the chain with
    the common S = 16 (the same entries in the same order), eager and replayed from a graph."""
    slots = calibrated_slots(4)
    say("per-layer S", slots)
    assert len(set(slots)) > 1 and max(slots) <= 16
    _, _, run_fixed, ys_fixed, _ = build_chain(T, 4)
    _, _, run, ys, hs = build_chain(T, 4, slots)
    run_fixed()
    run()
    torch.cuda.synchronize()
    if all(int(h.ovf_n.item()) == 0 for h in hs):
        assert torch.equal(ys[-1], ys_fixed[-1])
    else:
        assert rel_err(from_dev(ys[-1]), from_dev(ys_fixed[-1])) <= 2 ** -7
    eager = ys[-1].clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for i in range(2):
        ys[-1].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ys[-1], eager), f"replay {i}"
