"""GPU parity of the row-maximum histogram behind the dynamic slot count ([SFL] "Formato
Híbrido para Treinamento"): bit-exact against the oracle's histogram of the counts of the
GPU's own activations, consistent with the forward's overflow count, and a forward at the
chosen slot count keeps its overflow rows within the backup capacity."""
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


@pytest.mark.parametrize("T,d,f,W,S,hot,seed", [(600, 512, 2048, 128, 8, 64, 41), (333, 256, 1024, 64, 4, 0, 42),
                                                (40, 1024, 2048, 128, 3, 8, 43)])
def test_row_max_histogram_and_choice(T, d, f, W, S, hot, seed):
    say("row max histogram", T, d, f, W, S, hot)
    w = synth.C5.with_(T=T, d=d, f=f, tile_w=W, slots=S, hot_every=hot, seed=seed)
    g = synth.generate(w)
    x, w1t, w2 = (to_dev(g[k], "bf16") for k in ("x", "w1t", "w2"))
    b1 = to_dev(g["b1"], "f32")
    y, h = tw.twell_ffn_fwd(x, w1t, b1, w2, W, S, T)
    hz = tw.ffn_up_relu_dense(x, w1t, b1, torch.float32)
    hist = tw.twell_row_max_histogram(h)
    torch.cuda.synchronize()
    want = orc.row_max_histogram(orc.twell_pack(from_dev(hz), W, 1, 0)["counts"], W)
    got = from_dev(hist)
    assert np.array_equal(got, want)
    assert int(want[S + 1:].sum()) == int(h.ovf_n.item())
    cap = 16
    S2, nbytes = tw.twell_choose_slots(got, W, T, f, cap)
    assert (S2, nbytes) == orc.choose_slots(want, W, T, f, cap, 4)
    y2, h2 = tw.twell_ffn_fwd(x, w1t, b1, w2, W, S2, cap)
    assert tw.twell_sync_status(h2) == 0
    assert int(h2.ovf_n.item()) == int(want[S2 + 1:].sum()) <= cap
    assert rel_err(from_dev(y2), from_dev(y)) <= 1e-5


def test_row_max_histogram_overwrites_and_empty():
    w = synth.C5.with_(T=64, d=256, f=1024, tile_w=64, slots=4, seed=44)
    g = synth.generate(w)
    x, w1t, w2 = (to_dev(g[k], "bf16") for k in ("x", "w1t", "w2"))
    b1 = to_dev(g["b1"], "f32")
    y, h = tw.twell_ffn_fwd(x[:0], w1t, b1, w2, 64, 4, 4)
    hist = torch.full((65,), 7, dtype=torch.int32, device="cuda")
    tw.twell_row_max_histogram(h, hist)
    torch.cuda.synchronize()
    assert int(hist.abs().sum()) == 0
    y, h = tw.twell_ffn_fwd(x, w1t, b1, w2, 64, 4, 64)
    tw.twell_row_max_histogram(h, hist)
    tw.twell_row_max_histogram(h, hist)              # a second call does not accumulate
    torch.cuda.synchronize()
    assert int(hist.sum()) == 64
