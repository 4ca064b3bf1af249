"""GPU parity of the compact row-ELL of the hybrid training format and of the backward's
entry-sized workspace, through the C ABI.

"Sparser, Faster, Lighter Transformer Language Models", section "2. Metodologia", block
"Formato Híbrido para Treinamento": rows with few nonzeros in a compact ELL whose width
follows the data, the rest in a dense backup. The row-ELL is a TwELL with one tile per row,
so the oracle's packer with tile_w = cols is its reference; the width is chosen per step
from the row-nonzero histogram, in a short training loop checked against the oracle at
every step.
"""
import sys

import numpy as np
import pytest

import synth
from oracle import twell_oracle as orc
from tests.helpers import assert_twell_equal, from_dev, inputs64, rel_err, to_dev, twell_host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import activation_sparse_transformer_up_amd as tw  # noqa: E402

TOL = {"f32": 1e-5, "bf16": 2e-3}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def layer(w):
    g = synth.generate(w)
    dt = g["dtype"]
    return g, [to_dev(g[k], dt) for k in ("x", "w1t", "w2", "dy")] + [to_dev(g["b1"], "f32")]


def stored_entries(host, S):
    """Entries the backward stores: the nonzeros of every row (slots in use, or the nonzeros of
    its backup row)."""
    counts = host["counts"]
    backup = host["ovf_slot"] >= 0
    return int(np.minimum(counts[~backup], S).sum() + counts[backup].sum())


@pytest.mark.parametrize("T,d,f,W,S,hot,vdt", [(512, 512, 2048, 128, 8, 64, torch.float32),
                                               (300, 256, 1024, 64, 4, 32, torch.bfloat16),
                                               (70, 256, 512, 128, 16, 0, torch.float32)])
def test_row_ell_bit_exact_and_backward_equal(T, d, f, W, S, hot, vdt):
    """The row-ELL built from the forward's TwELL equals the oracle's packer with one tile per
    row (bit for bit, backup rows included); its width comes from the library's histogram and
    chooser, which agree with the oracle's. The backward on it gives the same bits as the
    backward on the TwELL (the two give the same entries in the same order), and both match
    the oracle's backward on that pattern."""
    say("row-ELL", T, d, f, W, S, hot)
    w = synth.C5.with_(T=T, d=d, f=f, tile_w=W, slots=S, hot_every=hot)
    g, (x, w1t, w2, dy, b1) = layer(w)
    y, h = tw.twell_ffn_fwd(x, w1t, b1, w2, W, S, T, vdt)
    hz = tw.ffn_up_relu_dense(x, w1t, b1, torch.float32)
    hist = tw.twell_row_nnz_histogram(h)
    torch.cuda.synchronize()
    host = twell_host(h)
    assert np.array_equal(from_dev(hist), orc.row_nnz_histogram(host["counts"], f + 1))
    cap = 8
    vb = 4 if vdt == torch.float32 else 2
    N, b = tw.twell_choose_row_ell_width(from_dev(hist), T, f, cap, vdt)
    assert (N, b) == orc.choose_row_ell_width(from_dev(hist), T, f, cap, vb)
    e = tw.twell_to_row_ell(h, N, cap)
    torch.cuda.synchronize()
    h64 = from_dev(hz)
    if vdt == torch.bfloat16:
        h64 = orc.widen(synth.f32_to_bf16_bits(h64.astype(np.float32)), "bf16")
    want = orc.twell_pack(h64, f, N, cap)
    got = twell_host(e)
    assert_twell_equal(got, want)
    assert tw.twell_sync_status(e) == 0
    say("width", N, "overflow rows", got["ovf_n"], "stash", b, "TwELL stash",
        tw.twell_stash_bytes(T, f, W, S, host["ovf_n"], vdt))
    # the down projection on the row-ELL: the same y bits as the forward on the rows that are
    # in neither backup (a backup row is summed in another order), within 1e-6 elsewhere
    y2 = tw.twell_down(e, w2)
    a = tw.twell_ffn_bwd(x, w1t, w2, h, dy, w.l1_coef)
    bb = tw.twell_ffn_bwd(x, w1t, w2, e, dy, w.l1_coef)
    torch.cuda.synchronize()
    plain = (host["ovf_slot"] < 0) & (got["ovf_slot"] < 0)
    assert np.array_equal(from_dev(y)[plain], from_dev(y2)[plain])
    assert rel_err(from_dev(y2), from_dev(y)) <= 1e-6
    for name, u, v in zip(("dx", "dw1t", "dw2", "db1"), a, bb):
        assert torch.equal(u, v), name
    xr, w1r, b1r, w2r, dyr = inputs64(g)
    ref = orc.ffn_bwd(xr, w1r, w2r, dyr, w.l1_coef, orc.twell_unpack(got))
    for name, u in zip(("dx", "dw1t", "dw2", "db1"), bb):
        err = rel_err(from_dev(u), ref[name])
        assert err <= TOL["bf16"], (name, err)


def test_row_ell_capacity_follows_the_source():
    """A source beyond its backup capacity lost entries: the row-ELL reports a capacity error
    too, and the backward on it returns NaN."""
    w = synth.C5.with_(T=300, d=256, f=1024, hot_every=16)
    g, (x, w1t, w2, dy, b1) = layer(w)
    y, h = tw.twell_ffn_fwd(x, w1t, b1, w2, 128, 8, 2)
    e = tw.twell_to_row_ell(h, 64, 300)
    outs = tw.twell_ffn_bwd(x, w1t, w2, e, dy, 2e-5)
    torch.cuda.synchronize()
    assert tw.twell_sync_status(h) == -5 and tw.twell_sync_status(e) == -5
    for t in outs:
        assert bool(torch.isnan(t).all())


def test_backward_workspace_sized_by_entries():
    """A workspace sized for the call's stored entries (twell_ffn_bwd_workspace_bytes with nnz)
    gives the same bits as the capacity-sized one; one sized for 256 entries less (arrays are
    rounded up to 256 bytes, so fewer would not change the size) poisons every output."""
    w = synth.C5.with_(T=600, d=512, f=2048, hot_every=100)
    g, (x, w1t, w2, dy, b1) = layer(w)
    T, d, f = w.T, w.d, w.f
    y, h = tw.twell_ffn_fwd(x, w1t, b1, w2, 128, 8, 64)
    torch.cuda.synchronize()
    nnz = stored_entries(twell_host(h), 8)
    full = tw.twell_ffn_bwd_workspace_bytes(T, d, f, h, x.dtype)
    exact = tw.twell_ffn_bwd_workspace_bytes(T, d, f, h, x.dtype, nnz=nnz)
    short = tw.twell_ffn_bwd_workspace_bytes(T, d, f, h, x.dtype, nnz=nnz - 256)
    say("workspace bytes: capacity", full, "entries", exact, "nnz", nnz)
    assert short < exact < full
    ref = tw.twell_ffn_bwd(x, w1t, w2, h, dy, 2e-5)
    got = tw.twell_ffn_bwd(x, w1t, w2, h, dy, 2e-5,
                           workspace=torch.empty((exact,), dtype=torch.uint8, device="cuda"))
    bad = tw.twell_ffn_bwd(x, w1t, w2, h, dy, 2e-5,
                           workspace=torch.empty((short,), dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    for u, v, z in zip(ref, got, bad):
        assert torch.equal(u, v)
        assert bool(torch.isnan(z).all())


def test_training_loop_dynamic_width():
    """Four SGD steps of a c5-shaped layer (T = 512, d = 256, f = 1024, bf16, W = 128, S = 8, hot
    tokens): each step runs the forward, takes the row-nonzero histogram, chooses the row-ELL
    width for that step's stash, converts, and runs the backward on the row-ELL with a
    workspace sized by the step's entries. Every step's stash equals the oracle's packer and
    every step's gradients match the oracle's backward on the step's pattern; the weights move,
    so the pattern (and the width) change from step to step."""
    w = synth.C5.with_(T=512, d=256, f=1024, hot_every=128)
    g = synth.generate(w)
    T, d, f = w.T, w.d, w.f
    x, dy = to_dev(g["x"], "bf16"), to_dev(g["dy"], "bf16")
    w1 = torch.from_numpy(orc.widen(g["w1t"], "bf16").astype(np.float32)).cuda()
    w2f = torch.from_numpy(orc.widen(g["w2"], "bf16").astype(np.float32)).cuda()
    b1 = to_dev(g["b1"], "f32")
    lr, cap = 0.5, 24
    widths = []
    for step in range(4):
        w1t, w2 = w1.to(torch.bfloat16), w2f.to(torch.bfloat16)
        y, h = tw.twell_ffn_fwd(x, w1t, b1, w2, 128, 8, T)
        hist = tw.twell_row_nnz_histogram(h).cpu().numpy()
        N, stash = tw.twell_choose_row_ell_width(hist, T, f, cap)
        e = tw.twell_to_row_ell(h, N, cap)
        nnz = int((hist * np.arange(len(hist))).sum())
        ws = torch.empty((tw.twell_ffn_bwd_workspace_bytes(T, d, f, e, x.dtype, nnz=nnz),), dtype=torch.uint8,
                         device="cuda")
        dx, dw1t, dw2, db1 = tw.twell_ffn_bwd(x, w1t, w2, e, dy, w.l1_coef, workspace=ws)
        torch.cuda.synchronize()
        assert tw.twell_sync_status(e) == 0
        got = twell_host(e)
        h64 = orc.twell_unpack(twell_host(h))
        assert_twell_equal(got, orc.twell_pack(h64, f, N, cap))
        ref = orc.ffn_bwd(orc.widen(g["x"], "bf16"), from_dev(w1t), from_dev(w2), orc.widen(g["dy"], "bf16"),
                          w.l1_coef, orc.twell_unpack(got))
        errs = {k: rel_err(from_dev(v), ref[k]) for k, v in (("dx", dx), ("dw1t", dw1t), ("dw2", dw2), ("db1", db1))}
        say("step", step, "width", N, "overflow rows", got["ovf_n"], "stash", stash, "errs", errs)
        assert max(errs.values()) <= TOL["bf16"], errs
        widths.append((N, int(got["ovf_n"]), int(hist[1:].argmax())))
        w1 -= lr * dw1t
        w2f -= lr * dw2
        b1 -= lr * db1
    assert len(set(widths)) > 1, widths            # the data moved between steps
