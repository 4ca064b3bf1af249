"""Out-of-bounds write checks: every output buffer of every entry point sits inside a larger
allocation whose guard zones (4 KB on each side) hold a fill pattern; after calls at ragged
sizes that take each kernel path (256 x 256 and 64 x 128 tiles, the decode kernels, overflow
rows, the chunked gated stage, the backward) the guards must be untouched."""
import ctypes
import sys

import numpy as np
import pytest

import synth
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import activation_sparse_transformer_up_amd as tw  # noqa: E402

PAD, FILL = 4096, 0xA5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class Guarded:
    """A tensor of the given shape inside a guarded byte buffer."""

    def __init__(self, shape, dtype, zero=False):
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        self.n = max(n, 16)
        self.raw = torch.full((self.n + 2 * PAD,), FILL, dtype=torch.uint8, device="cuda")
        self.t = self.raw[PAD:PAD + n].view(dtype).view(shape)
        if zero:
            self.t.zero_()

    def intact(self) -> bool:
        return bool((self.raw[:PAD] == FILL).all()) and bool((self.raw[PAD + self.n:] == FILL).all())


def guarded_matrix(T, f, W, S, cap, vdt=torch.float32):
    h = tw.TwellMatrix(T, f, W, S, cap, vdt)
    gs = {}
    for name in ("counts", "col_idx", "vals", "ovf_n", "ovf_rows", "ovf_slot", "ovf_dense", "ovf_bits",
                 "row_nnz", "row_list"):
        t = getattr(h, name)
        g = Guarded(tuple(t.shape), t.dtype, zero=(name == "ovf_n"))   # scratch keeps the fill bytes
        setattr(h, name, g.t)
        gs[name] = g
    return h, gs


def layer(T, d, f, seed, dt="bf16", bias=-2.326, hot=0):
    base = synth.C2 if dt == "bf16" else synth.C1
    w = base.with_(T=T, d=d, f=f, seed=seed, bias=bias, hot_every=hot, with_dy=True)
    g = synth.generate(w)
    return [to_dev(g[k], dt) for k in ("x", "w1t", "w2", "dy")] + [to_dev(g["b1"], "f32")]


def all_intact(gs):
    bad = [k for k, g in gs.items() if not g.intact()]
    assert not bad, bad


# (T, d, f, W, S, dtype, hot): large tiles with overflow rows, the 4-wave large tiles (W = 64,
# S > 32), 64 x 128 tiles, the decode K split, the one-token W1 stream, fp32 tiles
FWD = [(600, 256, 1024, 128, 4, "bf16", 64), (600, 256, 1024, 64, 40, "bf16", 64), (100, 256, 640, 64, 2, "bf16", 0),
       (40, 512, 1024, 128, 3, "bf16", 8), (1, 2048, 512, 64, 16, "bf16", 0), (70, 256, 512, 64, 4, "f32", 16)]


@pytest.mark.parametrize("T,d,f,W,S,dt,hot", FWD)
def test_fwd_bwd_guards(T, d, f, W, S, dt, hot):
    say("guards fwd/bwd", T, d, f, W, S, dt)
    x, w1t, w2, dy, b1 = layer(T, d, f, T + d, dt, hot=hot)
    h, gs = guarded_matrix(T, f, W, S, T)
    y = Guarded((T, d), torch.float32)
    tw.twell_ffn_fwd(x, w1t, b1, w2, W, S, T, h=h, y=y.t)
    gs["y"] = y
    hz = Guarded((T, f), x.dtype)
    tw.ffn_up_relu_dense(x, w1t, b1, x.dtype, out=hz.t)
    gs["h_dense"] = hz
    hist = Guarded((W + 1,), torch.int32)
    tw.twell_row_max_histogram(h, hist.t)
    gs["hist"] = hist
    L = tw.lib()
    outs = {k: Guarded(s, torch.float32) for k, s in (("dx", (T, d)), ("dw1t", (f, d)), ("dw2", (f, d)), ("db1", (f,)))}
    nb = tw.twell_ffn_bwd_workspace_bytes(T, d, f, h, x.dtype)
    ws = Guarded((nb,), torch.uint8)
    m = h.c()
    st = L.twell_ffn_bwd(x.data_ptr(), w1t.data_ptr(), w2.data_ptr(), tw._dt(x.dtype), T, d, f, ctypes.byref(m),
                         dy.data_ptr(), 2e-5, outs["dx"].t.data_ptr(), outs["dw1t"].t.data_ptr(),
                         outs["dw2"].t.data_ptr(), outs["db1"].t.data_ptr(), ws.t.data_ptr(), nb,
                         tw._stream(x.device))
    assert st == 0
    torch.cuda.synchronize()
    gs.update(outs)
    gs["bwd_ws"] = ws
    all_intact(gs)
    assert int(h.ovf_n.item()) <= T


@pytest.mark.parametrize("T,d,f,dt", [(600, 256, 1024, "bf16"), (77, 256, 640, "bf16"), (2, 2048, 512, "bf16"),
                                      (9, 512, 512, "bf16"), (33, 256, 512, "f32")])
def test_nm_guards(T, d, f, dt):
    say("guards nm", T, d, f, dt)
    x, w1t, w2, _, b1 = layer(T, d, f, 7 + T, dt, bias=0.0)
    L = tw.lib()
    gs = {}
    for n, m in ((2, 4), (4, 8), (8, 16), (16, 32)):
        v = Guarded((T, f // m, n), x.dtype)
        i = Guarded((T, f // m, n), torch.uint8)
        tw.ffn_up_relu_nm(x, w1t, b1, n, m, vals=v.t, idx=i.t)
        h = tw.ffn_up_relu_dense(x, w1t, b1, x.dtype)
        v2 = Guarded((T, f // m, n), x.dtype)
        i2 = Guarded((T, f // m, n), torch.uint8)
        assert L.nm_prune(h.data_ptr(), tw._dt(x.dtype), T, f, n, m, v2.t.data_ptr(), i2.t.data_ptr(),
                          tw._stream(x.device)) == 0
        gs.update({f"up_nm_v{m}": v, f"up_nm_i{m}": i, f"prune_v{m}": v2, f"prune_i{m}": i2})
        if dt == "bf16" and m >= 16:
            y = Guarded((T, d), torch.float32)
            tw.nm_ffn_down(v.t, i.t, n, m, w2, y=y.t)
            gs[f"nm_down_y{m}"] = y
    torch.cuda.synchronize()
    all_intact(gs)


@pytest.mark.parametrize("T,W,S", [(600, 128, 4), (50, 64, 8)])
def test_gated_and_pack_guards(T, W, S):
    say("guards gated/pack", T, W, S)
    d, f = 2048, 1024
    x, wgt, w2, _, bg = layer(T, d, f, 3 + T, "bf16", bias=-1.0)
    wut = to_dev(synth.f32_to_bf16_bits((np.random.default_rng(T).standard_normal((f, d)) / np.sqrt(d))
                                        .astype(np.float32)), "bf16")
    h, gs = guarded_matrix(T, f, W, S, T)
    y = Guarded((T, d), torch.float32)
    need = tw.twell_gate_up_workspace_bytes(T, d, f, h)
    ws = Guarded((max(need, 16),), torch.uint8)
    tw.twell_gated_ffn_fwd(x, wgt, bg, wut, w2, W, S, T, h=h, y=y.t, workspace=ws.t)
    gs.update({"y": y, "gate_ws": ws})
    hd = tw.ffn_up_relu_dense(x, wgt, bg, torch.float32)
    hp, gp = guarded_matrix(T, f, W, S, T)
    L = tw.lib()
    mp = hp.c()
    assert L.twell_pack(hd.data_ptr(), 0, ctypes.byref(mp), tw._stream(x.device)) == 0
    torch.cuda.synchronize()
    gs.update({"pack_" + k: v for k, v in gp.items()})
    all_intact(gs)
