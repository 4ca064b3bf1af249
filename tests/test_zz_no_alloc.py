"""The allocation-free backward (twell_ffn_bwd_noalloc: the library's fixed per-GPU scratch in
place of a workspace argument) against twell_ffn_bwd with a caller workspace, through the C
ABI: two calls in a row, the second on a smaller problem of another dtype, must give the same
bits (the two share every kernel). A problem whose workspace exceeds the fixed scratch is
refused with TWELL_ERR_WORKSPACE before anything is enqueued."""
import ctypes
import sys

import pytest

import synth
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import activation_sparse_transformer_up_amd as tw  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def layer(T, d, f, W, S, cap, dt, seed, hot):
    base = synth.C5 if dt == "bf16" else synth.C1.with_(with_dy=True, l1_coef=2e-5)
    w = base.with_(T=T, d=d, f=f, tile_w=W, slots=S, seed=seed, hot_every=hot)
    g = synth.generate(w)
    x, w1t, w2, dy = (to_dev(g[k], dt) for k in ("x", "w1t", "w2", "dy"))
    b1 = to_dev(g["b1"], "f32")
    y, h = tw.twell_ffn_fwd(x, w1t, b1, w2, W, S, cap)
    return x, w1t, w2, dy, h, w.l1_coef


def test_noalloc_matches_workspace_backward_twice():
    for (T, d, f, W, S, cap, dt, seed, hot) in [(300, 256, 1024, 128, 8, 64, "bf16", 91, 32),
                                                 (70, 128, 512, 64, 4, 16, "f32", 92, 16)]:
        say("noalloc bwd", T, d, f, W, S, cap, dt)
        x, w1t, w2, dy, h, lam = layer(T, d, f, W, S, cap, dt, seed, hot)
        need = tw.twell_ffn_bwd_workspace_bytes(T, d, f, h, x.dtype)
        assert 0 < need <= tw.NOALLOC_SCRATCH_BYTES
        ref = tw.twell_ffn_bwd(x, w1t, w2, h, dy, lam)
        got = tw.twell_ffn_bwd_noalloc(x, w1t, w2, h, dy, lam)
        torch.cuda.synchronize()
        assert int(h.ovf_n.item()) > 0          # backup rows are part of the pattern
        for name, a, b in zip(("dx", "dw1t", "dw2", "db1"), got, ref):
            assert torch.equal(a, b), name


def test_noalloc_refuses_beyond_its_scratch():
    T, d, f = 4096, 2048, 8192
    m = tw.TwellMatrixC(T, f, 128, 16, 64, 0, *([0x10000] * 10))
    need = tw.lib().twell_ffn_bwd_workspace_bytes(T, d, f, 1, ctypes.byref(m))
    assert need > tw.NOALLOC_SCRATCH_BYTES
    F = 0x10000
    st = tw.lib().twell_ffn_bwd_noalloc(F, F, F, 1, T, d, f, ctypes.byref(m), F, 0.0, F, F, F, F, None)
    assert st == -4
