"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function
include/twell.h declares, and rejects invalid arguments with the documented status codes
before anything is enqueued. Fake device addresses are used only in calls that fail
validation; on a machine with a GPU these cases run in the GPU suite with real buffers."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "twell.h")

import activation_sparse_transformer_up_amd as tw  # noqa: E402

ARG, SHAPE, ALIGN, WS, UNSUP = -1, -2, -3, -4, -7


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M)))


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for n in ["twell_pack", "twell_ffn_fwd", "twell_ffn_bwd", "nm_prune", "twell_abi_version",
              "twell_status_str", "twell_sync_status", "nm_ffn_down", "ffn_up_relu_dense",
              "twell_down", "twell_ffn_bwd_workspace_bytes", "twell_ovf_bits_words",
              "twell_row_list_bytes", "twell_up_gemm", "twell_up_finish", "twell_fwd_down",
              "twell_gate_up", "twell_gated_ffn_fwd", "ffn_up_relu_nm"]:
        assert n in names, n


def test_library_exports_every_declared_symbol():
    L = tw.lib()
    for n in declared_functions():
        assert hasattr(L, n), n


def test_version_and_status_strings():
    assert tw.twell_abi_version() == 4
    L = tw.lib()
    for code in [0, -1, -2, -3, -4, -5, -6, -7]:
        s = L.twell_status_str(code).decode()
        assert s.startswith(tw.STATUS[code])
    assert L.twell_status_str(12345).decode() == "TWELL_UNKNOWN_STATUS"
    assert L.twell_ovf_bits_words(100, 1024, 64) == 16 * 4
    assert L.twell_ovf_bits_words(-1, 1024, 64) == 0


def test_row_list_bytes_with_decode_workspace():
    L = tw.lib()
    # above 64 rows: the lists only (8 bytes per slot)
    assert L.twell_row_list_bytes(65, 14336, 128, 16) == 65 * 112 * 16 * 8
    assert L.twell_row_list_bytes(4096, 1024, 64, 8) == 4096 * 16 * 8 * 8
    # up to 64 rows: lists rounded up to 256 bytes, then two 64 x 128 fp32 half sums and a
    # 64-bit ticket per 128 columns (the tickets rounded up to 256 bytes)
    assert L.twell_row_list_bytes(64, 14336, 128, 16) == 64 * 112 * 16 * 8 + 112 * 65536 + 1024
    assert L.twell_row_list_bytes(1, 1984, 64, 3) == 768 + 16 * 65536 + 256     # 15.5 tiles -> 16
    assert L.twell_row_list_bytes(0, 512, 128, 8) == 0 + 4 * 65536 + 256


def gpu_present():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


pytestmark_nogpu = pytest.mark.skipif(gpu_present(), reason="fake-pointer checks run only without a GPU")

FAKE = 0x10000          # 16-byte aligned, never dereferenced: every call below fails validation
MIS = 0x10004           # misaligned


def mat(rows=64, cols=512, W=128, S=8, cap=4, dt=0, **kw):
    m = tw.TwellMatrixC(rows, cols, W, S, cap, dt, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    for k, v in kw.items():
        setattr(m, k, v)
    return m


def fwd(m, x=FAKE, w1t=FAKE, b1=FAKE, w2=FAKE, dt=1, T=64, d=256, f=512, y=FAKE, ydt=0):
    return tw.lib().twell_ffn_fwd(x, w1t, b1, w2, dt, T, d, f, ctypes.byref(m), y, ydt, None)


@pytestmark_nogpu
@pytest.mark.parametrize("kw,want", [
    (dict(x=None), ARG), (dict(w2=None), ARG), (dict(b1=None), ARG), (dict(y=None), ARG),
    (dict(dt=7), ARG), (dict(ydt=3), ARG), (dict(T=-1), SHAPE), (dict(d=0), SHAPE),
    (dict(f=0), SHAPE), (dict(d=100), ALIGN), (dict(x=MIS), ALIGN), (dict(y=MIS), ALIGN),
    (dict(T=32), SHAPE), (dict(f=1024), SHAPE),
])
def test_fwd_rejects(kw, want):
    assert fwd(mat(), **kw) == want


@pytestmark_nogpu
@pytest.mark.parametrize("mkw,want", [
    (dict(tile_w=96), UNSUP), (dict(cols=500), SHAPE), (dict(slots=0), SHAPE),
    (dict(slots=65), SHAPE), (dict(W=64, slots=65), SHAPE), (dict(ovf_cap=-1), SHAPE),
    (dict(counts=None), ARG), (dict(ovf_n=None), ARG), (dict(ovf_bits=None), ARG),
    (dict(val_dtype=5), ARG), (dict(ovf_rows=None), ARG), (dict(ovf_dense=MIS), ALIGN),
    (dict(counts=MIS + 1), ALIGN), (dict(row_list=None), ARG), (dict(row_nnz=MIS + 1), ALIGN),
])
def test_fwd_rejects_bad_matrix(mkw, want):
    W = mkw.pop("W", 128)
    m = mat(W=W)
    for k, v in mkw.items():
        setattr(m, k, v)
    assert fwd(m) == want


@pytestmark_nogpu
def test_pack_and_down_reject():
    L = tw.lib()
    m = mat()
    assert L.twell_pack(None, 0, ctypes.byref(m), None) == ARG
    assert L.twell_pack(FAKE, 9, ctypes.byref(m), None) == ARG
    assert L.twell_pack(MIS, 0, ctypes.byref(m), None) == ALIGN
    m16 = mat(dt=1)
    assert L.twell_pack(FAKE, 0, ctypes.byref(m16), None) == UNSUP       # fp32 h -> bf16 vals
    assert L.twell_down(ctypes.byref(m), FAKE, 1, 100, FAKE, 0, None) == ALIGN
    assert L.twell_down(ctypes.byref(m), None, 1, 256, FAKE, 0, None) == ARG
    assert L.twell_down(ctypes.byref(m), FAKE, 1, 0, FAKE, 0, None) == SHAPE
    # W2 rows are addressed with 32-bit byte offsets: 2 GiB of w2 (or of y) is refused
    wide = mat(rows=64, cols=65536)
    assert L.twell_down(ctypes.byref(wide), FAKE, 1, 16384, FAKE, 0, None) == UNSUP
    assert L.twell_fwd_down(ctypes.byref(wide), FAKE, 0, 8192, FAKE, 0, None) == UNSUP
    assert L.twell_down(ctypes.byref(mat(rows=1 << 17, cols=512)), FAKE, 1, 4096, FAKE, 0, None) == UNSUP
    assert L.ffn_up_relu_dense(FAKE, FAKE, None, 1, 4, 256, 512, FAKE, 0, None) == ARG
    assert L.ffn_up_relu_dense(FAKE, FAKE, FAKE, 1, 4, 250, 512, FAKE, 0, None) == ALIGN
    assert L.twell_sync_status(None, None) == ARG


@pytestmark_nogpu
def test_gated_entry_points_reject():
    L = tw.lib()
    m = mat()
    # twell_gate_up(h, x, w_up_t, dtype, T, d, f, workspace, workspace_bytes, stream)
    assert L.twell_gate_up(None, FAKE, FAKE, 1, 64, 256, 512, None, 0, None) == ARG
    assert L.twell_gate_up(ctypes.byref(m), FAKE, None, 1, 64, 256, 512, None, 0, None) == ARG
    assert L.twell_gate_up(ctypes.byref(m), FAKE, FAKE, 7, 64, 256, 512, None, 0, None) == ARG
    assert L.twell_gate_up(ctypes.byref(m), MIS, FAKE, 1, 64, 256, 512, None, 0, None) == ALIGN
    assert L.twell_gate_up(ctypes.byref(m), FAKE, FAKE, 1, 64, 100, 512, None, 0, None) == ALIGN
    assert L.twell_gate_up(ctypes.byref(m), FAKE, FAKE, 1, 32, 256, 512, None, 0, None) == SHAPE
    assert L.twell_gate_up(ctypes.byref(mat(row_list=None)), FAKE, FAKE, 1, 64, 256, 512, None, 0, None) == ARG
    # from 512 tokens on the up products need the workspace (16 column chunks x 512 x 4 x 8 floats)
    big = mat(rows=512)
    need = L.twell_gate_up_workspace_bytes(512, 2048, 512, 1, ctypes.byref(big))
    assert need == 16 * 512 * 4 * 8 * 4
    assert L.twell_gate_up_workspace_bytes(511, 2048, 512, 1, ctypes.byref(mat(rows=511))) == 0
    assert L.twell_gate_up(ctypes.byref(big), FAKE, FAKE, 1, 512, 2048, 512, None, 0, None) == WS
    assert L.twell_gate_up(ctypes.byref(big), FAKE, FAKE, 1, 512, 2048, 512, FAKE, need - 16, None) == WS
    assert L.twell_gate_up(ctypes.byref(big), FAKE, FAKE, 1, 512, 2048, 512, MIS, need, None) == ALIGN
    # the up GEMM alone needs row_list at decode sizes (its K-split workspace), not above
    up = lambda m, T: L.twell_up_gemm(FAKE, FAKE, FAKE, 1, T, 256, 512, ctypes.byref(m), None)
    assert up(mat(rows=4, row_list=None), 4) == ARG
    assert up(mat(rows=64, row_list=None), 64) == ARG

    def gfwd(mm=m, **kw):
        a = dict(x=FAKE, wg=FAKE, bg=FAKE, wu=FAKE, w2=FAKE, dt=1, T=64, d=256, f=512, y=FAKE, ydt=0, ws=None,
                 wsb=0)
        a.update(kw)
        return L.twell_gated_ffn_fwd(a["x"], a["wg"], a["bg"], a["wu"], a["w2"], a["dt"], a["T"], a["d"], a["f"],
                                     ctypes.byref(mm), a["y"], a["ydt"], a["ws"], a["wsb"], None)
    assert gfwd(wu=None) == ARG
    assert gfwd(w2=None) == ARG
    assert gfwd(bg=None) == ARG
    assert gfwd(ydt=4) == ARG
    assert gfwd(wu=MIS) == ALIGN
    assert gfwd(f=1024) == SHAPE
    assert gfwd(mm=big, T=512, d=2048) == WS
    assert gfwd(mm=big, T=512, d=2048, ws=FAKE, wsb=need - 1) == WS


@pytestmark_nogpu
def test_up_nm_rejects():
    L = tw.lib()

    def up_nm(**kw):
        a = dict(x=FAKE, w1t=FAKE, b1=FAKE, dt=1, T=64, d=256, f=512, n=8, m=16, vals=FAKE, idx=FAKE)
        a.update(kw)
        return L.ffn_up_relu_nm(a["x"], a["w1t"], a["b1"], a["dt"], a["T"], a["d"], a["f"], a["n"], a["m"],
                                a["vals"], a["idx"], None)
    assert up_nm(b1=None) == ARG
    assert up_nm(vals=None) == ARG
    assert up_nm(idx=None) == ARG
    assert up_nm(w1t=None) == ARG
    assert up_nm(dt=3) == ARG
    assert up_nm(n=3) == SHAPE
    assert up_nm(n=8, m=32) == SHAPE
    assert up_nm(f=520) == SHAPE                  # d_ff not a multiple of m
    assert up_nm(T=-1) == SHAPE
    assert up_nm(d=100) == ALIGN
    assert up_nm(vals=MIS) == ALIGN
    assert up_nm(idx=MIS) == ALIGN
    assert up_nm(b1=MIS + 2) == ALIGN
    assert up_nm(T=0, vals=None, idx=None) == 0   # nothing to do, nothing touched


@pytestmark_nogpu
def test_nm_down_rejects():
    L = tw.lib()

    def down(**kw):
        # nm_ffn_down(vals, idx, dtype, T, d_ff, n, m, w2 [d_ff][d_model], d_model, y, y_dtype, stream)
        a = dict(vals=FAKE, idx=FAKE, dt=1, T=64, f=512, n=8, m=16, w2=FAKE, d=256, y=FAKE, ydt=0)
        a.update(kw)
        return L.nm_ffn_down(a["vals"], a["idx"], a["dt"], a["T"], a["f"], a["n"], a["m"], a["w2"], a["d"],
                             a["y"], a["ydt"], None)
    assert down(w2=None) == ARG
    assert down(vals=None) == ARG
    assert down(ydt=5) == ARG
    assert down(n=2, m=4) == UNSUP
    assert down(n=3) == SHAPE
    assert down(dt=0) == UNSUP                    # fp32 values
    assert down(f=528) == SHAPE                   # d_ff not a multiple of 32
    assert down(d=260) == SHAPE                   # d_model not a multiple of 8
    assert down(w2=MIS) == ALIGN
    assert down(y=MIS) == ALIGN
    assert down(f=1 << 20, d=1024) == UNSUP       # w2 of 2 GiB
    assert down(f=1 << 23, d=8) == UNSUP          # 256 rows of packed values of 2 GiB
