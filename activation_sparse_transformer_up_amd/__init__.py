"""Activation-sparse transformer FFN (TwELL) on AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libtwell.so`` (declared in include/twell.h): the
functions below only check tensors, allocate outputs with torch and pass raw device
pointers plus the current HIP stream. Every step of the computation runs in the HIP
kernels of the library; there is no fallback path. If the library is missing, every call
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "TwellError", "TwellMatrix", "lib", "twell_abi_version", "twell_pack", "twell_ffn_fwd",
    "twell_down", "twell_fwd_down", "twell_up_gemm", "twell_up_finish", "ffn_up_relu_dense",
    "twell_gate_up", "twell_gated_ffn_fwd", "twell_gated_ffn_infer", "twell_gate_up_workspace_bytes", "twell_ffn_bwd",
    "twell_ffn_bwd_workspace_bytes", "twell_ffn_bwd_noalloc",
    "nm_prune", "ffn_up_relu_nm", "nm_ffn_down", "twell_sync_status", "twell_row_max_histogram",
    "twell_stash_bytes", "twell_choose_slots", "twell_to_row_ell", "twell_row_nnz_histogram",
    "twell_choose_row_ell_width", "F32", "BF16",
]

F32, BF16 = 0, 1
STATUS = {0: "TWELL_OK", -1: "TWELL_ERR_ARG", -2: "TWELL_ERR_SHAPE", -3: "TWELL_ERR_ALIGN",
          -4: "TWELL_ERR_WORKSPACE", -5: "TWELL_ERR_OVF_CAPACITY", -6: "TWELL_ERR_HIP",
          -7: "TWELL_ERR_UNSUPPORTED"}
# token count up to which the up GEMM takes its decode kernels (include/twell.h, row_list)
DECODE_MAX_T = 64
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtwell.so")

_c = ctypes
_P, _I, _F, _Z = _c.c_void_p, _c.c_int32, _c.c_float, _c.c_size_t


class TwellError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


class TwellMatrixC(_c.Structure):
    _fields_ = [("rows", _I), ("cols", _I), ("tile_w", _I), ("slots", _I), ("ovf_cap", _I),
                ("val_dtype", _I), ("counts", _P), ("col_idx", _P), ("vals", _P), ("ovf_n", _P),
                ("ovf_rows", _P), ("ovf_slot", _P), ("ovf_dense", _P), ("ovf_bits", _P),
                ("row_nnz", _P), ("row_list", _P)]


_SIGS = {
    "twell_abi_version": ([], _I),
    "twell_status_str": ([_I], _c.c_char_p),
    "twell_ovf_bits_words": ([_I, _I, _I], _Z),
    "twell_row_list_bytes": ([_I, _I, _I, _I], _Z),
    "twell_pack": ([_P, _I, _P, _P], _I),
    "twell_ffn_fwd": ([_P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _I, _P], _I),
    "twell_down": ([_P, _P, _I, _I, _P, _I, _P], _I),
    "twell_fwd_down": ([_P, _P, _I, _I, _P, _I, _P], _I),
    "twell_up_gemm": ([_P, _P, _P, _I, _I, _I, _I, _P, _P], _I),
    "twell_up_finish": ([_P, _P, _P, _I, _I, _I, _I, _P, _P], _I),
    "ffn_up_relu_dense": ([_P, _P, _P, _I, _I, _I, _I, _P, _I, _P], _I),
    "twell_gate_up_workspace_bytes": ([_I, _I, _I, _I, _P], _Z),
    "twell_gate_up": ([_P, _P, _P, _I, _I, _I, _I, _P, _Z, _P], _I),
    "twell_gated_ffn_fwd": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _I, _P, _Z, _P], _I),
    "twell_gated_ffn_infer": ([_P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _I, _P], _I),
    "twell_ffn_bwd_workspace_bytes": ([_I, _I, _I, _I, _P], _Z),
    "twell_ffn_bwd_workspace_bytes_nnz": ([_I, _I, _I, _I, _P, _c.c_int64], _Z),
    "twell_ffn_bwd": ([_P, _P, _P, _I, _I, _I, _I, _P, _P, _F, _P, _P, _P, _P, _P, _Z, _P], _I),
    "twell_ffn_bwd_noalloc": ([_P, _P, _P, _I, _I, _I, _I, _P, _P, _F, _P, _P, _P, _P, _P], _I),
    "nm_prune": ([_P, _I, _I, _I, _I, _I, _P, _P, _P], _I),
    "ffn_up_relu_nm": ([_P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P], _I),
    "nm_ffn_down": ([_P, _P, _I, _I, _I, _I, _I, _P, _I, _P, _I, _P], _I),
    "twell_sync_status": ([_P, _P], _I),
    "twell_to_row_ell": ([_P, _P, _P], _I),
    "twell_row_nnz_histogram": ([_P, _P, _I, _P], _I),
    "twell_choose_row_ell_width": ([_P, _I, _I, _I, _I, _I, _P], _I),
    "twell_row_max_histogram": ([_P, _P, _P], _I),
    "twell_stash_bytes": ([_I, _I, _I, _I, _I, _I], _Z),
    "twell_choose_slots": ([_P, _I, _I, _I, _I, _I, _P], _I),
}

_LIB = None


def lib():
    """Load libtwell.so (built in-tree by activation_sparse_transformer_up_amd.build)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m activation_sparse_transformer_up_amd.build`")
        L = _c.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _LIB = L
    return _LIB


def _check(status: int, where: str):
    if status != 0:
        raise TwellError(status, where)


def _dt(t: torch.dtype) -> int:
    if t == torch.float32:
        return F32
    if t == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t}")


def _tdt(code: int) -> torch.dtype:
    return torch.float32 if code == F32 else torch.bfloat16


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(device=None):
    return torch.cuda.current_stream(device).cuda_stream


def twell_abi_version() -> int:
    return lib().twell_abi_version()


class TwellMatrix:
    """Device buffers of a TwELL matrix (see twell_matrix_t in include/twell.h)."""

    def __init__(self, rows: int, cols: int, tile_w: int, slots: int, ovf_cap: int,
                 val_dtype: torch.dtype = torch.float32, device="cuda"):
        self.rows, self.cols, self.tile_w, self.slots, self.ovf_cap = rows, cols, tile_w, slots, ovf_cap
        self.val_dtype = val_dtype
        nt = cols // tile_w
        i32 = dict(dtype=torch.int32, device=device)
        self.counts = torch.empty((rows, nt), **i32)
        self.col_idx = torch.empty((rows, nt, slots), **i32)
        self.vals = torch.empty((rows, nt, slots), dtype=val_dtype, device=device)
        self.ovf_n = torch.zeros((1,), **i32)
        self.ovf_rows = torch.empty((max(ovf_cap, 1),), **i32)
        self.ovf_slot = torch.empty((rows,), **i32)
        self.ovf_dense = torch.empty((max(ovf_cap, 1), cols), dtype=val_dtype, device=device)
        words = lib().twell_ovf_bits_words(rows, cols, tile_w)
        self.ovf_bits = torch.empty((max(words, 1),), **i32)
        self.row_nnz = torch.empty((max(rows, 1),), **i32)
        lb = lib().twell_row_list_bytes(rows, cols, tile_w, slots)
        # up to DECODE_MAX_T rows the scratch also holds the decode GEMM's workspace and
        # tickets; none of it needs initialising
        self.row_list = torch.empty((max(lb // 8, 2),), dtype=torch.int64, device=device)

    def c(self) -> TwellMatrixC:
        return TwellMatrixC(self.rows, self.cols, self.tile_w, self.slots, self.ovf_cap,
                            _dt(self.val_dtype), _ptr(self.counts), _ptr(self.col_idx),
                            _ptr(self.vals), _ptr(self.ovf_n), _ptr(self.ovf_rows),
                            _ptr(self.ovf_slot), _ptr(self.ovf_dense), _ptr(self.ovf_bits),
                            _ptr(self.row_nnz), _ptr(self.row_list))

    @property
    def n_tiles(self) -> int:
        return self.cols // self.tile_w


def twell_pack(h: torch.Tensor, tile_w: int, slots: int, ovf_cap: int,
               val_dtype: torch.dtype | None = None, out: TwellMatrix | None = None) -> TwellMatrix:
    R, C = h.shape
    if out is None:
        out = TwellMatrix(R, C, tile_w, slots, ovf_cap, val_dtype or h.dtype, h.device)
    m = out.c()
    _check(lib().twell_pack(_ptr(h), _dt(h.dtype), _c.byref(m), _stream(h.device)), "twell_pack")
    return out


def twell_ffn_fwd(x, w1t, b1, w2, tile_w: int, slots: int, ovf_cap: int,
                  val_dtype=torch.float32, y_dtype=torch.float32, h: TwellMatrix | None = None,
                  y: torch.Tensor | None = None):
    """y = ReLU(x w1t^T + b1) w2 with the hidden activations packed in TwELL. Returns (y, h)."""
    T, d = x.shape
    f = w1t.shape[0]
    if w1t.dtype != x.dtype or w2.dtype != x.dtype:
        raise TypeError("x, w1t and w2 must share a dtype")
    if b1.dtype != torch.float32:
        raise TypeError("b1 must be float32")
    if h is None:
        h = TwellMatrix(T, f, tile_w, slots, ovf_cap, val_dtype, x.device)
    if y is None:
        y = torch.empty((T, d), dtype=y_dtype, device=x.device)
    m = h.c()
    _check(lib().twell_ffn_fwd(_ptr(x), _ptr(w1t), _ptr(b1), _ptr(w2), _dt(x.dtype), T, d, f,
                               _c.byref(m), _ptr(y), _dt(y.dtype), _stream(x.device)), "twell_ffn_fwd")
    return y, h


def twell_gate_up_workspace_bytes(T: int, d: int, f: int, h: TwellMatrix, dtype=torch.bfloat16) -> int:
    m = h.c()
    return lib().twell_gate_up_workspace_bytes(T, d, f, _dt(dtype), _c.byref(m))


def _gate_ws(T, d, f, h, dtype, device, workspace):
    need = twell_gate_up_workspace_bytes(T, d, f, h, dtype)
    if need and (workspace is None or workspace.numel() < need):
        workspace = torch.empty((need,), dtype=torch.uint8, device=device)
    return workspace


def twell_gated_ffn_fwd(x, wgt, bg, wut, w2, tile_w: int, slots: int, ovf_cap: int,
                        val_dtype=torch.float32, y_dtype=torch.float32, h: TwellMatrix | None = None,
                        y: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """y = (ReLU(x wgt^T + bg) * (x wut^T)) w2 with the gate activations packed in TwELL.
    Returns (y, h); h's slots hold the gate, its row lists the gated products. From 512 tokens
    on the up stage needs a workspace (allocated here unless a large enough one is given)."""
    T, d = x.shape
    f = wgt.shape[0]
    if wgt.dtype != x.dtype or wut.dtype != x.dtype or w2.dtype != x.dtype:
        raise TypeError("x, wgt, wut and w2 must share a dtype")
    if bg.dtype != torch.float32:
        raise TypeError("bg must be float32")
    if h is None:
        h = TwellMatrix(T, f, tile_w, slots, ovf_cap, val_dtype, x.device)
    if y is None:
        y = torch.empty((T, d), dtype=y_dtype, device=x.device)
    workspace = _gate_ws(T, d, f, h, x.dtype, x.device, workspace)
    m = h.c()
    _check(lib().twell_gated_ffn_fwd(_ptr(x), _ptr(wgt), _ptr(bg), _ptr(wut), _ptr(w2), _dt(x.dtype), T, d, f,
                                     _c.byref(m), _ptr(y), _dt(y.dtype), _ptr(workspace),
                                     workspace.numel() if workspace is not None else 0, _stream(x.device)),
           "twell_gated_ffn_fwd")
    return y, h


def twell_gated_ffn_infer(x, wgt, bg, wut, w2, tile_w: int, slots: int, val_dtype=torch.float32,
                          y_dtype=torch.float32, h: TwellMatrix | None = None, y: torch.Tensor | None = None):
    """Decode-size gated forward (T <= 64): the gate GEMM, then one fused kernel over the active
    units (up dot product and down multiply-add). Returns (y, h); h holds the gate's TwELL."""
    T, d = x.shape
    f = wgt.shape[0]
    if wgt.dtype != x.dtype or wut.dtype != x.dtype or w2.dtype != x.dtype:
        raise TypeError("x, wgt, wut and w2 must share a dtype")
    if bg.dtype != torch.float32:
        raise TypeError("bg must be float32")
    if h is None:
        h = TwellMatrix(T, f, tile_w, slots, 0, val_dtype, x.device)
    if y is None:
        y = torch.empty((T, d), dtype=y_dtype, device=x.device)
    m = h.c()
    _check(lib().twell_gated_ffn_infer(_ptr(x), _ptr(wgt), _ptr(bg), _ptr(wut), _ptr(w2), _dt(x.dtype), T, d, f,
                                       _c.byref(m), _ptr(y), _dt(y.dtype), _stream(x.device)),
           "twell_gated_ffn_infer")
    return y, h


def twell_gate_up(h: TwellMatrix, x, wut, workspace: torch.Tensor | None = None) -> TwellMatrix:
    """The up stage of the gated forward: row-list and backup values g <- g * (x[t] . wut[j])."""
    T, d = x.shape
    workspace = _gate_ws(T, d, wut.shape[0], h, x.dtype, x.device, workspace)
    m = h.c()
    _check(lib().twell_gate_up(_c.byref(m), _ptr(x), _ptr(wut), _dt(x.dtype), T, d, wut.shape[0], _ptr(workspace),
                               workspace.numel() if workspace is not None else 0, _stream(x.device)),
           "twell_gate_up")
    return h


def twell_up_gemm(x, w1t, b1, h: TwellMatrix) -> TwellMatrix:
    """Stage 1 of twell_ffn_fwd: up GEMM with the fused ReLU + TwELL epilogue."""
    T, d = x.shape
    m = h.c()
    _check(lib().twell_up_gemm(_ptr(x), _ptr(w1t), _ptr(b1), _dt(x.dtype), T, d, w1t.shape[0],
                               _c.byref(m), _stream(x.device)), "twell_up_gemm")
    return h


def twell_up_finish(x, w1t, b1, h: TwellMatrix) -> TwellMatrix:
    """Stage 2 of twell_ffn_fwd: overflow list, slots, count and dense backup rows."""
    T, d = x.shape
    m = h.c()
    _check(lib().twell_up_finish(_ptr(x), _ptr(w1t), _ptr(b1), _dt(x.dtype), T, d, w1t.shape[0],
                                 _c.byref(m), _stream(x.device)), "twell_up_finish")
    return h


def twell_down(h: TwellMatrix, w2: torch.Tensor, y_dtype=torch.float32, y=None) -> torch.Tensor:
    d = w2.shape[1]
    if y is None:
        y = torch.empty((h.rows, d), dtype=y_dtype, device=w2.device)
    m = h.c()
    _check(lib().twell_down(_c.byref(m), _ptr(w2), _dt(w2.dtype), d, _ptr(y), _dt(y.dtype),
                            _stream(w2.device)), "twell_down")
    return y


def twell_fwd_down(h: TwellMatrix, w2: torch.Tensor, y_dtype=torch.float32, y=None) -> torch.Tensor:
    """Stage 3 of twell_ffn_fwd: the down projection on the row lists twell_up_finish built."""
    d = w2.shape[1]
    if y is None:
        y = torch.empty((h.rows, d), dtype=y_dtype, device=w2.device)
    m = h.c()
    _check(lib().twell_fwd_down(_c.byref(m), _ptr(w2), _dt(w2.dtype), d, _ptr(y), _dt(y.dtype),
                                _stream(w2.device)), "twell_fwd_down")
    return y


def ffn_up_relu_dense(x, w1t, b1, h_dtype=torch.float32, out=None) -> torch.Tensor:
    T, d = x.shape
    f = w1t.shape[0]
    if out is None:
        out = torch.empty((T, f), dtype=h_dtype, device=x.device)
    _check(lib().ffn_up_relu_dense(_ptr(x), _ptr(w1t), _ptr(b1), _dt(x.dtype), T, d, f, _ptr(out),
                                   _dt(out.dtype), _stream(x.device)), "ffn_up_relu_dense")
    return out


def twell_ffn_bwd_workspace_bytes(T: int, d: int, f: int, h: TwellMatrix, dtype=torch.bfloat16,
                                  nnz: int | None = None) -> int:
    """Workspace bytes of twell_ffn_bwd: for all of h's entry capacity, or for ``nnz`` stored
    entries (the step's actual count, e.g. from twell_row_nnz_histogram)."""
    m = h.c()
    if nnz is None:
        return lib().twell_ffn_bwd_workspace_bytes(T, d, f, _dt(dtype), _c.byref(m))
    return lib().twell_ffn_bwd_workspace_bytes_nnz(T, d, f, _dt(dtype), _c.byref(m), int(nnz))


def twell_ffn_bwd(x, w1t, w2, h: TwellMatrix, dy, l1_coef: float, want_db1: bool = True,
                  workspace: torch.Tensor | None = None):
    """Gradients (dx, dw1t, dw2, db1) of <dy, y> + l1_coef * sum(h), fp32. A given workspace
    may be smaller than the capacity size (twell_ffn_bwd_workspace_bytes with nnz): the call's
    entries must fit, else the outputs are NaN."""
    T, d = x.shape
    f = w1t.shape[0]
    dev = x.device
    dx = torch.empty((T, d), dtype=torch.float32, device=dev)
    dw1t = torch.empty((f, d), dtype=torch.float32, device=dev)
    dw2 = torch.empty((f, d), dtype=torch.float32, device=dev)
    db1 = torch.empty((f,), dtype=torch.float32, device=dev) if want_db1 else None
    if workspace is None:
        nbytes = twell_ffn_bwd_workspace_bytes(T, d, f, h, x.dtype)
        workspace = torch.empty((max(nbytes, 16),), dtype=torch.uint8, device=dev)
    m = h.c()
    _check(lib().twell_ffn_bwd(_ptr(x), _ptr(w1t), _ptr(w2), _dt(x.dtype), T, d, f, _c.byref(m),
                               _ptr(dy), float(l1_coef), _ptr(dx), _ptr(dw1t), _ptr(dw2), _ptr(db1),
                               _ptr(workspace), workspace.numel(), _stream(dev)), "twell_ffn_bwd")
    return dx, dw1t, dw2, db1


# bytes of the fixed device scratch behind twell_ffn_bwd_noalloc (include/twell.h)
NOALLOC_SCRATCH_BYTES = 64 << 20


def twell_ffn_bwd_noalloc(x, w1t, w2, h: TwellMatrix, dy, l1_coef: float, out=None):
    """twell_ffn_bwd on the library's fixed per-GPU scratch (no workspace). ``out``: optional
    (dx, dw1t, dw2, db1) tensors to write (db1 may be None); allocated here if not given."""
    T, d = x.shape
    f = w1t.shape[0]
    dev = x.device
    if out is None:
        out = (torch.empty((T, d), dtype=torch.float32, device=dev),
               torch.empty((f, d), dtype=torch.float32, device=dev),
               torch.empty((f, d), dtype=torch.float32, device=dev),
               torch.empty((f,), dtype=torch.float32, device=dev))
    dx, dw1t, dw2, db1 = out
    m = h.c()
    _check(lib().twell_ffn_bwd_noalloc(_ptr(x), _ptr(w1t), _ptr(w2), _dt(x.dtype), T, d, f, _c.byref(m),
                                       _ptr(dy), float(l1_coef), _ptr(dx), _ptr(dw1t), _ptr(dw2), _ptr(db1),
                                       _stream(dev)), "twell_ffn_bwd_noalloc")
    return dx, dw1t, dw2, db1


def nm_prune(h: torch.Tensor, n: int, m: int):
    T, f = h.shape
    vals = torch.empty((T, f // m, n), dtype=h.dtype, device=h.device)
    idx = torch.empty((T, f // m, n), dtype=torch.uint8, device=h.device)
    _check(lib().nm_prune(_ptr(h), _dt(h.dtype), T, f, n, m, _ptr(vals), _ptr(idx), _stream(h.device)),
           "nm_prune")
    return vals, idx


def ffn_up_relu_nm(x, w1t, b1, n: int, m: int, vals=None, idx=None):
    """N:M-pruned h = ReLU(x W1 + b1) from the up GEMM's epilogue: (vals [T][f/m][n] in x's
    dtype, idx [T][f/m][n] uint8)."""
    T, d = x.shape
    f = w1t.shape[0]
    if vals is None:
        vals = torch.empty((T, f // m, n), dtype=x.dtype, device=x.device)
    if idx is None:
        idx = torch.empty((T, f // m, n), dtype=torch.uint8, device=x.device)
    _check(lib().ffn_up_relu_nm(_ptr(x), _ptr(w1t), _ptr(b1), _dt(x.dtype), T, d, f, n, m, _ptr(vals),
                                _ptr(idx), _stream(x.device)), "ffn_up_relu_nm")
    return vals, idx


def nm_ffn_down(vals, idx, n: int, m: int, w2: torch.Tensor, y_dtype=torch.float32, y=None):
    """w2: [d_ff][d_model] bf16, the down weight the TwELL entry points take."""
    T, G, _ = vals.shape
    f = G * m
    if w2.shape[0] != f:
        raise ValueError(f"nm_ffn_down: w2 has {w2.shape[0]} rows, the activations {f} columns")
    d = w2.shape[1]
    if y is None:
        y = torch.empty((T, d), dtype=y_dtype, device=vals.device)
    _check(lib().nm_ffn_down(_ptr(vals), _ptr(idx), _dt(vals.dtype), T, f, n, m, _ptr(w2), d, _ptr(y),
                             _dt(y.dtype), _stream(vals.device)), "nm_ffn_down")
    return y


def twell_sync_status(h: TwellMatrix) -> int:
    m = h.c()
    return lib().twell_sync_status(_c.byref(m), _stream(h.counts.device))


def twell_row_max_histogram(h: TwellMatrix, hist: torch.Tensor | None = None) -> torch.Tensor:
    """Device int32 [tile_w + 1]: rows of h by their largest per-tile true count."""
    if hist is None:
        hist = torch.empty((h.tile_w + 1,), dtype=torch.int32, device=h.counts.device)
    m = h.c()
    _check(lib().twell_row_max_histogram(_c.byref(m), _ptr(hist), _stream(h.counts.device)),
           "twell_row_max_histogram")
    return hist


def twell_stash_bytes(rows: int, cols: int, tile_w: int, slots: int, n_ovf: int,
                      val_dtype=torch.float32) -> int:
    return lib().twell_stash_bytes(rows, cols, tile_w, slots, n_ovf, _dt(val_dtype))


def twell_choose_slots(hist, tile_w: int, rows: int, cols: int, ovf_cap: int, val_dtype=torch.float32):
    """(S, stash bytes) from a host copy of the histogram (numpy or CPU tensor); raises
    TwellError (TWELL_ERR_OVF_CAPACITY) if no slot count fits ovf_cap."""
    import numpy as np
    hh = np.ascontiguousarray(np.asarray(hist.cpu() if hasattr(hist, "cpu") else hist), dtype=np.int32)
    out = _c.c_size_t(0)
    s = lib().twell_choose_slots(hh.ctypes.data_as(_c.c_void_p), tile_w, rows, cols, ovf_cap, _dt(val_dtype),
                                 _c.byref(out))
    _check(s if s < 0 else 0, "twell_choose_slots")
    return s, out.value


def twell_row_nnz_histogram(h: TwellMatrix, nbins: int | None = None,
                            hist: torch.Tensor | None = None) -> torch.Tensor:
    """Device int32 [nbins]: rows of h by their number of nonzeros (the last bin holds every
    row of nbins - 1 or more; default nbins = cols + 1, exact)."""
    nbins = nbins or h.cols + 1
    if hist is None:
        hist = torch.empty((nbins,), dtype=torch.int32, device=h.counts.device)
    m = h.c()
    _check(lib().twell_row_nnz_histogram(_c.byref(m), _ptr(hist), nbins, _stream(h.counts.device)),
           "twell_row_nnz_histogram")
    return hist


def twell_choose_row_ell_width(hist, rows: int, cols: int, ovf_cap: int, val_dtype=torch.float32):
    """(N, stash bytes) of the row-ELL from a host copy of a row-nonzero histogram; raises
    TwellError (TWELL_ERR_OVF_CAPACITY) if no width fits ovf_cap."""
    import numpy as np
    hh = np.ascontiguousarray(np.asarray(hist.cpu() if hasattr(hist, "cpu") else hist), dtype=np.int32)
    out = _c.c_size_t(0)
    n = lib().twell_choose_row_ell_width(hh.ctypes.data_as(_c.c_void_p), len(hh), rows, cols, ovf_cap,
                                         _dt(val_dtype), _c.byref(out))
    _check(n if n < 0 else 0, "twell_choose_row_ell_width")
    return n, out.value


def twell_to_row_ell(src: TwellMatrix, width: int, ovf_cap: int, val_dtype: torch.dtype | None = None,
                     out: TwellMatrix | None = None) -> TwellMatrix:
    """The compact row-ELL (one tile per row, ``width`` slots, dense backup for wider rows) of
    the TwELL src."""
    if out is None:
        out = TwellMatrix(src.rows, src.cols, src.cols, width, ovf_cap, val_dtype or src.val_dtype,
                          src.counts.device)
    ms, md = src.c(), out.c()
    _check(lib().twell_to_row_ell(_c.byref(ms), _c.byref(md), _stream(src.counts.device)), "twell_to_row_ell")
    return out
