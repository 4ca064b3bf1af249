"""Shared test plumbing: numpy <-> torch device transfers, oracle-side references and the
comparison rules of the parity tests."""
from __future__ import annotations

import numpy as np

from oracle import twell_oracle as orc


def to_dev(a: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    if dtype == "i32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    raise ValueError(dtype)


def from_dev(t) -> np.ndarray:
    """Device tensor -> numpy float64 (exact), int array, or uint8."""
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        bits = t.view(torch.int16).numpy().view(np.uint16)
        return orc.widen(bits, "bf16")
    if t.dtype == torch.float32:
        return t.numpy().astype(np.float64)
    return t.numpy()


def inputs64(g: dict):
    dt = g["dtype"]
    x = orc.widen(g["x"], dt)
    w1t = orc.widen(g["w1t"], dt)
    w2 = orc.widen(g["w2"], dt)
    b1 = g["b1"].astype(np.float64)
    dy = orc.widen(g["dy"], dt) if g.get("dy") is not None else None
    return x, w1t, b1, w2, dy


def rel_err(a: np.ndarray, ref: np.ndarray) -> float:
    den = np.abs(ref).max()
    return float(np.abs(a - ref).max() / (den if den > 0 else 1.0))


def twell_host(h) -> dict:
    """Device TwellMatrix -> dict shaped like the oracle's twell_pack output."""
    cap = h.ovf_cap
    n = int(from_dev(h.ovf_n)[0])
    k = min(n, cap)
    # only the stored backup rows: the rest of ovf_dense is uninitialised memory
    return {"counts": from_dev(h.counts), "col_idx": from_dev(h.col_idx), "vals": from_dev(h.vals),
            "ovf_n": n, "ovf_rows": from_dev(h.ovf_rows)[:k],
            "ovf_slot": from_dev(h.ovf_slot), "ovf_dense": from_dev(h.ovf_dense[:k]),
            "tile_w": h.tile_w, "slots": h.slots, "ovf_cap": cap, "shape": (h.rows, h.cols)}


def assert_twell_equal(got: dict, want: dict, check_dense: bool = True):
    """Bit-exact comparison of every integer field and of the stored values."""
    assert np.array_equal(got["counts"], want["counts"]), "counts differ"
    assert np.array_equal(got["col_idx"], want["col_idx"]), "col_idx differ"
    gv, wv = got["vals"], want["vals"]
    assert np.array_equal(gv, wv), "vals differ"
    assert not np.any(np.signbit(gv[got["col_idx"] < 0])), "pad must be +0.0"
    assert got["ovf_n"] == want["ovf_n"], (got["ovf_n"], want["ovf_n"])
    assert np.array_equal(got["ovf_rows"], want["ovf_rows"]), "ovf_rows differ"
    assert np.array_equal(got["ovf_slot"], want["ovf_slot"]), "ovf_slot differ"
    if check_dense:
        k = len(want["ovf_rows"])
        assert np.array_equal(got["ovf_dense"][:k], want["ovf_dense"][:k]), "ovf_dense differ"
