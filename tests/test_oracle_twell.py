"""Pins of the oracle's TwELL packer: a hand-built example, an independent brute-force
packer on tiny edge-case inputs, the exact round trip, the format invariants, and the
reduction to classic row ELL when one tile spans the whole row."""
import numpy as np
import pytest

from oracle import twell_oracle as orc


def brute_pack(h, W, S, cap):
    """Independent, loop-by-loop restatement of the format for tiny inputs."""
    R, C = h.shape
    nt = C // W
    counts = [[0] * nt for _ in range(R)]
    idx = [[[-1] * S for _ in range(nt)] for _ in range(R)]
    val = [[[0.0] * S for _ in range(nt)] for _ in range(R)]
    for r in range(R):
        for k in range(nt):
            found = []
            for c in range(k * W, (k + 1) * W):
                if h[r, c] != 0.0:
                    found.append(c)
            counts[r][k] = len(found)
            for s in range(min(S, len(found))):
                idx[r][k][s] = found[s]
                val[r][k][s] = h[r, found[s]]
    ovf = [r for r in range(R) if max(counts[r]) > S]
    return counts, idx, val, ovf


def check_invariants(h, tw):
    R, C = h.shape
    W, S = tw["tile_w"], tw["slots"]
    counts, col_idx, vals = tw["counts"], tw["col_idx"], tw["vals"]
    assert np.array_equal(counts.sum(1), (h != 0).sum(1))
    for r in range(R):
        for k in range(C // W):
            n = min(counts[r, k], S)
            cols = col_idx[r, k, :n]
            assert np.all(np.diff(cols) > 0)
            assert np.all((cols >= k * W) & (cols < (k + 1) * W))
            assert np.all(col_idx[r, k, n:] == -1)
            pad = vals[r, k, n:]
            assert np.all(pad == 0) and not np.any(np.signbit(pad))
            assert np.array_equal(vals[r, k, :n], h[r, cols])
    want = [r for r in range(R) if (counts[r] > S).any()]
    assert tw["ovf_n"] == len(want)
    assert list(tw["ovf_rows"]) == want[: tw["ovf_cap"]]


def test_hand_built_example():
    # h from the worked FFN example: rows [1, 0, 1.5, 0] and [0, 1.5, 0, 1].
    h = np.array([[1, 0, 1.5, 0], [0, 1.5, 0, 1]], float)
    tw = orc.twell_pack(h, tile_w=2, slots=1, ovf_cap=1)
    assert tw["counts"].tolist() == [[1, 1], [1, 1]]
    assert tw["col_idx"].tolist() == [[[0], [2]], [[1], [3]]]
    assert tw["vals"].tolist() == [[[1.0], [1.5]], [[1.5], [1.0]]]
    assert tw["ovf_n"] == 0 and tw["ovf_slot"].tolist() == [-1, -1]
    # One tile over the whole row with one slot: both rows overflow, only one fits.
    tw = orc.twell_pack(h, tile_w=4, slots=1, ovf_cap=1)
    assert tw["counts"].tolist() == [[2], [2]]
    assert tw["col_idx"].tolist() == [[[0]], [[1]]]
    assert tw["ovf_n"] == 2 and tw["ovf_rows"].tolist() == [0]
    assert tw["ovf_slot"].tolist() == [0, -1]
    assert tw["ovf_dense"].tolist() == [[1, 0, 1.5, 0]]


def edge_matrix(W=8, S=3):
    C = 4 * W
    rows = []
    rows.append(np.zeros(C))                                  # all zero
    rows.append(np.arange(1, C + 1, dtype=float))             # full tiles
    r = np.zeros(C); r[[0, 1, 2]] = [1, -2, 3]; rows.append(r)              # exactly S
    r = np.zeros(C); r[[W, W + 1, W + 2, W + 3]] = 5; rows.append(r)        # S+1 in tile 1
    r = np.zeros(C); r[[0, W - 1, W, 2 * W - 1, C - 1]] = 7; rows.append(r)  # tile edges
    r = np.zeros(C); r[[3, 4]] = [-0.0, 0.0]; r[5] = -1.0; rows.append(r)   # signed zeros
    r = np.zeros(C); r[[2, 9]] = [5e-324, -1e-310]; rows.append(r)          # subnormals
    r = np.zeros(C); r[2 * W:3 * W] = -1.0; rows.append(r)                  # negative full tile
    return np.array(rows)


@pytest.mark.parametrize("W,S,cap", [(8, 3, 0), (8, 3, 2), (8, 3, 16), (8, 8, 4), (4, 1, 3)])
def test_matches_brute_force_on_edge_cases(W, S, cap):
    h = edge_matrix(8, 3)
    C = h.shape[1]
    if C % W:
        pytest.skip("tile does not divide")
    tw = orc.twell_pack(h, W, S, cap)
    counts, idx, val, ovf = brute_pack(h, W, S, cap)
    assert tw["counts"].tolist() == counts
    assert tw["col_idx"].tolist() == idx
    assert np.array_equal(tw["vals"], np.array(val))
    assert tw["ovf_n"] == len(ovf)
    assert tw["ovf_rows"].tolist() == ovf[:cap]
    check_invariants(h, tw)


def test_signed_zero_counts_as_zero():
    h = np.array([[-0.0, 0.0, 2.0, -0.0]])
    tw = orc.twell_pack(h, 4, 2, 1)
    assert tw["counts"].tolist() == [[1]]
    assert tw["col_idx"].tolist() == [[[2, -1]]]


@pytest.mark.parametrize("seed", range(4))
def test_random_sparse_roundtrip_and_brute_force(seed):
    rng = np.random.default_rng(seed)
    R, W, nt = 37, 16, 5
    h = rng.standard_normal((R, W * nt)) * (rng.random((R, W * nt)) < 0.08 * (1 + seed))
    S = 2 + seed
    cap = 1000
    tw = orc.twell_pack(h, W, S, cap)
    counts, idx, val, ovf = brute_pack(h, W, S, cap)
    assert tw["counts"].tolist() == counts and tw["col_idx"].tolist() == idx
    assert tw["ovf_rows"].tolist() == ovf
    check_invariants(h, tw)
    back = orc.twell_unpack(tw)
    # slot-built rows hold +0.0 in empty places; backup rows are verbatim copies (-0.0 kept)
    want = np.where(tw["ovf_slot"][:, None] >= 0, h, h + 0.0)
    assert np.array_equal(back, h) and np.array_equal(np.signbit(back), np.signbit(want))


def test_unpack_refuses_rows_beyond_capacity():
    h = np.ones((3, 8))
    tw = orc.twell_pack(h, 8, 2, ovf_cap=1)
    assert tw["ovf_n"] == 3
    with pytest.raises(ValueError):
        orc.twell_unpack(tw)


def test_one_tile_is_classic_ell():
    rng = np.random.default_rng(3)
    h = rng.standard_normal((9, 24)) * (rng.random((9, 24)) < 0.2)
    tw = orc.twell_pack(h, tile_w=24, slots=24, ovf_cap=0)
    for r in range(9):
        nz = np.flatnonzero(h[r])
        assert tw["counts"][r, 0] == len(nz)
        assert tw["col_idx"][r, 0, :len(nz)].tolist() == nz.tolist()
        assert np.array_equal(tw["vals"][r, 0, :len(nz)], h[r, nz])
    assert tw["ovf_n"] == 0


def test_planted_mistake_is_caught():
    # A packer that keeps the *last* S nonzeros instead of the first must disagree with the
    # brute force on the edge matrix (guards against an order mistake in the comparison).
    h = edge_matrix()
    tw = orc.twell_pack(h, 8, 3, 4)
    bad = tw["col_idx"].copy()
    bad[1, 0] = [5, 6, 7]
    counts, idx, val, ovf = brute_pack(h, 8, 3, 4)
    assert bad.tolist() != idx
