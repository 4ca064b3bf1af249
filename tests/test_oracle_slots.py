"""Pins of the dynamic slot count (row-maximum histogram, stash bytes, choice of S) and
checks of the library's host-side chooser against the oracle (no GPU needed).

[SFL] "Formato Híbrido para Treinamento": the compact width follows the data and the rows
beyond it go to the dense backup."""
import numpy as np
import pytest

from oracle import twell_oracle as orc


def skewed_h(R, C, seed):
    """Rows with very different densities (some rows dense enough to overflow small S)."""
    rng = np.random.default_rng(seed)
    p = np.exp(rng.uniform(np.log(0.002), np.log(0.3), size=(R, 1)))
    h = np.where(rng.random((R, C)) < p, rng.standard_normal((R, C)), 0.0)
    h[rng.random((R, C)) < 0.01] = -0.0
    return h


@pytest.mark.parametrize("R,C,W,seed", [(37, 256, 64, 1), (50, 512, 128, 2), (0, 128, 64, 3)])
def test_histogram_brute_force(R, C, W, seed):
    h = skewed_h(R, C, seed)
    counts = orc.twell_pack(h, W, 1, R)["counts"]
    want = [0] * (W + 1)
    for r in range(R):
        best = 0
        for k in range(C // W):
            c = 0
            for j in range(k * W, (k + 1) * W):
                if h[r, j] != 0.0:
                    c += 1
            best = max(best, c)
        want[best] += 1
    got = orc.row_max_histogram(counts, W)
    assert got.tolist() == want
    assert got.sum() == R


def test_histogram_tail_is_the_packers_overflow_count():
    R, C, W = 80, 512, 64
    h = skewed_h(R, C, 7)
    hist = orc.row_max_histogram(orc.twell_pack(h, W, 1, R)["counts"], W)
    assert hist[W // 4:].sum() > 0                       # some rows overflow small S
    for S in range(1, W + 1):
        assert hist[S + 1:].sum() == orc.twell_pack(h, W, S, R)["ovf_n"], S


@pytest.mark.parametrize("vb", [4, 2])
def test_stash_bytes_equals_packer_arrays(vb):
    R, C, W = 60, 512, 128
    h = skewed_h(R, C, 11)
    for S in (1, 3, 8, 16, 64):
        n = orc.twell_pack(h, W, S, R)["ovf_n"]
        tw = orc.twell_pack(h, W, S, n)
        size = (tw["counts"].size * 4 + tw["col_idx"].size * 4 + tw["vals"].size * vb + tw["ovf_slot"].size * 4
                + tw["ovf_rows"].size * 4 + tw["ovf_dense"].size * vb)
        assert orc.stash_bytes(R, C, W, S, n, vb) == size, S


def test_choose_slots_brute_force():
    R, C, W = 70, 512, 64
    h = skewed_h(R, C, 5)
    hist = orc.row_max_histogram(orc.twell_pack(h, W, 1, R)["counts"], W)
    for cap in (0, 3, 10, R):
        best = (None, None)
        for S in range(1, W + 1):
            tw = orc.twell_pack(h, W, S, R)
            n = tw["ovf_n"]
            if n > cap:
                continue
            b = (tw["counts"].size + tw["col_idx"].size + tw["vals"].size + R + n + n * C) * 4
            if best[1] is None or b < best[1]:
                best = (S, b)
        assert orc.choose_slots(hist, W, R, C, cap, 4) == best, cap


# ------------------------------------------------------------ the library's host chooser

tw = pytest.importorskip("activation_sparse_transformer_up_amd")


@pytest.mark.parametrize("W,R,C,cap,seed", [(128, 16384, 14336, 1024, 1), (64, 300, 1024, 0, 2),
                                            (128, 500, 4096, 20, 3), (64, 0, 512, 0, 4)])
def test_library_choose_slots_matches_oracle(W, R, C, cap, seed):
    import torch
    rng = np.random.default_rng(seed)
    # a geometric-like spread of row maxima, as skewed per-unit activity produces
    hist = np.zeros(W + 1, np.int64)
    if R:
        np.add.at(hist, np.minimum(rng.geometric(0.25, size=R), W), 1)
    for vdt, vb in ((torch.float32, 4), (torch.bfloat16, 2)):
        S, b = orc.choose_slots(hist, W, R, C, cap, vb)
        if S is None:
            with pytest.raises(tw.TwellError) as e:
                tw.twell_choose_slots(hist, W, R, C, cap, vdt)
            assert e.value.status == -5
            continue
        assert tw.twell_choose_slots(hist, W, R, C, cap, vdt) == (S, b)
        for s in (1, 8, min(W, 64)):
            n = int(hist[s + 1:].sum())
            assert tw.twell_stash_bytes(R, C, W, s, n, vdt) == orc.stash_bytes(R, C, W, s, n, vb)


def test_library_choose_slots_no_fit_and_rejects():
    import ctypes
    hist = np.zeros(129, np.int32)
    hist[100] = 5                                    # five rows above the 64-slot limit: never fit cap 4
    with pytest.raises(tw.TwellError) as e:
        tw.twell_choose_slots(hist, 128, 5, 256, 4)
    assert e.value.status == -5
    assert orc.choose_slots(hist, 128, 5, 256, 4, 4) == (None, None)
    assert tw.twell_choose_slots(hist, 128, 5, 256, 5)[0] == 1
    L = tw.lib()
    out = ctypes.c_size_t(0)
    assert L.twell_choose_slots(None, 64, 5, 256, 5, 0, ctypes.byref(out)) == -1
    assert L.twell_choose_slots(hist.ctypes.data_as(ctypes.c_void_p), 96, 5, 288, 5, 0, None) == -2
    assert L.twell_choose_slots(hist.ctypes.data_as(ctypes.c_void_p), 64, 5, 250, 5, 0, None) == -2
    assert L.twell_stash_bytes(5, 250, 64, 8, 0, 0) == 0
    assert L.twell_row_max_histogram(None, None, None) == -1


# ------------------------------------------------------------ the compact row-ELL width

def test_row_nnz_histogram_tail_is_the_row_ell_overflow_count():
    R, C = 90, 768
    h = skewed_h(R, C, 11)
    counts = orc.twell_pack(h, 128, 1, R)["counts"]
    hist = orc.row_nnz_histogram(counts, C + 1)
    assert hist.sum() == R
    assert int((hist * np.arange(C + 1)).sum()) == int((h != 0).sum())
    for N in (1, 5, 20, 60, C):
        assert orc.twell_pack(h, C, N, R)["ovf_n"] == int(hist[N + 1:].sum()), N
    # a last bin below the widest row collects every wider row
    short = orc.row_nnz_histogram(counts, 10)
    assert short.sum() == R and short[9] == int((hist[9:]).sum())


def test_choose_row_ell_width_brute_force():
    R, C = 60, 384
    h = skewed_h(R, C, 12)
    hist = orc.row_nnz_histogram(orc.twell_pack(h, 64, 1, R)["counts"], C + 1)
    for cap in (0, 2, 9, R):
        best = (None, None)
        for N in range(1, C + 1):
            tw = orc.twell_pack(h, C, N, R)
            n = tw["ovf_n"]
            if n > cap:
                continue
            b = (tw["counts"].size + tw["col_idx"].size + tw["vals"].size + R + n + n * C) * 4
            if best[1] is None or b < best[1]:
                best = (N, b)
        assert orc.choose_row_ell_width(hist, R, C, cap, 4) == best, cap


@pytest.mark.parametrize("R,C,cap,seed", [(16384, 14336, 1024, 1), (300, 1024, 0, 2), (500, 4096, 20, 3)])
def test_library_row_ell_width_matches_oracle(R, C, cap, seed):
    import torch
    rng = np.random.default_rng(seed)
    hist = np.zeros(C + 1, np.int64)
    np.add.at(hist, np.minimum(rng.poisson(0.0125 * C, size=R) + (rng.random(R) < 0.01) * C // 4, C), 1)
    for nbins in (C + 1, 200):
        hb = hist if nbins == C + 1 else np.concatenate([hist[:nbins - 1], [hist[nbins - 1:].sum()]])
        for vdt, vb in ((torch.float32, 4), (torch.bfloat16, 2)):
            N, b = orc.choose_row_ell_width(hb, R, C, cap, vb)
            if N is None:
                with pytest.raises(tw.TwellError) as e:
                    tw.twell_choose_row_ell_width(hb, R, C, cap, vdt)
                assert e.value.status == -5
                continue
            assert tw.twell_choose_row_ell_width(hb, R, C, cap, vdt) == (N, b)
