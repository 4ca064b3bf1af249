"""Pins of the oracle's N:M activation pruning: exhaustive enumeration of every subset of
every block on tiny inputs (the kept set must maximise the sum of magnitudes and be the
index-smallest maximiser), the layout counts quoted on the N:M page (6 for 2:4, 12,870 for
8:16), hand-built tie cases, and the closed-form density after pruning."""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import twell_oracle as orc


def best_subset(block, n):
    """Exhaustive search in lexicographic order; the first subset with the largest exact sum
    of magnitudes wins. Returns (subset, number of subsets visited)."""
    best, best_sum, visited = None, None, 0
    mags = [Fraction(abs(float(v))) for v in block]
    for sub in itertools.combinations(range(len(block)), n):
        visited += 1
        s = sum(mags[i] for i in sub)
        if best_sum is None or s > best_sum:
            best, best_sum = sub, s
    return best, visited


def test_layout_counts_match_the_page():
    # The N:M page quotes 6 valid layouts per 2:4 block and 12,870 per 8:16 block.
    assert best_subset(np.zeros(4), 2)[1] == 6
    assert best_subset(np.zeros(16), 8)[1] == 12870
    assert math.comb(32, 16) == 601080390


@pytest.mark.parametrize("n,m", [(2, 4), (4, 8), (8, 16)])
@pytest.mark.parametrize("kind", ["ties", "bf16"])
def test_exhaustive_enumeration(n, m, kind):
    rng = np.random.default_rng(100 + m + (kind == "ties"))
    groups = 6 if m == 16 else 40
    if kind == "ties":
        h = rng.integers(-3, 4, size=(groups, m)).astype(float)     # many equal magnitudes
    else:
        bits = synth.f32_to_bf16_bits(rng.standard_normal((groups, m)).astype(np.float32))
        h = orc.widen(bits, "bf16")
    vals, idx = orc.nm_prune(h.reshape(1, -1), n, m)
    for g in range(groups):
        sub, _ = best_subset(h[g], n)
        assert idx[0, g].tolist() == list(sub)
        assert np.array_equal(vals[0, g], h[g, list(sub)])


def test_hand_built_ties():
    h = np.array([[0.5, -2, 2, 1, 1, -1, 1, 0, 0, 0, 0, 0, 0, 0, 0, 3]], float)
    vals, idx = orc.nm_prune(h, 2, 4)
    assert idx.tolist() == [[[1, 2], [0, 1], [0, 1], [0, 3]]]
    assert vals.tolist() == [[[-2, 2], [1, -1], [0, 0], [0, 3]]]


def test_signed_zeros_tie_by_index():
    h = np.array([[-0.0, 0.0, -0.0, 0.0]])
    vals, idx = orc.nm_prune(h, 2, 4)
    assert idx.tolist() == [[[0, 1]]]
    assert np.signbit(vals[0, 0, 0]) and not np.signbit(vals[0, 0, 1])


@pytest.mark.parametrize("n,m", [(8, 16), (16, 32)])
def test_characterisation_every_block(n, m):
    rng = np.random.default_rng(m)
    bits = synth.f32_to_bf16_bits(np.maximum(rng.standard_normal((64, 4 * m)), 0).astype(np.float32))
    h = orc.widen(bits, "bf16")
    vals, idx = orc.nm_prune(h, n, m)
    for r in range(h.shape[0]):
        for g in range(4):
            blk = h[r, g * m:(g + 1) * m]
            kept = set(idx[r, g].tolist())
            assert len(kept) == n and sorted(kept) == idx[r, g].tolist()
            for i in kept:
                for k in set(range(m)) - kept:
                    # every kept entry outranks every dropped one: larger |h|, or equal |h|
                    # and lower index
                    assert abs(blk[i]) > abs(blk[k]) or (abs(blk[i]) == abs(blk[k]) and i < k)
    back = orc.nm_unpack(vals, idx, m)
    assert np.all((back == 0) | (back == h))


@pytest.mark.parametrize("n,m,want", [(8, 16, 0.45090), (16, 32, 0.46501)])
def test_post_prune_density(n, m, want):
    assert abs(orc.nm_post_density(n, m) - want) < 5e-6
    # Monte-Carlo on the zero-bias workload's statistics: each entry active w.p. 1/2.
    rng = np.random.default_rng(7)
    h = np.maximum(rng.standard_normal((512, 64 * m)), 0)
    vals, idx = orc.nm_prune(h, n, m)
    dens = (vals != 0).sum() / h.size
    sd = math.sqrt(want * (1 - want) / h.size) * 3
    assert abs(dens - want) < 5 * sd
