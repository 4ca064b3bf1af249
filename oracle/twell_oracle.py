"""CPU oracle for the activation-sparse (TwELL) transformer feed-forward layer.

TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the benchmark's CPU
baseline leg may import this module; the library's product path never does.

Plain, slow, obviously correct numpy code in float64. Each function restates what the
method computes, as described on the pages (cited by page title and section):

  [SFL]  "Sparser, Faster, Lighter Transformer Language Models" (gist.science summary),
         sections "1. O Problema", "2. Metodologia" (blocks "Formato de Dados TwELL",
         "Kernels de Inferência", "Formato Híbrido para Treinamento",
         "Técnicas de Treinamento").
  [NM]   "Motivating Next-Gen Accelerators with Flexible (N:M) Activation Sparsity ..."
         (gist.science summary), section "2. Metodologia" (patterns and the magnitude
         criterion ACT) and section "5. Significado e Implicações" (layout counts).

Where the pages leave a step open, the reading taken is stated at the function.
Inputs arrive in their stored dtype (float32, or bf16 as uint16 bit patterns) and are
widened exactly to float64 before any arithmetic. Library primitives used as steps:
numpy matmul, sort/lexsort, cumsum.

Parity status: every function below is pinned by tests under tests/ against closed
forms, brute force or special cases (see each docstring); none is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np

U32 = 2.0 ** -24  # unit roundoff of fp32


# ----------------------------------------------------------------------------- inputs

def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of a stored array (bf16 bit patterns or float32)."""
    if dtype == "bf16":
        return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.asarray(a, np.float32).astype(np.float64)


# ----------------------------------------------------------------- forward definition

def preact(x: np.ndarray, w1t: np.ndarray, b1: np.ndarray) -> np.ndarray:
    """z = x . W1 + b1 with W1 = w1t^T (w1t row j holds unit j's input weights).

    [SFL] "1. O Problema": the feed-forward block's up projection is a dense product of the
    token activations with the first weight matrix; the bias is added last.
    """
    return x @ w1t.T + b1[None, :]


def relu(z: np.ndarray) -> np.ndarray:
    """h = max(z, 0); z == 0 is inactive (the derivative at 0 is taken as 0).

    [SFL] "Técnicas de Treinamento": the feed-forward activation is ReLU, which yields the
    exact zeros the sparse format skips.
    """
    return np.where(z > 0.0, z, 0.0)


def ffn_fwd(x: np.ndarray, w1t: np.ndarray, b1: np.ndarray, w2: np.ndarray):
    """y = ReLU(x . W1 + b1) . W2 with w2 row j = unit j's output weights.

    [SFL] "1. O Problema" (the dense FFN) and "Kernels de Inferência" (only active units
    contribute: a zero h entry adds nothing). Returns (z, h, y).
    """
    z = preact(x, w1t, b1)
    h = relu(z)
    y = h @ w2
    return z, h, y


def gather_rows(h: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """y[t] = sum over the nonzero h[t, j], in ascending j, of h[t, j] * w2[j] (fp64).

    [SFL] "Kernels de Inferência": iterate over the active units only. Skipping an exact
    zero leaves an IEEE sum unchanged, so this equals the dense product row by row.
    """
    T = h.shape[0]
    y = np.zeros((T, w2.shape[1]))
    for t in range(T):
        for j in np.flatnonzero(h[t]):
            y[t] += h[t, j] * w2[j]
    return y


# ------------------------------------------------------------------- gated feed-forward

def gated_ffn_fwd(x: np.ndarray, wgt: np.ndarray, bg: np.ndarray, wut: np.ndarray, w2: np.ndarray):
    """y = (ReLU(x . Wg + bg) * (x . Wu)) . W2, elementwise product of gate and up.

    [SFL] "Formato de Dados TwELL": the sparse format is produced by the dense product that
    computes the gate activations; "Kernels de Inferência": one kernel fuses the up and the
    down projections, iterating over the active units only (a dot product for the up
    projection, then the multiply-add with the unit's down row).
    Readings taken where the pages are silent: the gate is ReLU of its pre-activation with
    a bias (the bias is what makes the synthetic layers sparse); the up projection has no
    bias and no activation; a unit contributes gate * up; wgt / wut row j hold unit j's
    input weights (like w1t) and w2 row j its output weights. Returns (zg, g, u, h, y).
    """
    zg = preact(x, wgt, bg)
    g = relu(zg)
    u = x @ wut.T
    h = g * u
    return zg, g, u, h, h @ w2


def gated_gather(g: np.ndarray, x: np.ndarray, wut: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """The same y in the fused kernel's order: per token, for each active gate unit j in
    ascending order, u = x[t] . wut[j] and y[t] += (g[t, j] * u) * w2[j] (fp64).

    [SFL] "Kernels de Inferência". A unit with g = 0 adds nothing, so this equals
    ``gated_ffn_fwd`` up to the order of the fp64 sums.
    """
    T = g.shape[0]
    y = np.zeros((T, w2.shape[1]))
    for t in range(T):
        for j in np.flatnonzero(g[t]):
            u = float(x[t] @ wut[j])
            y[t] += (g[t, j] * u) * w2[j]
    return y


# ------------------------------------------------------------------------ TwELL format

def twell_pack(h: np.ndarray, tile_w: int, slots: int, ovf_cap: int) -> dict:
    """Tile-wise ELLPACK of an R x C matrix, with the row-level dense backup.

    [SFL] "Formato de Dados TwELL": the columns are cut into tiles of ``tile_w``; inside each
    (row, tile) the nonzero values and their column indices are stored aligned.
    [SFL] "Formato Híbrido para Treinamento": rows with too many nonzeros are routed to a
    dense backup matrix.

    Readings taken where the pages are silent:
      * nonzero means "not +0 and not -0";
      * a (row, tile) keeps its first min(count, slots) nonzeros in ascending column order;
        the stored index is the global column; unused slots hold (-1, +0.0);
      * ``counts`` is the true count (it may exceed ``slots``);
      * a row overflows iff some tile of it has count > slots; overflow rows are listed in
        ascending order; the first ``ovf_cap`` of them get a slot in ``ovf_dense`` holding
        the full row; ``ovf_n`` is the true number of overflow rows.
    """
    R, C = h.shape
    assert C % tile_w == 0 and 1 <= slots <= tile_w
    nt = C // tile_w
    nz = (h != 0.0).reshape(R, nt, tile_w)
    counts = nz.sum(axis=2).astype(np.int32)
    rank = np.cumsum(nz, axis=2) - 1                         # position among the tile's nonzeros
    keep = nz & (rank < slots)
    r_i, k_i, c_i = np.nonzero(keep)
    col_idx = np.full((R, nt, slots), -1, np.int32)
    vals = np.zeros((R, nt, slots), h.dtype)
    col_idx[r_i, k_i, rank[r_i, k_i, c_i]] = (k_i * tile_w + c_i).astype(np.int32)
    vals[r_i, k_i, rank[r_i, k_i, c_i]] = h.reshape(R, nt, tile_w)[r_i, k_i, c_i]
    row_ovf = (counts > slots).any(axis=1)
    ovf_all = np.flatnonzero(row_ovf).astype(np.int32)
    ovf_rows = ovf_all[:ovf_cap]
    ovf_slot = np.full(R, -1, np.int32)
    ovf_slot[ovf_rows] = np.arange(len(ovf_rows), dtype=np.int32)
    ovf_dense = np.zeros((ovf_cap, C), h.dtype)
    ovf_dense[: len(ovf_rows)] = h[ovf_rows]
    return {"counts": counts, "col_idx": col_idx, "vals": vals, "ovf_n": int(len(ovf_all)),
            "ovf_rows": ovf_rows, "ovf_slot": ovf_slot, "ovf_dense": ovf_dense,
            "tile_w": tile_w, "slots": slots, "ovf_cap": ovf_cap, "shape": (R, C)}


def twell_unpack(tw: dict) -> np.ndarray:
    """Inverse of ``twell_pack``: rows with a dense backup are copied from it, the others are
    rebuilt from their slots. Fails if an overflow row had no backup slot."""
    R, C = tw["shape"]
    nt, S = tw["col_idx"].shape[1], tw["slots"]
    if tw["ovf_n"] > tw["ovf_cap"]:
        raise ValueError("overflow rows beyond capacity cannot be rebuilt")
    h = np.zeros((R, C), tw["vals"].dtype)
    for r in range(R):
        s = tw["ovf_slot"][r]
        if s >= 0:
            h[r] = tw["ovf_dense"][s]
            continue
        for k in range(nt):
            n = min(int(tw["counts"][r, k]), S)
            h[r, tw["col_idx"][r, k, :n]] = tw["vals"][r, k, :n]
    return h


def row_max_histogram(counts: np.ndarray, tile_w: int) -> np.ndarray:
    """hist[m] = number of rows whose largest per-tile count is m, m = 0 .. tile_w.

    [SFL] "Formato Híbrido para Treinamento": the compact part holds rows up to some width
    and the rest go to the dense backup; with the per-(row, tile) layout a row fits S slots
    iff its largest tile count is at most S, so the overflow rows for S are the rows counted
    in hist[S + 1 ..]. Pinned against the packer's own overflow count for every S.
    """
    R = counts.shape[0]
    hist = np.zeros(tile_w + 1, np.int64)
    if R == 0:
        return hist
    for m in counts.max(axis=1):
        hist[int(m)] += 1
    return hist


def stash_bytes(rows: int, cols: int, tile_w: int, slots: int, n_ovf: int, val_bytes: int) -> int:
    """Bytes of the TwELL kept for the backward: counts and ovf_slot (int32 per row-tile /
    row), one int32 index and one value per slot, and per overflow row its int32 row id and
    a dense row of values (the layout of ``twell_pack``; pinned against its array sizes)."""
    cells = rows * (cols // tile_w)
    return cells * 4 + cells * slots * (4 + val_bytes) + rows * 4 + n_ovf * (4 + cols * val_bytes)


def choose_slots(hist: np.ndarray, tile_w: int, rows: int, cols: int, ovf_cap: int, val_bytes: int):
    """The dynamic width of the hybrid format ([SFL] "Formato Híbrido para Treinamento"),
    read as: among S = 1 .. min(tile_w, 64) whose overflow rows fit the backup capacity,
    take the one with the smallest stash (the smaller S on equal bytes). Returns (S, bytes)
    or (None, None) if no S fits."""
    best = (None, None)
    for S in range(1, min(tile_w, 64) + 1):
        n_ovf = int(hist[S + 1:].sum())
        if n_ovf > ovf_cap:
            continue
        b = stash_bytes(rows, cols, tile_w, S, n_ovf, val_bytes)
        if best[1] is None or b < best[1]:
            best = (S, b)
    return best


def row_nnz_histogram(counts: np.ndarray, nbins: int) -> np.ndarray:
    """hist[min(n_t, nbins - 1)] = number of rows t with n_t nonzeros (the sum of the row's
    true tile counts).

    [SFL] "Formato Híbrido para Treinamento": the compact ELL keeps a row's entries up to a
    width chosen from the data, and wider rows go to the dense backup; with a single tile per
    row a row fits N slots iff it has at most N nonzeros, so the rows above N are counted in
    hist[N + 1 ..]. Pinned against the packer's own overflow count with tile_w = cols.
    """
    hist = np.zeros(nbins, np.int64)
    for n in counts.sum(axis=1):
        hist[min(int(n), nbins - 1)] += 1
    return hist


def choose_row_ell_width(hist: np.ndarray, rows: int, cols: int, ovf_cap: int, val_bytes: int):
    """The width N of the compact row-ELL ([SFL] "Formato Híbrido para Treinamento"), read as
    for the slot count: among N = 1 .. min(len(hist) - 2, cols) whose rows with more than N
    nonzeros fit the backup capacity, the one with the smallest stash (one tile per row:
    ``stash_bytes`` with tile_w = cols), the smaller N on equal bytes. Returns (N, bytes) or
    (None, None)."""
    best = (None, None)
    for N in range(1, min(len(hist) - 2, cols) + 1):
        n_ovf = int(hist[N + 1:].sum())
        if n_ovf > ovf_cap:
            continue
        b = stash_bytes(rows, cols, cols, N, n_ovf, val_bytes)
        if best[1] is None or b < best[1]:
            best = (N, b)
    return best


# --------------------------------------------------------------------- N:M activations

def nm_prune(h: np.ndarray, n: int, m: int):
    """N:M activation pruning by magnitude.

    [NM] "2. Metodologia": in every block of ``m`` consecutive activations keep ``n``; the
    ACT criterion ranks activations by absolute value.
    Readings: blocks are contiguous along the hidden dimension; ties in |h| go to the lower
    index; the n kept entries are emitted in ascending index order with their signed
    values; a block with fewer than n nonzeros keeps zeros (so there are always n slots).
    Returns (vals [R, C/m, n] in h's dtype, idx [R, C/m, n] uint8 = index inside the block).
    """
    R, C = h.shape
    assert C % m == 0 and 1 <= n <= m
    g = h.reshape(R, C // m, m)
    mag = np.abs(g.astype(np.float64))
    pos = np.broadcast_to(np.arange(m), g.shape)
    # lexsort: last key is primary -> sort by descending magnitude, then ascending index.
    order = np.lexsort((pos, -mag), axis=2)
    kept = np.sort(order[:, :, :n], axis=2)
    vals = np.take_along_axis(g, kept, axis=2)
    return vals, kept.astype(np.uint8)


def nm_unpack(vals: np.ndarray, idx: np.ndarray, m: int) -> np.ndarray:
    """Dense matrix holding the kept N:M entries (zeros elsewhere)."""
    R, G, n = vals.shape
    out = np.zeros((R, G, m), vals.dtype)
    np.put_along_axis(out, idx.astype(np.int64), vals, axis=2)
    return out.reshape(R, G * m)


# ---------------------------------------------------------------------------- backward

def ffn_bwd(x, w1t, w2, dy, l1_coef, h):
    """Gradients of  L = <dy, y> + l1_coef * sum(h)  for y = ReLU(x W1 + b1) W2.

    [SFL] "Técnicas de Treinamento": an L1 penalty on the feed-forward activations
    (coefficient 2e-5 in the paper) is added to the loss; with ReLU its gradient is the
    coefficient on every active entry. [SFL] "Formato Híbrido para Treinamento": the
    training kernels work on the sparsity pattern P = {(t, j): h[t, j] > 0}.

    h is the forward activation (zero outside P). Returns dict with
      dh  = dy . W2^T                     (dense, for reference)
      dz  = (dh + l1_coef) on P, 0 elsewhere
      dx  = dz . w1t,   dw1t = dz^T . x,   dw2 = h^T . dy,   db1 = sum_t dz.
    """
    P = h > 0.0
    dh = dy @ w2.T
    dz = np.where(P, dh + l1_coef, 0.0)
    return {"dh": dh, "dz": dz, "dx": dz @ w1t, "dw1t": dz.T @ x, "dw2": h.T @ dy,
            "db1": dz.sum(axis=0)}


# ---------------------------------------------------------------------- analytic values

def phi_bar(x):
    """Upper tail of the standard normal."""
    return 0.5 * math.erfc(x / math.sqrt(2.0))


def p_active(b1: np.ndarray, w1t: np.ndarray) -> np.ndarray:
    """P(h_j > 0) for x ~ N(0, I): z_j ~ N(b_j, |w_j|^2), so p_j = P(N(0,1) > -b_j/|w_j|)."""
    nrm = np.sqrt((w1t ** 2).sum(axis=1))
    return np.array([phi_bar(-b / s) for b, s in zip(b1, nrm)])


def poisson_binomial_tail(p: np.ndarray, k: int) -> float:
    """P(sum of independent Bernoulli(p_i) > k), by the exact convolution recursion."""
    dist = np.zeros(len(p) + 1)
    dist[0] = 1.0
    for i, pi in enumerate(p):
        dist[1:i + 2] = dist[1:i + 2] * (1 - pi) + dist[0:i + 1] * pi
        dist[0] *= (1 - pi)
    return float(dist[k + 1:].sum())


def expected_overflow_rows(p: np.ndarray, tile_w: int, slots: int, rows: int) -> float:
    """Expected number of rows with some tile count > slots, units taken independent."""
    tiles = p.reshape(-1, tile_w)
    q = 1.0
    for pt in tiles:
        q *= 1.0 - poisson_binomial_tail(pt, slots)
    return rows * (1.0 - q)


def nm_post_density(n: int, m: int, p: float = 0.5) -> float:
    """Density after N:M pruning when each entry is nonzero with probability p: the block
    keeps min(#nonzeros, n) nonzeros, so density = E[min(Bin(m, p), n)] / m."""
    return sum(min(k, n) * math.comb(m, k) * p ** k * (1 - p) ** (m - k) for k in range(m + 1)) / m


def z_error_bound(x: np.ndarray, w1t: np.ndarray, b1: np.ndarray) -> np.ndarray:
    """Worst-case |fl32(z) - z| for any summation order of fp32 products and sums:
    gamma_{K+2} * (sum_i |x_i w_ji| + |b_j|), gamma_n = n u / (1 - n u), u = 2^-24."""
    K = x.shape[1] + 2
    g = K * U32 / (1 - K * U32)
    return g * (np.abs(x) @ np.abs(w1t).T + np.abs(b1)[None, :])
