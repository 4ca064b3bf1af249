// Per-row bookkeeping of a TwELL matrix, shared by the producers (pack, up-GEMM finish)
// and the down projection:
//  - the compact per-row lists of the stored slots, which the row gathers walk;
//  - the overflow scan of "Sparser, Faster, Lighter Transformer Language Models", section
//    "2. Metodologia", block "Formato Híbrido para Treinamento": rows with a row-tile count
//    above the slot budget go to a dense backup, listed in ascending row order.
#pragma once
#include "common.h"
#include "launch.h"

namespace tw {

// row_list[t][0 .. row_nnz[t]) = (column, fp32 value bits) of the stored slots of row t in
// ascending column order (an overflow row gets its truncated slots; consumers take such
// rows from the dense backup instead). One wave, 64 tiles at a time: lane k holds the
// count of tile k0 + k and its exclusive prefix off[k]; then lane e takes list entry e of
// the chunk (e, e + 64, ...), finds its tile as the last k with off[k] <= e by a binary
// search over the wave (ds_bpermute), and copies slot e - off[k]. A row costs a few wave
// loads and one coalesced 8-byte store per 64 entries, instead of one wave load per tile
// group and slot. The row is a chain of dependent memory round trips, so the next chunk's
// counts are loaded before this chunk's stores, and the slot loads of up to kListRounds
// rounds of 64 entries are all issued before their stores. Rows of 65 to 128 tiles take both
// chunks in one pass (row_list_wave2).
constexpr int kListRounds = 4;

// Rows per workgroup of the list kernels: a row is one wave's chain of dependent round trips,
// so the rows are spread over about one workgroup per CU (at most 16 rows, one per wave; the
// other waves exit at once). At c3 T = 64 one row per workgroup instead of 16 took the finish
// from five workgroups to 65 and the forward from 61.9-62.1 to 58.6-59.0 us (same box).
inline int list_rows_per_wg(int rows) { return rows < 256 ? 1 : (rows > 16 * 256 ? 16 : (rows + 255) / 256); }

// Stores of one list entry and of the list length (COH: agent-scope atomic stores).
template <bool COH> TW_DEV void list_store(uint2 *out, int e, uint32_t c, uint32_t v) {
  if constexpr (COH)
    __hip_atomic_store((uint64_t *)(out + e), (uint64_t)c | ((uint64_t)v << 32), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  else
    out[e] = make_uint2(c, v);
}

// The same list for rows of 65 to 128 tiles in one pass: both chunks' counts are loaded and
// scanned together (lane k holds tiles k and 64 + k), and entries of both chunks share the
// rounds of slot loads, so the second chunk's slots do not wait for the first chunk's.
// Entry e < tot0 lies in chunk 0, the others in chunk 1; each lane searches its chunk's
// prefix (both are shuffled at every step, the lane keeps its own).
template <typename VT, bool COH>
TW_DEV void row_list_wave2(const TwellIn &h, int t) {
  const int lane = lane_id();
  const int S = h.S, n_t = h.n_t;
  uint2 *out = h.row_list + (size_t)t * n_t * S;
  const VT *vals = (const VT *)h.vals;
  const int32_t *cnt = h.counts + (size_t)t * n_t;
  const int c0 = cnt[lane], c1 = cnt[64 + lane < n_t ? 64 + lane : n_t - 1];
  const int m0 = min(c0, S), m1 = 64 + lane < n_t ? min(c1, S) : 0;
  int tot0, tot1;
  const int off0 = wave_excl_scan(m0, &tot0);
  const int off1 = wave_excl_scan(m1, &tot1);
  const int tot = tot0 + tot1;
  const size_t rb = (size_t)t * n_t * S;                       // slot 0 of tile 0
  for (int e0 = 0; e0 < tot; e0 += kListRounds * 64) {
    uint32_t ci[kListRounds], cv[kListRounds];
#pragma unroll
    for (int r = 0; r < kListRounds; ++r) {
      const int e = e0 + r * 64 + lane;
      const bool in1 = e >= tot0;
      const int ee = in1 ? e - tot0 : e;
      int lo = 0;                                               // last tile of the chunk with off <= ee
#pragma unroll
      for (int step = 32; step > 0; step >>= 1) {
        const int o0 = __shfl(off0, lo + step, 64), o1 = __shfl(off1, lo + step, 64);
        const int o = in1 ? o1 : o0;
        lo = (lo + step < 64 && o <= ee) ? lo + step : lo;
      }
      const int b0 = __shfl(off0, lo, 64), b1 = __shfl(off1, lo, 64);
      const int tile = (in1 ? 64 : 0) + lo;
      const size_t si = rb + (e < tot ? (size_t)tile * S + (ee - (in1 ? b1 : b0)) : 0);
      ci[r] = (uint32_t)h.col_idx[si];
      cv[r] = __float_as_uint(Elem<VT>::load(vals, si));
    }
#pragma unroll
    for (int r = 0; r < kListRounds; ++r) {
      const int e = e0 + r * 64 + lane;
      if (e < tot) list_store<COH>(out, e, ci[r], cv[r]);
    }
  }
  if (lane == 0) {
    if constexpr (COH) __hip_atomic_store(h.row_nnz + t, tot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else h.row_nnz[t] = tot;
  }
}

// COH: the lists and lengths are written with agent-scope atomic stores, which reach the
// memory side directly, so that other XCDs can read them later in the same kernel.
template <typename VT, bool COH = false>
TW_DEV void row_list_wave(const TwellIn &h, int t) {
  if (h.n_t > 64 && h.n_t <= 128) {                            // wave-uniform
    row_list_wave2<VT, COH>(h, t);
    return;
  }
  const int lane = lane_id();
  const int S = h.S;
  const size_t stride = (size_t)h.n_t * S;
  uint2 *out = h.row_list + (size_t)t * stride;
  const VT *vals = (const VT *)h.vals;
  const int32_t *cnt = h.counts + (size_t)t * h.n_t;
  int n = 0;
  int cnext = h.n_t > 0 ? cnt[lane < h.n_t ? lane : h.n_t - 1] : 0;
  for (int k0 = 0; k0 < h.n_t; k0 += 64) {
    const int k = k0 + lane;
    const int m = k < h.n_t ? min(cnext, S) : 0;
    if (k0 + 64 < h.n_t) cnext = cnt[k + 64 < h.n_t ? k + 64 : h.n_t - 1];
    int tot;
    const int off = wave_excl_scan(m, &tot);
    const size_t rb = ((size_t)t * h.n_t + k0) * S;   // slot 0 of tile k0
    for (int e0 = 0; e0 < tot; e0 += kListRounds * 64) {
      uint32_t ci[kListRounds], cv[kListRounds];
#pragma unroll
      for (int r = 0; r < kListRounds; ++r) {
        const int e = e0 + r * 64 + lane;
        int lo = 0;                                   // last tile with off <= e (off[0] = 0)
#pragma unroll
        for (int step = 32; step > 0; step >>= 1) {
          const int o = __shfl(off, lo + step, 64);
          lo = (lo + step < 64 && o <= e) ? lo + step : lo;
        }
        const int base = __shfl(off, lo, 64);
        const size_t si = rb + (e < tot ? (size_t)lo * S + (e - base) : 0);
        ci[r] = (uint32_t)h.col_idx[si];
        cv[r] = __float_as_uint(Elem<VT>::load(vals, si));
      }
#pragma unroll
      for (int r = 0; r < kListRounds; ++r) {
        const int e = e0 + r * 64 + lane;
        if (e < tot) {
          if constexpr (COH)
            __hip_atomic_store((uint64_t *)(out + n + e), (uint64_t)ci[r] | ((uint64_t)cv[r] << 32), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
          else
            out[n + e] = make_uint2(ci[r], cv[r]);
        }
      }
    }
    n += tot;
  }
  if (lane == 0) {
    if constexpr (COH) __hip_atomic_store(h.row_nnz + t, n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else h.row_nnz[t] = n;
  }
}

// The overflow scan, by one workgroup of 1024 threads: the per-(tile, 32-row) overflow
// words are OR-reduced over the n_t tiles (a group of G lanes per word), their popcounts
// scanned (exclusive, carried across chunks of words), and every row's backup slot written:
// ovf_slot[row] = its rank among overflow rows if below cap, else -1; ovf_rows[rank] = row;
// *ovf_n = the number of overflow rows (may exceed cap).
TW_DEV void ovf_scan_block(const uint32_t *__restrict__ bits, int n_t, int words, int R, int cap,
                           int32_t *ovf_n, int32_t *ovf_rows, int32_t *ovf_slot) {
  __shared__ uint32_t fw[1024];
  __shared__ int pre[1024];
  __shared__ int wsum[16];
  __shared__ int carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int G = 1;
  while (G < 64 && G * 2 * min(words, 1024) <= 1024) G *= 2;
  const int wpc = 1024 / G;                       // words per chunk
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < words; base += wpc) {
    const int wi = tid / G, sub = tid % G;
    const int w = base + wi;
    // 16 loads in flight per lane, from clamped (always valid) addresses; see row_list_wave
    uint32_t f = 0;
    const int wc = min(w, words - 1);
    for (int k0 = sub; k0 < n_t; k0 += 16 * G) {
      uint32_t v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = bits[(size_t)min(k0 + i * G, n_t - 1) * words + wc];
#pragma unroll
      for (int i = 0; i < 16; ++i) f |= k0 + i * G < n_t ? v[i] : 0u;
    }
    if (w >= words) f = 0;
    for (int off = 1; off < G; off <<= 1) f |= (uint32_t)__shfl_xor((int)f, off, 64);
    // one value per word: lanes with sub == 0 hold it
    const int c = (sub == 0 && w < words) ? __popc(f) : 0;
    int tot;
    const int ex = wave_excl_scan(c, &tot);
    if (lane == 0) wsum[wave] = tot;
    __syncthreads();
    int wpre = 0, chunk_tot = 0;
    for (int i = 0; i < 16; ++i) {
      if (i < wave) wpre += wsum[i];
      chunk_tot += wsum[i];
    }
    const int carry = carry_s;
    if (sub == 0) {
      fw[wi] = f;
      pre[wi] = carry + wpre + ex;
    }
    __syncthreads();
    const int nrows = min(wpc * 32, R - base * 32);
    for (int i = tid; i < nrows; i += 1024) {
      const int row = base * 32 + i;
      const uint32_t ff = fw[i >> 5];
      const int bit = i & 31;
      int slot = -1;
      if ((ff >> bit) & 1u) {
        const int p = pre[i >> 5] + __popc(ff & ((1u << bit) - 1u));
        if (p < cap) {
          slot = p;
          ovf_rows[p] = row;
        }
      }
      ovf_slot[row] = slot;
    }
    __syncthreads();
    if (tid == 0) carry_s = carry + chunk_tot;
    __syncthreads();
  }
  if (tid == 0) *ovf_n = carry_s;
}

}  // namespace tw
