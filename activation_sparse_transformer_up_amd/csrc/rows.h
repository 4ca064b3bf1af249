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
// rows from the dense backup instead). One wave. Lane k holds the count of tile k0 + k;
// then each 16-lane group copies the slots of one tile per round (lane = slot), and all
// sixteen rounds' loads are issued before any store, so a row costs two memory latencies
// (counts, then slots) rather than one per slot.
template <typename VT>
TW_DEV void row_list_wave(const TwellIn &h, int t) {
  const int lane = lane_id(), g = lane >> 4, gl = lane & 15;
  const int S = h.S;
  const size_t stride = (size_t)h.n_t * S;
  uint2 *out = h.row_list + (size_t)t * stride;
  const VT *vals = (const VT *)h.vals;
  int n = 0;
  for (int k0 = 0; k0 < h.n_t; k0 += 64) {
    const int k = k0 + lane;
    const int m = k < h.n_t ? min(h.counts[(size_t)t * h.n_t + k], S) : 0;
    int tot;
    const int off = wave_excl_scan(m, &tot);
    for (int s0 = 0; s0 < S; s0 += 16) {
      const int s = s0 + gl;
      // row base of tile k0 (wave-uniform) + 32-bit lane offsets: one VGPR per load address
      const size_t rb = ((size_t)t * h.n_t + k0) * S;
      const char *ci_row = (const char *)(h.col_idx + rb);
      const char *cv_row = (const char *)(vals + rb);
      uint32_t ci[16], cv[16];
      int dst[16];
      // Loads are unconditional (lanes without a slot re-read slot 0 of tile k0): a load
      // under a divergent branch makes the compiler wait for every earlier load first.
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = 4 * r + g;                     // tile k0 + kk (count 0 past n_t)
        const int mk = __shfl(m, kk, 64), ok = __shfl(off, kk, 64);
        const bool on = s < mk;
        const uint32_t e = on ? (uint32_t)(kk * S + s) : 0u;
        ci[r] = *(const uint32_t *)(ci_row + 4u * e);
        cv[r] = __float_as_uint(Elem<VT>::load((const VT *)(cv_row + (uint32_t)sizeof(VT) * e), 0));
        dst[r] = on ? n + ok + s : -1;
      }
      // keep every load above the (branchy) stores: the compiler would otherwise sink a
      // round's loads into its store branch, behind a wait
#pragma unroll
      for (int r = 0; r < 16; ++r) asm volatile("" ::"v"(ci[r]), "v"(cv[r]));
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (dst[r] >= 0) out[dst[r]] = make_uint2(ci[r], cv[r]);
    }
    n += tot;
  }
  if (lane == 0) h.row_nnz[t] = n;
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
