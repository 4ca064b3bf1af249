// The compact row-ELL part of the hybrid training format.
//
// "Sparser, Faster, Lighter Transformer Language Models", section "2. Metodologia", block
// "Formato Híbrido para Treinamento": for training, rows with few nonzeros are kept in a
// compact ELL whose width follows the data, and the rows with more go to a dense backup. Here
// that compact ELL is a TwELL with a single tile per row (tile_w = cols): slots = the width
// N, counts [R][1] = the row's nonzeros, and the same ordered backup bookkeeping. It is built
// from the forward's TwELL (the up GEMM's epilogue writes per-tile slots; this keeps only the
// row's entries, so the stash for the backward shrinks from R * (C / W) * S slots to R * N),
// and every consumer of a TwELL (the down projection, the backward) takes it as it is.
//
//   k_rell_rows   one wave per row: the row's entries in ascending column order (from its
//                 slots, or from its dense backup row), their number into counts, the first
//                 min(count, N) into the row-ELL slots, pads after them
//   k_rell_words  the per-32-row overflow words (count > N) for the ordered overflow scan
//   k_ovf_scan    (pack.hip) ovf_rows, ovf_slot, ovf_n of the row-ELL
//   k_rell_backup one workgroup per backup row: the row assembled in LDS from the source's
//                 slots or backup row, written out densely
#include "common.h"
#include "launch.h"
#include "rows.h"

namespace tw {

// Calls emit(e, col, value) for the entries e = 0 .. n-1 of source row t in ascending column
// order, the lanes of the wave taking e = lane, lane + 64, ...; returns n (wave-uniform). A
// row with a backup slot is read from its dense row (its nonzeros), any other from its slots.
template <typename VT, typename F>
TW_DEV int row_entries(const TwellIn &h, int t, F &&emit) {
  const int lane = lane_id();
  const int slot = h.ovf_slot[t];
  int n = 0;
  if (slot >= 0) {
    const VT *row = (const VT *)h.ovf_dense + (size_t)slot * h.cols;
    for (int j0 = 0; j0 < h.cols; j0 += 64) {
      const int j = j0 + lane;
      const float v = j < h.cols ? Elem<VT>::load(row, j) : 0.f;
      const uint64_t m = ballot64(v != 0.f);
      if (v != 0.f) emit(n + (int)mbcnt64(m), j, v);
      n += __popcll(m);
    }
    return n;
  }
  const VT *vals = (const VT *)h.vals;
  const int32_t *cnt = h.counts + (size_t)t * h.n_t;
  for (int k0 = 0; k0 < h.n_t; k0 += 64) {
    const int k = k0 + lane;
    const int m = k < h.n_t ? min(cnt[k], h.S) : 0;
    int tot;
    const int off = wave_excl_scan(m, &tot);
    const size_t rb = ((size_t)t * h.n_t + k0) * h.S;
    for (int e0 = 0; e0 < tot; e0 += 64) {                     // uniform: every lane shuffles
      const int e = e0 + lane;
      int lo = 0;                                              // last tile with off <= e
#pragma unroll
      for (int step = 32; step > 0; step >>= 1) {
        const int o = __shfl(off, lo + step < 64 ? lo + step : 63, 64);
        lo = (lo + step < 64 && o <= e) ? lo + step : lo;
      }
      const int b = __shfl(off, lo, 64);
      if (e < tot) {
        const size_t si = rb + (size_t)lo * h.S + (e - b);
        emit(n + e, h.col_idx[si], Elem<VT>::load(vals, si));
      }
    }
    n += tot;
  }
  return n;
}

template <typename SVT, typename DVT>
__global__ __launch_bounds__(256) void k_rell_rows(TwellIn src, TwellOut dst) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= src.rows) return;
  const int N = dst.S;
  const size_t base = (size_t)t * N;
  DVT *dv = (DVT *)dst.vals;
  const int n = row_entries<SVT>(src, t, [&](int e, int col, float v) {
    if (e < N) {
      dst.col_idx[base + e] = col;
      Elem<DVT>::store(dv, base + e, v);
    }
  });
  for (int e = n + lane_id(); e < N; e += 64) {
    dst.col_idx[base + e] = -1;
    Elem<DVT>::store(dv, base + e, 0.f);
  }
  if (lane_id() == 0) dst.counts[t] = n;
}

// word w: bit i set iff row 32 w + i has more than N entries
__global__ __launch_bounds__(256) void k_rell_words(const int32_t *__restrict__ counts, int R, int N,
                                                    uint32_t *__restrict__ bits, int words) {
  const int w = blockIdx.x * 256 + threadIdx.x;
  if (w >= words) return;
  uint32_t word = 0;
  for (int i = 0; i < 32; ++i) {
    const int r = w * 32 + i;
    if (r < R && counts[r] > N) word |= 1u << i;
  }
  bits[w] = word;
}

// Backup row r < min(*ovf_n, cap) of the row-ELL = source row ovf_rows[r], densely.
template <typename SVT, typename DVT>
__global__ __launch_bounds__(256) void k_rell_backup(TwellIn src, const int32_t *__restrict__ ovf_n,
                                                     const int32_t *__restrict__ ovf_rows, int cap,
                                                     DVT *__restrict__ dense) {
  extern __shared__ float row_s[];
  const int r = blockIdx.x;
  const int n = min(*ovf_n, cap);
  if (r >= n) return;
  const int t = ovf_rows[r];
  const int C = src.cols;
  for (int j = threadIdx.x; j < C; j += 256) row_s[j] = 0.f;
  __syncthreads();
  if (threadIdx.x < 64) row_entries<SVT>(src, t, [&](int, int col, float v) { row_s[col] = v; });
  __syncthreads();
  for (int j = threadIdx.x; j < C; j += 256) Elem<DVT>::store(dense, (size_t)r * C + j, row_s[j]);
}

// A source row beyond the source's backup capacity lost entries and cannot be restored: then
// the row-ELL's *ovf_n is raised above its capacity, so that twell_sync_status reports it and
// the backward poisons its outputs.
__global__ void k_rell_src_capacity(const int32_t *__restrict__ src_ovf_n, int src_cap, int32_t *__restrict__ ovf_n,
                                    int cap) {
  if (*src_ovf_n > src_cap && *ovf_n <= cap) *ovf_n = cap + 1;
}

template <typename SVT, typename DVT>
static hipError_t rell_t(const TwellIn &src, const TwellOut &dst, int N, int cap, int32_t *ovf_n, int32_t *ovf_rows,
                         int32_t *ovf_slot, void *dense, hipStream_t s) {
  const int R = src.rows;
  hipLaunchKernelGGL((k_rell_rows<SVT, DVT>), dim3((R + 3) / 4), dim3(256), 0, s, src, dst);
  hipLaunchKernelGGL(k_rell_words, dim3((dst.words + 255) / 256), dim3(256), 0, s, dst.counts, R, N, dst.ovf_bits,
                     dst.words);
  TW_TRY_HIP(launch_ovf_scan(dst.ovf_bits, 1, dst.words, R, cap, ovf_n, ovf_rows, ovf_slot, s));
  if (cap > 0)
    hipLaunchKernelGGL((k_rell_backup<SVT, DVT>), dim3(cap), dim3(256), (size_t)src.cols * 4, s, src, ovf_n, ovf_rows, cap,
                       (DVT *)dense);
  hipLaunchKernelGGL(k_rell_src_capacity, dim3(1), dim3(1), 0, s, src.ovf_n, src.cap, ovf_n, cap);
  return hipGetLastError();
}

hipError_t launch_to_row_ell(const TwellIn &src, const TwellOut &dst, int N, int cap, int32_t *ovf_n,
                             int32_t *ovf_rows, int32_t *ovf_slot, void *dense, hipStream_t s) {
  if (src.rows == 0) return launch_set_int(ovf_n, 0, s);
  if (src.val_bf16) {
    if (dst.val_bf16) return rell_t<uint16_t, uint16_t>(src, dst, N, cap, ovf_n, ovf_rows, ovf_slot, dense, s);
    return rell_t<uint16_t, float>(src, dst, N, cap, ovf_n, ovf_rows, ovf_slot, dense, s);
  }
  return rell_t<float, float>(src, dst, N, cap, ovf_n, ovf_rows, ovf_slot, dense, s);
}

// hist[min(nnz_t, nbins - 1)] += 1 over the rows t, nnz_t = sum of the row's true tile counts
// (its nonzeros, also for rows in the backup). Integer atomics: exact and order-free.
__global__ __launch_bounds__(256) void k_row_nnz_hist(const int32_t *__restrict__ counts, int rows, int n_t,
                                                      int nbins, int32_t *__restrict__ hist) {
  const int lane = lane_id();
  for (int row = blockIdx.x * 4 + (threadIdx.x >> 6); row < rows; row += gridDim.x * 4) {
    int s = 0;
    for (int k = lane; k < n_t; k += 64) s += counts[(size_t)row * n_t + k];
    s = wave_sum(s);
    if (lane == 0) atomicAdd(&hist[min(s, nbins - 1)], 1);
  }
}

hipError_t launch_row_nnz_hist(const int32_t *counts, int rows, int n_t, int nbins, int32_t *hist, hipStream_t s) {
  TW_TRY_HIP(launch_zero_i32(hist, nbins, s));
  if (rows > 0)
    hipLaunchKernelGGL(k_row_nnz_hist, dim3(min((rows + 3) / 4, 1024)), dim3(256), 0, s, counts, rows, n_t, nbins, hist);
  return hipGetLastError();
}

}  // namespace tw
