// Sparse down projection: y[t] = sum over the active units j of token t of h[t, j] * w2[j].
//
// "Sparser, Faster, Lighter Transformer Language Models", section "2. Metodologia", block
// "Kernels de Inferência": the down projection iterates over the active units only, so the
// rows of W2 of inactive units are never read. Accumulation is fp32.
//
// Work item = (token t, column chunk c). A chunk is 16 lanes x 16 bytes of a W2 row (128
// bf16 or 64 fp32 columns); the wave's four 16-lane groups take every fourth entry of the
// token's active list, so one vector load instruction fetches four different W2 rows.
// The list (column, value) is staged in LDS: from the TwELL slots of normal rows, or from
// the nonzeros of the dense backup row of an overflow row.
//
// XCD-aware order: workgroup b runs on XCD b % 8 (round-robin dispatch), and all chunks
// handled by one XCD are congruent mod 8, so that XCD's L2 only ever holds its own column
// slices of W2; a chunk is finished for all tokens before the XCD moves to its next one.
#include "common.h"
#include "launch.h"

namespace tw {

template <typename VT> TW_DEV float ldv(const VT *p, size_t i) { return Elem<VT>::load(p, i); }

template <typename WT, typename VT, typename YT>
__global__ __launch_bounds__(64) void k_twell_down(TwellIn h, const WT *__restrict__ w2, int d,
                                                   YT *__restrict__ y, int nchunk) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int LCAP = 64 * h.S;
  int *lcol = (int *)lds;
  float *lval = (float *)(lds + (size_t)LCAP * 4);
  const int b = blockIdx.x, xcd = b & 7, i = b >> 3;
  const int T = h.rows;
  const int c = xcd + 8 * (i / T), t = i % T;
  if (c >= nchunk) return;
  constexpr int E = Vec16<WT>::N;
  constexpr int CW = 16 * E;
  const int lane = lane_id(), g = lane >> 4, gl = lane & 15;
  const int col = c * CW + gl * E;
  const bool cv = col < d;
  const VT *vals = (const VT *)h.vals;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;

  auto flush = [&](int n) {
    int e = g;
    for (; e + 12 < n; e += 16) {
      const int j0 = lcol[e], j1 = lcol[e + 4], j2 = lcol[e + 8], j3 = lcol[e + 12];
      const float v0 = lval[e], v1 = lval[e + 4], v2 = lval[e + 8], v3 = lval[e + 12];
      float r0[E], r1[E], r2[E], r3[E];
      if (cv) {
        Vec16<WT>::load(w2 + (size_t)j0 * d + col, r0);
        Vec16<WT>::load(w2 + (size_t)j1 * d + col, r1);
        Vec16<WT>::load(w2 + (size_t)j2 * d + col, r2);
        Vec16<WT>::load(w2 + (size_t)j3 * d + col, r3);
#pragma unroll
        for (int q = 0; q < E; ++q) {
          acc[q] = fmaf(v0, r0[q], acc[q]);
          acc[q] = fmaf(v1, r1[q], acc[q]);
          acc[q] = fmaf(v2, r2[q], acc[q]);
          acc[q] = fmaf(v3, r3[q], acc[q]);
        }
      }
    }
    for (; e < n; e += 4) {
      const int j = lcol[e];
      const float v = lval[e];
      float r[E];
      if (cv) {
        Vec16<WT>::load(w2 + (size_t)j * d + col, r);
#pragma unroll
        for (int q = 0; q < E; ++q) acc[q] = fmaf(v, r[q], acc[q]);
      }
    }
  };

  const int slot = h.ovf_slot[t];
  if (slot < 0) {
    for (int k0 = 0; k0 < h.n_t; k0 += 64) {
      const int k = k0 + lane;
      int m = 0;
      if (k < h.n_t) m = min(h.counts[(size_t)t * h.n_t + k], h.S);
      int tot;
      const int off = wave_excl_scan(m, &tot);
      const size_t sbase = ((size_t)t * h.n_t + k) * h.S;
      for (int s = 0; s < m; ++s) {
        lcol[off + s] = h.col_idx[sbase + s];
        lval[off + s] = ldv(vals, sbase + s);
      }
      __syncthreads();
      flush(tot);
      __syncthreads();
    }
  } else {
    const VT *row = (const VT *)h.ovf_dense + (size_t)slot * h.cols;
    int n = 0;
    for (int c0 = 0; c0 < h.cols; c0 += 64) {
      const int j = c0 + lane;
      const float v = j < h.cols ? ldv(row, j) : 0.f;
      const bool nz = v != 0.f;
      const uint64_t m = ballot64(nz);
      if (nz) {
        const int pos = n + (int)mbcnt64(m);
        lcol[pos] = j;
        lval[pos] = v;
      }
      n += __popcll(m);
      if (n > LCAP - 64 || c0 + 64 >= h.cols) {
        __syncthreads();
        flush(n);
        __syncthreads();
        n = 0;
      }
    }
  }
#pragma unroll
  for (int q = 0; q < E; ++q) {
    acc[q] += __shfl_xor(acc[q], 16, 64);
    acc[q] += __shfl_xor(acc[q], 32, 64);
  }
  if (g == 0 && cv) {
    const size_t o = (size_t)t * d + col;
#pragma unroll
    for (int q = 0; q < E; ++q) Elem<YT>::store(y, o + q, acc[q]);
  }
}

template <typename WT, typename VT, typename YT>
static hipError_t down_t(const TwellIn &h, const WT *w2, int d, YT *y, hipStream_t s) {
  constexpr int CW = 16 * Vec16<WT>::N;
  const int nchunk = (d + CW - 1) / CW;
  const long long per_xcd = (long long)h.rows * ((nchunk + 7) / 8);
  if (h.rows == 0) return hipSuccess;
  const size_t grid = 8 * (size_t)per_xcd;
  const size_t lds = (size_t)64 * h.S * 8;
  hipLaunchKernelGGL((k_twell_down<WT, VT, YT>), dim3((unsigned)grid), dim3(64), lds, s, h, w2, d, y, nchunk);
  return hipGetLastError();
}

hipError_t launch_twell_down(const TwellIn &h, const void *w2, int w_bf16, int d, void *y, int y_bf16,
                             hipStream_t s) {
  if (w_bf16) {
    const uint16_t *w = (const uint16_t *)w2;
    if (h.val_bf16) {
      if (y_bf16) return down_t<uint16_t, uint16_t, uint16_t>(h, w, d, (uint16_t *)y, s);
      return down_t<uint16_t, uint16_t, float>(h, w, d, (float *)y, s);
    }
    if (y_bf16) return down_t<uint16_t, float, uint16_t>(h, w, d, (uint16_t *)y, s);
    return down_t<uint16_t, float, float>(h, w, d, (float *)y, s);
  }
  const float *w = (const float *)w2;
  if (h.val_bf16) {
    if (y_bf16) return down_t<float, uint16_t, uint16_t>(h, w, d, (uint16_t *)y, s);
    return down_t<float, uint16_t, float>(h, w, d, (float *)y, s);
  }
  if (y_bf16) return down_t<float, float, uint16_t>(h, w, d, (uint16_t *)y, s);
  return down_t<float, float, float>(h, w, d, (float *)y, s);
}

}  // namespace tw
