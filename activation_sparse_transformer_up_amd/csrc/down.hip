// Sparse down projection: y[t] = sum over the active units j of token t of h[t, j] * w2[j].
//
// "Sparser, Faster, Lighter Transformer Language Models", section "2. Metodologia", block
// "Kernels de Inferência": the down projection iterates over the active units only, so the
// rows of W2 of inactive units are never read. Accumulation is fp32.
//
// First each normal row's TwELL slots are compacted once into a contiguous list of
// (column, value) pairs (k_row_list): the gather below is spread over all XCDs by column
// chunk, and reading the sparse slot blocks from every XCD would fetch whole cache lines
// for a handful of entries. Work item = (token t, column chunk c). A chunk is 16 lanes x
// 16 bytes of a W2 row (128 bf16 or 64 fp32 columns); the wave's four 16-lane groups take
// every fourth entry of the token's list, so one vector load instruction fetches four
// different W2 rows. Overflow rows take their entries from the dense backup row.
//
// XCD-aware order: workgroup b runs on XCD b % 8 (round-robin dispatch), and all chunks
// handled by one XCD are congruent mod 8, so that XCD's L2 only ever holds its own column
// slices of W2; a chunk is finished for all tokens before the XCD moves to its next one.
#include "common.h"
#include "launch.h"

namespace tw {

template <typename VT> TW_DEV float ldv(const VT *p, size_t i) { return Elem<VT>::load(p, i); }

// Compact list of each normal row: row_list[t][0 .. row_nnz[t]) = (column, fp32 value bits)
// in ascending column order, read once from the TwELL slots. Rows with a dense backup get
// row_nnz = -1 (their consumers read the backup row). One wave per row.
template <typename VT>
__global__ __launch_bounds__(256) void k_row_list(TwellIn h) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= h.rows) return;
  const int lane = lane_id();
  if (h.ovf_slot[t] >= 0) {
    if (lane == 0) h.row_nnz[t] = -1;
    return;
  }
  const size_t stride = (size_t)h.n_t * h.S;
  uint2 *out = h.row_list + (size_t)t * stride;
  const VT *vals = (const VT *)h.vals;
  int n = 0;
  for (int k0 = 0; k0 < h.n_t; k0 += 64) {
    const int k = k0 + lane;
    const int m = k < h.n_t ? min(h.counts[(size_t)t * h.n_t + k], h.S) : 0;
    int tot;
    const int off = wave_excl_scan(m, &tot);
    const size_t sb = ((size_t)t * h.n_t + k) * h.S;
    for (int s = 0; s < m; ++s)
      out[n + off + s] = make_uint2((uint32_t)h.col_idx[sb + s], __float_as_uint(ldv(vals, sb + s)));
    n += tot;
  }
  if (lane == 0) h.row_nnz[t] = n;
}

// y[t][chunk] from the compact list: batches of 64 (column, value) pairs are staged in LDS
// (one coalesced 8-byte load per lane); the four 16-lane groups take every fourth entry of
// a batch and issue all their W2 row loads (up to 16) before the FMAs.
template <typename WT, typename VT, typename YT>
__global__ __launch_bounds__(64) void k_twell_down(TwellIn h, const WT *__restrict__ w2, int d,
                                                   YT *__restrict__ y, int nchunk) {
  __shared__ uint2 lst[64];
  const int b = blockIdx.x, xcd = b & 7, i = b >> 3;
  const int T = h.rows;
  const int c = xcd + 8 * (i / T), t = i % T;
  if (c >= nchunk) return;
  constexpr int E = Vec16<WT>::N;
  constexpr int CW = 16 * E;
  const int lane = lane_id(), g = lane >> 4, gl = lane & 15;
  const int col = c * CW + gl * E;
  const bool cv = col < d;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;

  auto consume = [&](int n) {
    uint4 raw[16];
    float vv[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int e = g + 4 * j;
      vv[j] = 0.f;
      raw[j] = make_uint4(0, 0, 0, 0);
      if (e < n) {
        const uint2 p = lst[e];
        vv[j] = __uint_as_float(p.y);
        if (cv) raw[j] = *(const uint4 *)(w2 + (size_t)p.x * d + col);
      }
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      float r[E];
      if constexpr (sizeof(WT) == 2) {
        const uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          r[2 * q] = __uint_as_float(w[q] << 16);
          r[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
        }
      } else {
        r[0] = __uint_as_float(raw[j].x); r[1] = __uint_as_float(raw[j].y);
        r[2] = __uint_as_float(raw[j].z); r[3] = __uint_as_float(raw[j].w);
      }
#pragma unroll
      for (int q = 0; q < E; ++q) acc[q] = fmaf(vv[j], r[q], acc[q]);
    }
  };

  const int nnz = h.row_nnz[t];
  if (nnz >= 0) {
    const uint2 *src = h.row_list + (size_t)t * h.n_t * h.S;
    for (int base = 0; base < nnz; base += 64) {
      const int n = min(64, nnz - base);
      if (lane < n) lst[lane] = src[base + lane];
      __syncthreads();
      consume(n);
      __syncthreads();
    }
  } else {
    const VT *row = (const VT *)h.ovf_dense + (size_t)h.ovf_slot[t] * h.cols;
    for (int c0 = 0; c0 < h.cols; c0 += 64) {
      const int j = c0 + lane;
      const float v = j < h.cols ? ldv(row, j) : 0.f;
      const bool nz = v != 0.f;
      const uint64_t m = ballot64(nz);
      if (m == 0) continue;
      if (nz) lst[mbcnt64(m)] = make_uint2((uint32_t)j, __float_as_uint(v));
      __syncthreads();
      consume(__popcll(m));
      __syncthreads();
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
  hipLaunchKernelGGL((k_row_list<VT>), dim3((h.rows + 3) / 4), dim3(256), 0, s, h);
  hipLaunchKernelGGL((k_twell_down<WT, VT, YT>), dim3((unsigned)grid), dim3(64), 0, s, h, w2, d, y, nchunk);
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
