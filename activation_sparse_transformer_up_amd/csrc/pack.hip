// Standalone dense -> TwELL packing and the row-overflow bookkeeping.
//
// "Sparser, Faster, Lighter Transformer Language Models", section "2. Metodologia":
//  - block "Formato de Dados TwELL": per (row, column tile) the nonzeros and their column
//    indices are stored aligned inside the tile. k_pack builds that layout from a dense
//    matrix already in memory (the conversion step the fused GEMM epilogue makes
//    unnecessary; kept as a building block).
//  - block "Formato Híbrido para Treinamento": rows with too many nonzeros go to a dense
//    backup. k_ovf_scan (ovf_scan_block) turns the per-(tile, 32-row) overflow bit words
//    into the ordered list of overflow rows, each row's backup slot, and the true overflow
//    count; the backup rows themselves are copied by k_ovf_copy (or recomputed by the up
//    GEMM).
#include "common.h"
#include "launch.h"
#include "rows.h"

namespace tw {

// One wave per (32-row block, tile). A lane holds V = W/64 consecutive columns; the slot of
// a nonzero is the number of nonzeros at lower columns of the tile (lower lanes via mbcnt,
// plus this lane's lower elements).
template <typename HT, int W>
__global__ __launch_bounds__(256) void k_pack(const HT *__restrict__ h, int R, int C, TwellOut o) {
  constexpr int V = W / 64;
  const int wave_g = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nblk = (R + 31) >> 5;
  if (wave_g >= nblk * o.n_t) return;
  const int kt = wave_g % o.n_t, rb = wave_g / o.n_t;
  const int lane = lane_id();
  const int S = o.S;
  uint32_t ovf_word = 0;
  for (int i = 0; i < 32; ++i) {
    const int row = rb * 32 + i;
    if (row >= R) break;
    const size_t src = (size_t)row * C + (size_t)kt * W + lane * V;
    uint32_t bits[V];
    bool nz[V];
#pragma unroll
    for (int e = 0; e < V; ++e) {
      if constexpr (sizeof(HT) == 4) {
        bits[e] = __float_as_uint(((const float *)h)[src + e]);
        nz[e] = (bits[e] & 0x7FFFFFFFu) != 0;
      } else {
        bits[e] = ((const uint16_t *)h)[src + e];
        nz[e] = (bits[e] & 0x7FFFu) != 0;
      }
    }
    int cnt = 0, before = 0;
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const uint64_t m = ballot64(nz[e]);
      cnt += __popcll(m);
      before += mbcnt64(m);
    }
    const size_t base = ((size_t)row * o.n_t + kt) * (size_t)S;
    int slot = before;
#pragma unroll
    for (int e = 0; e < V; ++e) {
      if (nz[e]) {
        if (slot < S) {
          o.col_idx[base + slot] = kt * W + lane * V + e;
          if (o.val_bf16) ((uint16_t *)o.vals)[base + slot] = (uint16_t)bits[e];
          else ((uint32_t *)o.vals)[base + slot] = sizeof(HT) == 4 ? bits[e] : (bits[e] << 16);
        }
        ++slot;
      }
    }
    for (int s = lane; s < S; s += 64) {
      if (s >= cnt) {
        o.col_idx[base + s] = -1;
        if (o.val_bf16) ((uint16_t *)o.vals)[base + s] = 0;
        else ((uint32_t *)o.vals)[base + s] = 0;
      }
    }
    if (lane == 0) o.counts[(size_t)row * o.n_t + kt] = cnt;
    if (cnt > S) ovf_word |= 1u << i;
  }
  if (lane == 0 && rb < o.words) o.ovf_bits[(size_t)kt * o.words + rb] = ovf_word;
}

__global__ __launch_bounds__(1024) void k_ovf_scan(const uint32_t *__restrict__ bits, int n_t, int words,
                                                   int R, int cap, int32_t *ovf_n, int32_t *ovf_rows,
                                                   int32_t *ovf_slot) {
  ovf_scan_block(bits, n_t, words, R, cap, ovf_n, ovf_rows, ovf_slot);
}

// Backup row r < min(*ovf_n, cap) = source row ovf_rows[r], copied (bf16 -> fp32 widening
// is exact).
template <typename HT, typename DT>
__global__ __launch_bounds__(256) void k_ovf_copy(const HT *__restrict__ h, int C, const int32_t *__restrict__ ovf_n,
                                                  const int32_t *__restrict__ ovf_rows, int cap, DT *__restrict__ dense) {
  const int r = blockIdx.x;
  const int n = min(*ovf_n, cap);
  if (r >= n) return;
  const size_t src = (size_t)ovf_rows[r] * C, dst = (size_t)r * C;
  for (int c = threadIdx.x; c < C; c += 256) Elem<DT>::store(dense, dst + c, Elem<HT>::load(h, src + c));
}

__global__ void k_set_int(int32_t *p, int v) { *p = v; }

// ------------------------------------------------------------------ host launchers

hipError_t launch_pack(const void *h, int h_bf16, int R, int C, const TwellOut &o, int W, hipStream_t s) {
  const int waves = ((R + 31) / 32) * o.n_t;
  dim3 grid((waves + 3) / 4);
  if (h_bf16) {
    if (W == 64) hipLaunchKernelGGL((k_pack<uint16_t, 64>), grid, dim3(256), 0, s, (const uint16_t *)h, R, C, o);
    else hipLaunchKernelGGL((k_pack<uint16_t, 128>), grid, dim3(256), 0, s, (const uint16_t *)h, R, C, o);
  } else {
    if (W == 64) hipLaunchKernelGGL((k_pack<float, 64>), grid, dim3(256), 0, s, (const float *)h, R, C, o);
    else hipLaunchKernelGGL((k_pack<float, 128>), grid, dim3(256), 0, s, (const float *)h, R, C, o);
  }
  return hipGetLastError();
}

hipError_t launch_ovf_scan(const uint32_t *bits, int n_t, int words, int R, int cap, int32_t *ovf_n,
                           int32_t *ovf_rows, int32_t *ovf_slot, hipStream_t s) {
  hipLaunchKernelGGL(k_ovf_scan, dim3(1), dim3(1024), 0, s, bits, n_t, words, R, cap, ovf_n, ovf_rows, ovf_slot);
  return hipGetLastError();
}

hipError_t launch_ovf_copy(const void *h, int h_bf16, int R, int C, const int32_t *ovf_n, const int32_t *ovf_rows,
                           int cap, void *dense, int dense_bf16, hipStream_t s) {
  (void)R;
  if (cap <= 0) return hipSuccess;
  dim3 grid(cap);
  if (h_bf16 && dense_bf16)
    hipLaunchKernelGGL((k_ovf_copy<uint16_t, uint16_t>), grid, dim3(256), 0, s, (const uint16_t *)h, C, ovf_n, ovf_rows, cap, (uint16_t *)dense);
  else if (h_bf16)
    hipLaunchKernelGGL((k_ovf_copy<uint16_t, float>), grid, dim3(256), 0, s, (const uint16_t *)h, C, ovf_n, ovf_rows, cap, (float *)dense);
  else
    hipLaunchKernelGGL((k_ovf_copy<float, float>), grid, dim3(256), 0, s, (const float *)h, C, ovf_n, ovf_rows, cap, (float *)dense);
  return hipGetLastError();
}

// Row-maximum histogram of a TwELL's true counts ("Formato Híbrido para Treinamento": the
// compact width is chosen from the data, and rows beyond it go to the dense backup).
// hist[m] = number of rows whose largest per-tile count is m (0 <= m <= W). A wave reduces
// one row's n_t counts at a time; each workgroup gathers its rows in an LDS histogram and
// adds its nonzero bins to hist with integer atomics (exact and order-free).
__global__ __launch_bounds__(256) void k_zero_i32(int32_t *__restrict__ p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

__global__ __launch_bounds__(256) void k_rowmax_hist(const int32_t *__restrict__ counts, int rows, int n_t, int W,
                                                     int32_t *__restrict__ hist) {
  __shared__ int32_t lh[129];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i <= W; i += 256) lh[i] = 0;
  __syncthreads();
  for (int row = blockIdx.x * 4 + wave; row < rows; row += gridDim.x * 4) {
    const int32_t *c = counts + (size_t)row * n_t;
    int m = 0;
    for (int k = lane; k < n_t; k += 64) m = max(m, c[k]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = max(m, __shfl_xor(m, o, 64));
    if (lane == 0) atomicAdd(&lh[min(max(m, 0), W)], 1);
  }
  __syncthreads();
  for (int i = tid; i <= W; i += 256)
    if (lh[i]) atomicAdd(&hist[i], lh[i]);
}

hipError_t launch_rowmax_hist(const int32_t *counts, int rows, int n_t, int W, int32_t *hist, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_i32, dim3((W + 1 + 255) / 256), dim3(256), 0, s, hist, W + 1);
  if (rows > 0) {
    const int grid = min((rows + 3) / 4, 1024);
    hipLaunchKernelGGL(k_rowmax_hist, dim3(grid), dim3(256), 0, s, counts, rows, n_t, W, hist);
  }
  return hipGetLastError();
}

hipError_t launch_zero_i32(int32_t *p, int n, hipStream_t s) {
  if (n > 0) hipLaunchKernelGGL(k_zero_i32, dim3((n + 255) / 256), dim3(256), 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_set_int(int32_t *p, int v, hipStream_t s) {
  hipLaunchKernelGGL(k_set_int, dim3(1), dim3(1), 0, s, p, v);
  return hipGetLastError();
}

}  // namespace tw
