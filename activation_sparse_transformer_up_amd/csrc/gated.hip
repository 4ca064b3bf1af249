// Gated feed-forward: the up projection over the gate's active units only.
//
// "Sparser, Faster, Lighter Transformer Language Models", section "2. Metodologia": the
// TwELL layout is produced by the dense product that computes the gate activations (block
// "Formato de Dados TwELL"), and the inference kernel iterates over the active units only,
// taking a dot product with the up weights and then multiplying-adding the unit's down row
// (block "Kernels de Inferência"). Here the dot products are a stage of their own between
// the gate's finish (row lists, overflow backup) and the down gather: for every entry
// (j, g) of a token's row list g <- g * (x[t] . w_up[j]), and the same for every nonzero
// of a dense backup row. The gather then sums (g u)_j w2[j].
//
// A wave takes ENT list entries at a time. Lane l holds 16-byte pieces l, l + 64, ... of
// x[t] (8 bf16 or 4 fp32 per piece), loads the same pieces of the ENT up rows before any
// arithmetic, and accumulates with v_dot2_f32_bf16 (bf16; two products per instruction,
// fp32 accumulation) or fp32 FMAs; the ENT sums are reduced across the wave and lane 0
// rewrites the entries' values.
#include "common.h"
#include "launch.h"

namespace tw {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kGateEnt = 4;      // list entries per wave and round

template <typename XT> TW_DEV float dot16(uint4 a, uint4 b, float acc) {
  if constexpr (sizeof(XT) == 2) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x), __builtin_bit_cast(bf16x2_t, b.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y), __builtin_bit_cast(bf16x2_t, b.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z), __builtin_bit_cast(bf16x2_t, b.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w), __builtin_bit_cast(bf16x2_t, b.w), acc, false);
  } else {
    acc = fmaf(__uint_as_float(a.x), __uint_as_float(b.x), acc);
    acc = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), acc);
    acc = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), acc);
    acc = fmaf(__uint_as_float(a.w), __uint_as_float(b.w), acc);
  }
  return acc;
}

// u[k] = x_row . wu[col[k]] for k < ENT (col[k] < 0: no entry, u = 0), summed over the wave.
// NP 16-byte pieces per lane are in flight at once (NP = 4 covers 2048 bf16 columns; fewer
// registers than needed for larger rows would cost occupancy for nothing at small d).
template <typename XT, int NP>
TW_DEV void wave_dots(const XT *__restrict__ xrow, const XT *__restrict__ wu, int d, const int (&col)[kGateEnt],
                      float (&u)[kGateEnt]) {
  constexpr int EPL = 16 / sizeof(XT);
  const int lane = lane_id();
  const int npc = (d + 64 * EPL - 1) / (64 * EPL);
#pragma unroll
  for (int k = 0; k < kGateEnt; ++k) u[k] = 0.f;
  for (int c0 = 0; c0 < npc; c0 += NP) {
    uint4 xv[NP], wv[kGateEnt][NP];
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const int i = ((c0 + q) * 64 + lane) * EPL;
      const bool ok = i < d;                                    // d is a multiple of EPL
      xv[q] = ok ? *(const uint4 *)(xrow + i) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int k = 0; k < kGateEnt; ++k)
        wv[k][q] = (ok && col[k] >= 0) ? *(const uint4 *)(wu + (size_t)col[k] * d + i) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < NP; ++q)
#pragma unroll
      for (int k = 0; k < kGateEnt; ++k) u[k] = dot16<XT>(xv[q], wv[k][q], u[k]);
  }
#pragma unroll
  for (int k = 0; k < kGateEnt; ++k) u[k] = wave_sumf(u[k]);
}

// Row lists: workgroup (t, p) of 4 waves; wave w takes the entry groups p * 4 + w,
// p * 4 + w + 4 P, ... of ENT entries each. Overflow rows are skipped (their backup row
// carries them).
template <typename XT, int NP>
__global__ __launch_bounds__(256) void k_gate_dot(TwellIn h, const XT *__restrict__ x, const XT *__restrict__ wu,
                                                  int d, int P) {
  const int t = blockIdx.x / P, p = blockIdx.x % P;
  if (t >= h.rows || h.ovf_slot[t] >= 0) return;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  const int nnz = h.row_nnz[t];
  uint2 *lst = h.row_list + (size_t)t * h.n_t * h.S;
  const XT *xrow = x + (size_t)t * d;
  for (int e0 = (p * 4 + wave) * kGateEnt; e0 < nnz; e0 += P * 4 * kGateEnt) {
    int col[kGateEnt];
#pragma unroll
    for (int k = 0; k < kGateEnt; ++k) col[k] = e0 + k < nnz ? (int)lst[e0 + k].x : -1;
    float u[kGateEnt];
    wave_dots<XT, NP>(xrow, wu, d, col, u);
    if (lane == 0)
#pragma unroll
      for (int k = 0; k < kGateEnt; ++k)
        if (col[k] >= 0) lst[e0 + k].y = __float_as_uint(__uint_as_float(lst[e0 + k].y) * u[k]);
  }
}

// Backup rows: one wave per (overflow row r < min(ovf_n, cap), 64-column block); the
// block's nonzero gates are taken ENT at a time in ascending column order.
template <typename XT, typename VT>
__global__ __launch_bounds__(256) void k_gate_dot_backup(TwellIn h, const XT *__restrict__ x,
                                                         const XT *__restrict__ wu, int d) {
  const int wave_g = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nblk = (h.cols + 63) / 64;
  const int r = wave_g / nblk, blk = wave_g % nblk;
  if (r >= min(*h.ovf_n, h.cap)) return;                        // wave-uniform
  const int lane = lane_id();
  const int t = h.ovf_rows[r];
  VT *row = (VT *)h.ovf_dense + (size_t)r * h.cols;
  const int j = blk * 64 + lane;
  const float g = j < h.cols ? Elem<VT>::load(row, j) : 0.f;
  uint64_t m = ballot64(g != 0.f);
  while (m) {
    int col[kGateEnt];
#pragma unroll
    for (int k = 0; k < kGateEnt; ++k) {
      col[k] = m ? blk * 64 + (int)__builtin_ctzll(m) : -1;
      m &= m ? m - 1 : 0;
    }
    float u[kGateEnt];
    wave_dots<XT, 8>(x + (size_t)t * d, wu, d, col, u);
#pragma unroll
    for (int k = 0; k < kGateEnt; ++k) {
      const float gk = __shfl(g, col[k] & 63, 64);
      if (lane == 0 && col[k] >= 0) Elem<VT>::store(row, col[k], gk * u[k]);
    }
  }
}

hipError_t launch_gate_up(const TwellIn &h, const void *x, const void *wu, int bf16, int d, hipStream_t s) {
  if (h.rows == 0) return hipSuccess;
  // enough workgroups to keep every CU busy at few tokens, without more entry groups per
  // token than a full list has
  const int groups = (h.n_t * h.S + 4 * kGateEnt - 1) / (4 * kGateEnt);
  const int P = max(1, min(groups, (2048 + h.rows - 1) / h.rows));
  const dim3 grid((unsigned)((size_t)h.rows * P));
  const size_t nb = (size_t)h.cap * ((h.cols + 63) / 64);
  const dim3 gridb((unsigned)((nb + 3) / 4));
  if (bf16) {
    const uint16_t *xx = (const uint16_t *)x, *ww = (const uint16_t *)wu;
    if (d <= 2048) hipLaunchKernelGGL((k_gate_dot<uint16_t, 4>), grid, dim3(256), 0, s, h, xx, ww, d, P);
    else hipLaunchKernelGGL((k_gate_dot<uint16_t, 8>), grid, dim3(256), 0, s, h, xx, ww, d, P);
    if (nb) {
      if (h.val_bf16) hipLaunchKernelGGL((k_gate_dot_backup<uint16_t, uint16_t>), gridb, dim3(256), 0, s, h, xx, ww, d);
      else hipLaunchKernelGGL((k_gate_dot_backup<uint16_t, float>), gridb, dim3(256), 0, s, h, xx, ww, d);
    }
  } else {
    const float *xx = (const float *)x, *ww = (const float *)wu;
    if (d <= 1024) hipLaunchKernelGGL((k_gate_dot<float, 4>), grid, dim3(256), 0, s, h, xx, ww, d, P);
    else hipLaunchKernelGGL((k_gate_dot<float, 8>), grid, dim3(256), 0, s, h, xx, ww, d, P);
    if (nb) {
      if (h.val_bf16) hipLaunchKernelGGL((k_gate_dot_backup<float, uint16_t>), gridb, dim3(256), 0, s, h, xx, ww, d);
      else hipLaunchKernelGGL((k_gate_dot_backup<float, float>), gridb, dim3(256), 0, s, h, xx, ww, d);
    }
  }
  return hipGetLastError();
}

}  // namespace tw
