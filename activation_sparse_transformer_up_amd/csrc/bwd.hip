// Backward pass of the activation-sparse FFN on the stored sparsity pattern.
//
// "Sparser, Faster, Lighter Transformer Language Models", section "2. Metodologia":
//  - block "Formato Híbrido para Treinamento": training kernels run on the sparse pattern,
//    normal rows from their compact slots, overflow rows from the dense backup;
//  - block "Técnicas de Treinamento": an L1 penalty on the ReLU activations adds its
//    coefficient to dh on every active entry.
// For L = <dy, y> + l1 * sum(h), y = ReLU(x W1 + b1) W2, on the pattern P = {h > 0}:
//   dz = (dy W2^T + l1) on P;  dx = dz w1t;  dw1t = dz^T x;  dw2 = h^T dy;  db1 = sum_t dz.
//
// Steps (all on the caller's stream, scratch in the caller's workspace):
//   1. row_nnz + scan        -> row_ptr: per-token entry counts (CSR offsets)
//   2. csr_fill              -> (col, h) per entry, ascending column within a token
//   3. sddmm                 -> dz per entry: one wave per token, dy[t] held in registers,
//                               bf16 dot2 against the W2 rows of its active units
//   4. list_gather (w1t)     -> dx
//   5. col_mask, col_tot, scan, col_off, csc_fill -> the same entries by unit (CSC), tokens
//      ascending inside a unit, positions computed without a serial pass: per 32-token
//      block every unit keeps the bit mask of its tokens; an entry's rank inside its unit
//      is the block offset plus the popcount of the mask bits of earlier tokens
//   6. list_gather dual (dy, x) -> dw2, dw1t; col_sum -> db1
#include "common.h"
#include "launch.h"

namespace tw {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ 1. counts / scan

// nnz[t] = entries of row t: the nonzeros of its backup row (counted in that row, so the
// fill below writes exactly this many), else the stored slots.
template <typename VT>
__global__ __launch_bounds__(256) void k_row_nnz(TwellIn h, int32_t *__restrict__ nnz) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= h.rows) return;
  const int lane = lane_id();
  const int slot = h.ovf_slot[t];
  int s = 0;
  if (slot >= 0) {
    const VT *row = (const VT *)h.ovf_dense + (size_t)slot * h.cols;
    for (int j = lane; j < h.cols; j += 64) s += Elem<VT>::load(row, j) != 0.f;
  } else {
    for (int k = lane; k < h.n_t; k += 64) s += min(h.counts[(size_t)t * h.n_t + k], h.S);
  }
  s = wave_sum(s);
  if (lane == 0) nnz[t] = s;
}

// out[i] = in[0] + ... + in[i-1] for i <= n (out may alias in). One workgroup.
__global__ __launch_bounds__(1024) void k_scan_excl(const int32_t *in, int n, int32_t *out) {
  constexpr int IPT = 8;
  __shared__ int wsum[16];
  __shared__ int carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < n; base += 1024 * IPT) {
    int v[IPT];
    int local = 0;
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int idx = base + tid * IPT + i;
      v[i] = idx < n ? in[idx] : 0;
      local += v[i];
    }
    int tot;
    const int ex = wave_excl_scan(local, &tot);
    if (lane == 0) wsum[wave] = tot;
    __syncthreads();
    int wpre = 0, ctot = 0;
    for (int i = 0; i < 16; ++i) {
      if (i < wave) wpre += wsum[i];
      ctot += wsum[i];
    }
    int run = carry_s + wpre + ex;
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int idx = base + tid * IPT + i;
      if (idx < n) out[idx] = run;
      run += v[i];
    }
    __syncthreads();
    if (tid == 0) carry_s += ctot;
    __syncthreads();
  }
  if (tid == 0) out[n] = carry_s;
}

// --------------------------------------------------------------------- 2. CSR fill

template <typename VT>
__global__ __launch_bounds__(256) void k_csr_fill(TwellIn h, const int32_t *__restrict__ row_ptr,
                                                  int32_t *__restrict__ col, float *__restrict__ hval) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= h.rows) return;
  const int lane = lane_id();
  const int base = row_ptr[t], lim = row_ptr[t + 1];
  const int slot = h.ovf_slot[t];
  const VT *vals = (const VT *)h.vals;
  int n = 0;
  if (slot >= 0) {
    const VT *row = (const VT *)h.ovf_dense + (size_t)slot * h.cols;
    for (int c0 = 0; c0 < h.cols; c0 += 64) {
      const int j = c0 + lane;
      const float v = j < h.cols ? Elem<VT>::load(row, j) : 0.f;
      const bool nz = v != 0.f;
      const uint64_t m = ballot64(nz);
      const int pos = base + n + (int)mbcnt64(m);
      if (nz && pos < lim) {
        col[pos] = j;
        hval[pos] = v;
      }
      n += __popcll(m);
    }
  } else {
    for (int k0 = 0; k0 < h.n_t; k0 += 64) {
      const int k = k0 + lane;
      const int m = k < h.n_t ? min(h.counts[(size_t)t * h.n_t + k], h.S) : 0;
      int tot;
      const int off = wave_excl_scan(m, &tot);
      const size_t sb = ((size_t)t * h.n_t + k) * h.S;
      for (int s = 0; s < m; ++s) {
        const int pos = base + n + off + s;
        if (pos < lim) {
          col[pos] = h.col_idx[sb + s];
          hval[pos] = Elem<VT>::load(vals, sb + s);
        }
      }
      n += tot;
    }
  }
}

// ------------------------------------------------------------------------ 3. SDDMM

// dz[e] = dy[t] . w2[col[e]] + l1 for the entries e of token t. One wave per token; the
// token's dy row lives in registers (16-byte chunks, chunk c of lane l covers elements
// c * 64 * EPC + l * EPC ...), two W2 rows are in flight per step.
template <typename T, int MAXC>
__global__ __launch_bounds__(256) void k_sddmm(int T_rows, int d, const T *__restrict__ dy,
                                               const T *__restrict__ w2, const int32_t *__restrict__ row_ptr,
                                               const int32_t *__restrict__ col, float l1,
                                               float *__restrict__ dz) {
  constexpr int EPC = 16 / sizeof(T);
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T_rows) return;
  const int lane = lane_id();
  const int nch = (d + 64 * EPC - 1) / (64 * EPC);
  uint4 a[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int e0 = c * 64 * EPC + lane * EPC;
    a[c] = (c < nch && e0 < d) ? *(const uint4 *)(dy + (size_t)t * d + e0) : make_uint4(0, 0, 0, 0);
  }
  auto dot = [&](const uint4 &x, const uint4 &y, float acc) -> float {
    if constexpr (sizeof(T) == 2) {
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x.x), __builtin_bit_cast(bf16x2_t, y.x), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x.y), __builtin_bit_cast(bf16x2_t, y.y), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x.z), __builtin_bit_cast(bf16x2_t, y.z), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x.w), __builtin_bit_cast(bf16x2_t, y.w), acc, false);
    } else {
      acc = fmaf(__uint_as_float(x.x), __uint_as_float(y.x), acc);
      acc = fmaf(__uint_as_float(x.y), __uint_as_float(y.y), acc);
      acc = fmaf(__uint_as_float(x.z), __uint_as_float(y.z), acc);
      acc = fmaf(__uint_as_float(x.w), __uint_as_float(y.w), acc);
    }
    return acc;
  };
  const int start = row_ptr[t], end = row_ptr[t + 1];
  int e = start;
  for (; e + 1 < end; e += 2) {
    const int j0 = col[e], j1 = col[e + 1];
    uint4 b0[MAXC], b1[MAXC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int e0 = c * 64 * EPC + lane * EPC;
      const bool ok = c < nch && e0 < d;
      b0[c] = ok ? *(const uint4 *)(w2 + (size_t)j0 * d + e0) : make_uint4(0, 0, 0, 0);
      b1[c] = ok ? *(const uint4 *)(w2 + (size_t)j1 * d + e0) : make_uint4(0, 0, 0, 0);
    }
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      s0 = dot(a[c], b0[c], s0);
      s1 = dot(a[c], b1[c], s1);
    }
    s0 = wave_sumf(s0);
    s1 = wave_sumf(s1);
    if (lane == 0) {
      dz[e] = s0 + l1;
      dz[e + 1] = s1 + l1;
    }
  }
  if (e < end) {
    const int j0 = col[e];
    float s0 = 0.f;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int e0 = c * 64 * EPC + lane * EPC;
      if (c < nch && e0 < d) s0 = dot(a[c], *(const uint4 *)(w2 + (size_t)j0 * d + e0), s0);
    }
    s0 = wave_sumf(s0);
    if (lane == 0) dz[e] = s0 + l1;
  }
}

// ------------------------------------------------------------------ 4/6. list gathers

// out[r][c..] = sum over entries e of list r of val[e] * M[idx[e]][c..] (fp32 accumulation).
// DUAL: a second value array / matrix / output sharing the same index list.
// Work item (r, chunk); chunk = 16 lanes x 16 bytes; XCD-aware order as in the forward
// down projection (chunks congruent mod 8 stay on one XCD).
template <typename MT, bool DUAL>
__global__ __launch_bounds__(64) void k_list_gather(int R, int d, int nchunk, const int32_t *__restrict__ ptr,
                                                    const int32_t *__restrict__ idx,
                                                    const float *__restrict__ va, const MT *__restrict__ Ma,
                                                    float *__restrict__ outa, const float *__restrict__ vb,
                                                    const MT *__restrict__ Mb, float *__restrict__ outb) {
  const int b = blockIdx.x, xcd = b & 7, i = b >> 3;
  const int c = xcd + 8 * (i / R), r = i % R;
  if (c >= nchunk) return;
  constexpr int E = Vec16<MT>::N;
  constexpr int CW = 16 * E;
  const int lane = lane_id(), g = lane >> 4, gl = lane & 15;
  const int colo = c * CW + gl * E;
  const bool cv = colo < d;
  float acc_a[E], acc_b[E];
#pragma unroll
  for (int q = 0; q < E; ++q) acc_a[q] = acc_b[q] = 0.f;
  const int start = ptr[r], end = ptr[r + 1];
  int e = start + g;
  for (; e + 12 < end; e += 16) {
    int j[4];
    float v[4], w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      j[u] = idx[e + 4 * u];
      v[u] = va[e + 4 * u];
      if (DUAL) w[u] = vb[e + 4 * u];
    }
    if (cv) {
      float ra[4][E], rb[4][E];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        Vec16<MT>::load(Ma + (size_t)j[u] * d + colo, ra[u]);
        if (DUAL) Vec16<MT>::load(Mb + (size_t)j[u] * d + colo, rb[u]);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < E; ++q) {
          acc_a[q] = fmaf(v[u], ra[u][q], acc_a[q]);
          if (DUAL) acc_b[q] = fmaf(w[u], rb[u][q], acc_b[q]);
        }
    }
  }
  for (; e < end; e += 4) {
    const int jj = idx[e];
    const float vv = va[e];
    const float ww = DUAL ? vb[e] : 0.f;
    if (cv) {
      float ra[E], rb[E];
      Vec16<MT>::load(Ma + (size_t)jj * d + colo, ra);
      if (DUAL) Vec16<MT>::load(Mb + (size_t)jj * d + colo, rb);
#pragma unroll
      for (int q = 0; q < E; ++q) {
        acc_a[q] = fmaf(vv, ra[q], acc_a[q]);
        if (DUAL) acc_b[q] = fmaf(ww, rb[q], acc_b[q]);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < E; ++q) {
    acc_a[q] += __shfl_xor(acc_a[q], 16, 64);
    acc_a[q] += __shfl_xor(acc_a[q], 32, 64);
    if (DUAL) {
      acc_b[q] += __shfl_xor(acc_b[q], 16, 64);
      acc_b[q] += __shfl_xor(acc_b[q], 32, 64);
    }
  }
  if (g == 0 && cv) {
    const size_t o = (size_t)r * d + colo;
#pragma unroll
    for (int q = 0; q < E; q += 4) {
      *(float4 *)(outa + o + q) = make_float4(acc_a[q], acc_a[q + 1], acc_a[q + 2], acc_a[q + 3]);
      if (DUAL) *(float4 *)(outb + o + q) = make_float4(acc_b[q], acc_b[q + 1], acc_b[q + 2], acc_b[q + 3]);
    }
  }
}

// ------------------------------------------------------------------- 5. CSR -> CSC

// Per 32-token block b: mask[b][j] bit (t - 32 b) set iff token t has unit j active;
// cnt[b][j] = popcount. LDS holds the block's masks for all units.
__global__ __launch_bounds__(256) void k_col_mask(int T_rows, int f, const int32_t *__restrict__ row_ptr,
                                                  const int32_t *__restrict__ col, uint32_t *__restrict__ mask,
                                                  int32_t *__restrict__ cnt) {
  extern __shared__ uint32_t lm[];
  const int b = blockIdx.x, tid = threadIdx.x;
  for (int j = tid; j < f; j += 256) lm[j] = 0u;
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63;
  for (int tt = wave; tt < 32; tt += 4) {
    const int t = b * 32 + tt;
    if (t >= T_rows) break;
    const int s = row_ptr[t], e = row_ptr[t + 1];
    for (int k = s + lane; k < e; k += 64) atomicOr(&lm[col[k]], 1u << tt);
  }
  __syncthreads();
  for (int j = tid; j < f; j += 256) {
    const uint32_t m = lm[j];
    mask[(size_t)b * f + j] = m;
    cnt[(size_t)b * f + j] = __popc(m);
  }
}

// tot[j] = sum_b cnt[b][j]
__global__ __launch_bounds__(256) void k_col_tot(int NB, int f, const int32_t *__restrict__ cnt,
                                                 int32_t *__restrict__ tot) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= f) return;
  int s = 0;
  for (int b = 0; b < NB; ++b) s += cnt[(size_t)b * f + j];
  tot[j] = s;
}

// cnt[b][j] <- col_ptr[j] + sum_{b' < b} cnt[b'][j]  (first position of block b in unit j)
__global__ __launch_bounds__(256) void k_col_off(int NB, int f, const int32_t *__restrict__ col_ptr,
                                                 int32_t *__restrict__ cnt) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= f) return;
  int run = col_ptr[j];
  for (int b = 0; b < NB; ++b) {
    const int c = cnt[(size_t)b * f + j];
    cnt[(size_t)b * f + j] = run;
    run += c;
  }
}

// Every CSR entry (t, j) goes to position off[t/32][j] + popc(mask[t/32][j] & lower bits).
__global__ __launch_bounds__(256) void k_csc_fill(int T_rows, int f, const int32_t *__restrict__ row_ptr,
                                                  const int32_t *__restrict__ col, const float *__restrict__ hval,
                                                  const float *__restrict__ dz, const uint32_t *__restrict__ mask,
                                                  const int32_t *__restrict__ off, int32_t *__restrict__ tok,
                                                  float *__restrict__ hv, float *__restrict__ dzv) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T_rows) return;
  const int lane = lane_id();
  const int b = t >> 5, bit = t & 31;
  const uint32_t lower = (1u << bit) - 1u;
  const int s = row_ptr[t], e = row_ptr[t + 1];
  for (int k = s + lane; k < e; k += 64) {
    const int j = col[k];
    const size_t bj = (size_t)b * f + j;
    const int pos = off[bj] + __popc(mask[bj] & lower);
    tok[pos] = t;
    hv[pos] = hval[k];
    dzv[pos] = dz[k];
  }
}

// db1[j] = sum of dz over unit j's entries
__global__ __launch_bounds__(256) void k_col_sum(int f, const int32_t *__restrict__ col_ptr,
                                                 const float *__restrict__ dzv, float *__restrict__ db1) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= f) return;
  float s = 0.f;
  for (int k = col_ptr[j]; k < col_ptr[j + 1]; ++k) s += dzv[k];
  db1[j] = s;
}

// ------------------------------------------------------------------ host side

// Register-resident dy needs ceil(d / (64 * EPC)) 16-byte chunks per lane (<= 16).
template <typename T>
static void sddmm_t(dim3 grid, hipStream_t s, int T_rows, int d, const T *dy, const T *w2, const int32_t *row_ptr,
                    const int32_t *col, float l1, float *dz) {
  constexpr int EPC = 16 / sizeof(T);
  const int nch = (d + 64 * EPC - 1) / (64 * EPC);
  if (nch <= 1) hipLaunchKernelGGL((k_sddmm<T, 1>), grid, dim3(256), 0, s, T_rows, d, dy, w2, row_ptr, col, l1, dz);
  else if (nch <= 2) hipLaunchKernelGGL((k_sddmm<T, 2>), grid, dim3(256), 0, s, T_rows, d, dy, w2, row_ptr, col, l1, dz);
  else if (nch <= 4) hipLaunchKernelGGL((k_sddmm<T, 4>), grid, dim3(256), 0, s, T_rows, d, dy, w2, row_ptr, col, l1, dz);
  else if (nch <= 8) hipLaunchKernelGGL((k_sddmm<T, 8>), grid, dim3(256), 0, s, T_rows, d, dy, w2, row_ptr, col, l1, dz);
  else hipLaunchKernelGGL((k_sddmm<T, 16>), grid, dim3(256), 0, s, T_rows, d, dy, w2, row_ptr, col, l1, dz);
}

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t bwd_workspace_bytes(int T, int d, int f, int n_t, int S, int cap) {
  (void)d;
  const size_t NZ = (size_t)T * n_t * S + (size_t)(cap < T ? cap : T) * f;
  const size_t NB = ((size_t)T + 31) / 32;
  size_t b = 0;
  b += al256(4 * ((size_t)T + 1));          // row_ptr
  b += 3 * al256(4 * NZ);                   // col, hval, dz
  b += 2 * al256(4 * NB * f);               // mask, cnt/off
  b += al256(4 * ((size_t)f + 1));          // col_ptr
  b += 3 * al256(4 * NZ);                   // tok, hv, dzv
  return b;
}

hipError_t launch_bwd(const BwdArgs &a, hipStream_t s) {
  const TwellIn &h = a.h;
  const int T = h.rows, f = h.cols, d = a.d;
  const size_t NZ = (size_t)T * h.n_t * h.S + (size_t)(a.cap < T ? a.cap : T) * f;
  const size_t NB = ((size_t)T + 31) / 32;
  char *p = (char *)a.ws;
  auto take = [&](size_t bytes) { char *q = p; p += al256(bytes); return q; };
  int32_t *row_ptr = (int32_t *)take(4 * ((size_t)T + 1));
  int32_t *col = (int32_t *)take(4 * NZ);
  float *hval = (float *)take(4 * NZ);
  float *dz = (float *)take(4 * NZ);
  uint32_t *mask = (uint32_t *)take(4 * NB * f);
  int32_t *cnt = (int32_t *)take(4 * NB * f);
  int32_t *col_ptr = (int32_t *)take(4 * ((size_t)f + 1));
  int32_t *tok = (int32_t *)take(4 * NZ);
  float *hv = (float *)take(4 * NZ);
  float *dzv = (float *)take(4 * NZ);
  const dim3 rows4((T + 3) / 4);
  if (T > 0) {
    if (h.val_bf16) hipLaunchKernelGGL(k_row_nnz<uint16_t>, rows4, dim3(256), 0, s, h, row_ptr);
    else hipLaunchKernelGGL(k_row_nnz<float>, rows4, dim3(256), 0, s, h, row_ptr);
  }
  hipLaunchKernelGGL(k_scan_excl, dim3(1), dim3(1024), 0, s, row_ptr, T, row_ptr);
  if (T > 0) {
    if (h.val_bf16) hipLaunchKernelGGL(k_csr_fill<uint16_t>, rows4, dim3(256), 0, s, h, row_ptr, col, hval);
    else hipLaunchKernelGGL(k_csr_fill<float>, rows4, dim3(256), 0, s, h, row_ptr, col, hval);
    if (a.bf16) sddmm_t<uint16_t>(rows4, s, T, d, (const uint16_t *)a.dy, (const uint16_t *)a.w2, row_ptr, col, a.l1, dz);
    else sddmm_t<float>(rows4, s, T, d, (const float *)a.dy, (const float *)a.w2, row_ptr, col, a.l1, dz);
  }
  const int cw = a.bf16 ? 128 : 64;
  const int nchunk = (d + cw - 1) / cw;
  // dx = dz . w1t
  if (T > 0) {
    const size_t grid = 8 * (size_t)T * ((nchunk + 7) / 8);
    if (a.bf16) hipLaunchKernelGGL((k_list_gather<uint16_t, false>), dim3((unsigned)grid), dim3(64), 0, s, T, d, nchunk,
                                   row_ptr, col, dz, (const uint16_t *)a.w1t, a.dx, nullptr, nullptr, nullptr);
    else hipLaunchKernelGGL((k_list_gather<float, false>), dim3((unsigned)grid), dim3(64), 0, s, T, d, nchunk,
                            row_ptr, col, dz, (const float *)a.w1t, a.dx, nullptr, nullptr, nullptr);
  }
  // CSC
  if (T > 0) {
    hipLaunchKernelGGL(k_col_mask, dim3((unsigned)NB), dim3(256), (size_t)f * 4, s, T, f, row_ptr, col, mask, cnt);
    hipLaunchKernelGGL(k_col_tot, dim3((f + 255) / 256), dim3(256), 0, s, (int)NB, f, cnt, col_ptr);
  } else {
    hipLaunchKernelGGL(k_col_tot, dim3((f + 255) / 256), dim3(256), 0, s, 0, f, cnt, col_ptr);
  }
  hipLaunchKernelGGL(k_scan_excl, dim3(1), dim3(1024), 0, s, col_ptr, f, col_ptr);
  if (T > 0) {
    hipLaunchKernelGGL(k_col_off, dim3((f + 255) / 256), dim3(256), 0, s, (int)NB, f, col_ptr, cnt);
    hipLaunchKernelGGL(k_csc_fill, rows4, dim3(256), 0, s, T, f, row_ptr, col, hval, dz, mask, cnt, tok, hv, dzv);
  }
  // dw2 = h^T dy, dw1t = dz^T x  (every unit row written, zero if it has no entry)
  {
    const size_t grid = 8 * (size_t)f * ((nchunk + 7) / 8);
    if (a.bf16) hipLaunchKernelGGL((k_list_gather<uint16_t, true>), dim3((unsigned)grid), dim3(64), 0, s, f, d, nchunk,
                                   col_ptr, tok, hv, (const uint16_t *)a.dy, a.dw2, dzv, (const uint16_t *)a.x, a.dw1t);
    else hipLaunchKernelGGL((k_list_gather<float, true>), dim3((unsigned)grid), dim3(64), 0, s, f, d, nchunk,
                            col_ptr, tok, hv, (const float *)a.dy, a.dw2, dzv, (const float *)a.x, a.dw1t);
  }
  if (a.db1) hipLaunchKernelGGL(k_col_sum, dim3((f + 255) / 256), dim3(256), 0, s, f, col_ptr, dzv, a.db1);
  return hipGetLastError();
}

}  // namespace tw
