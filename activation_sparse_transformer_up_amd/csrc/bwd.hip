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
//   3. sddmm                 -> dz per entry, in two kernels: per 16-byte-per-lane column
//                               chunk the partial dot products of dy[t] with the W2 rows of
//                               its active units (the gathers' decomposition, so each XCD
//                               reads only its slices of W2), then their sum in chunk order
//                               plus l1, stored as the (unit, dz) pairs of the dx gather
//   4. gather (w1t rows)     -> dx
//   5. col_mask, scan, col_off, csc_fill -> the same entries by unit (CSC), tokens
//      ascending inside a unit, positions computed without a serial pass: per 32-token
//      block every unit keeps the bit mask of its tokens; an entry's rank inside its unit
//      is the block offset plus the popcount of the mask bits of earlier tokens. Writes
//      the (token, h) and (token, dz) pairs of the two dW gathers
//   6. gather (dy rows) -> dw2; gather (x rows) -> dw1t, with db1 = sum of dz
// The three gathers share the 4-lists-per-wave core of the forward down projection.
#include <algorithm>

#include "common.h"
#include "gather.h"
#include "launch.h"

namespace tw {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ 1. counts / scan

// A dense backup row is walked by one wave, 64 columns per step; the loads of kDenseBatch
// steps are issued before any is used (addresses clamped into the row; columns past the
// row read as zero), so the walk waits for memory once per batch rather than once per step.
constexpr int kDenseBatch = 32;

template <typename VT>
TW_DEV void dense_batch(const VT *row, int cols, int j0, float (&v)[kDenseBatch]) {
#pragma unroll
  for (int u = 0; u < kDenseBatch; ++u) {
    const int j = j0 + u * 64;
    const float x = Elem<VT>::load(row, j < cols ? j : cols - 1);
    v[u] = j < cols ? x : 0.f;
  }
}

// nnz[t] = entries of row t: the nonzeros of its backup row (counted in that row, so the
// fill below writes exactly this many), else the stored slots.
// Also clears tot[0 .. f] (the per-unit totals k_col_mask accumulates into).
template <typename VT>
__global__ __launch_bounds__(256) void k_row_nnz(TwellIn h, int32_t *__restrict__ nnz, int32_t *__restrict__ tot,
                                                 int f) {
  for (int j = blockIdx.x * 256 + threadIdx.x; j <= f; j += gridDim.x * 256) tot[j] = 0;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= h.rows) return;
  const int lane = lane_id();
  const int slot = h.ovf_slot[t];
  int s = 0;
  if (slot >= 0) {
    const VT *row = (const VT *)h.ovf_dense + (size_t)slot * h.cols;
    for (int j0 = 0; j0 < h.cols; j0 += 64 * kDenseBatch) {
      float v[kDenseBatch];
      dense_batch<VT>(row, h.cols, j0 + lane, v);
#pragma unroll
      for (int u = 0; u < kDenseBatch; ++u) s += v[u] != 0.f;
    }
  } else {
    for (int k = lane; k < h.n_t; k += 64) s += min(h.counts[(size_t)t * h.n_t + k], h.S);
  }
  s = wave_sum(s);
  if (lane == 0) nnz[t] = s;
}

// out[i] = in[0] + ... + in[i-1] for i <= n (out may alias in). One workgroup.
__global__ __launch_bounds__(1024) void k_scan_excl(const int32_t *in, int n, int32_t *out) {
  // wave w of a chunk covers values base + w 1024 + i 64 + lane (i < 16): every load and store
  // is one coalesced 256-byte row per wave; the 16 rows are scanned in order with a running
  // carry. Every value of a chunk is read before the barrier that precedes its stores (in may
  // be out).
  constexpr int IPT = 16;
  __shared__ int wsum[16];
  __shared__ int carry_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < n; base += 1024 * IPT) {
    const int wb = base + wave * 64 * IPT;
    int v[IPT];
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int idx = wb + i * 64 + lane;
      v[i] = idx < n ? in[idx] : 0;
    }
    int ex[IPT], run = 0;
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      int tot;
      ex[i] = run + wave_excl_scan(v[i], &tot);
      run += tot;
    }
    if (lane == 0) wsum[wave] = run;
    __syncthreads();
    int wpre = 0, ctot = 0;
    for (int i = 0; i < 16; ++i) {
      if (i < wave) wpre += wsum[i];
      ctot += wsum[i];
    }
    const int c = carry_s + wpre;
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int idx = wb + i * 64 + lane;
      if (idx < n) out[idx] = c + ex[i];
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
                                                  int32_t *__restrict__ col, float *__restrict__ hval, size_t nzcap) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= h.rows || (size_t)row_ptr[h.rows] > nzcap) return;   // entries beyond the workspace
  const int lane = lane_id();
  const int base = row_ptr[t], lim = row_ptr[t + 1];
  const int slot = h.ovf_slot[t];
  const VT *vals = (const VT *)h.vals;
  int n = 0;
  if (slot >= 0) {
    const VT *row = (const VT *)h.ovf_dense + (size_t)slot * h.cols;
    for (int c0 = 0; c0 < h.cols; c0 += 64 * kDenseBatch) {
      float v[kDenseBatch];
      dense_batch<VT>(row, h.cols, c0 + lane, v);
#pragma unroll
      for (int u = 0; u < kDenseBatch; ++u) {
        const int j = c0 + u * 64 + lane;
        const bool nz = v[u] != 0.f;
        const uint64_t m = ballot64(nz);
        const int pos = base + n + (int)mbcnt64(m);
        if (nz && pos < lim) {
          col[pos] = j;
          hval[pos] = v[u];
        }
        n += __popcll(m);
      }
    }
  } else if (h.n_t == 1) {
    // one tile per row (the compact row-ELL): the lanes take the slots
    const int m = min(h.counts[t], h.S);
    const size_t sb = (size_t)t * h.S;
    for (int s = lane; s < m; s += 64) {
      const int pos = base + s;
      if (pos < lim) {
        col[pos] = h.col_idx[sb + s];
        hval[pos] = Elem<VT>::load(vals, sb + s);
      }
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

// The 16-byte dot product of a chunk of dy with a chunk of a W2 row, fp32 accumulation
// (bf16 pairs through v_dot2_f32_bf16).
template <typename T>
TW_DEV float dot16(const uint4 &x, const uint4 &y) {
  float acc = 0.f;
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
}

// part[c][e] = dy[t][chunk c] . w2[col[e]][chunk c] for the entries e of token t. Block b
// runs on XCD b % 8 with chunk b % 8 + 8 * ((b / 8) / ntb) and token block (b / 8) % ntb of
// 16 tokens (taken in the order perm), one per 16-lane group; lane l holds 16 bytes of
// dy[t]. Per round the group
// loads its next 16 columns (coalesced), broadcasts them, issues the 16 W2 row loads, and
// the 16 per-lane dot products are summed across the group so that lane l stores entry l
// (a coalesced 64-byte store per round).
template <typename T>
__global__ __launch_bounds__(256) void k_sddmm_part(int T_rows, int d, int nchunk, int ntb, const T *__restrict__ dy,
                                                    const T *__restrict__ w2, const int32_t *__restrict__ row_ptr,
                                                    const int32_t *__restrict__ perm,
                                                    const int32_t *__restrict__ col, size_t nz,
                                                    float *__restrict__ part) {
  constexpr int E = Vec16<T>::N;
  constexpr int CW = 16 * E;
  const int b = blockIdx.x, xcd = b & 7, i = b >> 3;
  const int c = xcd + 8 * (i / ntb), tb = i % ntb;
  if (c >= nchunk || (size_t)row_ptr[T_rows] > nz) return;     // nz: the workspace's entry capacity
  const int lane = lane_id(), g = lane >> 4, gl = lane & 15;
  const int ti = tb * 16 + (threadIdx.x >> 6) * 4 + g;
  const int t = ti < T_rows ? perm[ti] : T_rows;
  const int colo = c * CW + gl * E;
  const bool cv = colo < d;
  int start = 0, n = 0;
  if (t < T_rows) {
    start = row_ptr[t];
    n = row_ptr[t + 1] - start;
  }
  int nw = max(n, __shfl_xor(n, 16, 64));
  nw = max(nw, __shfl_xor(nw, 32, 64));
  const uint4 a = (t < T_rows && cv) ? *(const uint4 *)(dy + (size_t)t * d + colo) : make_uint4(0, 0, 0, 0);
  const int32_t *cp = col + start;
  float *out = part + (size_t)c * nz + start;
  int jn = gl < n ? cp[gl] : 0;
  for (int base = 0; base < nw; base += 16) {
    const int jq = jn;
    if (base + 16 < nw) jn = base + 16 + gl < n ? cp[base + 16 + gl] : 0;
    uint4 raw[16];
    static_for<16>([&](auto J) {
      constexpr int j = decltype(J)::value;
      const uint32_t jj = row_bcast<j>((uint32_t)jq);
      raw[j] = make_uint4(0, 0, 0, 0);
      if (base + j < n && cv) raw[j] = *(const uint4 *)(w2 + (size_t)jj * d + colo);
    });
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) v[j] = dot16<T>(a, raw[j]);
    const float tot = group16_transpose_sum(v, gl);
    if (base + gl < n) out[base + gl] = tot;
  }
}

// dz[e] = (sum over chunks c of part[c][e], in chunk order) + l1, stored as (col[e], dz),
// for the row_ptr[T] entries in use (grid-stride over a fixed grid). Each thread has the loads
// of 16 chunks in flight (clamped to valid addresses) before it adds them in order.
__global__ __launch_bounds__(256) void k_sddmm_sum(int T_rows, const int32_t *__restrict__ row_ptr, size_t nz,
                                                   int nchunk, const float *__restrict__ part,
                                                   const int32_t *__restrict__ col, float l1,
                                                   uint2 *__restrict__ dz) {
  const size_t total = (size_t)row_ptr[T_rows];
  if (total > nz) return;
  for (size_t e = (size_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (size_t)gridDim.x * 256) {
    float s = 0.f;
    for (int c0 = 0; c0 < nchunk; c0 += 16) {
      float v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = part[(size_t)min(c0 + j, nchunk - 1) * nz + e];
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (c0 + j < nchunk) s += v[j];
    }
    dz[e] = make_uint2((uint32_t)col[e], __float_as_uint(s + l1));
  }
}

// --------------------------------------------------------- list order for the gathers

// perm = the R lists ordered by length, longest first, in 64 buckets of 16 entries (the
// gathers walk a list 16 entries per round, so the four lists of a wave then take the same
// number of rounds; lists of 1008 entries and more share the first bucket and start
// first). The order inside a bucket depends on atomic arrival order; every output row is
// still summed by one group in list order, so results do not depend on it. One workgroup.
__global__ __launch_bounds__(1024) void k_order_by_len(int R, const int32_t *__restrict__ ptr, int32_t *__restrict__ perm) {
  constexpr int NB = 64;
  __shared__ int hist[NB];
  const int tid = threadIdx.x;
  if (tid < NB) hist[tid] = 0;
  __syncthreads();
  auto bucket = [&](int r) { return NB - 1 - min(NB - 1, (ptr[r + 1] - ptr[r]) >> 4); };
  for (int r = tid; r < R; r += 1024) atomicAdd(&hist[bucket(r)], 1);
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int b = 0; b < NB; ++b) {
      const int c = hist[b];
      hist[b] = run;
      run += c;
    }
  }
  __syncthreads();
  for (int r = tid; r < R; r += 1024) perm[atomicAdd(&hist[bucket(r)], 1)] = r;
}

// ------------------------------------------------------------------ 4/6. gathers

// out[r][chunk] = sum over the pairs (i, v) of list r of v * M[i][chunk], lists r given by
// CSR offsets ptr. Block b runs on XCD b % 8 and takes chunk b % 8 + 8 * ((b / 8) / ntb)
// and row block (b / 8) % ntb of 16 lists (chunks congruent mod 8 stay on one XCD, whose L2
// then holds only those column slices of M). Rows without entries are written as zero.
// rowsum (optional): rowsum[r] = sum of list r's values, written by the chunk-0 blocks.
// Rows are taken in the order perm (k_order_by_len).
template <typename MT>
__global__ __launch_bounds__(256) void k_gather_csr4(int R, int d, int nchunk, int ntb,
                                                     const int32_t *__restrict__ ptr,
                                                     const int32_t *__restrict__ perm,
                                                     const uint2 *__restrict__ pairs, const MT *__restrict__ M,
                                                     float *__restrict__ out, float *__restrict__ rowsum,
                                                     const int32_t *__restrict__ total, size_t nzcap) {
  constexpr int E = Vec16<MT>::N;
  constexpr int CW = 16 * E;
  const int b = blockIdx.x, xcd = b & 7, i = b >> 3;
  const int c = xcd + 8 * (i / ntb), rb = i % ntb;
  if (c >= nchunk || (size_t)*total > nzcap) return;
  const int lane = lane_id(), g = lane >> 4, gl = lane & 15;
  const int ri = rb * 16 + (threadIdx.x >> 6) * 4 + g;
  const int r = ri < R ? perm[ri] : R;
  const int col = c * CW + gl * E;
  const bool cv = col < d;
  int start = 0, n = 0;
  if (r < R) {
    start = ptr[r];
    n = ptr[r + 1] - start;
  }
  int nw = max(n, __shfl_xor(n, 16, 64));
  nw = max(nw, __shfl_xor(nw, 32, 64));
  float acc[E];
#pragma unroll
  for (int q = 0; q < E; ++q) acc[q] = 0.f;
  const float vs = gather_list16<MT>(pairs + start, n, nw, M, d, col, cv, acc);
  if (r < R && cv) {
    const size_t o = (size_t)r * d + col;
    store_out_nt<float, E>(out, o, acc);
  }
  if (rowsum && c == 0) {                        // uniform for the block
    const float sv = group16_sum(vs);
    if (gl == 0 && r < R) rowsum[r] = sv;
  }
}

// ------------------------------------------------------------------- 5. CSR -> CSC

// Per 32-token block b: mask[b][j] bit (t - 32 b) set iff token t has unit j active;
// cnt[b][j] = popcount, also added to tot[j] (integer atomics: the sum is exact and
// independent of order). LDS holds the block's masks for all units.
__global__ __launch_bounds__(256) void k_col_mask(int T_rows, int f, const int32_t *__restrict__ row_ptr,
                                                  const int32_t *__restrict__ col, uint32_t *__restrict__ mask,
                                                  int32_t *__restrict__ cnt, int32_t *__restrict__ tot, size_t nzcap) {
  extern __shared__ uint32_t lm[];
  const int b = blockIdx.x, tid = threadIdx.x;
  if ((size_t)row_ptr[T_rows] > nzcap) return;
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
    if (m) atomicAdd(&tot[j], __popc(m));
  }
}

// cnt[b][j] <- col_ptr[j] + sum_{b' < b} cnt[b'][j]  (first position of block b in unit j).
// A workgroup owns 64 units; its 16 waves split the NB blocks into consecutive ranges, sum
// their range, exchange the range sums through LDS, and rewrite their range with offsets.
__global__ __launch_bounds__(1024) void k_col_off(int NB, int f, const int32_t *__restrict__ col_ptr,
                                                  int32_t *__restrict__ cnt) {
  __shared__ int part[16][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = blockIdx.x * 64 + lane;
  const int per = (NB + 15) / 16;
  const int b0 = min(NB, w * per), b1 = min(NB, b0 + per);
  int sum = 0;
  if (j < f)
    for (int b = b0; b < b1; ++b) sum += cnt[(size_t)b * f + j];
  part[w][lane] = sum;
  __syncthreads();
  if (j >= f) return;
  int run = col_ptr[j];
  for (int k = 0; k < w; ++k) run += part[k][lane];
  for (int b = b0; b < b1; ++b) {
    const int c = cnt[(size_t)b * f + j];
    cnt[(size_t)b * f + j] = run;
    run += c;
  }
}

constexpr int kCscBatch = 4;

// Every CSR entry (t, j) goes to position off[t/32][j] + popc(mask[t/32][j] & lower bits)
// of the unit-major lists: (t, h) for dw2, (t, dz) for dw1t.
__global__ __launch_bounds__(256) void k_csc_fill(int T_rows, int f, const int32_t *__restrict__ row_ptr,
                                                  const int32_t *__restrict__ col, const float *__restrict__ hval,
                                                  const uint2 *__restrict__ dz, const uint32_t *__restrict__ mask,
                                                  const int32_t *__restrict__ off, uint2 *__restrict__ th,
                                                  uint2 *__restrict__ tdz, size_t nzcap) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T_rows || (size_t)row_ptr[T_rows] > nzcap) return;
  const int lane = lane_id();
  const int b = t >> 5, bit = t & 31;
  const uint32_t lower = (1u << bit) - 1u;
  const int s = row_ptr[t], e = row_ptr[t + 1];
  // kCscBatch rounds of 64 entries: their loads (clamped to entry s) are all issued before
  // the scattered stores, which would otherwise hold back the next round's loads
  for (int k0 = s; k0 < e; k0 += 64 * kCscBatch) {
    int j[kCscBatch];
    uint32_t hv[kCscBatch], dv[kCscBatch];
#pragma unroll
    for (int u = 0; u < kCscBatch; ++u) {
      const int k = k0 + u * 64 + lane;
      const int kc = k < e ? k : s;
      j[u] = col[kc];
      hv[u] = __float_as_uint(hval[kc]);
      dv[u] = dz[kc].y;
    }
    int pos[kCscBatch];
#pragma unroll
    for (int u = 0; u < kCscBatch; ++u) {
      const size_t bj = (size_t)b * f + j[u];
      pos[u] = off[bj] + __popc(mask[bj] & lower);
    }
#pragma unroll
    for (int u = 0; u < kCscBatch; ++u) {
      if (k0 + u * 64 + lane < e) {
        th[pos[u]] = make_uint2((uint32_t)t, hv[u]);
        tdz[pos[u]] = make_uint2((uint32_t)t, dv[u]);
      }
    }
  }
}

// More overflow rows than backup slots (*ovf_n > cap): the rows beyond the backup kept only
// their first S entries per tile, so their gradients cannot be formed. Or more entries than
// the workspace holds (the kernels after the row scan then did nothing). In both cases every
// output is overwritten with a quiet NaN, so that the condition cannot pass unnoticed;
// otherwise the kernel exits at once (two scalar loads per workgroup).
__global__ __launch_bounds__(256) void k_bwd_poison(const int32_t *__restrict__ ovf_n, int cap,
                                                    const int32_t *__restrict__ total, size_t nzcap, float *dx,
                                                    size_t ndx, float *dw1t, float *dw2, size_t ndw, float *db1,
                                                    size_t ndb) {
  if (*ovf_n <= cap && (size_t)*total <= nzcap) return;
  const float qnan = __uint_as_float(0x7FC00000u);
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < ndw; i += stride) {
    dw1t[i] = qnan;
    dw2[i] = qnan;
    if (i < ndx) dx[i] = qnan;
    if (db1 && i < ndb) db1[i] = qnan;
  }
  for (size_t i = ndw + (size_t)blockIdx.x * 256 + threadIdx.x; i < ndx; i += stride) dx[i] = qnan;
}

__global__ __launch_bounds__(256) void k_fill_zero(int32_t *p, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0;
}

// ------------------------------------------------------------------ host side

static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

static int sddmm_chunks(int d, int bf16) {
  const int cw = bf16 ? 128 : 64;
  return (d + cw - 1) / cw;
}

size_t bwd_entry_capacity(int T, int f, int n_t, int S, int cap) {
  return (size_t)T * n_t * S + (size_t)(cap < T ? cap : T) * f;
}

// Workspace for at most NZ stored entries (slots in use plus nonzeros of the backup rows).
size_t bwd_workspace_bytes(int T, int d, int f, size_t NZ, int bf16) {
  const size_t NB = ((size_t)T + 31) / 32;
  size_t b = 0;
  b += al256(4 * NZ * (size_t)sddmm_chunks(d, bf16));   // SDDMM partial dot products
  b += al256(4 * ((size_t)T + 1));          // row_ptr
  b += 2 * al256(4 * NZ);                   // col, hval
  b += al256(8 * NZ);                       // (col, dz) pairs
  b += 2 * al256(4 * NB * f);               // mask, cnt/off
  b += al256(4 * ((size_t)f + 1));          // col_ptr
  b += 2 * al256(8 * NZ);                   // (token, h), (token, dz) pairs
  b += al256(4 * (size_t)T) + al256(4 * (size_t)f);   // list orders
  return b;
}

// The largest entry count up to NZmax whose workspace fits in `bytes` (bytes grows with it);
// SIZE_MAX if not even an empty one fits.
size_t bwd_fit_entries(int T, int d, int f, size_t bytes, size_t NZmax, int bf16) {
  if (bwd_workspace_bytes(T, d, f, 0, bf16) > bytes) return SIZE_MAX;
  if (bwd_workspace_bytes(T, d, f, NZmax, bf16) <= bytes) return NZmax;
  size_t lo = 0, hi = NZmax;                // fits(lo), !fits(hi)
  while (hi - lo > 1) {
    const size_t mid = lo + (hi - lo) / 2;
    if (bwd_workspace_bytes(T, d, f, mid, bf16) <= bytes) lo = mid;
    else hi = mid;
  }
  return lo;
}

hipError_t launch_bwd(const BwdArgs &a, hipStream_t s) {
  const TwellIn &h = a.h;
  const int T = h.rows, f = h.cols, d = a.d;
  const size_t NZ = a.nz;                   // entry capacity of the workspace (checked on the device)
  const size_t NB = ((size_t)T + 31) / 32;
  const int nchunk = sddmm_chunks(d, a.bf16);
  char *p = (char *)a.ws;
  auto take = [&](size_t bytes) { char *q = p; p += al256(bytes); return q; };
  float *part = (float *)take(4 * NZ * (size_t)nchunk);
  int32_t *row_ptr = (int32_t *)take(4 * ((size_t)T + 1));
  int32_t *col = (int32_t *)take(4 * NZ);
  float *hval = (float *)take(4 * NZ);
  uint2 *dz = (uint2 *)take(8 * NZ);
  uint32_t *mask = (uint32_t *)take(4 * NB * f);
  int32_t *cnt = (int32_t *)take(4 * NB * f);
  int32_t *col_ptr = (int32_t *)take(4 * ((size_t)f + 1));
  uint2 *th = (uint2 *)take(8 * NZ);
  uint2 *tdz = (uint2 *)take(8 * NZ);
  int32_t *perm_t = (int32_t *)take(4 * (size_t)T);
  int32_t *perm_u = (int32_t *)take(4 * (size_t)f);
  const dim3 rows4((T + 3) / 4);
  if (T > 0) {
    if (h.val_bf16) hipLaunchKernelGGL(k_row_nnz<uint16_t>, rows4, dim3(256), 0, s, h, row_ptr, col_ptr, f);
    else hipLaunchKernelGGL(k_row_nnz<float>, rows4, dim3(256), 0, s, h, row_ptr, col_ptr, f);
  } else {
    hipLaunchKernelGGL(k_fill_zero, dim3((f + 256) / 256), dim3(256), 0, s, col_ptr, f + 1);
  }
  hipLaunchKernelGGL(k_scan_excl, dim3(1), dim3(1024), 0, s, row_ptr, T, row_ptr);
  if (T > 0) {
    if (h.val_bf16) hipLaunchKernelGGL(k_csr_fill<uint16_t>, rows4, dim3(256), 0, s, h, row_ptr, col, hval, NZ);
    else hipLaunchKernelGGL(k_csr_fill<float>, rows4, dim3(256), 0, s, h, row_ptr, col, hval, NZ);
    hipLaunchKernelGGL(k_order_by_len, dim3(1), dim3(1024), 0, s, T, row_ptr, perm_t);
    const int ntb = (T + 15) / 16;
    const size_t grid = 8 * (size_t)ntb * ((nchunk + 7) / 8);
    if (a.bf16) hipLaunchKernelGGL((k_sddmm_part<uint16_t>), dim3((unsigned)grid), dim3(256), 0, s, T, d, nchunk, ntb,
                                   (const uint16_t *)a.dy, (const uint16_t *)a.w2, row_ptr, perm_t, col, NZ, part);
    else hipLaunchKernelGGL((k_sddmm_part<float>), dim3((unsigned)grid), dim3(256), 0, s, T, d, nchunk, ntb,
                            (const float *)a.dy, (const float *)a.w2, row_ptr, perm_t, col, NZ, part);
    const unsigned sum_grid = (unsigned)std::max<size_t>(1, std::min<size_t>((NZ + 255) / 256, 4096));
    hipLaunchKernelGGL(k_sddmm_sum, dim3(sum_grid), dim3(256), 0, s, T, row_ptr, NZ, nchunk, part, col, a.l1, dz);
  }
  auto gather = [&](int R, const int32_t *ptr, const int32_t *perm, const uint2 *pairs, const void *M, float *out,
                    float *rowsum) {
    const int ntb = (R + 15) / 16;
    const size_t grid = 8 * (size_t)ntb * ((nchunk + 7) / 8);
    if (a.bf16) hipLaunchKernelGGL((k_gather_csr4<uint16_t>), dim3((unsigned)grid), dim3(256), 0, s, R, d, nchunk, ntb,
                                   ptr, perm, pairs, (const uint16_t *)M, out, rowsum, row_ptr + T, NZ);
    else hipLaunchKernelGGL((k_gather_csr4<float>), dim3((unsigned)grid), dim3(256), 0, s, R, d, nchunk, ntb, ptr,
                            perm, pairs, (const float *)M, out, rowsum, row_ptr + T, NZ);
  };
  // dx = dz . w1t
  if (T > 0) gather(T, row_ptr, perm_t, dz, a.w1t, a.dx, nullptr);
  // CSC
  if (T > 0)
    hipLaunchKernelGGL(k_col_mask, dim3((unsigned)NB), dim3(256), (size_t)f * 4, s, T, f, row_ptr, col, mask, cnt,
                       col_ptr, NZ);
  hipLaunchKernelGGL(k_scan_excl, dim3(1), dim3(1024), 0, s, col_ptr, f, col_ptr);
  if (T > 0) {
    hipLaunchKernelGGL(k_col_off, dim3((f + 63) / 64), dim3(1024), 0, s, (int)NB, f, col_ptr, cnt);
    hipLaunchKernelGGL(k_csc_fill, rows4, dim3(256), 0, s, T, f, row_ptr, col, hval, dz, mask, cnt, th, tdz, NZ);
  }
  // dw2 = h^T dy, dw1t = dz^T x (every unit row written, zero if it has no entry), db1
  hipLaunchKernelGGL(k_order_by_len, dim3(1), dim3(1024), 0, s, f, col_ptr, perm_u);
  gather(f, col_ptr, perm_u, th, a.dy, a.dw2, nullptr);
  gather(f, col_ptr, perm_u, tdz, a.x, a.dw1t, a.db1);
  hipLaunchKernelGGL(k_bwd_poison, dim3(256), dim3(256), 0, s, h.ovf_n, a.cap, row_ptr + T, NZ, a.dx, (size_t)T * d,
                     a.dw1t, a.dw2, (size_t)f * d, a.db1, (size_t)f);
  return hipGetLastError();
}

}  // namespace tw
