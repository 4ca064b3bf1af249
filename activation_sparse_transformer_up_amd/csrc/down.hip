// Sparse down projection: y[t] = sum over the active units j of token t of h[t, j] * w2[j].
//
// "Sparser, Faster, Lighter Transformer Language Models", section "2. Metodologia", block
// "Kernels de Inferência": the down projection iterates over the active units only, so the
// rows of W2 of inactive units are never read. Accumulation is fp32.
//
// First each row's TwELL slots are compacted once into a contiguous list of
// (column, value) pairs (k_row_list): the gathers below are spread over all XCDs by column
// chunk, and reading the sparse slot blocks from every XCD would fetch whole cache lines
// for a handful of entries. A chunk is 16 lanes x 16 bytes of a W2 row (128 bf16 or 64
// fp32 columns), so one vector load instruction fetches four different W2 rows. Three
// work decompositions, chosen by the number of tokens:
//   many tokens (k_down_rows4): a wave owns four tokens of one chunk, one per 16-lane
//     group; each group walks its own list, so no cross-lane reduction is needed. The
//     rate is set by the texture-address path of each CU (one 16-byte load per lane and
//     W2 row), which this keeps busiest.
//   medium (k_twell_down): a wave owns one (token, chunk); its four groups take every
//     fourth list entry and are summed at the end.
//   few tokens (k_down_split): a 4-wave workgroup owns one (token, chunk), so sixteen
//     groups split the list and all W2 row loads of a token leave in one round; this is
//     the HBM-latency-bound decode case.
// Overflow rows take their entries from the dense backup row.
//
// XCD-aware order: workgroup b runs on XCD b % 8 (round-robin dispatch), and all chunks
// handled by one XCD are congruent mod 8, so that XCD's L2 only ever holds its own column
// slices of W2; a chunk is finished for all tokens before the XCD moves to its next one.
#include "common.h"
#include "gather.h"
#include "launch.h"
#include "rows.h"

namespace tw {

template <typename VT> TW_DEV float ldv(const VT *p, size_t i) { return Elem<VT>::load(p, i); }

// The compact list of every row (row_list_wave), rpw rows per workgroup.
template <typename VT>
__global__ __launch_bounds__(1024) void k_row_list(TwellIn h, int rpw) {
  const int w = threadIdx.x >> 6;
  if (w >= rpw) return;
  const int t = blockIdx.x * rpw + w;
  if (t < h.rows) row_list_wave<VT>(h, t);
}

// The finish step of the fused forward in one launch: workgroup 0 runs the overflow scan
// (ovf_scan_block), the others build the row lists, which do not depend on the scan
// (consumers tell overflow rows by ovf_slot).
template <typename VT>
__global__ __launch_bounds__(1024) void k_lists_scan(TwellIn h, const uint32_t *__restrict__ bits, int words,
                                                     int32_t *ovf_n, int32_t *ovf_rows, int32_t *ovf_slot, int rpw) {
  if (blockIdx.x == 0) {
    ovf_scan_block(bits, h.n_t, words, h.rows, h.cap, ovf_n, ovf_rows, ovf_slot);
    return;
  }
  const int w = threadIdx.x >> 6;
  if (w >= rpw) return;
  const int t = (blockIdx.x - 1) * rpw + w;
  if (t < h.rows) row_list_wave<VT>(h, t);
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
  const __amdgpu_buffer_rsrc_t rs = rows_rsrc(w2, rows_bytes<WT>(h.cols, d));
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
        if (cv) raw[j] = ld16<WT>(rs, p.x * (uint32_t)d + (uint32_t)col);
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

  // the overflow slot and the list length in one round trip
  const int slot0 = h.ovf_slot[t], nnz0 = h.row_nnz[t];
  if (slot0 < 0) {
    const int nnz = list_len(h, nnz0);
    const uint2 *src = h.row_list + (size_t)t * h.n_t * h.S;
    for (int base = 0; base < nnz; base += 64) {
      const int n = min(64, nnz - base);
      if (lane < n) lst[lane] = src[base + lane];
      __syncthreads();
      consume(n);
      __syncthreads();
    }
  } else {
    const VT *row = (const VT *)h.ovf_dense + (size_t)slot0 * h.cols;
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
    store_out_nt<YT, E>(y, o, acc);
  }
}


TW_DEV void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Backup row r of the overflow list, one chunk, by one wave: the dense row is read kBkSteps
// steps of 64 columns at a time (every load before any use; addresses clamped into the row),
// its nonzeros are appended to this wave's LDS list (CAP entries) in column order, and the list
// is gathered whenever it might not take another full step, and at the end: the four groups
// take every fourth entry, 16 entries per round. The group sums are added and written by
// group 0. A row is then a few round trips per kBkSteps steps and per 16 entries, instead of
// one per step for the row and one per step with a nonzero for W2.
constexpr int kBkSteps = 8, kBkList = 192;            // list entries per wave

template <typename WT, typename VT, typename YT, int CAP>
TW_DEV void backup_row(const TwellIn &h, const WT *__restrict__ w2, int d, YT *__restrict__ y, int r, int c,
                       uint2 *lst) {
  static_assert(CAP >= 128, "a flush must leave room for a full step");
  constexpr int E = Vec16<WT>::N;
  constexpr int CW = 16 * E;
  const int lane = lane_id(), g = lane >> 4, gl = lane & 15;
  const int col = c * CW + gl * E;
  const bool cv = col < d;
  const int t = h.ovf_rows[r];
  const int cols = h.cols;
  const VT *row = (const VT *)h.ovf_dense + (size_t)r * cols;
  const __amdgpu_buffer_rsrc_t rs = rows_rsrc(w2, rows_bytes<WT>(cols, d));
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  int cnt = 0;                                                 // pending list entries (uniform)
  auto flush = [&]() {
    wave_sync_lds();
    for (int e0 = 0; e0 < cnt; e0 += 16) {
      uint4 raw[4];
      float vv[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int e = e0 + g + 4 * k;
        vv[k] = 0.f;
        raw[k] = make_uint4(0, 0, 0, 0);
        if (e < cnt) {
          const uint2 p = lst[e];
          vv[k] = __uint_as_float(p.y);
          if (cv) raw[k] = ld16<WT>(rs, p.x * (uint32_t)d + (uint32_t)col);
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) fma16<WT, E>(acc, vv[k], raw[k]);
    }
    wave_sync_lds();
    cnt = 0;
  };
  for (int c0 = 0; c0 < cols; c0 += 64 * kBkSteps) {
    float v[kBkSteps];
#pragma unroll
    for (int u = 0; u < kBkSteps; ++u) {
      const int j = c0 + u * 64 + lane;
      const float x = ldv(row, j < cols ? j : cols - 1);
      v[u] = j < cols ? x : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kBkSteps; ++u) {
      const bool nz = v[u] != 0.f;
      const uint64_t m = ballot64(nz);
      if (m == 0) continue;                                    // uniform
      if (cnt > CAP - 64) flush();                             // uniform
      if (nz) lst[cnt + (int)mbcnt64(m)] = make_uint2((uint32_t)(c0 + u * 64 + lane), __float_as_uint(v[u]));
      cnt += (int)__popcll(m);
    }
  }
  if (cnt > 0) flush();
#pragma unroll
  for (int q = 0; q < E; ++q) {
    acc[q] += __shfl_xor(acc[q], 16, 64);
    acc[q] += __shfl_xor(acc[q], 32, 64);
  }
  if (g == 0 && cv) {
    const size_t o = (size_t)t * d + col;
    store_out_nt<YT, E>(y, o, acc);
  }
}

// Many tokens. Workgroups [0, nmain): block b runs on XCD b % 8 and takes chunk
// c = b % 8 + 8 * ((b / 8) / ntb) and token block (b / 8) % ntb of 16 tokens; wave w, group
// g owns token 16 * block + 4 w + g and walks its list with gather_list16.
// Workgroups [nmain, ...): the backup rows, one (row, chunk) per wave.
template <typename WT, typename VT, typename YT>
__global__ __launch_bounds__(256) void k_down_rows4(TwellIn h, const WT *__restrict__ w2, int d,
                                                    YT *__restrict__ y, int nchunk, int ntb, int nmain) {
  __shared__ uint2 lst[4][kBkList];
  constexpr int E = Vec16<WT>::N;
  constexpr int CW = 16 * E;
  const int b = blockIdx.x;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  if (b >= nmain) {
    const int i = b - nmain;
    const int c = i % nchunk, r = (i / nchunk) * 4 + wave;
    if (r >= min(*h.ovf_n, h.cap)) return;               // wave-uniform
    backup_row<WT, VT, YT, kBkList>(h, w2, d, y, r, c, lst[wave]);
    return;
  }
  const int xcd = b & 7, i = b >> 3;
  const int c = xcd + 8 * (i / ntb), tb = i % ntb;
  if (c >= nchunk) return;
  const int g = lane >> 4, gl = lane & 15;
  const int t = tb * 16 + wave * 4 + g;
  const int col = c * CW + gl * E;
  const bool cv = col < d;
  const int tc = t < h.rows ? t : 0;                       // slot and length in one round trip
  const int slot0 = h.ovf_slot[tc], nnz0 = h.row_nnz[tc];
  const bool normal = t < h.rows && slot0 < 0;
  const int nnz = normal ? list_len(h, nnz0) : 0;
  int n = max(nnz, __shfl_xor(nnz, 16, 64));
  n = max(n, __shfl_xor(n, 32, 64));
  const uint2 *lp = h.row_list + (size_t)(t < h.rows ? t : 0) * h.n_t * h.S;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  gather_list16<WT>(lp, nnz, n, w2, d, col, cv, acc, rows_bytes<WT>(h.cols, d));
  if (normal && t < h.rows && cv) {
    const size_t o = (size_t)t * d + col;
    store_out_nt<YT, E>(y, o, acc);
  }
}

// Few tokens: one (token, chunk) per workgroup of 4 waves = 16 groups. The list window of
// up to 256 entries is read into LDS together with the count (speculatively: the scratch
// row always holds n_t * S entries); group G takes entries G, G + 16, ..., so its (at most
// 16) W2 row loads leave at once. Group sums are added across lanes and then across waves.
template <typename WT, typename VT, typename YT>
__global__ __launch_bounds__(256) void k_down_split(TwellIn h, const WT *__restrict__ w2, int d,
                                                    YT *__restrict__ y, int nchunk) {
  constexpr int LW = 256, NG = 16, PER = LW / NG;
  constexpr int E = Vec16<WT>::N;
  constexpr int CW = 16 * E;
  __shared__ uint2 lst[LW];
  __shared__ float red[3][16 * E];
  const int T = h.rows;
  const int b = blockIdx.x, xcd = b & 7, i = b >> 3;
  const int c = xcd + 8 * (i / T), t = i % T;
  if (c >= nchunk) return;                                  // uniform for the workgroup
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = wave * 4 + (lane >> 4), gl = lane & 15;
  const int col = c * CW + gl * E;
  const bool cv = col < d;
  const __amdgpu_buffer_rsrc_t rs = rows_rsrc(w2, rows_bytes<WT>(h.cols, d));
  const int cap = h.n_t * h.S;
  const uint2 *src = h.row_list + (size_t)t * cap;
  if (tid < LW) lst[tid] = tid < cap ? src[tid] : make_uint2(0, 0);
  const int slot = h.ovf_slot[t], nnz = list_len(h, h.row_nnz[t]);   // one round trip with the list
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  if (slot >= 0) {                                          // backup row: one wave does it
    if (wave == 0) backup_row<WT, VT, YT, LW>(h, w2, d, y, slot, c, lst);
    return;
  }
  __syncthreads();
  for (int base = 0; base < nnz; base += LW) {
    if (base > 0) {
      __syncthreads();
      if (tid < LW) lst[tid] = base + tid < cap ? src[base + tid] : make_uint2(0, 0);
      __syncthreads();
    }
    const int n = min(LW, nnz - base);
    uint4 raw[PER];
    float vv[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = G + NG * j;
      vv[j] = 0.f;
      raw[j] = make_uint4(0, 0, 0, 0);
      if (e < n) {
        const uint2 p = lst[e];
        vv[j] = __uint_as_float(p.y);
        if (cv) raw[j] = ld16<WT>(rs, p.x * (uint32_t)d + (uint32_t)col);
      }
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) fma16<WT, E>(acc, vv[j], raw[j]);
  }
#pragma unroll
  for (int q = 0; q < E; ++q) {
    acc[q] += __shfl_xor(acc[q], 16, 64);
    acc[q] += __shfl_xor(acc[q], 32, 64);
  }
  if (wave > 0 && lane < 16)
#pragma unroll
    for (int q = 0; q < E; ++q) red[wave - 1][lane * E + q] = acc[q];
  __syncthreads();
  if (wave == 0 && lane < 16 && cv) {
#pragma unroll
    for (int w = 0; w < 3; ++w)
#pragma unroll
      for (int q = 0; q < E; ++q) acc[q] += red[w][lane * E + q];
    const size_t o = (size_t)t * d + col;
    store_out_nt<YT, E>(y, o, acc);
  }
}

// Medium token counts at wide rows: a workgroup of NW waves owns one (token, chunk of 64
// lanes x 16 bytes: 512 bf16 or 256 fp32 columns), so every W2 row piece is one contiguous
// 1 KB wave load. Chunk c runs on XCD c % 8 as in the other decompositions. Wave w takes
// entries [NW PE k + PE w, NW PE k + PE w + PE) of the token's list, k = 0, 1, ...: lanes
// 0 .. PE-1 load the pairs (the first ones speculatively with the count, the next round's
// while the rows are in flight) and readlane broadcasts them, so the row addresses are
// scalar. The wave sums are added in wave order through LDS. A backup row is taken by the
// first four waves as four 16-lane chunks (backup_row).
constexpr int kWideNW = 8, kWidePE = 4;                 // measured at c3 T = 64, d = 4096

template <typename WT, typename VT, typename YT, int NW, int PE>
__global__ __launch_bounds__(64 * NW) void k_down_wide(TwellIn h, const WT *__restrict__ w2, int d,
                                                        YT *__restrict__ y, int nchunk) {
  constexpr int E = Vec16<WT>::N;
  constexpr int CW = 64 * E;
  constexpr int RW = NW * PE;                               // entries per round
  static_assert(NW >= 4 && PE <= 64, "shape");
  __shared__ uint2 lst[4][kBkList];
  __shared__ float red[NW - 1][64 * E];
  const int T = h.rows;
  const int b = blockIdx.x, xcd = b & 7, i = b >> 3;
  const int c = xcd + 8 * (i / T), t = i % T;
  if (c >= nchunk) return;                                  // uniform for the workgroup
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cap = h.n_t * h.S;
  const uint2 *src = h.row_list + (size_t)t * cap;
  const int e0 = PE * wave + lane;
  uint2 pn = (lane < PE && e0 < cap) ? src[e0] : make_uint2(0, 0);
  const int slot = h.ovf_slot[t], nnz = list_len(h, h.row_nnz[t]);   // one round trip with the list
  if (slot >= 0) {
    if (wave < 4) {
      const int cn = 4 * c + wave;                          // this wave's 16-lane chunk
      if (cn * 16 * E < d) backup_row<WT, VT, YT, kBkList>(h, w2, d, y, slot, cn, lst[wave]);
    }
    return;
  }
  const int col = c * CW + lane * E;
  const bool cv = col < d;
  const __amdgpu_buffer_rsrc_t rs = rows_rsrc(w2, rows_bytes<WT>(h.cols, d));
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  for (int base = PE * wave; base < nnz; base += RW) {
    const uint2 q = pn;
    const int nb = base + RW;
    if (nb < nnz) pn = (lane < PE && nb + lane < nnz) ? src[nb + lane] : make_uint2(0, 0);
    uint4 raw[PE];
    float vv[PE];
    static_for<PE>([&](auto J) {
      constexpr int j = decltype(J)::value;
      const uint32_t ij = (uint32_t)__builtin_amdgcn_readlane((int)q.x, j);
      const float vj = __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)q.y, j));
      const bool ok = base + j < nnz;
      vv[j] = ok ? vj : 0.f;
      raw[j] = make_uint4(0, 0, 0, 0);
      if (ok && cv) raw[j] = ld16<WT>(rs, ij * (uint32_t)d + (uint32_t)col);
    });
#pragma unroll
    for (int j = 0; j < PE; ++j) fma16<WT, E>(acc, vv[j], raw[j]);
  }
  if (wave > 0)
#pragma unroll
    for (int q = 0; q < E; ++q) red[wave - 1][lane * E + q] = acc[q];
  __syncthreads();
  if (wave == 0 && cv) {
#pragma unroll
    for (int w = 0; w < NW - 1; ++w)
#pragma unroll
      for (int q = 0; q < E; ++q) acc[q] += red[w][lane * E + q];
    const size_t o = (size_t)t * d + col;
    store_out_nt<YT, E>(y, o, acc);
  }
}

// Token-count thresholds between the three decompositions (measured at d = 2048 and 4096).
constexpr int kRows4MinT = 512, kSplitMaxT = 16;

template <typename WT, typename VT, typename YT>
static hipError_t down_t(const TwellIn &h, const WT *w2, int d, YT *y, bool build_lists, hipStream_t s) {
  constexpr int CW = 16 * Vec16<WT>::N;
  const int nchunk = (d + CW - 1) / CW;
  const size_t per_xcd_chunks = (nchunk + 7) / 8;
  if (h.rows == 0) return hipSuccess;
  if (build_lists) {
    const int rpw = list_rows_per_wg(h.rows);
    hipLaunchKernelGGL((k_row_list<VT>), dim3((h.rows + rpw - 1) / rpw), dim3(1024), 0, s, h, rpw);
  }
  if (h.rows >= kRows4MinT) {
    const int ntb = (h.rows + 15) / 16;
    const size_t nmain = 8 * per_xcd_chunks * (size_t)ntb;
    const size_t nback = (size_t)nchunk * ((h.cap + 3) / 4);
    hipLaunchKernelGGL((k_down_rows4<WT, VT, YT>), dim3((unsigned)(nmain + nback)), dim3(256), 0, s, h, w2, d, y,
                       nchunk, ntb, (int)nmain);
  } else if (h.rows <= kSplitMaxT) {
    hipLaunchKernelGGL((k_down_split<WT, VT, YT>), dim3((unsigned)(8 * per_xcd_chunks * h.rows)), dim3(256), 0, s,
                       h, w2, d, y, nchunk);
  } else if ((d + 64 * Vec16<WT>::N - 1) / (64 * Vec16<WT>::N) >= 8) {
    const int nwide = (d + 64 * Vec16<WT>::N - 1) / (64 * Vec16<WT>::N);
    hipLaunchKernelGGL((k_down_wide<WT, VT, YT, kWideNW, kWidePE>), dim3((unsigned)(8 * ((nwide + 7) / 8) * h.rows)),
                       dim3(64 * kWideNW), 0, s, h, w2, d, y, nwide);
  } else {
    hipLaunchKernelGGL((k_twell_down<WT, VT, YT>), dim3((unsigned)(8 * per_xcd_chunks * h.rows)), dim3(64), 0, s,
                       h, w2, d, y, nchunk);
  }
  return hipGetLastError();
}

hipError_t launch_twell_down(const TwellIn &h, const void *w2, int w_bf16, int d, void *y, int y_bf16,
                             bool build_lists, hipStream_t s) {
  if (w_bf16) {
    const uint16_t *w = (const uint16_t *)w2;
    if (h.val_bf16) {
      if (y_bf16) return down_t<uint16_t, uint16_t, uint16_t>(h, w, d, (uint16_t *)y, build_lists, s);
      return down_t<uint16_t, uint16_t, float>(h, w, d, (float *)y, build_lists, s);
    }
    if (y_bf16) return down_t<uint16_t, float, uint16_t>(h, w, d, (uint16_t *)y, build_lists, s);
    return down_t<uint16_t, float, float>(h, w, d, (float *)y, build_lists, s);
  }
  const float *w = (const float *)w2;
  if (h.val_bf16) {
    if (y_bf16) return down_t<float, uint16_t, uint16_t>(h, w, d, (uint16_t *)y, build_lists, s);
    return down_t<float, uint16_t, float>(h, w, d, (float *)y, build_lists, s);
  }
  if (y_bf16) return down_t<float, float, uint16_t>(h, w, d, (uint16_t *)y, build_lists, s);
  return down_t<float, float, float>(h, w, d, (float *)y, build_lists, s);
}

hipError_t launch_lists_scan(const TwellIn &h, const uint32_t *bits, int words, int32_t *ovf_n, int32_t *ovf_rows,
                            int32_t *ovf_slot, hipStream_t s) {
  const int rpw = list_rows_per_wg(h.rows);
  const dim3 grid(1 + (h.rows + rpw - 1) / rpw);
  if (h.val_bf16) hipLaunchKernelGGL((k_lists_scan<uint16_t>), grid, dim3(1024), 0, s, h, bits, words, ovf_n, ovf_rows, ovf_slot, rpw);
  else hipLaunchKernelGGL((k_lists_scan<float>), grid, dim3(1024), 0, s, h, bits, words, ovf_n, ovf_rows, ovf_slot, rpw);
  return hipGetLastError();
}

}  // namespace tw
