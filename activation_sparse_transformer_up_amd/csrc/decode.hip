// The forward of up to 16 tokens after the W1 stream, in one launch.
//
// "Sparser, Faster, Lighter Transformer Language Models", section "2. Metodologia": the
// TwELL of h = ReLU(x W1 + b1) (block "Formato de Dados TwELL") and y = h W2 over the
// nonzeros of h only, with rows that overflow the slot budget kept in a dense backup (block
// "Formato Híbrido para Treinamento"). At decode sizes the up projection's stream kernels
// (gemm.hip) leave the half sums zp[half][t][u] of z = x W1^T in the decode workspace; here
// every (token, 128-column chunk) workgroup of the down projection rebuilds its token's
// active list from them in LDS and multiplies-adds the W2 row pieces of its chunk, and the
// chunk-0 workgroup of each token also writes the token's TwELL. No row lists go through
// memory and no finish kernel runs between the two products.
#include "common.h"
#include "gather.h"
#include "launch.h"
#include "stage.h"

namespace tw {

// A workgroup of kFdThreads threads; a thread holds kFdUPT consecutive units of a segment of
// kFdThreads kFdUPT units (a whole row at d_ff up to 16384: one round trip for its half sums).
constexpr int kFdThreads = 1024, kFdUPT = 16, kFdSeg = kFdThreads * kFdUPT;
// Entries per gather round (as in the split gather, k_down_split) and the waves that gather
// them: group G (16 lanes) of the first kFdGW waves takes entries G, G + 4 kFdGW, ...
constexpr int kFdLW = 256, kFdGW = 8;

// Grid: 8 ceil(nchunk / 8) M workgroups of kFdThreads threads; workgroup b runs on XCD b % 8 and
// takes chunk c = b % 8 + 8 ((b / 8) / M) (CW = 16 E columns, E = 16 bytes of W2 elements) of
// token t = (b / 8) % M, as k_down_split does.
//
// Per segment of units: each thread loads its kFdUPT units' half sums and biases (all loads
// first), marks the active ones (z > -b1, value z - (-b1) as the TwELL stores it, read back
// in the value type) and a block scan of the per-thread counts places the active (unit,
// value) entries, in ascending unit order, after the entries still pending in LDS. Every
// complete round of kFdLW pending entries is gathered at once by the first kFdGW waves (group G
// of 16 lanes takes entries G, G + 4 kFdGW, ..., all row loads issued before the FMAs), and the rest
// moves to the front for the next segment. An overflow row (a tile above S) is gathered the same way from
// all its active units: the products are those of its dense backup row.
//
// The chunk-0 workgroup of each token also writes the token's TwELL: the lanes of a tile
// (W / 16 consecutive lanes) take its count and slot base from the scan (shuffles), store the
// first S active units in ascending column order and pad the rest (-1, +0). The chunk-0
// workgroups then meet on one 64-bit word of the decode workspace, zeroed by the stream
// kernel of the same call (each adds 1 plus its overflow flag at bit 32 + t; one token needs
// no meeting); the last to arrive writes the overflow scan (rank among overflow rows, below
// cap) and the backup rows ReLU(z + b1), and zeroes the word again. The row lists and the
// overflow words are not written (they are library scratch).
template <int W, typename WT, typename VT, typename YT>
__global__ __launch_bounds__(kFdThreads) void k_dec_fused_down(const float *__restrict__ zp, const float *__restrict__ b1,
                                                        int M, int N, TwellOut o, TwellFinish f,
                                                        const WT *__restrict__ w2, int d, YT *__restrict__ y,
                                                        int nchunk) {
  constexpr int E = Vec16<WT>::N, CW = 16 * E, NG = 4 * kFdGW, PER = kFdLW / NG;
  constexpr int L = W / kFdUPT;                                // lanes of a tile
  static_assert(W % kFdUPT == 0 && 64 % L == 0 && kFdSeg % W == 0, "tile lanes");
  __shared__ uint2 lst[kFdLW + kFdSeg];
  __shared__ float red[kFdGW - 1][16 * E];
  __shared__ int wsum[kFdThreads / 64];
  __shared__ int ovf_s, last_s;
  __shared__ int slot_s[16];
  const int b = blockIdx.x, xcd = b & 7, i = b >> 3;
  const int c = xcd + 8 * (i / M), t = i % M;
  if (c >= nchunk) return;                                     // uniform for the workgroup
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bool gatherer = wave < kFdGW;                          // the NG groups of the gather
  const int G = wave * 4 + (lane >> 4), gl = lane & 15;
  const int col = c * CW + gl * E;
  const bool cv = col < d;
  const bool writer = c == 0;
  const __amdgpu_buffer_rsrc_t rs = rows_rsrc(w2, rows_bytes<WT>(N, d));
  const float *z0 = zp + (size_t)t * N, *z1 = zp + ((size_t)M + t) * N;
  const int S = o.S, n_t = o.n_t;
  if (tid == 0) ovf_s = 0;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;

  // one gather round over lst[base .. base + n) (the first four waves)
  auto round = [&](int base, int n) {
    if (!gatherer) return;
    uint4 raw[PER];
    float vv[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = G + NG * j;
      vv[j] = 0.f;
      raw[j] = make_uint4(0, 0, 0, 0);
      if (e < n) {
        const uint2 p = lst[base + e];
        vv[j] = __uint_as_float(p.y);
        if (cv) raw[j] = ld16<WT>(rs, p.x * (uint32_t)d + (uint32_t)col);
      }
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) fma16<WT, E>(acc, vv[j], raw[j]);
  };

  int rem = 0;                                                 // pending entries (uniform)
  for (int s0 = 0; s0 < N; s0 += kFdSeg) {
    const int ub = s0 + tid * kFdUPT;
    const bool valid = ub < N;                                 // N is a multiple of 16
    const int uc = valid ? ub : 0;
    float za[kFdUPT], zb[kFdUPT], nb[kFdUPT];
#pragma unroll
    for (int q = 0; q < kFdUPT / 4; ++q) {                    // the half sums are 256-byte aligned rows
      const float4 a = *(const float4 *)(z0 + uc + 4 * q), bb = *(const float4 *)(z1 + uc + 4 * q);
      za[4 * q] = a.x; za[4 * q + 1] = a.y; za[4 * q + 2] = a.z; za[4 * q + 3] = a.w;
      zb[4 * q] = bb.x; zb[4 * q + 1] = bb.y; zb[4 * q + 2] = bb.z; zb[4 * q + 3] = bb.w;
    }
#pragma unroll
    for (int e = 0; e < kFdUPT; ++e) nb[e] = b1[uc + e];     // b1 is only 4-byte aligned
    __builtin_amdgcn_sched_barrier(0);                         // every load before the first use
    uint32_t on = 0;
    float v[kFdUPT];
#pragma unroll
    for (int e = 0; e < kFdUPT; ++e) {
      const float z = za[e] + zb[e], nbe = -nb[e];
      v[e] = z - nbe;
      on |= (valid && z > nbe ? 1u : 0u) << e;
    }
    const int cnt = __popc(on);
    int tot;
    const int ex = wave_excl_scan(cnt, &tot);
    if (lane == 0) wsum[wave] = tot;
    __syncthreads();                                           // also: the last round read lst
    int off = ex, segtot = 0;
#pragma unroll
    for (int w = 0; w < kFdThreads / 64; ++w) {
      if (w < wave) off += wsum[w];
      segtot += wsum[w];
    }
    {
      int k = rem + off;
#pragma unroll
      for (int e = 0; e < kFdUPT; ++e)
        if ((on >> e) & 1u) lst[k++] = make_uint2((uint32_t)(ub + e), __float_as_uint(Elem<VT>::load_rounded(v[e])));
    }
    if (writer) {
      // the tile's lanes are lane & ~(L - 1) .. + L - 1 of this wave
      const int first = lane & ~(L - 1);
      const int tile_off = __shfl(off, first, 64);
      const int tile_cnt = __shfl(off + cnt, first + L - 1, 64) - tile_off;
      if (valid) {
        const int kt = ub / W;
        const size_t base = ((size_t)t * n_t + kt) * S;
        int slot = off - tile_off;
#pragma unroll
        for (int e = 0; e < kFdUPT; ++e) {
          if ((on >> e) & 1u) {
            if (slot < S) {
              o.col_idx[base + slot] = ub + e;
              Elem<VT>::store((VT *)o.vals, base + slot, v[e]);
            }
            ++slot;
          }
        }
        for (int p = lane & (L - 1); p < S; p += L)
          if (p >= tile_cnt) {
            o.col_idx[base + p] = -1;
            Elem<VT>::store((VT *)o.vals, base + p, 0.f);
          }
        if ((lane & (L - 1)) == 0) {
          o.counts[(size_t)t * n_t + kt] = tile_cnt;
          if (tile_cnt > S) ovf_s = 1;
        }
      }
    }
    __syncthreads();                                           // the entries are in lst
    const int total = rem + segtot, nfull = total / kFdLW;
    for (int r = 0; r < nfull; ++r) round(r * kFdLW, kFdLW);
    rem = total - nfull * kFdLW;
    if (nfull > 0 && rem > 0) {                                // the rest to the front
      __syncthreads();
      const uint2 e = tid < rem ? lst[nfull * kFdLW + tid] : make_uint2(0, 0);
      __syncthreads();
      if (tid < rem) lst[tid] = e;
    }
    __syncthreads();
  }
  if (rem > 0) round(0, rem);

  // group sums: across the four groups of a wave, then across waves in order
#pragma unroll
  for (int q = 0; q < E; ++q) {
    acc[q] += __shfl_xor(acc[q], 16, 64);
    acc[q] += __shfl_xor(acc[q], 32, 64);
  }
  if (wave > 0 && wave < kFdGW && lane < 16)
#pragma unroll
    for (int q = 0; q < E; ++q) red[wave - 1][lane * E + q] = acc[q];
  __syncthreads();
  if (wave == 0 && lane < 16 && cv) {
#pragma unroll
    for (int w = 0; w < kFdGW - 1; ++w)
#pragma unroll
      for (int q = 0; q < E; ++q) acc[q] += red[w][lane * E + q];
    store_out_nt<YT, E>(y, (size_t)t * d + col, acc);
  }
  if (!writer) return;

  // the tokens' chunk-0 workgroups meet: the last one has every overflow flag
  if (tid == 0) {
    const uint64_t mine = 1ull | ((uint64_t)(ovf_s ? 1u : 0u) << (32 + t));
    const uint64_t old = M == 1 ? 0ull : __hip_atomic_fetch_add(o.dec_ticket, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_s = (int)(old & 0xFFFFFFFFull) == M - 1;
    if (last_s) {
      const uint32_t flags = (uint32_t)((old + mine) >> 32);
      int r = 0;
      for (int k = 0; k < M; ++k) {
        int sl = -1;
        if ((flags >> k) & 1u) {
          if (r < f.cap) {
            sl = r;
            f.ovf_rows[r] = k;
          }
          ++r;
        }
        slot_s[k] = sl;
        f.ovf_slot[k] = sl;
      }
      *f.ovf_n = r;
      if (M > 1) __hip_atomic_store(o.dec_ticket, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();
  if (!last_s) return;
  for (int k = 0; k < M; ++k) {
    const int sl = slot_s[k];
    if (sl < 0) continue;                                      // uniform
    VT *row = (VT *)f.ovf_dense + (size_t)sl * N;
    const float *a0 = zp + (size_t)k * N, *a1 = zp + ((size_t)M + k) * N;
    for (int u = tid; u < N; u += kFdThreads) {
      float h = a0[u] + a1[u] + b1[u];
      h = h > 0.f ? h : 0.f;
      Elem<VT>::store(row, u, h);
    }
  }
}

template <int W, typename WT, typename VT, typename YT>
static hipError_t fused_t(const float *b1, int M, int N, const TwellOut &o, const TwellFinish &f, const WT *w2, int d,
                          YT *y, hipStream_t s) {
  constexpr int CW = 16 * Vec16<WT>::N;
  const int nchunk = (d + CW - 1) / CW;
  hipLaunchKernelGGL((k_dec_fused_down<W, WT, VT, YT>), dim3((unsigned)(8 * ((nchunk + 7) / 8) * M)), dim3(kFdThreads), 0, s,
                     o.dec_part, b1, M, N, o, f, w2, d, y, nchunk);
  return hipGetLastError();
}

template <typename WT, typename VT, typename YT>
static hipError_t fused_w(const float *b1, int M, int N, const TwellOut &o, const TwellFinish &f, const WT *w2, int d,
                          YT *y, int W, hipStream_t s) {
  if (W == 64) return fused_t<64, WT, VT, YT>(b1, M, N, o, f, w2, d, y, s);
  return fused_t<128, WT, VT, YT>(b1, M, N, o, f, w2, d, y, s);
}

hipError_t launch_dec_fused_down(const float *b1, int M, int N, const TwellOut &o, const TwellFinish &f, const void *w2,
                                 int d, void *y, int y_bf16, int W, hipStream_t s) {
  if (M < 1 || M > 16 || (W != 64 && W != 128) || N % W || !o.dec_part || !o.dec_ticket || !f.ovf_n || !f.ovf_slot ||
      (f.cap > 0 && (!f.ovf_rows || !f.ovf_dense)))
    return hipErrorInvalidValue;
  const uint16_t *w = (const uint16_t *)w2;
  if (o.val_bf16) {
    if (y_bf16) return fused_w<uint16_t, uint16_t, uint16_t>(b1, M, N, o, f, w, d, (uint16_t *)y, W, s);
    return fused_w<uint16_t, uint16_t, float>(b1, M, N, o, f, w, d, (float *)y, W, s);
  }
  if (y_bf16) return fused_w<uint16_t, float, uint16_t>(b1, M, N, o, f, w, d, (uint16_t *)y, W, s);
  return fused_w<uint16_t, float, float>(b1, M, N, o, f, w, d, (float *)y, W, s);
}

}  // namespace tw
