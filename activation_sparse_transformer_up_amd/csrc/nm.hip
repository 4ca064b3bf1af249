// N:M activation pruning and the packed N:M down projection.
//
// "Motivating Next-Gen Accelerators with Flexible (N:M) Activation Sparsity ...", section
// "2. Metodologia": in every block of M consecutive activations keep the N of largest
// magnitude (criterion ACT); patterns 2:4, 4:8, 8:16 and 16:32. Section "5. Significado e
// Implicações": without hardware that executes the N:M format the products are not
// reduced; gfx950 has no N:M matrix instruction, so the down projection expands each block
// back to dense bf16 in LDS and multiplies on MFMA (only the activation bytes shrink).
#include "common.h"
#include "launch.h"

namespace tw {

// ------------------------------------------------------------------------ nm_prune
// One thread per block of M. Entry i is kept iff its rank
//   rank_i = #{k : |h_k| > |h_i|} + #{k < i : |h_k| == |h_i|}
// is below N (magnitudes compared as sign-cleared bit patterns: exact and monotone for
// finite values, +-0 equal); output position = kept entries of lower index.
// bf16: the ranks are those of the unique keys (magnitude << log2 M) | (M - 1 - i); every
// supported pattern keeps N = M / 2, and the N largest keys are found by sorting each half
// of the block (bitonic network, descending) and taking c_i = max(a_i, b_{N-1-i}), whose
// minimum is the N-th largest key. fp32 (31-bit magnitudes) counts the ranks directly.
// Outputs are staged in LDS per wave and written with 16-byte stores.

// Bitonic sort of L keys, descending; every index is a compile-time constant.
template <int L> TW_DEV void bitonic_desc(uint32_t (&a)[L]) {
  static_for<31 - __builtin_clz(L)>([&](auto KS) {              // k = 2, 4, ..., L
    constexpr int k = 2 << decltype(KS)::value;
    static_for<decltype(KS)::value + 1>([&](auto JS) {          // j = k/2, ..., 1
      constexpr int j = (k >> 1) >> decltype(JS)::value;
      static_for<L>([&](auto IS) {
        constexpr int i = decltype(IS)::value, l = i ^ j;
        if constexpr (l > i) {
          const uint32_t x = a[i], y = a[l];
          const uint32_t hi = x > y ? x : y, lo = x > y ? y : x;
          if constexpr ((i & k) == 0) { a[i] = hi; a[l] = lo; }
          else { a[i] = lo; a[l] = hi; }
        }
      });
    });
  });
}
template <typename HT, int N, int M>
__global__ __launch_bounds__(256) void k_nm_prune(const HT *__restrict__ h, size_t groups, HT *__restrict__ vals,
                                                  uint8_t *__restrict__ idx) {
  constexpr uint32_t MAGMASK = sizeof(HT) == 2 ? 0x7FFFu : 0x7FFFFFFFu;
  __shared__ __attribute__((aligned(16))) HT sv[4][64 * N];
  __shared__ __attribute__((aligned(16))) uint8_t si[4][64 * N];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t g0 = ((size_t)blockIdx.x * 4 + wave) * 64;
  if (g0 >= groups) return;
  const size_t g = g0 + lane;
  const bool gv = g < groups;
  uint32_t bits[M];
  if (gv) {
    // M values = W32 words, fetched with the widest aligned vector loads
    constexpr int W32 = M * (int)sizeof(HT) / 4;
    uint32_t w[W32];
    if constexpr (W32 % 4 == 0) {
      const uint4 *src = (const uint4 *)(h + g * M);
#pragma unroll
      for (int v = 0; v < W32 / 4; ++v) {
        const uint4 u = src[v];
        w[4 * v] = u.x; w[4 * v + 1] = u.y; w[4 * v + 2] = u.z; w[4 * v + 3] = u.w;
      }
    } else {
      const uint2 *src = (const uint2 *)(h + g * M);
#pragma unroll
      for (int v = 0; v < W32 / 2; ++v) {
        const uint2 u = src[v];
        w[2 * v] = u.x; w[2 * v + 1] = u.y;
      }
    }
#pragma unroll
    for (int i = 0; i < M; ++i) {
      if constexpr (sizeof(HT) == 2) bits[i] = (w[i / 2] >> (16 * (i & 1))) & 0xFFFFu;
      else bits[i] = w[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < M; ++i) bits[i] = 0;
  }
  bool keep[M];
  if constexpr (sizeof(HT) == 2) {
    static_assert(2 * N == M, "bf16 path keeps half of each block");
    constexpr int LOGM = 31 - __builtin_clz(M);
    uint32_t key[M], a[N], b[N];
    static_for<M>([&](auto I) {
      constexpr int i = decltype(I)::value;
      key[i] = ((bits[i] & MAGMASK) << LOGM) | (uint32_t)(M - 1 - i);
      if constexpr (i < N) a[i] = key[i];
      else b[i - N] = key[i];
    });
    bitonic_desc<N>(a);
    bitonic_desc<N>(b);
    uint32_t th = 0xFFFFFFFFu;
    static_for<N>([&](auto I) {
      constexpr int i = decltype(I)::value;
      const uint32_t c = a[i] > b[N - 1 - i] ? a[i] : b[N - 1 - i];
      th = c < th ? c : th;
    });
    static_for<M>([&](auto I) { keep[decltype(I)::value] = key[decltype(I)::value] >= th; });
  } else {
#pragma unroll
    for (int i = 0; i < M; ++i) {
      const uint32_t mi = bits[i] & MAGMASK;
      int rank = 0;
#pragma unroll
      for (int k = 0; k < M; ++k) {
        if (k == i) continue;
        const uint32_t mk = bits[k] & MAGMASK;
        rank += (k < i) ? (mk >= mi) : (mk > mi);
      }
      keep[i] = rank < N;
    }
  }
  int pos = 0;
#pragma unroll
  for (int i = 0; i < M; ++i) {
    if (keep[i]) {
      if constexpr (sizeof(HT) == 2) ((uint16_t *)sv[wave])[lane * N + pos] = (uint16_t)bits[i];
      else ((uint32_t *)sv[wave])[lane * N + pos] = bits[i];
      si[wave][lane * N + pos] = (uint8_t)i;
      ++pos;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // copy out this wave's 64 groups (contiguous in the outputs)
  const size_t ng = groups - g0 < 64 ? groups - g0 : 64;
  const size_t vbytes = ng * N * sizeof(HT), ibytes = ng * N;
  char *dv = (char *)(vals + g0 * N);
  char *di = (char *)(idx + g0 * N);
  const char *lv = (const char *)sv[wave];
  const char *li = (const char *)si[wave];
  if (ng == 64) {
    for (size_t o = (size_t)lane * 16; o < vbytes; o += 64 * 16) *(uint4 *)(dv + o) = *(const uint4 *)(lv + o);
    for (size_t o = (size_t)lane * 8; o < ibytes; o += 64 * 8) *(uint2 *)(di + o) = *(const uint2 *)(li + o);
  } else {
    for (size_t o = lane; o < vbytes; o += 64) dv[o] = lv[o];
    for (size_t o = lane; o < ibytes; o += 64) di[o] = li[o];
  }
}

template <typename HT>
static hipError_t prune_t(const HT *h, size_t groups, int n, int m, HT *vals, uint8_t *idx, hipStream_t s) {
  const dim3 grid((unsigned)((groups + 255) / 256));
  if (n == 2 && m == 4) hipLaunchKernelGGL((k_nm_prune<HT, 2, 4>), grid, dim3(256), 0, s, h, groups, vals, idx);
  else if (n == 4 && m == 8) hipLaunchKernelGGL((k_nm_prune<HT, 4, 8>), grid, dim3(256), 0, s, h, groups, vals, idx);
  else if (n == 8 && m == 16) hipLaunchKernelGGL((k_nm_prune<HT, 8, 16>), grid, dim3(256), 0, s, h, groups, vals, idx);
  else hipLaunchKernelGGL((k_nm_prune<HT, 16, 32>), grid, dim3(256), 0, s, h, groups, vals, idx);
  return hipGetLastError();
}

hipError_t launch_nm_prune(const void *h, int bf16, int T, int f, int n, int m, void *vals, uint8_t *idx,
                           hipStream_t s) {
  const size_t groups = (size_t)T * (f / m);
  if (groups == 0) return hipSuccess;
  if (bf16) return prune_t<uint16_t>((const uint16_t *)h, groups, n, m, (uint16_t *)vals, idx, s);
  return prune_t<float>((const float *)h, groups, n, m, (float *)vals, idx, s);
}

// ------------------------------------------------------------------- nm_ffn_down
// y[t][c] = sum_k H[t][k] w2t[c][k] with H expanded from (vals, idx) per K step. Tile 256 x
// 256, 4 waves of 128 x 128, 32x32x16 bf16 MFMA, K step 32. B (w2t rows) is staged by
// buffer_load ... lds; A is built by the threads: zero the step's 32 columns of a row, then
// write its N kept values (two groups per row for M = 16, one for M = 32). Two LDS stages:
// the packed data of step k+1 is loaded into registers while step k is multiplied.
// Patterns: 8:16 and 16:32 (M must be a multiple of 8 for the 16-byte zero fill).
typedef uint32_t u32x4n_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void nm_lds_t;

template <int N, int M>
__global__ __launch_bounds__(256) void k_nm_down(const uint16_t *__restrict__ vals, const uint8_t *__restrict__ idx,
                                                 int T, int f, const uint16_t *__restrict__ w2t, int d,
                                                 void *__restrict__ y, int y_bf16) {
  constexpr int BM = 256, BN = 256, RB = 64, STAGE = (BM + BN) * RB;
  constexpr int GPR = 32 / M;                    // groups of a row per K step
  constexpr int GPT = BM * GPR / 256;            // groups per thread per K step
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int G = f / M;                           // groups per row
  const int nk = f / 32;
  // B operand via LDS DMA: 16 wave-loads of 16 rows per stage, 4 per wave
  constexpr uint32_t OOB = 0x80000000u;
  const size_t row_bytes = (size_t)f * 2;
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc((void *)w2t, (short)0,
                                                                      (int)((size_t)d * row_bytes), 0x00020000);
  const int lrow = lane >> 2, cl = (lane & 3) ^ ((lrow >> 2) & 3);
  uint32_t voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = wave + 4 * i;
    const int gr = n0 + q * 16 + lrow;
    voff[i] = gr < d ? (uint32_t)((size_t)gr * row_bytes) + cl * 16 : OOB;
  }
  auto issue_b = [&](int kt) {
    char *st = smem + (kt & 1) * STAGE + BM * RB;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (nm_lds_t *)(st + (wave + 4 * i) * 1024), 16, voff[i],
                                               kt * 64, 0, 0);
  };
  // A operand: thread -> (row, group-in-step) pairs
  uint4 pv[GPT][(N * 2 + 15) / 16];
  uint32_t pi[GPT][(N + 3) / 4];
  auto load_a = [&](int kt) {
#pragma unroll
    for (int u = 0; u < GPT; ++u) {
      const int q = tid + 256 * u;
      const int r = q / GPR, gi = q % GPR;
      const int t = m0 + r;
      const int gg = kt * GPR + gi;
      if (t < T) {
        const size_t base = ((size_t)t * G + gg) * N;
#pragma unroll
        for (int v = 0; v < (N * 2 + 15) / 16; ++v) pv[u][v] = ((const uint4 *)(vals + base))[v];
#pragma unroll
        for (int v = 0; v < (N + 3) / 4; ++v) pi[u][v] = ((const uint32_t *)(idx + base))[v];
      } else {
#pragma unroll
        for (int v = 0; v < (N * 2 + 15) / 16; ++v) pv[u][v] = make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < (N + 3) / 4; ++v) pi[u][v] = 0;
      }
    }
  };
  auto store_a = [&](int kt) {
    char *sa = smem + (kt & 1) * STAGE;
#pragma unroll
    for (int u = 0; u < GPT; ++u) {
      const int q = tid + 256 * u;
      const int r = q / GPR, gi = q % GPR;
      // zero the group's M columns (M / 8 chunks of 16 bytes)
#pragma unroll
      for (int c = 0; c < M / 8; ++c) {
        const int lc = gi * (M / 8) + c;
        *(uint4 *)(sa + r * RB + ((lc ^ ((r >> 2) & 3)) << 4)) = make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < N; ++e) {
        const uint32_t w = ((const uint32_t *)pv[u])[e / 2];
        const uint16_t v = (uint16_t)((w >> (16 * (e & 1))) & 0xFFFFu);
        const int k = gi * M + ((pi[u][e / 4] >> (8 * (e & 3))) & 0xFF);
        const int lc = k >> 3;
        *(uint16_t *)(sa + r * RB + ((lc ^ ((r >> 2) & 3)) << 4) + (k & 7) * 2) = v;
      }
    }
  };
  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};
  const int lr = lane & 31, lh = lane >> 5;
  load_a(0);
  issue_b(0);
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt & 1 was last read by compute(kt - 2), finished before the previous barrier
    store_a(kt);
    __builtin_amdgcn_s_waitcnt((0) | (7 << 4) | (15 << 8));      // B of step kt landed
    asm volatile("" ::: "memory");
    __syncthreads();
    if (kt + 1 < nk) {
      issue_b(kt + 1);                             // its stage was last read by compute(kt - 1)
      load_a(kt + 1);
    }
    const char *sa = smem + (kt & 1) * STAGE;
    const char *sb = sa + BM * RB;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int c = 2 * u + lh;
      u32x4n_t a[4], b[4];
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int r = wm * 128 + mb * 32 + lr;
        a[mb] = *(const u32x4n_t *)(sa + r * RB + ((c ^ ((r >> 2) & 3)) << 4));
      }
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int r = wn * 128 + nb * 32 + lr;
        b[nb] = *(const u32x4n_t *)(sb + r * RB + ((c ^ ((r >> 2) & 3)) << 4));
      }
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[mb]),
                                                                __builtin_bit_cast(bf16x8_t, b[nb]), acc[mb][nb], 0, 0, 0);
    }
  }
  // epilogue: y[row][col]
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int col = n0 + wn * 128 + nb * 32 + lr;
    if (col >= d) continue;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 128 + mb * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
        if (row >= T) continue;
        const size_t o = (size_t)row * d + col;
        if (y_bf16) ((uint16_t *)y)[o] = (uint16_t)f32_to_bf16(acc[mb][nb][r]);
        else ((float *)y)[o] = acc[mb][nb][r];
      }
  }
}

hipError_t launch_nm_down(const void *vals, const uint8_t *idx, int T, int f, int n, int m, const void *w2t, int d,
                          void *y, int y_bf16, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid((d + 255) / 256, (T + 255) / 256);
  const uint16_t *v = (const uint16_t *)vals, *w = (const uint16_t *)w2t;
  if (n == 8 && m == 16) hipLaunchKernelGGL((k_nm_down<8, 16>), grid, dim3(256), 0, s, v, idx, T, f, w, d, y, y_bf16);
  else hipLaunchKernelGGL((k_nm_down<16, 32>), grid, dim3(256), 0, s, v, idx, T, f, w, d, y, y_bf16);
  return hipGetLastError();
}

}  // namespace tw
