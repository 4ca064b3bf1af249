// N:M activation pruning and the packed N:M down projection.
//
// "Motivating Next-Gen Accelerators with Flexible (N:M) Activation Sparsity ...", section
// "2. Metodologia": in every block of M consecutive activations keep the N of largest
// magnitude (criterion ACT); patterns 2:4, 4:8, 8:16 and 16:32. Section "5. Significado e
// Implicações": without hardware that executes the N:M format the products are not
// reduced. gfx950's sparse matrix instructions (v_smfmac) take only a 2:4 structure, at
// most two nonzeros in every four consecutive entries, which 8:16 and 16:32 blocks do not
// have; so the down projection expands each block back to dense bf16 in LDS and multiplies
// on MFMA (only the activation bytes shrink).
#include "common.h"
#include "launch.h"
#include "nmsel.h"
#include "stage.h"

namespace tw {

// ------------------------------------------------------------------------ nm_prune
// fp32 blocks: one thread per block of M (M words, read as 16-byte vectors); the kept set
// is chosen by nm_keep32 (nmsel.h), and the kept positions are emitted in ascending order with
// their signed values. Outputs are staged in LDS per wave and written with 16-byte stores.
template <int N, int M>
__global__ __launch_bounds__(256) void k_nm_prune32(const float *__restrict__ h, size_t groups,
                                                    float *__restrict__ vals, uint8_t *__restrict__ idx) {
  static_assert(M % 4 == 0, "whole 16-byte vectors per block");
  __shared__ __attribute__((aligned(16))) uint32_t sv[4][64 * N];
  __shared__ __attribute__((aligned(16))) uint8_t si[4][64 * N];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t g0 = ((size_t)blockIdx.x * 4 + wave) * 64;
  if (g0 >= groups) return;
  const size_t g = g0 + lane;
  uint32_t bits[M];
  if (g < groups) {
    const uint4 *src = (const uint4 *)(h + g * M);
#pragma unroll
    for (int v = 0; v < M / 4; ++v) {
      const uint4 u = src[v];
      bits[4 * v] = u.x; bits[4 * v + 1] = u.y; bits[4 * v + 2] = u.z; bits[4 * v + 3] = u.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < M; ++i) bits[i] = 0;
  }
  bool keep[M];
  nm_keep32<N, M>(bits, keep);
  int pos = 0;
#pragma unroll
  for (int i = 0; i < M; ++i) {
    if (keep[i]) {
      sv[wave][lane * N + pos] = bits[i];
      si[wave][lane * N + pos] = (uint8_t)i;
      ++pos;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // copy out this wave's 64 groups (contiguous in the outputs)
  const size_t ng = groups - g0 < 64 ? groups - g0 : 64;
  const size_t vbytes = ng * N * 4, ibytes = ng * N;
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

// bf16 blocks. A wave owns 64 consecutive blocks, one per lane: 128 M contiguous bytes,
// staged through LDS with coalesced loads. Each lane reads its block back, takes the kept
// set as a mask (nm_kept_mask) and walks it with count-leading-zeros, which yields the kept
// entries in ascending order; each value is re-read from the staged block and each index
// packed into bytes, so nothing branches on the data.
template <int N, int M>
__global__ __launch_bounds__(256) void k_nm_prune16(const uint16_t *__restrict__ h, size_t groups,
                                                    uint16_t *__restrict__ vals, uint8_t *__restrict__ idx) {
  constexpr int RB = 2 * M;                      // bytes per block
  constexpr int CH = RB >= 16 ? 16 : 8;          // bytes per staged load
  constexpr int CPL = RB / CH;                   // loads per lane
  constexpr int NV = N / 2, NI = (N + 3) / 4;    // packed value words, index words
  __shared__ __attribute__((aligned(16))) uint32_t raw[4][64 * RB / 4];
  __shared__ __attribute__((aligned(16))) uint32_t sv[4][64 * NV];
  __shared__ __attribute__((aligned(16))) uint8_t si[4][64 * N];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t g0 = ((size_t)blockIdx.x * 4 + wave) * 64;
  if (g0 >= groups) return;
  const size_t ng = groups - g0 < 64 ? groups - g0 : 64;
  const char *src = (const char *)(h + g0 * M);
  char *rw = (char *)raw[wave];
  const int nch = (int)ng * CPL;                 // loads that fall inside this wave's blocks
  if constexpr (CH == 16) {
    uint4 u[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int ch = c * 64 + lane;
      u[c] = *(const uint4 *)(src + (size_t)(ch < nch ? ch : 0) * 16);
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int ch = c * 64 + lane;
      *(uint4 *)(rw + ch * 16) = ch < nch ? u[c] : make_uint4(0, 0, 0, 0);
    }
  } else {
    const uint2 u = *(const uint2 *)(src + (size_t)(lane < nch ? lane : 0) * 8);
    *(uint2 *)(rw + lane * 8) = lane < nch ? u : make_uint2(0, 0);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const char *row = rw + lane * RB;
  uint32_t w[RB / 4];
  if constexpr (CH == 16) {
#pragma unroll
    for (int v = 0; v < RB / 16; ++v) {
      const uint4 u = *(const uint4 *)(row + v * 16);
      w[4 * v] = u.x; w[4 * v + 1] = u.y; w[4 * v + 2] = u.z; w[4 * v + 3] = u.w;
    }
  } else {
    const uint2 u = *(const uint2 *)row;
    w[0] = u.x; w[1] = u.y;
  }
  uint32_t bits[M];
#pragma unroll
  for (int i = 0; i < M; ++i) bits[i] = (w[i / 2] >> (16 * (i & 1))) & 0xFFFFu;
  uint32_t km = nm_kept_mask<N, M>(bits);
  const uint16_t *rowh = (const uint16_t *)row;
  uint32_t vw[NV], iw[NI];
  static_for<N>([&](auto J) {
    constexpr int j = decltype(J)::value;
    const uint32_t e = (uint32_t)__builtin_clz(km);   // km holds N - j set bits here
    km ^= 0x80000000u >> e;
    const uint32_t v = rowh[e];
    if constexpr (j & 1) vw[j / 2] |= v << 16;
    else vw[j / 2] = v;
    if constexpr (j % 4 == 0) iw[j / 4] = e;
    else iw[j / 4] |= e << (8 * (j % 4));
  });
#pragma unroll
  for (int q = 0; q < NV; ++q) sv[wave][lane * NV + q] = vw[q];
  if constexpr (N >= 4) {
#pragma unroll
    for (int q = 0; q < NI; ++q) ((uint32_t *)si[wave])[lane * NI + q] = iw[q];
  } else {
    ((uint16_t *)si[wave])[lane] = (uint16_t)iw[0];
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const size_t vbytes = ng * N * 2, ibytes = ng * N;
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

template <int N, int M>
static void prune_launch(const void *h, size_t groups, void *vals, uint8_t *idx, int bf16, hipStream_t s) {
  const dim3 grid((unsigned)((groups + 255) / 256));
  if (bf16)
    hipLaunchKernelGGL((k_nm_prune16<N, M>), grid, dim3(256), 0, s, (const uint16_t *)h, groups, (uint16_t *)vals, idx);
  else
    hipLaunchKernelGGL((k_nm_prune32<N, M>), grid, dim3(256), 0, s, (const float *)h, groups, (float *)vals, idx);
}

hipError_t launch_nm_prune(const void *h, int bf16, int T, int f, int n, int m, void *vals, uint8_t *idx,
                           hipStream_t s) {
  const size_t groups = (size_t)T * (f / m);
  if (groups == 0) return hipSuccess;
  if (n == 2 && m == 4) prune_launch<2, 4>(h, groups, vals, idx, bf16, s);
  else if (n == 4 && m == 8) prune_launch<4, 8>(h, groups, vals, idx, bf16, s);
  else if (n == 8 && m == 16) prune_launch<8, 16>(h, groups, vals, idx, bf16, s);
  else prune_launch<16, 32>(h, groups, vals, idx, bf16, s);
  return hipGetLastError();
}

// ------------------------------------------------------------------- nm_ffn_down
// y[t][c] = sum_k H[t][k] w2t[c][k] with H expanded from (vals, idx) per 32-column stage.
// Tile 256 tokens x 256 output columns, 8 waves of 64 x 128 (two per SIMD, so one wave's
// expansion and loads overlap the other's MFMAs), v_mfma_f32_16x16x32_bf16, a ring of four
// stages of 64-byte rows (A: 256 expanded H rows, B: 256 w2t rows), read as in the up GEMM
// (16-row fragments, XOR-swizzled 16-byte chunks).
//  - B arrives by buffer_load ... lds three stages ahead of its use.
//  - A: tile row r is built by the neighbouring lanes 2r and 2r + 1. A stage of a row holds
//    32 N / M = 16 kept entries (8:16 and 16:32): each lane loads 8 values and 8 indices
//    (16 + 8 bytes), clears its 32-byte half of the row, then writes its values at their
//    columns, which may lie in either half. The two lanes are in one wave, whose LDS writes
//    execute in issue order, so both clears precede every value.
// Step kt: wait for stage kt + 1, barrier; load the packed A of stage kt + 3; the MFMAs of
// stage kt with the fragment reads of stage kt + 1 and the B loads of stage kt + 3 between
// them; then build the A of stage kt + 3. Stage kt + 3 reuses the buffer of stage kt - 1,
// whose fragments were read in step kt - 2. (With 4 waves of 128 x 128 and the packed A
// loaded a step earlier the kernel took 0.56 / 0.57 ms at c4 instead of 0.48 / 0.49 ms.)
// Patterns: 8:16 and 16:32 (d_ff a multiple of 32).
// One thread's half of a row's packed stage: 8 values (bf16) and 8 indices (u8).
struct NmPack {
  uint4 v;
  uint2 ix;
};

template <int N, int M>
__global__ __launch_bounds__(512) void k_nm_down(const uint16_t *__restrict__ vals, const uint8_t *__restrict__ idx,
                                                 int T, int f, const uint16_t *__restrict__ w2t, int d,
                                                 void *__restrict__ y, int y_bf16) {
  static_assert(32 % M == 0 && 32 / M * N == 16, "16 kept entries per 32 columns");
  constexpr int BM = 256, BN = 256, RB = 64, NS = 4, STAGE = (BM + BN) * RB;
  constexpr int WM = 64, WN = 128, FM = WM / 16, FN = WN / 16;
  constexpr int NM = FM * FN, NR = FM + FN;
  constexpr int LPW = BN / 16 / 8;               // B wave-loads per wave per stage
  constexpr int LA = 2;                          // packed-A loads per thread per stage
  __shared__ __attribute__((aligned(16))) char smem[NS * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int nk = f / 32;
  const size_t E = (size_t)f / M * N;            // kept entries per row

  // B: stage rows of w2t through LDS DMA (16-row blocks q = wave + 8 i of the B half)
  constexpr uint32_t OOB = 0x80000000u;
  const size_t row_bytes = (size_t)f * 2;
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc((void *)w2t, (short)0, (int)((size_t)d * row_bytes), 0x00020000);
  const int lrow = lane >> 2, cl = (lane & 3) ^ ((lrow >> 2) & 3);
  uint32_t voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int gr = n0 + (wave + 8 * i) * 16 + lrow;
    voff[i] = gr < d ? (uint32_t)((size_t)gr * row_bytes) + cl * 16 : OOB;
  }
  auto issue_b = [&](int kt, int i) {
    char *st = smem + (kt % NS) * STAGE + BM * RB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t *)(st + (wave + 8 * i) * 1024), 16, voff[i], kt * 64,
                                             0, 0);
  };
  // A: tile row tid / 2, whose 16 kept entries per stage this thread shares with its
  // neighbour lane: half hf = tid % 2 takes entries 8 hf .. 8 hf + 7 (rows past T read row
  // T - 1 and are built as zeros)
  const int arow = tid >> 1, hf = tid & 1;
  const bool trow = m0 + arow < T;
  const size_t prow = (size_t)min(m0 + arow, T - 1) * E;
  const uint4 *pv = (const uint4 *)(vals + prow);
  const uint2 *pi = (const uint2 *)(idx + prow);
  auto load_a = [&](int kt, NmPack &p) {
    p.v = pv[2 * kt + hf];
    p.ix = pi[2 * kt + hf];
  };
  // The stores are inline assembly: the compiler cannot tell them apart from the B ring's
  // pending LDS DMA and would wait for all of it (vmcnt(0)) before each build. They write
  // the A half of stage kt, which no DMA targets; the LDS wait before every barrier covers
  // them.
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char_t *)smem;
  const int swz = (arow >> 2) & 3;
  auto a_row = [&](int kt) { return lds0 + (uint32_t)((kt % NS) * STAGE + arow * RB); };
  // each thread clears its 32-byte half of the row, then writes its 8 entries anywhere in the
  // row: the two halves' threads are neighbouring lanes of one wave, whose LDS writes execute
  // in issue order, so both clears precede every entry write
  auto build_zero = [&](uint32_t row) {
    const u32x4_t z = {0u, 0u, 0u, 0u};
    const uint32_t h = row + 32u * (uint32_t)hf;
    asm volatile("ds_write_b128 %0, %1\n\tds_write_b128 %0, %1 offset:16" ::"v"(h), "v"(z));
  };
  auto build_entry = [&](uint32_t row, const NmPack &p, int e) {     // entry 8 hf + e of the stage
    const uint32_t iw = e < 4 ? p.ix.x : p.ix.y;
    const uint32_t vw = e < 2 ? p.v.x : e < 4 ? p.v.y : e < 6 ? p.v.z : p.v.w;
    const int ee = 8 * hf + e;
    const int col = (ee / N) * M + (int)((iw >> (8 * (e % 4))) & (M - 1));
    const uint32_t v = trow ? (vw >> (16 * (e & 1))) & 0xFFFFu : 0u;
    const uint32_t a = row + (uint32_t)((((col >> 3) ^ swz) << 4) + (col & 7) * 2);
    asm volatile("ds_write_b16 %0, %1" ::"v"(a), "v"(v));
  };
  auto build_a = [&](int kt, const NmPack &p) {
    const uint32_t row = a_row(kt);
    build_zero(row);
#pragma unroll
    for (int e = 0; e < 8; ++e) build_entry(row, p, e);
  };
  // fragments (as in the up GEMM's 16 x 16 x 32 loop)
  typedef u32x4_t FA[FM];
  typedef u32x4_t FB[FN];
  const int l16 = lane & 15, c4 = lane >> 4;
  auto read1 = [&](int kt, int j, FA &a, FB &b) {
    const char *sa = smem + (kt % NS) * STAGE;
    if (j < FM) {
      const int r = wm * WM + j * 16 + l16;
      a[j] = *(const u32x4_t *)(sa + r * RB + ((c4 ^ ((r >> 2) & 3)) << 4));
    } else {
      const int r = wn * WN + (j - FM) * 16 + l16;
      b[j - FM] = *(const u32x4_t *)(sa + BM * RB + r * RB + ((c4 ^ ((r >> 2) & 3)) << 4));
    }
  };
  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{};
  auto mma = [&](int i, const FA &a, const FB &b) {
    acc[i / FN][i % FN] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[i / FN]),
                                                                  __builtin_bit_cast(bf16x8_t, b[i % FN]),
                                                                  acc[i / FN][i % FN], 0, 0, 0);
  };
  // prologue: stages 0 .. 2 built and loaded
  NmPack pa;
#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    if (st < nk) {
      load_a(st, pa);
      build_a(st, pa);
    }
#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    if (st < nk)
#pragma unroll
      for (int i = 0; i < LPW; ++i) issue_b(st, i);
  wait_vmcnt<0>();
  block_barrier_lds();
  FA a0, a1;
  FB b0, b1;
#pragma unroll
  for (int j = 0; j < NR; ++j) read1(0, j, a0, b0);

  constexpr int RI = NM / NR;                    // a fragment read after every RI MFMAs
  constexpr int DI = NM / LPW;                   // a B load after every DI MFMAs
  // A step of the steady state (kt + 3 < nk): the packed loads of stage kt + 3, then (between
  // the MFMAs of stage kt, with the fragment reads of stage kt + 1) the B loads of stage
  // kt + 3; after the MFMAs the A of stage kt + 3 is built from those packed registers, whose
  // loads are the ones issued before the LPW B loads. At the start of step kt the loads issued
  // after stage kt + 1's B are step kt - 1's (LA + LPW). Stage kt + 3 reuses the buffer of
  // stage kt - 1, whose fragments were read in step kt - 2.
  auto step = [&](int kt, const FA &ac, const FB &bc, FA &an, FB &bn) {
    wait_vmcnt<LA + LPW>();
    block_barrier_lds();
    load_a(kt + 3, pa);
    __builtin_amdgcn_sched_barrier(0);
    static_for<NM>([&](auto I) {
      constexpr int i = decltype(I)::value;
      mma(i, ac, bc);
      if constexpr (i % RI == 0 && i / RI < NR) read1(kt + 1, i / RI, an, bn);
      if constexpr (i % DI == DI - 1) issue_b(kt + 3, i / DI);
      __builtin_amdgcn_sched_barrier(0);
    });
    wait_vmcnt<LPW>();
    build_a(kt + 3, pa);
    __builtin_amdgcn_sched_barrier(0);
  };
  // The last steps (kt + 3 >= nk for the second of a pair or later): what exists is issued,
  // waits are complete ones, and the next fragment set is copied into the current one.
  auto tail_step = [&](int kt) {
    wait_vmcnt<0>();
    block_barrier_lds();
    if (kt + 3 < nk) load_a(kt + 3, pa);
    static_for<NM>([&](auto I) {
      constexpr int i = decltype(I)::value;
      mma(i, a0, b0);
      if constexpr (i % RI == 0 && i / RI < NR) read1(kt + 1, i / RI, a1, b1);
      __builtin_amdgcn_sched_barrier(0);
    });
    if (kt + 3 < nk) {
#pragma unroll
      for (int i = 0; i < LPW; ++i) issue_b(kt + 3, i);
      build_a(kt + 3, pa);
    }
    wait_vmcnt<0>();
#pragma unroll
    for (int j = 0; j < FM; ++j) a0[j] = a1[j];
#pragma unroll
    for (int j = 0; j < FN; ++j) b0[j] = b1[j];
  };
  int kt = 0;
  for (; kt + 4 < nk; kt += 2) {
    step(kt, a0, b0, a1, b1);
    step(kt + 1, a1, b1, a0, b0);
  }
  for (; kt + 1 < nk; ++kt) tail_step(kt);
#pragma unroll
  for (int i = 0; i < NM; ++i) mma(i, a0, b0);

  // epilogue: y[row][col], register r of block (fm, fn): row 16 fm + 4 (lane / 16) + r,
  // column 16 fn + lane % 16
#pragma unroll
  for (int fn = 0; fn < FN; ++fn) {
    const int col = n0 + wn * WN + fn * 16 + l16;
    if (col >= d) continue;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + wm * WM + fm * 16 + 4 * c4 + r;
        if (row >= T) continue;
        const size_t o = (size_t)row * d + col;
        if (y_bf16) ((uint16_t *)y)[o] = (uint16_t)f32_to_bf16(acc[fm][fn][r]);
        else ((float *)y)[o] = acc[fm][fn][r];
      }
  }
}

hipError_t launch_nm_down(const void *vals, const uint8_t *idx, int T, int f, int n, int m, const void *w2t, int d,
                          void *y, int y_bf16, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid((d + 255) / 256, (T + 255) / 256);
  const uint16_t *v = (const uint16_t *)vals, *w = (const uint16_t *)w2t;
  if (n == 8 && m == 16) hipLaunchKernelGGL((k_nm_down<8, 16>), grid, dim3(512), 0, s, v, idx, T, f, w, d, y, y_bf16);
  else hipLaunchKernelGGL((k_nm_down<16, 32>), grid, dim3(512), 0, s, v, idx, T, f, w, d, y, y_bf16);
  return hipGetLastError();
}

}  // namespace tw
