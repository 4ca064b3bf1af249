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
#include "nmsel.h"
#include "stage.h"

namespace tw {

// ------------------------------------------------------------------------ nm_prune
// One thread per block of M; the kept set is chosen by nm_keep (nmsel.h), and the kept
// positions are emitted in ascending order with their signed values. Outputs are staged in
// LDS per wave and written with 16-byte stores.
template <typename HT, int N, int M>
__global__ __launch_bounds__(256) void k_nm_prune(const HT *__restrict__ h, size_t groups, HT *__restrict__ vals,
                                                  uint8_t *__restrict__ idx) {
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
  nm_keep<(int)sizeof(HT), N, M>(bits, keep);
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
// y[t][c] = sum_k H[t][k] w2t[c][k] with H expanded from (vals, idx) per 32-column stage.
// Tile 256 tokens x 256 output columns, 4 waves of 128 x 128, v_mfma_f32_16x16x32_bf16, a
// ring of four stages of 64-byte rows (A: 256 expanded H rows, B: 256 w2t rows), read as in
// the up GEMM (16-row fragments, XOR-swizzled 16-byte chunks).
//  - B arrives by buffer_load ... lds three stages ahead of its use.
//  - A: thread r owns tile row r. A stage of a row holds 32 N / M = 16 kept entries (8:16
//    and 16:32): 32 bytes of values and 16 bytes of indices, loaded into registers one step
//    before the stage is built. Building writes zeros over the row's 64 bytes, then each
//    kept value at its column (one thread's LDS writes execute in order).
// Step kt: wait for stage kt + 1, barrier; load the packed A of stage kt + 4; the MFMAs of
// stage kt with the fragment reads of stage kt + 1 and the B loads of stage kt + 3 between
// them; then build the A of stage kt + 3 from the registers loaded in step kt - 1. Stage
// kt + 3 reuses the buffer of stage kt - 1, whose fragments were read in step kt - 2.
// Patterns: 8:16 and 16:32 (d_ff a multiple of 32).
struct NmPack {
  uint4 v0, v1, ix;                              // 16 values (bf16) and 16 indices (u8)
};

template <int N, int M>
__global__ __launch_bounds__(256) void k_nm_down(const uint16_t *__restrict__ vals, const uint8_t *__restrict__ idx,
                                                 int T, int f, const uint16_t *__restrict__ w2t, int d,
                                                 void *__restrict__ y, int y_bf16) {
  static_assert(32 % M == 0 && 32 / M * N == 16, "16 kept entries per 32 columns");
  constexpr int BM = 256, BN = 256, RB = 64, NS = 4, STAGE = (BM + BN) * RB;
  constexpr int WM = 128, WN = 128, FM = WM / 16, FN = WN / 16;
  constexpr int NM = FM * FN, NR = FM + FN;
  constexpr int LPW = BN / 16 / 4;               // B wave-loads per wave per stage
  constexpr int LA = 3;                          // packed-A loads per thread per stage
  __shared__ __attribute__((aligned(16))) char smem[NS * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int nk = f / 32;
  const size_t E = (size_t)f / M * N;            // kept entries per row

  // B: stage rows of w2t through LDS DMA (16-row blocks q = wave + 4 i of the B half)
  constexpr uint32_t OOB = 0x80000000u;
  const size_t row_bytes = (size_t)f * 2;
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc((void *)w2t, (short)0, (int)((size_t)d * row_bytes), 0x00020000);
  const int lrow = lane >> 2, cl = (lane & 3) ^ ((lrow >> 2) & 3);
  uint32_t voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int gr = n0 + (wave + 4 * i) * 16 + lrow;
    voff[i] = gr < d ? (uint32_t)((size_t)gr * row_bytes) + cl * 16 : OOB;
  }
  auto issue_b = [&](int kt, int i) {
    char *st = smem + (kt % NS) * STAGE + BM * RB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t *)(st + (wave + 4 * i) * 1024), 16, voff[i], kt * 64,
                                             0, 0);
  };
  // A: this thread's row (rows past T read row T - 1 and are built as zeros)
  const bool trow = m0 + tid < T;
  const size_t prow = (size_t)min(m0 + tid, T - 1) * E;
  const uint4 *pv = (const uint4 *)(vals + prow);
  const uint4 *pi = (const uint4 *)(idx + prow);
  auto load_a = [&](int kt, NmPack &p) {
    p.v0 = pv[2 * kt];
    p.v1 = pv[2 * kt + 1];
    p.ix = pi[kt];
  };
  // The stores are inline assembly: the compiler cannot tell them apart from the B ring's
  // pending LDS DMA and would wait for all of it (vmcnt(0)) before each build. They write
  // the A half of stage kt, which no DMA targets; the LDS wait before every barrier covers
  // them.
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char_t *)smem;
  const int swz = (tid >> 2) & 3;
  auto a_row = [&](int kt) { return lds0 + (uint32_t)((kt % NS) * STAGE + tid * RB); };
  auto build_zero = [&](uint32_t row) {
    const u32x4_t z = {0u, 0u, 0u, 0u};
    asm volatile("ds_write_b128 %0, %1\n\tds_write_b128 %0, %1 offset:16\n\t"
                 "ds_write_b128 %0, %1 offset:32\n\tds_write_b128 %0, %1 offset:48" ::"v"(row), "v"(z));
  };
  auto build_entry = [&](uint32_t row, const NmPack &p, int e) {
    const uint32_t iw = e < 4 ? p.ix.x : e < 8 ? p.ix.y : e < 12 ? p.ix.z : p.ix.w;
    const uint32_t vw = e < 8 ? (e < 2 ? p.v0.x : e < 4 ? p.v0.y : e < 6 ? p.v0.z : p.v0.w)
                              : (e < 10 ? p.v1.x : e < 12 ? p.v1.y : e < 14 ? p.v1.z : p.v1.w);
    const int col = (e / N) * M + (int)((iw >> (8 * (e % 4))) & (M - 1));
    const uint32_t v = trow ? (vw >> (16 * (e & 1))) & 0xFFFFu : 0u;
    const uint32_t a = row + (uint32_t)((((col >> 3) ^ swz) << 4) + (col & 7) * 2);
    asm volatile("ds_write_b16 %0, %1" ::"v"(a), "v"(v));
  };
  auto build_a = [&](int kt, const NmPack &p) {
    const uint32_t row = a_row(kt);
    build_zero(row);
#pragma unroll
    for (int e = 0; e < 16; ++e) build_entry(row, p, e);
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
  // prologue: stages 0 .. 2 built and loaded, the packed A of stage 3 in registers
  NmPack pa0, pa1;
#pragma unroll
  for (int st = 0; st < NS - 1; ++st)
    if (st < nk) {
      load_a(st, pa0);
      build_a(st, pa0);
    }
  if (NS - 1 < nk) load_a(NS - 1, pa1);
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

  // A step of the steady state (kt + 4 < nk): packed loads of stage kt + 4 into pl, build of
  // stage kt + 3 from pb. Issue order per step: packed loads, then B loads, so that at the
  // start of step kt the loads issued after stage kt + 1's B are step kt - 1's (LA + LPW),
  // and at the build those issued after stage kt + 3's packed loads are 2 LPW + LA.
  constexpr int RI = NM / NR;                    // a fragment read after every RI MFMAs
  constexpr int DI = NM / LPW;                   // a B load after every DI MFMAs
  // A step of the steady state (kt + 4 < nk). Issue order: the packed loads of stage kt + 4,
  // then (between the MFMAs of stage kt, with the fragment reads of stage kt + 1) the B loads
  // of stage kt + 3; after the MFMAs the A of stage kt + 3 is built from the registers
  // loaded in step kt - 1. So at the start of step kt the loads issued after stage kt + 1's B
  // are step kt - 1's (LA + LPW), and at the build those issued after stage kt + 3's packed
  // loads are 2 LPW + LA. (Interleaving the build with the MFMAs measured slower: with one
  // wave per SIMD its VALU work delays the MFMA issue.)
  auto step = [&](int kt, const FA &ac, const FB &bc, FA &an, FB &bn, NmPack &pl, const NmPack &pb) {
    wait_vmcnt<LA + LPW>();
    block_barrier_lds();
    load_a(kt + 4, pl);
    __builtin_amdgcn_sched_barrier(0);
    static_for<NM>([&](auto I) {
      constexpr int i = decltype(I)::value;
      mma(i, ac, bc);
      if constexpr (i % RI == 0 && i / RI < NR) read1(kt + 1, i / RI, an, bn);
      if constexpr (i % DI == DI - 1) issue_b(kt + 3, i / DI);
      __builtin_amdgcn_sched_barrier(0);
    });
    wait_vmcnt<2 * LPW + LA>();
    build_a(kt + 3, pb);
    __builtin_amdgcn_sched_barrier(0);
  };
  // The last steps (kt + 4 >= nk): what exists is issued, waits are complete ones, and the
  // next fragment set and packed registers are copied into the current ones afterwards.
  auto tail_step = [&](int kt) {
    wait_vmcnt<0>();
    block_barrier_lds();
    if (kt + 4 < nk) load_a(kt + 4, pa0);
    static_for<NM>([&](auto I) {
      constexpr int i = decltype(I)::value;
      mma(i, a0, b0);
      if constexpr (i % RI == 0 && i / RI < NR) read1(kt + 1, i / RI, a1, b1);
      __builtin_amdgcn_sched_barrier(0);
    });
    if (kt + 3 < nk) {
#pragma unroll
      for (int i = 0; i < LPW; ++i) issue_b(kt + 3, i);
      build_a(kt + 3, pa1);
    }
    wait_vmcnt<0>();
#pragma unroll
    for (int j = 0; j < FM; ++j) a0[j] = a1[j];
#pragma unroll
    for (int j = 0; j < FN; ++j) b0[j] = b1[j];
    pa1 = pa0;
  };
  int kt = 0;
  for (; kt + 5 < nk; kt += 2) {
    step(kt, a0, b0, a1, b1, pa0, pa1);          // loads stage kt + 4 (even parity) into pa0
    step(kt + 1, a1, b1, a0, b0, pa1, pa0);      // builds stage kt + 4 from pa0
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
  if (n == 8 && m == 16) hipLaunchKernelGGL((k_nm_down<8, 16>), grid, dim3(256), 0, s, v, idx, T, f, w, d, y, y_bf16);
  else hipLaunchKernelGGL((k_nm_down<16, 32>), grid, dim3(256), 0, s, v, idx, T, f, w, d, y, y_bf16);
  return hipGetLastError();
}

}  // namespace tw
