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
// y[t][c] = sum_k H[t][k] w2[k][c] with H expanded from (vals, idx) per 32-column stage and
// w2 [d_ff][d_model] (the down weight as the TwELL path reads it, so one copy serves both).
// Tile 256 tokens x 256 output columns, 8 waves of 64 x 128 (two per SIMD, so one wave's
// expansion and stores overlap the other's MFMAs), v_mfma_f32_16x16x32_bf16, a ring of four
// LDS stages, each A: 256 expanded H rows of 64 bytes (16-row fragments read with 16-byte
// loads from XOR-swizzled chunks, as in the up GEMM) and B: 32 rows of w2, 512 bytes each.
//  - B: the MFMA wants 8 consecutive k of one column per lane, while w2 rows run along the
//    columns, so its fragments are read with gfx950's transposing LDS load
//    (ds_read_b64_tr_b16): in each 16-lane group, lane a + 4 e points at row k0 + e, columns
//    4 a .. 4 a + 3, and lane i receives the four values of column i at rows k0 .. k0 + 3;
//    two such loads give 8 k. Row k's 16-byte chunk j sits at chunk j ^ (key(k) << 1),
//    key(k) = (k & 3) | ((k >> 3) & 3) << 2: the 16 rows one load touches (k = 8 q + e or
//    8 q + 4 + e, q, e < 4) get distinct even chunk offsets, so its 32 chunks fall on
//    distinct bank groups.
//    B travels through registers (two 16-byte buffer loads per thread and stage, then
//    16-byte LDS stores), not by buffer_load ... lds: the compiler cannot tell a transposing
//    read from a write of a pending LDS DMA and would wait for every DMA in flight before
//    each such read, which stalls the ring on the load just issued.
//  - A: tile row r is built by the neighbouring lanes 2r and 2r + 1. A stage of a row holds
//    32 N / M = 16 kept entries (8:16 and 16:32): each lane loads 8 values and 8 indices
//    (16 + 8 bytes; rows past T load as zeros through the buffer's range check), clears its
//    32-byte half of the row, then stores its values at their columns (which for 16:32 may
//    lie in either half). The two lanes are in one wave, whose LDS writes execute in issue
//    order, so both clears precede every value. The LDS byte of column c in row r is
//    2 (c ^ 8 swz(r)), swz(r) = (r >> 2) & 3, so each index byte becomes a byte offset with
//    one XOR and one shift per 4 indices, and a value's store address with one add.
//    These value stores are the kernel's largest cost beyond the GEMM itself (about 40 %
//    of its time at 4096 x 14336 x 4096): each takes one entry of 32 rows, and since the
//    t-th kept column of every row lies near column 2 t, the lanes of rows in one 16-bank
//    group meet in a bank (3.6 at a time on average). Stores of 4 or 8 rows with 16 or 8
//    lanes per row meet 1 or 2 at a time, but need 2- and 4-byte loads per entry (4 to 8
//    times the load instructions and twice the registers) or a pass through LDS; measured,
//    each of those was slower.
// Step kt: barrier (stage kt + 1 is in LDS, nobody reads stage kt - 1 any more); the A and
// B loads of stage kt + 3 into registers; the MFMAs of stage kt in B-fragment order, each
// B fragment reloaded with stage kt + 1 once its four MFMAs are issued, the A fragments of
// stage kt + 1 read early into the other A set; then stage kt + 3's A is built and its B
// stored into the buffer of stage kt - 1.
// Patterns: 8:16 and 16:32 (d_ff a multiple of 32).
typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s_t lds_v4s_t;
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

TW_DEV int nm_b_key(int k) { return (k & 3) | (((k >> 3) & 3) << 2); }

template <int N, int M>
__global__ __launch_bounds__(512) void k_nm_down(const uint16_t *__restrict__ vals, const uint8_t *__restrict__ idx,
                                                 int T, int f, const uint16_t *__restrict__ w2, int d,
                                                 void *__restrict__ y, int y_bf16) {
  static_assert(32 % M == 0 && 32 / M * N == 16, "16 kept entries per 32 columns");
  constexpr int BM = 256, BN = 256, RB = 64, NS = 4;
  constexpr int ASZ = BM * RB, BSZ = 32 * BN * 2, STAGE = ASZ + BSZ;
  constexpr int WM = 64, WN = 128, FM = WM / 16, FN = WN / 16, NM = FM * FN;
  __shared__ __attribute__((aligned(16))) char smem[NS * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int nk = f / 32;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char_t *)smem;

  // B: thread load i in {0, 1} of a stage is wave-load q = wave + 8 i, rows 2 q and 2 q + 1
  // of the stage; lane l stores LDS chunk l % 32 of row 2 q + l / 32, which holds the row's
  // global chunk (l % 32) ^ (key << 1). Columns past d read as zeros (range check).
  constexpr uint32_t OOB = 0x80000000u;
  const uint32_t wrow = (uint32_t)d * 2;
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc((void *)w2, (short)0, (int)((size_t)f * wrow), 0x00020000);
  uint32_t gb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int k = 2 * (wave + 8 * i) + (lane >> 5);
    const int col = n0 + 8 * ((lane & 31) ^ (nm_b_key(k) << 1));
    gb[i] = col < d ? (uint32_t)k * wrow + (uint32_t)col * 2 : OOB;
  }
  typedef u32x4_t PB[2];
  auto load_b = [&](int kt, PB &p) {
#pragma unroll
    for (int i = 0; i < 2; ++i) p[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, gb[i], kt * 32 * (int)wrow, 0);
  };
  auto store_b = [&](int kt, const PB &p) {
    const uint32_t base = lds0 + (uint32_t)((kt % NS) * STAGE + ASZ) + (uint32_t)lane * 16;
#pragma unroll
    for (int i = 0; i < 2; ++i)
      asm volatile("ds_write_b128 %0, %1" ::"v"(base + (uint32_t)(wave + 8 * i) * 1024), "v"(p[i]));
  };

  // A: tile row tid / 2; half hf = tid % 2 takes entries 8 hf .. 8 hf + 7 of each stage.
  const int arow = tid >> 1, hf = tid & 1;
  const uint32_t E = (uint32_t)f / M * N;                 // kept entries per row
  const uint32_t nrows = (uint32_t)min(BM, T - m0);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(vals + (size_t)m0 * E), (short)0, (int)(nrows * E * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t ri = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(idx + (size_t)m0 * E), (short)0, (int)(nrows * E), 0x00020000);
  const uint32_t gv = (uint32_t)arow * E * 2 + 16u * hf, gi = (uint32_t)arow * E + 8u * hf;
  struct PA {
    u32x4_t v;
    u32x2_t ix;
  };
  auto load_a = [&](int kt, PA &p) {
    p.v = __builtin_amdgcn_raw_buffer_load_b128(rv, gv, kt * 32, 0);
    p.ix = __builtin_amdgcn_raw_buffer_load_b64(ri, gi, kt * 16, 0);
  };
  // column c of the row sits at byte 2 (c ^ 8 swz): for 8:16 the half's columns are 16 hf +
  // idx, for 16:32 they are idx
  const int swz = (arow >> 2) & 3;
  const uint32_t xw = (M == 16 ? 8u * (uint32_t)(swz & 1) : 8u * (uint32_t)swz) * 0x01010101u;
  const uint32_t hb = M == 16 ? 32u * (uint32_t)(hf ^ (swz >> 1)) : 0u;
  constexpr uint32_t IM = (uint32_t)(M - 1) * 0x01010101u;
  // The stores are inline assembly so that they stay in issue order after the clears; the
  // LDS wait before every barrier covers them.
  auto build_a = [&](int kt, const PA &p) {
    const uint32_t row = lds0 + (uint32_t)((kt % NS) * STAGE + arow * RB);
    const u32x4_t z = {0u, 0u, 0u, 0u};
    const uint32_t h = row + 32u * (uint32_t)hf;
    asm volatile("ds_write_b128 %0, %1\n\tds_write_b128 %0, %1 offset:16" ::"v"(h), "v"(z));
    const uint32_t base = row + hb;
    const uint32_t w0 = ((p.ix.x & IM) ^ xw) << 1, w1 = ((p.ix.y & IM) ^ xw) << 1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t w = e < 4 ? w0 : w1;
      const uint32_t a = base + ((w >> (8 * (e & 3))) & 0xFFu);
      const uint32_t v = p.v[e >> 1];
      if (e & 1) asm volatile("ds_write_b16_d16_hi %0, %1" ::"v"(a), "v"(v));
      else asm volatile("ds_write_b16 %0, %1" ::"v"(a), "v"(v));
    }
  };

  // fragments
  typedef u32x4_t FA[FM];
  typedef u32x4_t FB[FN];
  const int l16 = lane & 15, c4 = lane >> 4;
  auto read_a = [&](int kt, int j, FA &a) {
    const int r = wm * WM + j * 16 + l16;
    a[j] = *(const u32x4_t *)(smem + (kt % NS) * STAGE + r * RB + ((c4 ^ ((r >> 2) & 3)) << 4));
  };
  // transposing B reads: lane l (group q = l / 16, source lane s = l % 16: a = s % 4,
  // e = s / 4) points at row 8 q + 4 half + e, columns 16 fn' + 4 a of the tile, fn' = wn *
  // 8 + fn, i.e. chunk 2 fn' + (a >> 1) at its swizzled place, byte (a & 1) * 8
  const int tq = lane >> 4, ta = lane & 3, te = (lane >> 2) & 3;
  uint32_t boff[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int k = 8 * tq + 4 * hh + te;
    boff[hh] = (uint32_t)(k * 512 + (((ta >> 1) ^ (nm_b_key(k) << 1)) << 4) + (ta & 1) * 8);
  }
  auto read_b = [&](int kt, int fn, FB &b) {
    // the stage offset sits above bit 13 and the fragment's chunk bits in bits 5 .. 8, so
    // XORing after the add equals adding after the XOR; XORing last keeps the address tied
    // to the stage, so it is formed at the read instead of held in a register per fragment
    const uint32_t so = (uint32_t)((kt % NS) * STAGE + ASZ);
    const uint32_t cx = (uint32_t)(2 * (wn * FN + fn)) << 4;
    const v4s_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t *)(smem + ((so + boff[0]) ^ cx)));
    const v4s_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s_t *)(smem + ((so + boff[1]) ^ cx)));
    const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
    b[fn] = u32x4_t{l2.x, l2.y, h2.x, h2.y};
  };
  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{};
  auto mma = [&](int fm, int fn, const FA &a, const FB &b) {
    acc[fm][fn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[fm]),
                                                          __builtin_bit_cast(bf16x8_t, b[fn]), acc[fm][fn], 0, 0, 0);
  };

  // prologue: stages 0 .. 2 built and stored, stage 0's fragments read
  {
    PA pa[NS - 1];
    PB pb[NS - 1];
#pragma unroll
    for (int st = 0; st < NS - 1; ++st)
      if (st < nk) {
        load_a(st, pa[st]);
        load_b(st, pb[st]);
      }
#pragma unroll
    for (int st = 0; st < NS - 1; ++st)
      if (st < nk) {
        build_a(st, pa[st]);
        store_b(st, pb[st]);
      }
  }
  block_barrier_lds();
  FA a0, a1;
  FB b;
#pragma unroll
  for (int j = 0; j < FM; ++j) read_a(0, j, a0);
#pragma unroll
  for (int j = 0; j < FN; ++j) read_b(0, j, b);

  // One step. LOAD: stage kt + 3 exists; NEXT: stage kt + 1 exists.
  PA pa;
  PB pb;
  auto step = [&](int kt, const FA &ac, FA &an, bool load, bool next) {
    block_barrier_lds();
    if (load) {
      load_a(kt + 3, pa);
      load_b(kt + 3, pb);
    }
    __builtin_amdgcn_sched_barrier(0);
    static_for<NM>([&](auto I) {
      constexpr int i = decltype(I)::value, fn = i / FM, fm = i % FM;
      mma(fm, fn, ac, b);
      if (next) {
        if constexpr (fm == FM - 1) read_b(kt + 1, fn, b);
        if constexpr (i % 2 == 0 && i / 2 < FM) read_a(kt + 1, i / 2, an);
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    if (load) {
      build_a(kt + 3, pa);
      store_b(kt + 3, pb);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  int kt = 0;
  for (; kt + 4 < nk; kt += 2) {
    step(kt, a0, a1, true, true);
    step(kt + 1, a1, a0, true, true);
  }
  for (; kt < nk; ++kt) {
    step(kt, a0, a1, kt + 3 < nk, kt + 1 < nk);
#pragma unroll
    for (int j = 0; j < FM; ++j) a0[j] = a1[j];
  }

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

hipError_t launch_nm_down(const void *vals, const uint8_t *idx, int T, int f, int n, int m, const void *w2, int d,
                          void *y, int y_bf16, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid((d + 255) / 256, (T + 255) / 256);
  const uint16_t *v = (const uint16_t *)vals, *w = (const uint16_t *)w2;
  if (n == 8 && m == 16) hipLaunchKernelGGL((k_nm_down<8, 16>), grid, dim3(512), 0, s, v, idx, T, f, w, d, y, y_bf16);
  else hipLaunchKernelGGL((k_nm_down<16, 32>), grid, dim3(512), 0, s, v, idx, T, f, w, d, y, y_bf16);
  return hipGetLastError();
}

}  // namespace tw
