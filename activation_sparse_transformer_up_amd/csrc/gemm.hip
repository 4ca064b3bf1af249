// Up projection of the activation-sparse FFN on gfx950 matrix cores (MFMA).
//
// "Sparser, Faster, Lighter Transformer Language Models", section "2. Metodologia",
// block "Formato de Dados TwELL": the up projection stays a dense GEMM, and the TwELL
// layout of its ReLU output is produced inside that GEMM's epilogue, so no separate
// conversion kernel and no synchronisation between workgroups is needed.
//
// z[t, j] = sum_i x[t, i] * w1t[j, i] (+ b1[j] in the epilogue). Both operands are
// K-contiguous ("NT"). A workgroup computes a BM x BN tile; each wave a WM x WN sub-tile
// made of 32x32 MFMA blocks with fp32 accumulators in registers.
//
// Operand staging: every K step moves 64 bytes of each operand row (32 bf16 or 16 fp32)
// = 4 chunks of 16 bytes straight from HBM into LDS (buffer_load ... lds: lane l of a
// wave writes bytes [16 l, 16 l + 16) of a 1 KB block), through a ring of NS stages, so
// that NS - 1 K steps of loads are in flight while one is multiplied. Rows past the
// operand's end and k past K are fetched as zeros by the buffer range check (no
// branches). Chunk c of LDS row r sits at position c ^ ((r >> 2) & 3): the 16 rows that
// one quarter-wave reads then start in 16 different bank groups.
//
// Accumulation order of one output element depends only on K and the fixed step order,
// not on the tile shape or the row's position, so every epilogue (TwELL, dense, backup
// rows) sees bit-identical z values.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "nmsel.h"
#include "rows.h"
#include "stage.h"

namespace tw {


template <typename T> struct MfmaOps;

// bf16: one v_mfma_f32_32x32x16_bf16 per step; lanes 0-31 bring one 16-byte chunk
// (8 k values), lanes 32-63 the next one.
template <> struct MfmaOps<uint16_t> {
  static constexpr int KPT = 32;   // k values per 64-byte row
  static TW_DEV void step(f32x16_t &acc, u32x4_t a, u32x4_t b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  }
};

// fp32: a 16-byte chunk holds 4 k values; four v_mfma_f32_32x32x2_f32 consume them, lane
// half h bringing k = 4h + s in the s-th one (A and B use the same assignment).
template <> struct MfmaOps<float> {
  static constexpr int KPT = 16;
  static TW_DEV void step(f32x16_t &acc, u32x4_t a, u32x4_t b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
};

template <int BM_, int BN_, int WM_, int WN_, int EPIW, int NS_ = 4, int MI_ = 32>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int NWM = BM / WM, NWN = BN / WN, NW = NWM * NWN, NT = NW * 64;
  static constexpr int MB = WM / 32, NB = WN / 32;
  // MFMA shape: 32 (v_mfma_f32_32x32x16_bf16 / 32x32x2_f32, f32x16_t accumulators per
  // 32 x 32 block) or 16 (v_mfma_f32_16x16x32_bf16, f32x4_t per 16 x 16 block: FM x FN)
  static constexpr int MI = MI_;
  static constexpr int FM = WM / 16, FN = WN / 16;
  static constexpr int RB = 64;                           // bytes of a row per K step
  static constexpr int NS = NS_;                          // pipeline stages
  static constexpr int STAGE = (BM + BN) * RB;            // bytes per stage (A rows, then B rows)
  static constexpr int LDS_BYTES = NS * STAGE;
  static constexpr int LPW = (BM + BN) / 16 / NW;         // 1 KB wave-loads per wave per stage
  static constexpr int EPI_WAVE = EPIW;                   // TwELL epilogue LDS per wave
  static constexpr int EPI_BYTES = NW * EPI_WAVE;
  static constexpr int SMEM = LDS_BYTES > EPI_BYTES ? LDS_BYTES : EPI_BYTES;
  static_assert((BM + BN) % (16 * NW) == 0 && BM % 16 == 0, "tile");
};

// TwELL epilogue LDS of one wave: slot indices and values for 32 rows x RS slots (+ one
// junk element per lane) and the counts. RS = (WN / W) * S slots per row.
constexpr int epi_wave_bytes(int rs, int tpw, int vbytes) {
  return ((4 * (32 * rs + 64) + vbytes * (32 * rs + 64) + 15) & ~15) + 4 * (32 * tpw + 64);
}

// Many tokens: 256 x 256 tiles. TileL8 has 8 waves of 64 x 128 (two per SIMD, so one
// wave's LDS and memory instructions overlap the other's MFMAs); its epilogue LDS allows
// up to 64 slots per row per wave. TileL (4 waves of 128 x 128) takes the larger slot
// counts (W = 64 with S > 32). Few tokens: 64 x 128 tiles. Waves are 128 columns wide so
// that a 64- or 128-wide TwELL tile never straddles two waves.
typedef Tile<256, 256, 64, 128, epi_wave_bytes(64, 2, 4), 4, 16> TileL8;
typedef Tile<256, 256, 128, 128, epi_wave_bytes(128, 2, 4), 4, 16> TileL;
typedef Tile<64, 128, 32, 128, epi_wave_bytes(128, 2, 4), 4, 16> TileS;
typedef Tile<64, 128, 32, 128, epi_wave_bytes(128, 2, 4)> TileSF;      // fp32 operands
// Decode (at most 64 tokens): one wave owns a 64 x 128 tile over a quarter of K with its
// own 6-stage ring (TileD); the quarters are added in a fixed order (decode section below).
typedef Tile<64, 128, 64, 128, epi_wave_bytes(128, 2, 4), 6> TileD;

// A operand row r of the tile reads global row arow[m0 + r] (if arow) or m0 + r; rows at or
// beyond a_rows are zero. B operand rows at or beyond b_rows are zero. a_total rows exist
// in A (bounds of the buffer resource). Operands must be smaller than 2 GiB.
// K split: the loop covers k in [kofs, kofs + K) of rows that are lda elements long (lda = 0:
// lda = K); vwave >= 0 makes the calling wave act as wave vwave of G (a wave running its
// own one-wave tile with its own smem ring passes 0).
//
// Software pipeline of one K step (two half-steps u = 0, 1 of 16 (bf16) k each):
//   read fragments (kt, u=1)    | MFMAs on fragments (kt, u=0)
//   wait for stage kt+1's loads, barrier
//   read fragments (kt+1, u=0)  | MFMAs on fragments (kt, u=1), with the loads of stage
//                                 kt+NS-1 issued between them
// so LDS reads are always one half-step ahead of the MFMAs that consume them. The stage
// overwritten by the loads issued after the barrier of step kt is (kt-1) mod NS, whose last
// fragments every wave has consumed before reaching that barrier.
template <typename T, class G>
TW_DEV void mainloop(const T *__restrict__ A, const int32_t *__restrict__ arow, int a_rows, int a_total,
                     const T *__restrict__ B, int b_rows, int K, int m0, int n0,
                     f32x16_t (&acc)[G::MB][G::NB], char *smem, int lda = 0, int kofs = 0, int vwave = -1) {
  static_assert(G::NS >= 3, "stages");
  constexpr int EPC = 16 / sizeof(T);                     // elements per 16-byte chunk
  constexpr int KPT = G::RB / sizeof(T);                  // k per stage
  constexpr int NMMA = G::MB * G::NB;
  constexpr uint32_t OOB = 0x80000000u;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = vwave >= 0 ? vwave : __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / G::NWN, wn = wave % G::NWN;
  const size_t row_bytes = (size_t)(lda ? lda : K) * sizeof(T);
  const size_t shift = (size_t)kofs * sizeof(T);
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(A + kofs), (short)0, (int)((size_t)a_total * row_bytes - shift), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(B + kofs), (short)0, (int)((size_t)b_rows * row_bytes - shift), 0x00020000);

  // This lane's part of each of its wave-loads: LDS row lr16 = l / 4 of a 16-row block,
  // physical chunk l % 4 holding logical chunk c.
  const int lrow = lane >> 2;
  const int cl = (lane & 3) ^ ((lrow >> 2) & 3);
  uint32_t voff[G::LPW];
  bool isA[G::LPW];
  int ldsq[G::LPW];
#pragma unroll
  for (int i = 0; i < G::LPW; ++i) {
    const int q = wave + G::NW * i;                       // 16-row block of [A rows; B rows]
    const int r = q * 16 + lrow;
    ldsq[i] = q * 1024;
    isA[i] = q * 16 < G::BM;                              // wave-uniform
    if (isA[i]) {
      const int gr = m0 + r;
      voff[i] = gr < a_rows ? (uint32_t)((size_t)(arow ? arow[gr] : gr) * row_bytes) + cl * 16 : OOB;
    } else {
      const int gr = n0 + (r - G::BM);
      voff[i] = gr < b_rows ? (uint32_t)((size_t)gr * row_bytes) + cl * 16 : OOB;
    }
  }
  const int nk = (K + KPT - 1) / KPT;
  const int kc = cl * EPC;                                // this lane's k offset in a stage

  auto issue1 = [&](int kt, int i) {
    const int k0 = kt * KPT;
    char *st = smem + (kt % G::NS) * G::STAGE;
    const uint32_t vo = (k0 + kc < K) ? voff[i] : OOB;
    lds_void_t *dst = (lds_void_t *)(st + ldsq[i]);
    if (isA[i]) __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, vo, k0 * (int)sizeof(T), 0, 0);
    else __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, dst, 16, vo, k0 * (int)sizeof(T), 0, 0);
  };
  const int lr = lane & 31, lh = lane >> 5;
  typedef u32x4_t FA[G::MB];
  typedef u32x4_t FB[G::NB];
  auto read = [&](int kt, int u, FA &a, FB &b) {
    const char *sa = smem + (kt % G::NS) * G::STAGE;
    const char *sb = sa + G::BM * G::RB;
    const int c = 2 * u + lh;
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb) {
      const int r = wm * G::WM + mb * 32 + lr;
      a[mb] = *(const u32x4_t *)(sa + r * G::RB + ((c ^ ((r >> 2) & 3)) << 4));
    }
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb) {
      const int r = wn * G::WN + nb * 32 + lr;
      b[nb] = *(const u32x4_t *)(sb + r * G::RB + ((c ^ ((r >> 2) & 3)) << 4));
    }
  };
  auto mma = [&](const FA &a, const FB &b) {
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb) MfmaOps<T>::step(acc[mb][nb], a[mb], b[nb]);
  };
  if (nk == 0) return;
#pragma unroll
  for (int s = 0; s < G::NS - 1; ++s)
    if (s < nk)
#pragma unroll
      for (int i = 0; i < G::LPW; ++i) issue1(s, i);
  if (nk >= G::NS - 1) wait_vmcnt<(G::NS - 2) * G::LPW>();
  else wait_vmcnt<0>();
  block_barrier();
  FA a0, a1;
  FB b0, b1;
  read(0, 0, a0, b0);
  // Step kt < nk - 1; LOAD: stage kt + NS - 1 exists and is loaded during this step. The
  // scheduling barriers keep the compiler from moving MFMAs across the phases.
  auto step = [&](int kt, auto load_tag) {
    constexpr bool LOAD = decltype(load_tag)::value;
    read(kt, 1, a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    mma(a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    if (LOAD) wait_vmcnt<(G::NS - 3) * G::LPW>();        // stage kt + 1 has landed
    else wait_vmcnt<0>();
    block_barrier_lds();
    read(kt + 1, 0, a0, b0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NMMA; ++i) {
      MfmaOps<T>::step(acc[i / G::NB][i % G::NB], a1[i / G::NB], b1[i % G::NB]);
      if (LOAD && (i & 1) && (i >> 1) < G::LPW) issue1(kt + G::NS - 1, i >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (LOAD)
#pragma unroll
      for (int i = NMMA / 2; i < G::LPW; ++i) issue1(kt + G::NS - 1, i);
    __builtin_amdgcn_sched_barrier(0);
  };
  int kt = 0;
  for (; kt + G::NS - 1 < nk; ++kt) step(kt, std::integral_constant<bool, true>());
  for (; kt + 1 < nk; ++kt) step(kt, std::integral_constant<bool, false>());
  read(kt, 1, a1, b1);
  __builtin_amdgcn_sched_barrier(0);
  mma(a0, b0);
  mma(a1, b1);
}

// The same operand staging with v_mfma_f32_16x16x32_bf16 (bf16 only; Tile::MI == 16). A
// 16 x 16 x 32 MFMA takes a 16-row block of a whole stage (16 rows x 32 k: lane l reads row
// l % 16, 16-byte chunk l / 16), so each stage is read as FM + FN fragments. Against the
// 32 x 32 x 16 form the accumulator traffic per multiply-add halves, which lowers the power
// of the loop and so raises the clock the chip sustains under it (the K loop is
// power-limited on gfx950). One barrier per stage:
//   wait for stage kt + 1's loads, barrier
//   MFMAs on the fragments of stage kt, interleaved with the reads of stage kt + 1 (into
//   the other fragment set) and with the loads of stage kt + NS - 1
// The stage overwritten by those loads, (kt - 1) mod NS, was read during step kt - 2.
template <class G>
TW_DEV void mainloop16(const uint16_t *__restrict__ A, const int32_t *__restrict__ arow, int a_rows, int a_total,
                       const uint16_t *__restrict__ B, int b_rows, int K, int m0, int n0,
                       f32x4_t (&acc)[G::FM][G::FN], char *smem) {
  static_assert(G::NS >= 3 && G::MI == 16, "stages / shape");
  constexpr int KPT = G::RB / 2;                          // k per stage
  constexpr int NM = G::FM * G::FN;                       // MFMAs per stage
  constexpr int NR = G::FM + G::FN;                       // fragment reads per stage
  constexpr int RI = NM / NR >= 2 ? NM / NR : 1;          // a read after every RI MFMAs
  constexpr int DI = NM / G::LPW >= 1 ? NM / G::LPW : 1;  // a stage load after every DI MFMAs
  constexpr uint32_t OOB = 0x80000000u;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / G::NWN, wn = wave % G::NWN;
  const size_t row_bytes = (size_t)K * 2;
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void *)A, (short)0, (int)((size_t)a_total * row_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc((void *)B, (short)0, (int)((size_t)b_rows * row_bytes), 0x00020000);
  // stage loads: as in mainloop (LDS row lrow of a 16-row block, physical chunk cl)
  const int lrow = lane >> 2;
  const int cl = (lane & 3) ^ ((lrow >> 2) & 3);
  uint32_t voff[G::LPW];
  bool isA[G::LPW];
  int ldsq[G::LPW];
#pragma unroll
  for (int i = 0; i < G::LPW; ++i) {
    const int q = wave + G::NW * i;
    const int r = q * 16 + lrow;
    ldsq[i] = q * 1024;
    isA[i] = q * 16 < G::BM;
    if (isA[i]) {
      const int gr = m0 + r;
      voff[i] = gr < a_rows ? (uint32_t)((size_t)(arow ? arow[gr] : gr) * row_bytes) + cl * 16 : OOB;
    } else {
      const int gr = n0 + (r - G::BM);
      voff[i] = gr < b_rows ? (uint32_t)((size_t)gr * row_bytes) + cl * 16 : OOB;
    }
  }
  const int nk = (K + KPT - 1) / KPT;
  const int kc = cl * 8;
  auto issue1 = [&](int kt, int i) {
    const int k0 = kt * KPT;
    char *st = smem + (kt % G::NS) * G::STAGE;
    const uint32_t vo = (k0 + kc < K) ? voff[i] : OOB;
    lds_void_t *dst = (lds_void_t *)(st + ldsq[i]);
    if (isA[i]) __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, vo, k0 * 2, 0, 0);
    else __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, dst, 16, vo, k0 * 2, 0, 0);
  };
  typedef u32x4_t FA[G::FM];
  typedef u32x4_t FB[G::FN];
  const int l16 = lane & 15, c4 = lane >> 4;
  // fragment j of stage kt: j < FM the A block j, else the B block j - FM
  auto read1 = [&](int kt, int j, FA &a, FB &b) {
    const char *sa = smem + (kt % G::NS) * G::STAGE;
    if (j < G::FM) {
      const int r = wm * G::WM + j * 16 + l16;
      a[j] = *(const u32x4_t *)(sa + r * G::RB + ((c4 ^ ((r >> 2) & 3)) << 4));
    } else {
      const int r = wn * G::WN + (j - G::FM) * 16 + l16;
      b[j - G::FM] = *(const u32x4_t *)(sa + G::BM * G::RB + r * G::RB + ((c4 ^ ((r >> 2) & 3)) << 4));
    }
  };
  auto mma = [&](int i, const FA &a, const FB &b) {
    acc[i / G::FN][i % G::FN] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        __builtin_bit_cast(bf16x8_t, a[i / G::FN]), __builtin_bit_cast(bf16x8_t, b[i % G::FN]),
        acc[i / G::FN][i % G::FN], 0, 0, 0);
  };
  if (nk == 0) return;
#pragma unroll
  for (int st = 0; st < G::NS - 1; ++st)
    if (st < nk)
#pragma unroll
      for (int i = 0; i < G::LPW; ++i) issue1(st, i);
  if (nk >= G::NS - 1) wait_vmcnt<(G::NS - 2) * G::LPW>();
  else wait_vmcnt<0>();
  block_barrier();
  FA a0, a1;
  FB b0, b1;
#pragma unroll
  for (int j = 0; j < NR; ++j) read1(0, j, a0, b0);
  // step kt < nk - 1: MFMAs on (ac, bc) = stage kt, reads of stage kt + 1 into (an, bn);
  // LOAD: stage kt + NS - 1 exists and is loaded in this step
  auto step = [&](int kt, const FA &ac, const FB &bc, FA &an, FB &bn, auto load_tag) {
    constexpr bool LOAD = decltype(load_tag)::value;
    if (LOAD) wait_vmcnt<(G::NS - 3) * G::LPW>();          // stage kt + 1 has landed
    else wait_vmcnt<0>();
    block_barrier_lds();
    __builtin_amdgcn_sched_barrier(0);
    static_for<NM>([&](auto I) {
      constexpr int i = decltype(I)::value;
      mma(i, ac, bc);
      if constexpr (i % RI == 0 && i / RI < NR) read1(kt + 1, i / RI, an, bn);
      if constexpr (LOAD && i % DI == DI - 1 && i / DI < G::LPW) issue1(kt + G::NS - 1, i / DI);
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (NM / RI < NR)
#pragma unroll
      for (int j = NM / RI; j < NR; ++j) read1(kt + 1, j, an, bn);
    if constexpr (LOAD && NM / DI < G::LPW)
#pragma unroll
      for (int i = NM / DI; i < G::LPW; ++i) issue1(kt + G::NS - 1, i);
    __builtin_amdgcn_sched_barrier(0);
  };
  const std::integral_constant<bool, true> ld;
  const std::integral_constant<bool, false> nold;
  auto settle = [&]() {                   // next fragment set -> current (tail steps only)
#pragma unroll
    for (int j = 0; j < G::FM; ++j) a0[j] = a1[j];
#pragma unroll
    for (int j = 0; j < G::FN; ++j) b0[j] = b1[j];
  };
  // Steps kt < nl load stage kt + NS - 1; the last NS - 2 steps (fewer if nk is small) do
  // not. Loading steps run in pairs (the fragment sets alternate); an odd one and the
  // non-loading ones copy the next set into the current one after the step.
  const int nl = nk >= G::NS ? nk - G::NS + 1 : 0;
  int kt = 0;
  for (; kt + 1 < nl; kt += 2) {
    step(kt, a0, b0, a1, b1, ld);
    step(kt + 1, a1, b1, a0, b0, ld);
  }
  if (kt < nl) {
    step(kt, a0, b0, a1, b1, ld);
    settle();
    ++kt;
  }
  for (; kt + 1 < nk; ++kt) {
    step(kt, a0, b0, a1, b1, nold);
    settle();
  }
#pragma unroll
  for (int i = 0; i < NM; ++i) mma(i, a0, b0);
}

// 16-byte copy from LDS to global memory with a nontemporal store (the TwELL output is not
// read again by this kernel, so it should not displace operand lines in L2).
typedef int i32x4_t __attribute__((ext_vector_type(4)));
TW_DEV void st_nt16(void *dst, const void *src) {
  __builtin_nontemporal_store(*(const i32x4_t *)src, (i32x4_t *)dst);
}

// Output position of accumulator register r of a 32x32 block, for this lane:
//   row = 8 * (r / 4) + 4 * (lane / 32) + r % 4,   col = lane % 32.
TW_DEV int acc_row(int r, int lh) { return 8 * (r >> 2) + 4 * lh + (r & 3); }

// ---------------------------------------------------------------- TwELL epilogue
// "Formato de Dados TwELL": per (row, tile) the wave ballots h > 0 over the tile's columns
// (each 32x32 block contributes 32 columns of two rows: lanes 0-31 one row, lanes 32-63
// the row 4 below), the popcount is the count, and a lane's slot is the number of set
// bits of lower columns. Slots below S receive (column, value); the rest are padded.
// A row-tile with count > S sets its row's bit in ovf_bits[tile][row / 32].
//
// At one wave per SIMD every instruction costs a full issue slot and scalar<->vector
// dependencies stall, so the work per 32-column block is a handful of independent vector
// operations: the lane's half of the ballot, a popcount of the lower bits (slot) and of
// all bits (running count). Per 32-row block the wave fills its LDS copy of the slot
// blocks with the pad pattern, writes the active (column, value) pairs into their slots
// (lanes with nothing to write hit a private junk word, so no branches), and copies the
// block out with 16-byte stores. Blocks whose ballot is empty are skipped (a scalar test).
template <class G, int W, typename VT>
TW_DEV void epi_twell(f32x16_t (&acc)[G::MB][G::NB], const float (&nbias)[G::NB], int M, int N,
                      int m0, int n0, const TwellOut &o, char *smem, int only_mb = -1) {
  constexpr int BPT = W / 32;                   // 32-column blocks per TwELL tile
  constexpr int TPW = G::WN / W;                // TwELL tiles per wave
  static_assert(G::WN % W == 0, "a TwELL tile must sit inside one wave");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // only_mb >= 0: this wave packs only 32-row block only_mb of a one-wave-wide tile (the
  // tile's other blocks are packed by other waves), in its own LDS area
  const int wm = only_mb >= 0 ? 0 : wave / G::NWN, wn = only_mb >= 0 ? 0 : wave % G::NWN;
  const int lh = lane >> 5, li = lane & 31;
  const int row0 = m0 + wm * G::WM, col0 = n0 + wn * G::WN;
  const int S = o.S;
  const int kt0 = col0 / W;
  const int tiles = min(TPW, o.n_t - kt0);      // tiles of this wave inside the matrix
  if (tiles <= 0) return;
  const int RS = TPW * S;                        // LDS slots per row (all tiles of the wave)
  // wave-private LDS (<= 32 KB): idx [32][RS] + junk[64] | vals [32][RS] + junk[64] |
  // counts [32][TPW] + junk[64]
  char *base = smem + wave * G::EPI_WAVE;
  int32_t *lidx = (int32_t *)base;
  VT *lval = (VT *)(lidx + 32 * RS + 64);
  int32_t *lcnt = (int32_t *)(base + ((4 * (32 * RS + 64) + (int)sizeof(VT) * (32 * RS + 64) + 15) & ~15));
  const int JI = 32 * RS + lane;                 // this lane's junk element in lidx / lval
  const uint32_t below = (1u << li) - 1u;
  const bool vec_ok = (S * (int)sizeof(VT)) % 16 == 0;
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb) {
    if (only_mb >= 0 && mb != only_mb) continue;  // wave-uniform
    const int rb0 = row0 + mb * 32;
    if (rb0 >= M) break;                         // wave-uniform
    // 1. pad pattern
    for (int i = lane; i < 32 * RS / 4; i += 64) ((int4 *)lidx)[i] = make_int4(-1, -1, -1, -1);
    for (int i = lane; i < 32 * RS * (int)sizeof(VT) / 16; i += 64) ((int4 *)lval)[i] = make_int4(0, 0, 0, 0);
    wave_lds_order();
    // 2. active units -> slots
    uint32_t ovfv[TPW];                          // rows of this lane's half that overflow
#pragma unroll
    for (int q = 0; q < TPW; ++q) ovfv[q] = 0;
#pragma unroll
    for (int q = 0; q < TPW; ++q) {
      const int kt = kt0 + q;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lrow = 8 * (r >> 2) + (r & 3) + 4 * lh;    // row of this lane in the block
        int pre = 0;                                          // this lane's row: count so far
#pragma unroll
        for (int b = 0; b < BPT; ++b) {
          const int nb = q * BPT + b;
          const float zb = acc[mb][nb][r];
          const bool on = zb > nbias[nb];
          const uint64_t bal = ballot64(on);
          if (bal == 0) continue;                             // wave-uniform
          const uint32_t hm = lh ? (uint32_t)(bal >> 32) : (uint32_t)bal;
          const int slot = pre + __popc(hm & below);
          const bool act = on && slot < S;
          const int e = act ? lrow * RS + q * S + slot : JI;
          lidx[e] = kt * W + b * 32 + li;
          Elem<VT>::store(lval, e, zb - nbias[nb]);
          pre += __popc(hm);
        }
        const int e = li == 0 ? lrow * TPW + q : 32 * TPW + lane;
        lcnt[e] = pre;
        ovfv[q] |= (pre > S ? 1u : 0u) << lrow;
      }
    }
    wave_lds_order();
    // 3. copy out rows rb0 .. rb0 + 31: row r's slots of tiles kt0 .. kt0 + tiles - 1 are
    //    contiguous in the output (tiles * S elements at (row * n_t + kt0) * S)
    const int nrow = min(32, M - rb0);
    const int relem = tiles * S;
    if (vec_ok) {
      const int ci = relem / 4, cv = relem * (int)sizeof(VT) / 16;   // 16-byte chunks per row
      for (int i = lane; i < nrow * ci; i += 64) {
        const int rr = i / ci, c = i - rr * ci;
        const size_t g = ((size_t)(rb0 + rr) * o.n_t + kt0) * S;
        st_nt16(o.col_idx + g + 4 * c, lidx + rr * RS + 4 * c);
      }
      constexpr int EV = 16 / sizeof(VT);
      for (int i = lane; i < nrow * cv; i += 64) {
        const int rr = i / cv, c = i - rr * cv;
        const size_t g = ((size_t)(rb0 + rr) * o.n_t + kt0) * S;
        st_nt16((VT *)o.vals + g + EV * c, lval + rr * RS + EV * c);
      }
    } else {
      for (int i = lane; i < nrow * relem; i += 64) {
        const int rr = i / relem, c = i - rr * relem;
        const size_t g = ((size_t)(rb0 + rr) * o.n_t + kt0) * S + c;
        o.col_idx[g] = lidx[rr * RS + c];
        ((VT *)o.vals)[g] = lval[rr * RS + c];
      }
    }
    for (int i = lane; i < nrow * tiles; i += 64) {
      const int rr = i / tiles, c = i - rr * tiles;
      o.counts[(size_t)(rb0 + rr) * o.n_t + kt0 + c] = lcnt[rr * TPW + c];
    }
    // overflow words: lanes 0 / 32 hold the bits of rows 8i+{0..3} / 8i+{4..7}
    const uint32_t valid = nrow >= 32 ? 0xFFFFFFFFu : ((1u << nrow) - 1u);
#pragma unroll
    for (int q = 0; q < TPW; ++q) {
      const uint32_t word = (uint32_t)__builtin_amdgcn_readlane((int)ovfv[q], 0) |
                            (uint32_t)__builtin_amdgcn_readlane((int)ovfv[q], 32);
      if (q < tiles && lane == 0) o.ovf_bits[(size_t)(kt0 + q) * o.words + (rb0 >> 5)] = word & valid;
    }
    wave_lds_order();
  }
}

// The TwELL epilogue on 16 x 16 accumulator blocks (Tile::MI == 16): register i of block
// (fm, fn) holds row fm * 16 + 4 * (lane / 16) + i, column fn * 16 + lane % 16, so one
// ballot covers 16 columns of four rows (lane group g = lane / 16 owns row 4 g + i). The
// steps per 16-row block are those of epi_twell: pad the LDS slot block, scatter the active
// (column, value) pairs into their slots, copy the block out with 16-byte stores. Overflow
// bits are gathered per 32-row word over two 16-row blocks.
template <class G, int W, typename VT>
TW_DEV void epi_twell16(f32x4_t (&acc)[G::FM][G::FN], const float (&nbias)[G::FN], int M, int N, int m0,
                        int n0, const TwellOut &o, char *smem) {
  constexpr int BPT = W / 16;                   // 16-column blocks per TwELL tile
  constexpr int TPW = G::WN / W;                // TwELL tiles per wave
  static_assert(G::WN % W == 0 && G::FM % 2 == 0, "a TwELL tile must sit inside one wave");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / G::NWN, wn = wave % G::NWN;
  const int g = lane >> 4, li = lane & 15;
  const int row0 = m0 + wm * G::WM, col0 = n0 + wn * G::WN;
  const int S = o.S;
  const int kt0 = col0 / W;
  const int tiles = min(TPW, o.n_t - kt0);
  if (tiles <= 0) return;
  const int RS = TPW * S;
  // wave-private LDS at fixed offsets (so that a slot's value sits VOFF bytes after its column
  // for fp32 values, one address for both stores): idx [16][RS] + junk[64] at 0 | vals
  // [16][RS] + junk[64] at VOFF | counts [16][TPW] + junk[64] at 2 VOFF. RSX is the largest RS
  // the wave's EPI_WAVE bytes hold (epi_wave_bytes(RSX / 2, 2, 4)); the host keeps RS <= RSX.
  constexpr int RSX = (G::EPI_WAVE - 1024) / 128;
  static_assert(epi_wave_bytes(RSX / 2, 2, 4) == G::EPI_WAVE, "epilogue LDS layout");
  constexpr int VOFF = 4 * (16 * RSX + 64);
  char *base = smem + wave * G::EPI_WAVE;
  int32_t *lidx = (int32_t *)base;
  VT *lval = (VT *)(base + VOFF);
  int32_t *lcnt = (int32_t *)(base + 2 * VOFF);
  const int JI = 16 * RS + lane;
  const int jaddr = 4 * JI;                                    // this lane's junk word
  const uint32_t below = (1u << li) - 1u;
  const bool vec_ok = (S * (int)sizeof(VT)) % 16 == 0;
  // copy-out positions: the lane's first (row, 16-byte chunk) and the step between its
  // chunks i and i + 64, divided once here (the chunk counts per row are runtime values)
  const int relem = tiles * S;
  const int ci = relem / 4, cv = relem * (int)sizeof(VT) / 16;   // 16-byte chunks per row
  const int ri0 = vec_ok ? lane / ci : 0, ci0 = vec_ok ? lane - ri0 * ci : 0;
  const int rq = vec_ok ? 64 / ci : 0, rm = vec_ok ? 64 - rq * ci : 0;
  const int rv0 = vec_ok ? lane / cv : 0, cv0 = vec_ok ? lane - rv0 * cv : 0;
  const int vq = vec_ok ? 64 / cv : 0, vm = vec_ok ? 64 - vq * cv : 0;
  uint32_t ovfv[TPW];                            // overflow bits of this lane's rows, 32-row word
  int colv[TPW][BPT];                            // this lane's column in each 16-column block
#pragma unroll
  for (int q = 0; q < TPW; ++q)
#pragma unroll
    for (int b = 0; b < BPT; ++b) colv[q][b] = (kt0 + q) * W + b * 16 + li;
#pragma unroll
  for (int fm = 0; fm < G::FM; ++fm) {
    const int rb0 = row0 + fm * 16;
    if (rb0 >= M) break;                         // wave-uniform
    if (fm % 2 == 0)
#pragma unroll
      for (int q = 0; q < TPW; ++q) ovfv[q] = 0;
    for (int i = lane; i < 16 * RS / 4; i += 64) ((int4 *)lidx)[i] = make_int4(-1, -1, -1, -1);
    for (int i = lane; i < 16 * RS * (int)sizeof(VT) / 16; i += 64) ((int4 *)lval)[i] = make_int4(0, 0, 0, 0);
    wave_lds_order();
#pragma unroll
    for (int q = 0; q < TPW; ++q) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int lrow = 4 * g + r;                           // row of this lane in the block
        // the running slot counts from the word of slot 0 of (row, tile), so a slot's word is
        // `slot` and the budget test compares with `lim`
        const int row0w = lrow * RS + q * S, lim = row0w + S;
        int pre = row0w;
#pragma unroll
        for (int b = 0; b < BPT; ++b) {
          const int nb = q * BPT + b;
          const float zb = acc[fm][nb][r];
          const bool on = zb > nbias[nb];
          const uint64_t bal = ballot64(on);
          if (bal == 0) continue;                             // wave-uniform
          const uint32_t hm = (uint32_t)(bal >> (16 * g)) & 0xFFFFu;
          const int slot = pre + __popc(hm & below);
          const int a = (on && slot < lim) ? 4 * slot : jaddr;   // byte of the slot's column
          *(int32_t *)(base + a) = colv[q][b];
          if constexpr (sizeof(VT) == 4) *(float *)(base + VOFF + a) = zb - nbias[nb];
          else *(uint16_t *)(base + VOFF + (a >> 1)) = (uint16_t)f32_to_bf16(zb - nbias[nb]);
          pre += __popc(hm);
        }
        pre -= row0w;
        const int e = li == 0 ? lrow * TPW + q : 16 * TPW + lane;
        lcnt[e] = pre;
        ovfv[q] |= (pre > S ? 1u : 0u) << ((fm & 1) * 16 + lrow);
      }
    }
    wave_lds_order();
    const int nrow = min(16, M - rb0);
    if (vec_ok) {
      for (int i = lane, rr = ri0, c = ci0; i < nrow * ci; i += 64) {
        const size_t gi = ((size_t)(rb0 + rr) * o.n_t + kt0) * S;
        st_nt16(o.col_idx + gi + 4 * c, lidx + rr * RS + 4 * c);
        rr += rq;
        c += rm;
        if (c >= ci) {
          c -= ci;
          ++rr;
        }
      }
      constexpr int EV = 16 / sizeof(VT);
      for (int i = lane, rr = rv0, c = cv0; i < nrow * cv; i += 64) {
        const size_t gi = ((size_t)(rb0 + rr) * o.n_t + kt0) * S;
        st_nt16((VT *)o.vals + gi + EV * c, lval + rr * RS + EV * c);
        rr += vq;
        c += vm;
        if (c >= cv) {
          c -= cv;
          ++rr;
        }
      }
    } else {
      for (int i = lane; i < nrow * relem; i += 64) {
        const int rr = i / relem, c = i - rr * relem;
        const size_t gi = ((size_t)(rb0 + rr) * o.n_t + kt0) * S + c;
        o.col_idx[gi] = lidx[rr * RS + c];
        ((VT *)o.vals)[gi] = lval[rr * RS + c];
      }
    }
    if constexpr (TPW == 1) {
      if (lane < nrow) o.counts[(size_t)(rb0 + lane) * o.n_t + kt0] = lcnt[lane];
    } else {
      for (int i = lane; i < nrow * tiles; i += 64) {
        const int rr = i / tiles, c = i - rr * tiles;
        o.counts[(size_t)(rb0 + rr) * o.n_t + kt0 + c] = lcnt[rr * TPW + c];
      }
    }
    // after the second 16-row block of a 32-row word (or the last block inside the matrix)
    const bool last = fm == G::FM - 1 || rb0 + 16 >= M;
    if (fm % 2 == 1 || last) {
      const int wb0 = rb0 - (fm & 1) * 16;                    // first row of the word
      const int nw = min(32, M - wb0);
      const uint32_t valid = nw >= 32 ? 0xFFFFFFFFu : ((1u << nw) - 1u);
#pragma unroll
      for (int q = 0; q < TPW; ++q) {
        const uint32_t word = (uint32_t)__builtin_amdgcn_readlane((int)ovfv[q], 0) |
                              (uint32_t)__builtin_amdgcn_readlane((int)ovfv[q], 16) |
                              (uint32_t)__builtin_amdgcn_readlane((int)ovfv[q], 32) |
                              (uint32_t)__builtin_amdgcn_readlane((int)ovfv[q], 48);
        if (q < tiles && lane == 0) o.ovf_bits[(size_t)(kt0 + q) * o.words + (wb0 >> 5)] = word & valid;
      }
    }
    wave_lds_order();
  }
}

// ---------------------------------------------------------------- dense epilogue
// out[orow][col] = ReLU(z + b1) (or z + b1 without ReLU), fp32 or bf16, orow = tile row.
template <class G>
TW_DEV void epi_dense(f32x16_t (&acc)[G::MB][G::NB], const float *__restrict__ b1, int rows_valid,
                      int N, int m0, int n0, void *out, int out_bf16, int relu) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / G::NWN, wn = wave % G::NWN;
  const int lh = lane >> 5, li = lane & 31;
  const int row0 = m0 + wm * G::WM, col0 = n0 + wn * G::WN;
#pragma unroll
  for (int nb = 0; nb < G::NB; ++nb) {
    const int col = col0 + nb * 32 + li;
    if (col >= N) continue;
    const float bias = b1 ? b1[col] : 0.f;
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + mb * 32 + acc_row(r, lh);
        if (row >= rows_valid) continue;
        float z = acc[mb][nb][r] + bias;
        if (relu) z = z > 0.f ? z : 0.f;
        const size_t i = (size_t)row * N + col;
        if (out_bf16) ((uint16_t *)out)[i] = (uint16_t)f32_to_bf16(z);
        else ((float *)out)[i] = z;
      }
    }
  }
}

// epi_dense on 16 x 16 accumulator blocks (Tile::MI == 16).
template <class G>
TW_DEV void epi_dense16(f32x4_t (&acc)[G::FM][G::FN], const float *__restrict__ b1, int rows_valid, int N,
                        int m0, int n0, void *out, int out_bf16, int relu) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / G::NWN, wn = wave % G::NWN;
  const int g = lane >> 4, li = lane & 15;
  const int row0 = m0 + wm * G::WM, col0 = n0 + wn * G::WN;
#pragma unroll
  for (int fn = 0; fn < G::FN; ++fn) {
    const int col = col0 + fn * 16 + li;
    if (col >= N) continue;
    const float bias = b1 ? b1[col] : 0.f;
#pragma unroll
    for (int fm = 0; fm < G::FM; ++fm) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + fm * 16 + 4 * g + r;
        if (row >= rows_valid) continue;
        float z = acc[fm][fn][r] + bias;
        if (relu) z = z > 0.f ? z : 0.f;
        const size_t i = (size_t)row * N + col;
        if (out_bf16) ((uint16_t *)out)[i] = (uint16_t)f32_to_bf16(z);
        else ((float *)out)[i] = z;
      }
    }
  }
}

// ---------------------------------------------------------------- N:M epilogue
// "Motivating Next-Gen Accelerators with Flexible (N:M) Activation Sparsity ...", section
// "2. Metodologia": the activations are pruned to N:M by magnitude. Fused here into the up
// GEMM so that the dense h never goes to HBM: the workgroup's tile of h = ReLU(z + b1) is
// rounded to the output type and staged in LDS ([BM][BN], rows padded by 16 bytes), then
// every thread takes whole blocks of M columns. bf16 blocks: the kept set comes as a mask
// (nm_kept_mask), walked in ascending order by count-leading-zeros; the kept values are
// re-read from LDS and stored with the packed indices straight from registers. fp32 blocks:
// nm_keep32, then the kept (value, index) pairs are compacted in place over the block's own
// LDS bytes and copied out. h is formed exactly as the dense epilogue forms it, so the
// result equals the standalone pruning of ffn_up_relu_dense's output bit for bit.
template <typename HT> TW_DEV void put_h(char *p, float z) {
  z = z > 0.f ? z : 0.f;
  if constexpr (sizeof(HT) == 2) *(uint16_t *)p = (uint16_t)f32_to_bf16(z);
  else *(float *)p = z;
}

template <class G, typename HT> constexpr int nm_row_bytes() { return G::BN * (int)sizeof(HT) + 16; }
template <class G, typename HT> constexpr int nm_stage_bytes() { return G::BM * nm_row_bytes<G, HT>(); }

// 16 x 16 accumulator blocks: register i of block (fm, fn) is row fm * 16 + 4 (lane / 16) + i,
// column fn * 16 + lane % 16 of the wave's sub-tile.
template <class G, typename HT>
TW_DEV void stage_h16(const f32x4_t (&acc)[G::FM][G::FN], const float *__restrict__ b1, int N, int n0, char *lds) {
  constexpr int RS = nm_row_bytes<G, HT>();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / G::NWN, wn = wave % G::NWN;
  const int g = lane >> 4, li = lane & 15;
#pragma unroll
  for (int fn = 0; fn < G::FN; ++fn) {
    const int ct = wn * G::WN + fn * 16 + li;
    const float bias = n0 + ct < N ? b1[n0 + ct] : 0.f;
#pragma unroll
    for (int fm = 0; fm < G::FM; ++fm)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        put_h<HT>(lds + (wm * G::WM + fm * 16 + 4 * g + r) * RS + ct * (int)sizeof(HT), acc[fm][fn][r] + bias);
  }
}

// 32 x 32 accumulator blocks (register r of block (mb, nb): row acc_row(r, lane / 32), column
// lane % 32).
template <class G, typename HT>
TW_DEV void stage_h32(const f32x16_t (&acc)[G::MB][G::NB], const float *__restrict__ b1, int N, int n0, char *lds) {
  constexpr int RS = nm_row_bytes<G, HT>();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / G::NWN, wn = wave % G::NWN;
  const int lh = lane >> 5, li = lane & 31;
#pragma unroll
  for (int nb = 0; nb < G::NB; ++nb) {
    const int ct = wn * G::WN + nb * 32 + li;
    const float bias = n0 + ct < N ? b1[n0 + ct] : 0.f;
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        put_h<HT>(lds + (wm * G::WM + mb * 32 + acc_row(r, lh)) * RS + ct * (int)sizeof(HT), acc[mb][nb][r] + bias);
  }
}

// Copy NB bytes (a power of two, both sides NB-aligned up to 16) with the widest accesses.
template <int NB> TW_DEV void copy_bytes(char *dst, const char *src) {
  if constexpr (NB % 16 == 0) {
#pragma unroll
    for (int i = 0; i < NB / 16; ++i) ((uint4 *)dst)[i] = ((const uint4 *)src)[i];
  } else if constexpr (NB == 8) {
    *(uint2 *)dst = *(const uint2 *)src;
  } else if constexpr (NB == 4) {
    *(uint32_t *)dst = *(const uint32_t *)src;
  } else {
    static_assert(NB == 2, "size");
    *(uint16_t *)dst = *(const uint16_t *)src;
  }
}

// Store NB bytes (a power of two, dst NB-aligned up to 16) from packed words.
template <int NB, int NW> TW_DEV void store_words(char *dst, const uint32_t (&w)[NW]) {
  if constexpr (NB % 16 == 0) {
#pragma unroll
    for (int i = 0; i < NB / 16; ++i) ((uint4 *)dst)[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
  } else if constexpr (NB == 8) {
    *(uint2 *)dst = make_uint2(w[0], w[1]);
  } else if constexpr (NB == 4) {
    *(uint32_t *)dst = w[0];
  } else {
    static_assert(NB == 2, "size");
    *(uint16_t *)dst = (uint16_t)w[0];
  }
}

// Select the blocks of the staged tile (rows m0 .., columns n0 ..; rows at or beyond
// rows_valid and columns at or beyond N are skipped; N is a multiple of M). Outputs
// vals / idx [rows][N / M][NK]. Consecutive threads take consecutive blocks of a row, so the
// copies of a wave are contiguous.
template <typename HT, int NK, int M, int BM, int BN, int NT>
TW_DEV void nm_tile(char *lds, int rows_valid, int N, int m0, int n0, HT *__restrict__ vals,
                    uint8_t *__restrict__ idx) {
  constexpr int RS = BN * (int)sizeof(HT) + 16;
  constexpr int GPR = BN / M;                       // blocks per tile row
  constexpr int GB = M * (int)sizeof(HT);           // bytes of a block
  constexpr int VB = NK * (int)sizeof(HT);          // bytes of its kept values (= GB / 2)
  static_assert(BN % M == 0 && 2 * NK == M, "blocks");
  const int bpr = N / M;
  for (int gi = threadIdx.x; gi < BM * GPR; gi += NT) {
    const int r = gi / GPR, q = gi - r * GPR;
    const int row = m0 + r, col = n0 + q * M;
    if (row >= rows_valid || col >= N) continue;
    char *p = lds + r * RS + q * GB;
    uint32_t w[GB / 4];
    if constexpr (GB % 16 == 0) {
#pragma unroll
      for (int v = 0; v < GB / 16; ++v) {
        const uint4 u = ((const uint4 *)p)[v];
        w[4 * v] = u.x; w[4 * v + 1] = u.y; w[4 * v + 2] = u.z; w[4 * v + 3] = u.w;
      }
    } else {
      const uint2 u = *(const uint2 *)p;
      w[0] = u.x; w[1] = u.y;
    }
    uint32_t bits[M];
#pragma unroll
    for (int i = 0; i < M; ++i) {
      if constexpr (sizeof(HT) == 2) bits[i] = (w[i / 2] >> (16 * (i & 1))) & 0xFFFFu;
      else bits[i] = w[i];
    }
    const size_t o = ((size_t)row * bpr + col / M) * NK;
    if constexpr (sizeof(HT) == 2) {
      uint32_t km = nm_kept_mask<NK, M>(bits);
      const uint16_t *ph = (const uint16_t *)p;
      uint32_t vw[(NK + 1) / 2], iw[(NK + 3) / 4];
      static_for<NK>([&](auto J) {
        constexpr int j = decltype(J)::value;
        const uint32_t e = (uint32_t)__builtin_clz(km);   // km holds NK - j set bits here
        km ^= 0x80000000u >> e;
        const uint32_t v = ph[e];
        if constexpr (j & 1) vw[j / 2] |= v << 16;
        else vw[j / 2] = v;
        if constexpr (j % 4 == 0) iw[j / 4] = e;
        else iw[j / 4] |= e << (8 * (j % 4));
      });
      store_words<VB>((char *)(vals + o), vw);
      store_words<NK>((char *)(idx + o), iw);
    } else {
      bool keep[M];
      nm_keep32<NK, M>(bits, keep);
      // in place: entry i moves to position pos <= i, so nothing unread is overwritten
      int pos = 0;
#pragma unroll
      for (int i = 0; i < M; ++i) {
        if (keep[i]) {
          ((uint32_t *)p)[pos] = bits[i];
          ((uint8_t *)p)[VB + pos] = (uint8_t)i;
          ++pos;
        }
      }
      copy_bytes<VB>((char *)(vals + o), p);
      copy_bytes<NK>((char *)(idx + o), p + VB);
    }
  }
}

// ------------------------------------------------------------------------ kernels

template <typename T, class G, int W, typename VT>
__global__ __launch_bounds__(G::NT) void k_up_twell(const T *__restrict__ x, const T *__restrict__ w1t,
                                                    const float *__restrict__ b1, int M, int N, int K,
                                                    TwellOut o) {
  __shared__ __attribute__((aligned(16))) char smem[G::SMEM];
  const int n0 = blockIdx.x * G::BN, m0 = blockIdx.y * G::BM;
  const int wn = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) % G::NWN;
  if constexpr (G::MI == 16) {
    static_assert(std::is_same<T, uint16_t>::value, "16x16x32 MFMA tiles take bf16 operands");
    // -b1 of this lane's columns, fetched before the K loop so its latency is hidden
    float nbias[G::FN];
#pragma unroll
    for (int fn = 0; fn < G::FN; ++fn) {
      const int col = n0 + wn * G::WN + fn * 16 + (threadIdx.x & 15);
      nbias[fn] = col < N ? -b1[col] : 0.f;
    }
    f32x4_t acc[G::FM][G::FN];
#pragma unroll
    for (int fm = 0; fm < G::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < G::FN; ++fn) acc[fm][fn] = f32x4_t{};
    mainloop16<G>(x, nullptr, M, M, w1t, N, K, m0, n0, acc, smem);
    block_barrier();                    // every wave is done reading the operand stages
    epi_twell16<G, W, VT>(acc, nbias, M, N, m0, n0, o, smem);
  } else {
    float nbias[G::NB];
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb) {
      const int col = n0 + wn * G::WN + nb * 32 + (threadIdx.x & 31);
      nbias[nb] = col < N ? -b1[col] : 0.f;
    }
    f32x16_t acc[G::MB][G::NB];
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb) acc[mb][nb] = f32x16_t{};
    mainloop<T, G>(x, nullptr, M, M, w1t, N, K, m0, n0, acc, smem);
    block_barrier();
    epi_twell<G, W, VT>(acc, nbias, M, N, m0, n0, o, smem);
  }
}

// Dense ReLU(x W1 + b1). With arow != NULL the A rows are gathered: tile row i reads x row
// arow[i] for i < min(*n_rows_dev, M) (the overflow rows of a TwELL), and writes out row i.
template <typename T, class G>
__global__ __launch_bounds__(G::NT) void k_up_dense(const T *__restrict__ x, const T *__restrict__ w1t,
                                                    const float *__restrict__ b1, int M, int N, int K, int x_rows,
                                                    const int32_t *__restrict__ arow,
                                                    const int32_t *__restrict__ n_rows_dev, void *out,
                                                    int out_bf16, int relu) {
  __shared__ __attribute__((aligned(16))) char smem[G::LDS_BYTES];
  const int n0 = blockIdx.x * G::BN, m0 = blockIdx.y * G::BM;
  int rows = M;
  if (n_rows_dev) rows = min(rows, *n_rows_dev);
  if (m0 >= rows) return;
  if constexpr (G::MI == 16) {
    static_assert(std::is_same<T, uint16_t>::value, "16x16x32 MFMA tiles take bf16 operands");
    f32x4_t acc[G::FM][G::FN];
#pragma unroll
    for (int fm = 0; fm < G::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < G::FN; ++fn) acc[fm][fn] = f32x4_t{};
    mainloop16<G>(x, arow, rows, x_rows, w1t, N, K, m0, n0, acc, smem);
    epi_dense16<G>(acc, b1, rows, N, m0, n0, out, out_bf16, relu);
  } else {
    f32x16_t acc[G::MB][G::NB];
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb) acc[mb][nb] = f32x16_t{};
    mainloop<T, G>(x, arow, rows, x_rows, w1t, N, K, m0, n0, acc, smem);
    epi_dense<G>(acc, b1, rows, N, m0, n0, out, out_bf16, relu);
  }
}


// ------------------------------------------------------------------ decode (K in quarters)

// Decode (at most 64 tokens) is bound by the weight stream, and the stream rate grows with the
// number of CUs that keep loads in flight. The sum over K is taken in four quarters,
//   z = (q0 + q1) + (q2 + q3),   q_i over k in [i K / 4, (i + 1) K / 4),
// each quarter by one wave through its own ring:
//  - k_up_twell_dec spreads a 128-column tile over two workgroups of two waves (quarters
//    0-1 and 2-3): twice the workgroups of one per tile. The halves meet in a workspace: each
//    workgroup stores its half sum and takes a ticket; the second to arrive adds the other
//    half and runs the TwELL epilogue, its two waves on one 32-row block each.
//  - k_up_dense_dec keeps one workgroup of four waves per tile (no workspace).
// fp32 addition is commutative, so both add the same halves to the same bits whichever
// workgroup arrives last, and the dense path equals the TwELL path bit for bit.

// Fp32 of one wave's 64 x 128 accumulator tile, in register order: element r of block
// (mb, nb) of lane l at ((mb * NB + nb) * 16 + r) * 64 + l.
constexpr int kDecTileF = TileD::MB * TileD::NB * 16 * 64;
static_assert(kDecTileF * 4 == (int)kDecHalfBytes, "workspace layout");

TW_DEV void acc_to_lds(const f32x16_t (&acc)[TileD::MB][TileD::NB], float *red) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < TileD::MB * TileD::NB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(i * 16 + r) * 64 + lane] = acc[i / TileD::NB][i % TileD::NB][r];
}

TW_DEV void acc_add_lds(f32x16_t (&acc)[TileD::MB][TileD::NB], const float *red) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < TileD::MB * TileD::NB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i / TileD::NB][i % TileD::NB][r] += red[(i * 16 + r) * 64 + lane];
}

// Rows of register group g (registers 4g .. 4g + 3) of block row mb: mb * 32 + 8 g + 0..7. A
// group whose first row is at or beyond M holds only padding rows and is skipped as a whole
// (a uniform branch, so the loads of the kept groups are all issued before any wait).
TW_DEV bool dec_group_live(int mb, int g, int M) { return mb * 32 + 8 * g < M; }

constexpr int kDecodeSmem = 2 * TileD::LDS_BYTES > TileD::EPI_WAVE ? 2 * TileD::LDS_BYTES : TileD::EPI_WAVE;
static_assert(kDecodeSmem <= 160 * 1024, "LDS");

// The TwELL decode kernel splits the tail of a tile by 32-row block: wave w of a workgroup
// keeps block row w (rows 32 w .. 32 w + 31). kDecRowF floats hold one wave's block row in
// register order: element r of block nb of lane l at (nb * 16 + r) * 64 + l.
constexpr int kDecRowF = TileD::NB * 16 * 64;
constexpr int kDecTicketOff = kDecodeSmem - 16;   // LDS word that shares the ticket
static_assert(2 * kDecRowF * 4 <= kDecTicketOff && 2 * TileD::EPI_WAVE <= kDecTicketOff, "decode LDS layout");

TW_DEV void row_to_lds(const f32x16_t (&a)[TileD::NB], float *red) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int nb = 0; nb < TileD::NB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) red[(nb * 16 + r) * 64 + lane] = a[nb][r];
}

TW_DEV void row_add_lds(f32x16_t (&a)[TileD::NB], const float *red) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int nb = 0; nb < TileD::NB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) a[nb][r] += red[(nb * 16 + r) * 64 + lane];
}

// Cross-workgroup hand-over of the half sums (k_up_twell_dec). Every access
// to the workspace is an atomic of agent scope: such accesses are coherent across the XCDs'
// separate L2 caches on their own (stores write through, loads do not hit a stale line). The
// half sum is stored, its stores are waited for (vmcnt(0)) and only then is the ticket taken,
// so the workgroup that arrives second reads a completely stored other half: its loads are
// issued after the ticket's value has returned. An agent-scope release/acquire pair would
// add an L2 write-back and invalidate per workgroup (several microseconds per launch) that
// only plain stores need.
//
// The ticket is a 64-bit word that each of the tile's two workgroups swaps for its own tag
// (an arbitrary 64-bit constant per half). The workgroup that gets back the other half's tag
// arrived second: it zeroes the word and finishes the tile. Any other value it gets back
// (zero after an earlier launch, or whatever an uninitialised buffer holds) means it arrived
// first. So the workspace needs no initialisation; only a word that happens to hold one of
// the two tags before the first launch would mislead a tile (one chance in 2^63). Both waves
// of a workgroup store (and later load) their own block rows; wave 0 takes the one ticket
// after a barrier that follows both waves' store waits.
TW_DEV uint64_t dec_tag(int half) { return half ? 0xBB67AE8584CAA73Bull : 0x6A09E667F3BCC908ull; }

// true if this workgroup (half `half` of the tile) arrived second; then the ticket is zeroed.
TW_DEV bool dec_meet(uint64_t *ticket, int half) {
  const uint64_t old = __hip_atomic_exchange(ticket, dec_tag(half), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const bool second = old == dec_tag(1 - half);
  if (second) __hip_atomic_store(ticket, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return second;
}
// Half sum of block row MB to the workspace (element r of block (MB, nb) of lane l at
// ((MB * NB + nb) * 16 + r) * 64 + l), agent-scope stores of the live row groups only.
template <int MB> TW_DEV void dec_store_row(const f32x16_t (&acc)[TileD::MB][TileD::NB], int M, float *mine) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int nb = 0; nb < TileD::NB; ++nb)
#pragma unroll
    for (int g = 0; g < 4; ++g)
      if (dec_group_live(MB, g, M))
#pragma unroll
        for (int q = 0; q < 4; ++q)
          __hip_atomic_store(mine + ((MB * TileD::NB + nb) * 16 + 4 * g + q) * 64 + lane, acc[MB][nb][4 * g + q],
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// acc[MB] += the other half's block row MB (all loads issued before the adds).
template <int MB> TW_DEV void dec_add_row(f32x16_t (&acc)[TileD::MB][TileD::NB], int M, const float *other) {
  const int lane = threadIdx.x & 63;
  float ov[TileD::NB][16];
#pragma unroll
  for (int nb = 0; nb < TileD::NB; ++nb)
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        ov[nb][4 * g + q] = dec_group_live(MB, g, M)
                                ? __hip_atomic_load(other + ((MB * TileD::NB + nb) * 16 + 4 * g + q) * 64 + lane,
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                : 0.f;
#pragma unroll
  for (int nb = 0; nb < TileD::NB; ++nb)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[MB][nb][r] += ov[nb][r];
}

// Grid: 2 * ceil(N / 128) workgroups of 128 threads; workgroup b takes tile b % n_tiles and
// half b / n_tiles (quarters 2 half, 2 half + 1). Workspace o.dec_part [n_tiles][2][kDecTileF]
// fp32 and o.dec_ticket [n_tiles] (see dec_meet).
template <typename T, int W, typename VT>
__global__ __launch_bounds__(128) void k_up_twell_dec(const T *__restrict__ x, const T *__restrict__ w1t,
                                                      const float *__restrict__ b1, int M, int N, int K,
                                                      TwellOut o) {
  __shared__ __attribute__((aligned(16))) char smem[kDecodeSmem];
  const int n_tiles = (N + TileD::BN - 1) / TileD::BN;
  const int tile = blockIdx.x % n_tiles, half = blockIdx.x / n_tiles;
  const int n0 = tile * TileD::BN;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kq = K / 4;
  float nbias[TileD::NB];
#pragma unroll
  for (int nb = 0; nb < TileD::NB; ++nb) {
    const int col = n0 + nb * 32 + (threadIdx.x & 31);
    nbias[nb] = col < N ? -b1[col] : 0.f;
  }
  f32x16_t acc[TileD::MB][TileD::NB];
#pragma unroll
  for (int mb = 0; mb < TileD::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < TileD::NB; ++nb) acc[mb][nb] = f32x16_t{};
  mainloop<T, TileD>(x, nullptr, M, M, w1t, N, kq, 0, n0, acc, smem + w * TileD::LDS_BYTES, K, (2 * half + w) * kq, 0);
  // Wave w keeps block row w: it passes the other block row to the other wave through LDS
  // and adds the one it receives (q_2h + q_2h+1; fp32 addition is commutative, so either
  // wave's order gives the same bits).
  block_barrier_lds();                      // both rings are drained
  float *red = (float *)smem;
  if (w == 0) row_to_lds(acc[1], red + kDecRowF);
  else row_to_lds(acc[0], red);
  block_barrier_lds();
  if (w == 0) row_add_lds(acc[0], red);
  else row_add_lds(acc[1], red + kDecRowF);
  // Hand-over of the half sums (one ticket per workgroup):
  // both waves store their block rows and wait for the stores; after the barrier wave 0
  // takes the ticket and shares it through LDS.
  float *part = o.dec_part + (size_t)tile * 2 * kDecTileF;
  if (w == 0) dec_store_row<0>(acc, M, part + half * kDecTileF);
  else dec_store_row<1>(acc, M, part + half * kDecTileF);
  wait_vmcnt<0>();
  block_barrier_lds();
  uint32_t *tk = (uint32_t *)(smem + kDecTicketOff);
  const int lane = threadIdx.x & 63;
  if (w == 0 && lane == 0) *tk = dec_meet(o.dec_ticket + tile, half) ? 1u : 0u;
  block_barrier_lds();
  const uint32_t t = (uint32_t)__builtin_amdgcn_readfirstlane((int)*tk);
  if (t == 0) return;                       // first to arrive: the other workgroup finishes
  if (w == 0) dec_add_row<0>(acc, M, part + (1 - half) * kDecTileF);
  else dec_add_row<1>(acc, M, part + (1 - half) * kDecTileF);
  epi_twell<TileD, W, VT>(acc, nbias, M, N, 0, n0, o, smem, w);
}

// Four waves of TileDQ (3-stage rings, 36 KB each), wave w on quarter w; then
// (q0 + q1) + (q2 + q3) through LDS and the dense epilogue by wave 0.
typedef Tile<64, 128, 64, 128, 0, 3> TileDQ;
static_assert(4 * TileDQ::LDS_BYTES <= 160 * 1024 && 2 * kDecTileF * 4 <= 4 * TileDQ::LDS_BYTES, "LDS");

// One 128-column tile of the dense rows arow[i], i < rows (x row arow[i] if arow, else i): four
// waves, wave w on quarter w of K through its own ring, then (q0 + q1) + (q2 + q3) through LDS and
// the dense epilogue by wave 0. Waves 4 and up of a larger workgroup must have exited.
template <typename T>
TW_DEV void dense_dec_tile(const T *__restrict__ x, const T *__restrict__ w1t, const float *__restrict__ b1, int rows,
                           int N, int K, int x_rows, const int32_t *arow, int n0, void *out, int out_bf16, int relu,
                           char *smem) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kq = K / 4;
  f32x16_t acc[TileD::MB][TileD::NB];
#pragma unroll
  for (int mb = 0; mb < TileD::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < TileD::NB; ++nb) acc[mb][nb] = f32x16_t{};
  mainloop<T, TileDQ>(x, arow, rows, x_rows, w1t, N, kq, 0, n0, acc, smem + w * TileDQ::LDS_BYTES, K, w * kq, 0);
  block_barrier_lds();
  float *red = (float *)smem;
  if (w & 1) acc_to_lds(acc, red + (w >> 1) * kDecTileF);
  block_barrier_lds();
  if (!(w & 1)) acc_add_lds(acc, red + (w >> 1) * kDecTileF);   // waves 0, 2: q0 + q1, q2 + q3
  block_barrier_lds();
  if (w == 2) acc_to_lds(acc, red);
  block_barrier_lds();
  if (w != 0) return;
  acc_add_lds(acc, red);
  epi_dense<TileD>(acc, b1, rows, N, 0, n0, out, out_bf16, relu);
}

template <typename T>
__global__ __launch_bounds__(256) void k_up_dense_dec(const T *__restrict__ x, const T *__restrict__ w1t,
                                                      const float *__restrict__ b1, int M, int N, int K, int x_rows,
                                                      const int32_t *__restrict__ arow,
                                                      const int32_t *__restrict__ n_rows_dev, void *out,
                                                      int out_bf16, int relu) {
  __shared__ __attribute__((aligned(16))) char smem[4 * TileDQ::LDS_BYTES];
  int rows = M;
  if (n_rows_dev) rows = min(rows, *n_rows_dev);
  if (rows <= 0) return;
  dense_dec_tile<T>(x, w1t, b1, rows, N, K, x_rows, arow, blockIdx.x * TileDQ::BN, out, out_bf16, relu, smem);
}

// The finish of at most 64 rows after the decode tile GEMM, with the backup recompute in the
// same launch, in workgroups of four waves. Every workgroup that needs them finds the overflow
// rows from the overflow words itself (bit t % 32 of word t / 32 of any tile; at most 64 rows),
// ranked in ascending row order and cut at cap, which is the order of the overflow scan
// (ovf_scan_block). Workgroup 0 writes that scan (ovf_slot, ovf_rows, ovf_n); workgroups 1 ..
// nlist build one row list each (row_list_wave); workgroup 1 + nlist + i recomputes tile i of the
// backup rows ReLU(x W1 + b1) exactly as k_up_dense_dec does, so it waits for nothing, and with
// no overflow row it exits after the one read of the words.
template <typename T, typename VT>
__global__ __launch_bounds__(256) void k_finish_dec(TwellIn h, const uint32_t *__restrict__ bits, int words,
                                                    int32_t *ovf_n, int32_t *ovf_rows, int32_t *ovf_slot, int nlist,
                                                    const T *__restrict__ x, const T *__restrict__ w1t,
                                                    const float *__restrict__ b1, int K, void *dense, int dense_bf16) {
  __shared__ __attribute__((aligned(16))) char smem[4 * TileDQ::LDS_BYTES];
  __shared__ int32_t rows_s[64];
  __shared__ uint32_t ow[2];
  __shared__ int nr_s;
  const int b = blockIdx.x, tid = threadIdx.x;
  if (b >= 1 && b <= nlist) {
    if (tid >= 64) return;
    if (b - 1 < h.rows) row_list_wave<VT>(h, b - 1);
    return;
  }
  if (b > nlist && h.cap <= 0) return;                         // uniform: no backup rows
  // The words of all tiles, read as one flat run (word i belongs to row word i % words), OR-ed
  // into ow: four clamped loads in flight per lane.
  if (tid < 2) ow[tid] = 0u;
  __syncthreads();
  const int nw = h.n_t * words;
  uint32_t f0 = 0, f1 = 0;
  for (int i0 = tid; i0 < nw; i0 += 4 * 256) {
    uint32_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = bits[min(i0 + u * 256, nw - 1)];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * 256;
      if (i < nw && i % words == 0) f0 |= v[u];
      if (i < nw && i % words == 1) f1 |= v[u];
    }
  }
  if (f0) atomicOr(&ow[0], f0);
  if (f1) atomicOr(&ow[1], f1);
  __syncthreads();
  if (tid < 64) {
    const bool on = tid < h.rows && ((ow[tid >> 5] >> (tid & 31)) & 1u);
    const uint64_t m = ballot64(on);
    const int rank = __popcll(m & ((1ull << tid) - 1ull));
    const int slot = on && rank < h.cap ? rank : -1;
    if (slot >= 0) rows_s[slot] = tid;
    if (tid == 0) nr_s = min(__popcll(m), h.cap);
    if (b == 0) {                                              // the overflow scan's outputs
      if (tid < h.rows) ovf_slot[tid] = slot;
      if (slot >= 0) ovf_rows[slot] = tid;
      if (tid == 0) *ovf_n = __popcll(m);
    }
  }
  if (b == 0) return;
  __syncthreads();
  const int nr = nr_s;
  if (nr == 0) return;                                         // uniform
  dense_dec_tile<T>(x, w1t, b1, nr, h.cols, K, h.rows, rows_s, (b - 1 - nlist) * TileDQ::BN, dense, dense_bf16, 1,
                    smem);
}
// h = ReLU(x W1 + b1) pruned to NK:M inside the up GEMM (N:M epilogue above). The tiles,
// loops and accumulation order are those of k_up_dense for the same problem, so z is the
// same bit for bit.
template <typename T, class G, int NK, int M>
__global__ __launch_bounds__(G::NT) void k_up_nm(const T *__restrict__ x, const T *__restrict__ w1t,
                                                 const float *__restrict__ b1, int Mr, int N, int K,
                                                 T *__restrict__ vals, uint8_t *__restrict__ idx) {
  constexpr int SM = G::LDS_BYTES > nm_stage_bytes<G, T>() ? G::LDS_BYTES : nm_stage_bytes<G, T>();
  static_assert(SM <= 160 * 1024, "LDS");
  __shared__ __attribute__((aligned(16))) char smem[SM];
  const int n0 = blockIdx.x * G::BN, m0 = blockIdx.y * G::BM;
  if constexpr (G::MI == 16) {
    static_assert(std::is_same<T, uint16_t>::value, "16x16x32 MFMA tiles take bf16 operands");
    f32x4_t acc[G::FM][G::FN];
#pragma unroll
    for (int fm = 0; fm < G::FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < G::FN; ++fn) acc[fm][fn] = f32x4_t{};
    mainloop16<G>(x, nullptr, Mr, Mr, w1t, N, K, m0, n0, acc, smem);
    block_barrier();                    // every wave is done reading the operand stages
    stage_h16<G, T>(acc, b1, N, n0, smem);
  } else {
    f32x16_t acc[G::MB][G::NB];
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb) acc[mb][nb] = f32x16_t{};
    mainloop<T, G>(x, nullptr, Mr, Mr, w1t, N, K, m0, n0, acc, smem);
    block_barrier();
    stage_h32<G, T>(acc, b1, N, n0, smem);
  }
  block_barrier_lds();
  nm_tile<T, NK, M, G::BM, G::BN, G::NT>(smem, Mr, N, m0, n0, vals, idx);
}

// Decode form: the quarters of k_up_dense_dec, summed the same way by wave 0, then all four
// waves select.
template <typename T, int NK, int M>
__global__ __launch_bounds__(256) void k_up_nm_dec(const T *__restrict__ x, const T *__restrict__ w1t,
                                                   const float *__restrict__ b1, int Mr, int N, int K,
                                                   T *__restrict__ vals, uint8_t *__restrict__ idx) {
  __shared__ __attribute__((aligned(16))) char smem[4 * TileDQ::LDS_BYTES];
  static_assert(nm_stage_bytes<TileD, T>() <= 4 * TileDQ::LDS_BYTES, "LDS");
  const int n0 = blockIdx.x * TileDQ::BN;
  if (Mr <= 0) return;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kq = K / 4;
  f32x16_t acc[TileD::MB][TileD::NB];
#pragma unroll
  for (int mb = 0; mb < TileD::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < TileD::NB; ++nb) acc[mb][nb] = f32x16_t{};
  mainloop<T, TileDQ>(x, nullptr, Mr, Mr, w1t, N, kq, 0, n0, acc, smem + w * TileDQ::LDS_BYTES, K, w * kq, 0);
  block_barrier_lds();
  float *red = (float *)smem;
  if (w & 1) acc_to_lds(acc, red + (w >> 1) * kDecTileF);
  block_barrier_lds();
  if (!(w & 1)) acc_add_lds(acc, red + (w >> 1) * kDecTileF);   // waves 0, 2: q0 + q1, q2 + q3
  block_barrier_lds();
  if (w == 2) acc_to_lds(acc, red);
  block_barrier_lds();
  if (w == 0) acc_add_lds(acc, red);
  block_barrier_lds();                  // the partial sums are read before the tile overwrites them
  if (w == 0) stage_h32<TileD, T>(acc, b1, N, n0, smem);
  block_barrier_lds();
  nm_tile<T, NK, M, TileD::BM, TileD::BN, 256>(smem, Mr, N, 0, n0, vals, idx);
}

// ------------------------------------------------------------------ decode GEMV (T <= 2, bf16)
// With a handful of tokens the up projection is a stream of W1 with a few dot products per
// row. The tile kernels above fetch each W1 row in 64-byte pieces per stage; here every wave
// load is one contiguous kilobyte of a row. A wave takes 16 units over one half of K; lane l
// holds the 16-byte pieces
//   k = k0 + 8 (64 p + l),  p = 0 .. np - 1   (np = K / 1024 per half of K)
// of x (all tokens, in registers) and of the rows it streams, four units at a time with three
// (stream kernel) or two (dense kernel, whose waves have half the registers) groups of four
// in flight. Each (unit, token) partial is accumulated over the lane's pieces
// in order with v_dot2_f32_bf16, then the wave's 16 TT partials are summed over the 64 lanes
// by one transposing butterfly (gemv_reduce):
//   z = half_0 + half_1.
// TwELL: k_up_gemv_z streams W1 on one-wave workgroups (every CU streams; no workgroup waits
// for another) and stores the half sums in the decode workspace; k_dec_finish (one workgroup
// per token row) packs the TwELL from them and completes the matrix (row lists, overflow
// scan, dense backup rows), or k_dec_pack packs the TwELL alone. Dense and N:M:
// k_up_gemv_dense runs both halves of a 128-unit tile on the 8 waves of one workgroup and
// adds them in LDS. fp32 addition is commutative, so all of them see the same z bit for bit.
constexpr int kGemvMaxT = 2, kGemvNP = 4, kGemvUnits = 128;
constexpr int kGemvUPW = 16;                                // units per wave

typedef __bf16 bf16x2g_t __attribute__((ext_vector_type(2)));
TW_DEV float dot8_bf16(uint4 a, uint4 b, float c) {
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2g_t, a.x), __builtin_bit_cast(bf16x2g_t, b.x), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2g_t, a.y), __builtin_bit_cast(bf16x2g_t, b.y), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2g_t, a.z), __builtin_bit_cast(bf16x2g_t, b.z), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2g_t, a.w), __builtin_bit_cast(bf16x2g_t, b.w), c, false);
  return c;
}

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

// Sum over the 64 lanes of each of the V values v[j] (V a power of two, at most 64). Step s
// (m = 32 >> s) halves the set: a lane keeps the upper half of its values if bit m of its
// lane index is set, else the lower half, and adds the partner's (lane ^ m) copy of that
// half. After log2 V steps a lane holds one value, index gemv_value_index<V>(lane); the lanes
// that hold the same index then add their partials by an xor butterfly over the low bits, so
// every lane ends with its index's complete sum (identical bits in all of them: each addition
// is commutative). V - 1 + log2(64 / V) exchanges instead of 6 per value.
template <int V> TW_DEV float gemv_reduce(float (&v)[V]) {
  constexpr int LV = ilog2(V);
  static_assert((1 << LV) == V && V <= 64, "power of two");
  const int lane = lane_id();
  static_for<LV>([&](auto S) {
    constexpr int st = decltype(S)::value, m = 32 >> st, half = V >> (st + 1);
    const bool hi = lane & m;
    static_for<half>([&](auto J) {
      constexpr int k = decltype(J)::value;
      const float keep = hi ? v[k + half] : v[k];
      const float send = hi ? v[k] : v[k + half];
      v[k] = keep + __shfl_xor(send, m, 64);
    });
  });
  float r = v[0];
#pragma unroll
  for (int m = 32 >> LV; m > 0; m >>= 1) r += __shfl_xor(r, m, 64);
  return r;
}

template <int V> TW_DEV int gemv_value_index(int lane) {
  constexpr int LV = ilog2(V);
  int j = 0;
#pragma unroll
  for (int st = 0; st < LV; ++st) j += ((lane >> (5 - st)) & 1) * (V >> (st + 1));
  return j;
}

// One wave: units u0 .. u0 + 15 (rows at or beyond N read as zero) over half kh of K (NP =
// K / 1024 pieces per lane), token slots t < TT (x row arow[t] if arow, else t; slots at or
// beyond rows are zero). Returns the sum of value gemv_value_index<16 TT>(lane) = unit * TT +
// slot (complete in every lane). Unit addresses are clamped into the operand (row 0) before
// the predicate is applied, so no load can leave it whatever the compiler hoists.
template <int TT, int NP, int NG>
TW_DEV float gemv_wave(const uint16_t *__restrict__ x, const int32_t *__restrict__ arow, int rows,
                       const uint16_t *__restrict__ w1t, int N, int K, int u0, int kh) {
  const int lane = lane_id();
  const size_t k0 = (size_t)kh * (K / 2) + 8 * lane;
  uint4 xr[TT][NP];
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    const int tr = t < rows ? t : 0;
    const uint16_t *xp = x + (size_t)(arow ? arow[tr] : tr) * K + k0;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const uint4 v = *(const uint4 *)(xp + 512 * p);
      xr[t][p] = t < rows ? v : make_uint4(0, 0, 0, 0);
    }
  }
  const __amdgpu_buffer_rsrc_t rw = rows_rsrc(w1t);
  auto load = [&](int g, uint4 (&wr)[4][NP]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = u0 + 4 * g + i;
      const uint32_t wo = (uint32_t)((size_t)(u < N ? u : 0) * K + k0);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const uint4 v = ld16<uint16_t>(rw, wo + 512u * p);
        wr[i][p] = u < N ? v : make_uint4(0, 0, 0, 0);
      }
    }
  };
  float part[16 * TT];
  auto dot = [&](int g, const uint4 (&wr)[4][NP]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        float acc = 0.f;
#pragma unroll
        for (int p = 0; p < NP; ++p) acc = dot8_bf16(xr[t][p], wr[i][p], acc);
        part[(4 * g + i) * TT + t] = acc;
      }
  };
  static_assert(kGemvUPW == 16 && (NG == 2 || NG == 3), "four groups of four units, two or three in flight");
  uint4 wa[4][NP], wb[4][NP];
  if constexpr (NG == 3) {
    uint4 wc[4][NP];
    load(0, wa);
    load(1, wb);
    load(2, wc);
    dot(0, wa);
    load(3, wa);
    dot(1, wb);
    dot(2, wc);
    dot(3, wa);
  } else {
    load(0, wa);
    load(1, wb);
    dot(0, wa);
    load(2, wa);
    dot(1, wb);
    load(3, wb);
    dot(2, wa);
    dot(3, wb);
  }
  return gemv_reduce<16 * TT>(part);
}

// Grid: 2 * ceil(N / 16) one-wave workgroups; workgroup b takes units 16 (b % nb) .. + 15 and
// half b / nb of K, and stores its sums to zp[half][t][u] (fp32, t < M). With n_rows_dev the token
// count is min(M, *n_rows_dev) (nothing to do at zero). ticket (optional): the decode
// tickets of the matrix, unused on this path; like every call, it leaves them zero (plain
// stores: they are next read by a later launch). ovf_words (optional): the first word of each
// of the n_words tiles' overflow bits (stride words), zeroed for k_dec_pack.
template <int TT, int NP>
__global__ __launch_bounds__(64) void k_up_gemv_z(const uint16_t *__restrict__ x, const int32_t *__restrict__ arow,
                                                  const int32_t *__restrict__ n_rows_dev, int M,
                                                  const uint16_t *__restrict__ w1t, int N, int K,
                                                  float *__restrict__ zp, uint64_t *__restrict__ ticket,
                                                  uint32_t *__restrict__ ovf_words, int n_words, int words) {
  if (ticket && threadIdx.x == 0 && blockIdx.x < (N + kGemvUnits - 1) / kGemvUnits) ticket[blockIdx.x] = 0;
  if (ovf_words && threadIdx.x == 0 && blockIdx.x < n_words) ovf_words[(size_t)blockIdx.x * words] = 0;
  int rows = M;
  if (n_rows_dev) rows = min(rows, *n_rows_dev);
  if (rows <= 0) return;
  const int nb = (N + kGemvUPW - 1) / kGemvUPW;
  const int ub = blockIdx.x % nb, kh = blockIdx.x / nb;
  const float z = gemv_wave<TT, NP, 3>(x, arow, rows, w1t, N, K, ub * kGemvUPW, kh);
  const int lane = lane_id(), j = gemv_value_index<16 * TT>(lane);
  const int u = ub * kGemvUPW + j / TT, t = j % TT;
  if (lane % (64 / (16 * TT)) == 0 && u < N && t < M) zp[((size_t)kh * M + t) * N + u] = z;
}

// ------------------------------------------------------------ decode stream, 3 to 16 tokens
// From three tokens on, the dot products of the W1 stream go to the matrix cores: a wave
// still owns 16 units over one half of K, now as the A operand of v_mfma_f32_16x16x32_bf16
// loaded straight from memory (16 rows x 64 bytes per wave load, no LDS), with x^T as the B
// operand (token slots 0-15). kMsD steps of 32 k are in flight. The output stays the half
// sums zp[half][t][u] of the one- and two-token stream, so the same packing kernels follow.
constexpr int kMsMaxT = 16, kMsD = 16;

// Units u0 .. u0 + 15 over half kh of K for token slots t < rows <= 16 (x row arow[t] if arow,
// else t). Lane l loads the 16-byte piece l / 16 of every 32-k step of W1 row u0 + l % 16 and
// of x row l % 16; rows at or beyond N and slots at or beyond rows take an out-of-range
// offset and read zeros. Returns lane l's accumulators z[u0 + 4 (l / 16) + i][slot l % 16],
// i < 4, each the sum over the half's steps in order. K = 1024 NP.
template <int NP>
TW_DEV f32x4_t mstream_wave(const uint16_t *__restrict__ x, const int32_t *__restrict__ arow, int rows,
                            const uint16_t *__restrict__ w1t, int N, int K, int u0, int kh) {
  constexpr uint32_t OOB = 0x80000000u;
  constexpr int NS = 16 * NP;                                  // steps of the half (K = 1024 NP)
  const int lane = lane_id(), r = lane & 15, c = lane >> 4;
  const uint32_t rowb = (uint32_t)K * 2u, half = (uint32_t)kh * (uint32_t)K;   // bytes
  const int u = u0 + r;
  const uint32_t wo = u < N ? (uint32_t)u * rowb + half + 16u * (uint32_t)c : OOB;
  const uint32_t xo = r < rows ? (uint32_t)(arow ? arow[r] : r) * rowb + half + 16u * (uint32_t)c : OOB;
  const __amdgpu_buffer_rsrc_t rw = rows_rsrc(w1t), rx = rows_rsrc(x);
  // straight-line steps (fully unrolled), so that each MFMA waits for its own step's loads only
  u32x4_t a[kMsD], b[kMsD];
  static_for<kMsD>([&](auto D) {
    constexpr int d = decltype(D)::value;
    a[d] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(wo + 64u * d), 0, 0);
    b[d] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(xo + 64u * d), 0, 0);
  });
  __builtin_amdgcn_sched_barrier(0);            // the scheduler keeps the kMsD steps in flight
  f32x4_t acc = f32x4_t{};
  static_for<NS>([&](auto J) {
    constexpr int j = decltype(J)::value, d = j % kMsD;
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[d]), __builtin_bit_cast(bf16x8_t, b[d]),
                                                 acc, 0, 0, 0);
    if constexpr (j + kMsD < NS) {
      a[d] = __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(wo + 64u * (j + kMsD)), 0, 0);
      b[d] = __builtin_amdgcn_raw_buffer_load_b128(rx, (int)(xo + 64u * (j + kMsD)), 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  });
  return acc;
}

// Grid: 2 * ceil(N / 16) one-wave workgroups, as k_up_gemv_z: zp[half][t][u] (fp32, t < M).
template <int NP>
__global__ __launch_bounds__(64) void k_up_mstream_z(const uint16_t *__restrict__ x, const int32_t *__restrict__ arow,
                                                     const int32_t *__restrict__ n_rows_dev, int M,
                                                     const uint16_t *__restrict__ w1t, int N, int K,
                                                     float *__restrict__ zp, uint64_t *__restrict__ ticket,
                                                     uint32_t *__restrict__ ovf_words, int n_words, int words) {
  if (ticket && threadIdx.x == 0 && blockIdx.x < (N + kGemvUnits - 1) / kGemvUnits) ticket[blockIdx.x] = 0;
  if (ovf_words && threadIdx.x == 0 && blockIdx.x < n_words) ovf_words[(size_t)blockIdx.x * words] = 0;
  int rows = M;
  if (n_rows_dev) rows = min(rows, *n_rows_dev);
  if (rows <= 0) return;
  const int nb = (N + kGemvUPW - 1) / kGemvUPW;
  const int ub = blockIdx.x % nb, kh = blockIdx.x / nb;
  const f32x4_t z = mstream_wave<NP>(x, arow, rows, w1t, N, K, ub * kGemvUPW, kh);
  const int lane = lane_id(), t = lane & 15;
  if (t < M)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = ub * kGemvUPW + 4 * (lane >> 4) + i;
      if (u < N) zp[((size_t)kh * M + t) * N + u] = z[i];
    }
}

// TwELL of row t of one tile kt (a wave; lane l holds units V l .. V l + V - 1 of it, V = W / 64)
// from z and nb = -b1 of those units: unit u is active iff z > nb, value z - nb (the tile
// epilogues' arithmetic); a ballot per unit position, the count, the slots in ascending column
// order (the first S active units), pads (-1, +0) and the count. Returns min(count, S);
// *ovf = count > S; stored(slot, col, v) sees every stored slot.
template <int W, typename VT, class F>
TW_DEV int gemv_pack_row(const float (&z)[W / 64], const float (&nb)[W / 64], int t, int kt, const TwellOut &o,
                         bool *ovf, F &&stored) {
  constexpr int V = W / 64;
  const int lane = lane_id(), S = o.S, n_t = o.n_t;
  bool on[V];
  uint64_t m[V];
  int c = 0, before = 0;
#pragma unroll
  for (int e = 0; e < V; ++e) {
    on[e] = z[e] > nb[e];
    m[e] = ballot64(on[e]);
    c += __popcll(m[e]);
    before += mbcnt64(m[e]);
  }
  const size_t base = ((size_t)t * n_t + kt) * S;
  int slot = before;
#pragma unroll
  for (int e = 0; e < V; ++e) {
    if (on[e]) {
      if (slot < S) {
        const int col = kt * W + V * lane + e;
        const float v = z[e] - nb[e];
        o.col_idx[base + slot] = col;
        Elem<VT>::store((VT *)o.vals, base + slot, v);
        stored(slot, col, v);
      }
      ++slot;
    }
  }
  for (int s2 = min(c, S) + lane; s2 < S; s2 += 64) {
    o.col_idx[base + s2] = -1;
    Elem<VT>::store((VT *)o.vals, base + s2, 0.f);
  }
  if (lane == 0) o.counts[(size_t)t * n_t + kt] = c;
  *ovf = c > S;
  return min(c, S);
}

// The TwELL alone (no lists, scan or backup rows) of M <= 16 rows from the half sums
// zp[half][t][u] (z = zp[0] + zp[1]): one (tile, row) per wave, grid ceil(M n_t / 16)
// workgroups of 1024 threads. A row-tile above S slots sets its bit in the tile's overflow word
// (rows < 32) with an atomic OR; the stream kernel of the same call zeroed the words.
template <int W, typename VT>
__global__ __launch_bounds__(1024) void k_dec_pack(const float *__restrict__ zp, const float *__restrict__ b1, int M,
                                                   int N, TwellOut o) {
  constexpr int V = W / 64;
  const int wg = blockIdx.x * 16 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wg >= M * o.n_t) return;
  const int kt = wg % o.n_t, t = wg / o.n_t;
  float z[V], z1[V], nb[V];
#pragma unroll
  for (int e = 0; e < V; ++e) {
    const int u = kt * W + V * lane + e;
    nb[e] = b1[u];
    z[e] = zp[(size_t)t * N + u];
    z1[e] = zp[((size_t)M + t) * N + u];
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int e = 0; e < V; ++e) {
    nb[e] = -nb[e];
    z[e] += z1[e];
  }
  bool ovf;
  gemv_pack_row<W, VT>(z, nb, t, kt, o, &ovf, [](int, int, float) {});
  if (ovf && lane == 0)
    __hip_atomic_fetch_or(o.ovf_bits + (size_t)kt * o.words, 1u << t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The whole matrix of M <= 16 rows from the half sums: workgroup t (1024 threads) takes row t,
// in chunks of CH tiles (as many as the LDS stage holds):
//  1. per tile (one wave, up to kFinB tiles at once with every load issued first: the loads
//     are the cost) the TwELL of gemv_pack_row; the stored slots also go to an LDS stage as
//     (column, fp32 value bits);
//  2. with lists: the exclusive prefix over the chunk's tiles of min(count, S) (plus the carry
//     of earlier chunks) gives each tile's list offset, and the staged slots are copied to the
//     row's list;
// then the rows meet on one 64-bit word of the decode workspace (zeroed by the stream kernel of
// the same call; a single row needs no meeting): each adds 1 plus its overflow flag at bit
// 32 + t. The last to arrive has
// every flag, runs the overflow scan (rank among overflow rows, below cap), writes the dense
// backup row ReLU(z + b1) of each overflow row with a slot (formed as k_up_gemv_dense forms
// it, so it equals the recompute bit for bit) and zeroes the word again. Barriers wait for
// LDS only: nothing written to global memory is read back by this kernel.
constexpr int kFinB = 8;                                     // tiles per batch of a wave
constexpr int kFinStage = 12288;                             // LDS stage entries (96 KB)
constexpr int kFinMaxCH = 1024;

template <int W, typename VT>
__global__ __launch_bounds__(1024) void k_dec_finish(const float *__restrict__ zp, const float *__restrict__ b1, int M,
                                                     int N, TwellOut o, TwellFinish f) {
  constexpr int V = W / 64;
  __shared__ uint2 stage[kFinStage];
  __shared__ int off_s[kFinMaxCH], st_s[kFinMaxCH];
  __shared__ int wsum[16];
  __shared__ int carry_s, ovf_s, last_s;
  __shared__ int slot_s[kMsMaxT];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, t = blockIdx.x;
  const int S = o.S, n_t = o.n_t;
  const int CH = min(kFinMaxCH, kFinStage / S);
  if (tid == 0) {
    carry_s = 0;
    ovf_s = 0;
  }
  block_barrier_lds();
  const bool lists = f.row_nnz && f.row_list;
  const float *z0 = zp + (size_t)t * N, *z1 = zp + ((size_t)M + t) * N;
  uint2 *lrow = lists ? f.row_list + (size_t)t * n_t * S : nullptr;
  for (int c0 = 0; c0 < n_t; c0 += CH) {
    const int nc = min(CH, n_t - c0);
    for (int q0 = wave; q0 < nc; q0 += 16 * kFinB) {
      float z[kFinB][V], zb[kFinB][V], nb[kFinB][V];
#pragma unroll
      for (int bq = 0; bq < kFinB; ++bq) {
        const int q = q0 + 16 * bq < nc ? q0 + 16 * bq : q0;   // a valid tile for every load
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const int u = (c0 + q) * W + V * lane + e;
          nb[bq][e] = b1[u];
          z[bq][e] = z0[u];
          zb[bq][e] = z1[u];
        }
      }
      __builtin_amdgcn_sched_barrier(0);       // every load of the batch before the first sum
#pragma unroll
      for (int bq = 0; bq < kFinB; ++bq)
#pragma unroll
        for (int e = 0; e < V; ++e) {
          nb[bq][e] = -nb[bq][e];
          z[bq][e] += zb[bq][e];
        }
#pragma unroll
      for (int bq = 0; bq < kFinB; ++bq) {
        const int q = q0 + 16 * bq;
        if (q >= nc) break;                                    // wave-uniform
        bool ovf;
        const int cnt = gemv_pack_row<W, VT>(z[bq], nb[bq], t, c0 + q, o, &ovf, [&](int slot, int col, float v) {
          stage[q * S + slot] = make_uint2((uint32_t)col, __float_as_uint(Elem<VT>::load_rounded(v)));
        });
        if (lane == 0) {
          off_s[q] = cnt;
          st_s[q] = cnt;
          if (ovf) ovf_s = 1;
        }
      }
    }
    block_barrier_lds();
    if (lists) {
      const int c = tid < nc ? off_s[tid] : 0;
      int tot;
      const int ex = wave_excl_scan(c, &tot);
      if (lane == 0) wsum[wave] = tot;
      block_barrier_lds();
      int pre = carry_s, all = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i < wave) pre += wsum[i];
        all += wsum[i];
      }
      if (tid < nc) off_s[tid] = pre + ex;
      block_barrier_lds();                     // every thread has read carry_s
      if (tid == 0) carry_s += all;
      // copy: lane l of a wave takes slot l % S of a tile (64 / S tiles per pass when S <= 32)
      const int per = S <= 32 ? 64 / S : 1;
      const int sl = lane % S, sub = lane / S;
      for (int q0 = wave * per; q0 < nc; q0 += 16 * per) {
        const int q = q0 + sub;
        if (sub < per && q < nc && sl < st_s[q]) lrow[off_s[q] + sl] = stage[q * S + sl];
      }
    }
    block_barrier_lds();               // the stage and the offsets are free for the next chunk
  }
  if (tid == 0) {
    if (lists) f.row_nnz[t] = carry_s;
    const uint64_t mine = 1ull | ((uint64_t)(ovf_s ? 1u : 0u) << (32 + t));
    const uint64_t old = M == 1 ? 0ull : __hip_atomic_fetch_add(o.dec_ticket, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    last_s = (int)(old & 0xFFFFFFFFull) == M - 1;
    if (last_s) {
      const uint32_t flags = (uint32_t)((old + mine) >> 32);
      int r = 0;
      for (int i = 0; i < M; ++i) {
        int sl = -1;
        if ((flags >> i) & 1u) {
          if (r < f.cap) {
            sl = r;
            f.ovf_rows[r] = i;
          }
          ++r;
        }
        slot_s[i] = sl;
        f.ovf_slot[i] = sl;
      }
      *f.ovf_n = r;
      if (M > 1) __hip_atomic_store(o.dec_ticket, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  block_barrier_lds();
  if (!last_s) return;
  for (int i = 0; i < M; ++i) {
    const int sl = slot_s[i];
    if (sl < 0) continue;                      // uniform
    VT *row = (VT *)f.ovf_dense + (size_t)sl * N;
    const float *a0 = zp + (size_t)i * N, *a1 = zp + ((size_t)M + i) * N;
    for (int u = tid; u < N; u += 1024) {
      float h = a0[u] + a1[u] + b1[u];
      h = h > 0.f ? h : 0.f;
      Elem<VT>::store(row, u, h);
    }
  }
}

// Dense or N:M output of one 128-unit tile from its two half sums zs[half][u * TT + t] (token
// slots t < rows, columns n0 + u < N): (NK == 0) out[t][col] = ReLU(z + b1) (or z + b1) in fp32
// or bf16; (NK > 0) h rounded to bf16 and pruned NK:MM into vals / idx ([rows][N / MM][NK]),
// staged in hs.
template <int TT, int NK, int MM, int NT>
TW_DEV void gemv_dense_out(const float (&zs)[2][kGemvUnits * TT], char *hs, const float *__restrict__ b1, int rows,
                           int N, int n0, void *out, int out_bf16, int relu, uint8_t *__restrict__ idx) {
  const int tid = threadIdx.x;
  if constexpr (NK == 0) {
    for (int i = tid; i < kGemvUnits * TT; i += NT) {
      const int t = i / kGemvUnits, u = i % kGemvUnits, col = n0 + u;
      if (t >= rows || col >= N) continue;
      float h = zs[0][u * TT + t] + zs[1][u * TT + t] + b1[col];
      if (relu) h = h > 0.f ? h : 0.f;
      const size_t o = (size_t)t * N + col;
      if (out_bf16) ((uint16_t *)out)[o] = (uint16_t)f32_to_bf16(h);
      else ((float *)out)[o] = h;
    }
  } else {
    constexpr int RS = kGemvUnits * 2 + 16;
    for (int i = tid; i < kGemvUnits * TT; i += NT) {
      const int t = i / kGemvUnits, u = i % kGemvUnits, col = n0 + u;
      put_h<uint16_t>(hs + t * RS + u * 2, zs[0][u * TT + t] + zs[1][u * TT + t] + (col < N ? b1[col] : 0.f));
    }
    __syncthreads();
    nm_tile<uint16_t, NK, MM, TT, kGemvUnits, NT>(hs, rows, N, 0, n0, (uint16_t *)out, idx);
  }
}

// The dense and N:M forms for 3 to 16 tokens: one 128-unit tile per workgroup of 512 threads,
// wave w takes units 16 w .. 16 w + 15 over both halves of K in turn (mstream_wave), then
// gemv_dense_out with 16 token slots.
template <int NP, int NK, int MM>
__global__ __launch_bounds__(512) void k_up_mstream_dense(const uint16_t *__restrict__ x,
                                                          const uint16_t *__restrict__ w1t, const float *__restrict__ b1,
                                                          int M, int N, int K, const int32_t *__restrict__ arow,
                                                          const int32_t *__restrict__ n_rows_dev, void *out,
                                                          int out_bf16, int relu, uint8_t *__restrict__ idx) {
  constexpr int TT = kMsMaxT;
  __shared__ float zs[2][kGemvUnits * TT];
  __shared__ __attribute__((aligned(16))) char hs[NK > 0 ? TT * (kGemvUnits * 2 + 16) : 16];
  const int n0 = blockIdx.x * kGemvUnits, tid = threadIdx.x;
  int rows = M;
  if (n_rows_dev) rows = min(rows, *n_rows_dev);
  if (rows <= 0) return;
  const int w = tid >> 6, lane = tid & 63, t = lane & 15;
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    const f32x4_t z = mstream_wave<NP>(x, arow, rows, w1t, N, K, n0 + kGemvUPW * w, kh);
#pragma unroll
    for (int i = 0; i < 4; ++i) zs[kh][(kGemvUPW * w + 4 * (lane >> 4) + i) * TT + t] = z[i];
  }
  __syncthreads();
  gemv_dense_out<TT, NK, MM, 512>(zs, hs, b1, rows, N, n0, out, out_bf16, relu, idx);
}

// One 128-unit tile per workgroup of 512 threads: wave w takes units 16 w .. 16 w + 15 over
// both halves of K in turn, then (NK == 0) out[i][col] = ReLU(z + b1) (or z + b1) in fp32 or
// bf16 for token slots i < rows (x row arow[i] if arow), or (NK > 0) h rounded to bf16 and
// pruned NK:MM into vals / idx ([rows][N / MM][NK]).
template <int TT, int NP, int NK, int MM>
__global__ __launch_bounds__(512) void k_up_gemv_dense(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w1t,
                                                       const float *__restrict__ b1, int M, int N, int K,
                                                       const int32_t *__restrict__ arow,
                                                       const int32_t *__restrict__ n_rows_dev, void *out, int out_bf16,
                                                       int relu, uint8_t *__restrict__ idx) {
  __shared__ float zs[2][kGemvUnits * TT];
  __shared__ __attribute__((aligned(16))) char hs[NK > 0 ? TT * (kGemvUnits * 2 + 16) : 16];
  const int n0 = blockIdx.x * kGemvUnits, tid = threadIdx.x;
  int rows = M;
  if (n_rows_dev) rows = min(rows, *n_rows_dev);
  if (rows <= 0) return;
  const int w = tid >> 6, lane = tid & 63;
  const int vi = kGemvUPW * TT * w + gemv_value_index<16 * TT>(lane);
  const bool own = lane % (64 / (16 * TT)) == 0;
#pragma unroll
  for (int kh = 0; kh < 2; ++kh) {
    const float z = gemv_wave<TT, NP, 2>(x, arow, rows, w1t, N, K, n0 + kGemvUPW * w, kh);
    if (own) zs[kh][vi] = z;
  }
  __syncthreads();
  gemv_dense_out<TT, NK, MM, 512>(zs, hs, b1, rows, N, n0, out, out_bf16, relu, idx);
}

// bf16, 1 or 2 tokens (at c3 sizes: 26 / 28 us against 30 us for the tile kernel; from 3 tokens
// on the per-row dot products make it slower: 35 us at 3-4 tokens, 50 us at 8), K in
// {1024, 2048, 4096} (K / 2 in whole kilobyte pieces per lane).
static bool use_gemv(int bf16, int T_tokens, int K) {
  return bf16 && T_tokens >= 1 && T_tokens <= kGemvMaxT && (K == 1024 || K == 2048 || K == 4096);
}

// bf16, 3 to 16 tokens, K in {1024, 2048, 4096} (the steps are unrolled per K).
static bool use_mstream(int bf16, int T_tokens, int K) {
  return bf16 && T_tokens > kGemvMaxT && T_tokens <= kMsMaxT && (K == 1024 || K == 2048 || K == 4096);
}

// The decode kernels apply to at most 64 tokens and K a multiple of four stages.
template <typename T> static bool use_decode(int T_tokens, int K) {
  constexpr int KPT = TileD::RB / (int)sizeof(T);
  return T_tokens <= kDecodeMaxT && K % (4 * KPT) == 0;
}

// ------------------------------------------------------------------ host launchers

template <typename T, class G>
static hipError_t launch_twell_t(const T *x, const T *w1t, const float *b1, int M, int N, int K,
                                 const TwellOut &o, int W, hipStream_t s) {
  static_assert(G::SMEM <= 160 * 1024, "LDS");
  dim3 grid((N + G::BN - 1) / G::BN, (M + G::BM - 1) / G::BM);
  if (o.val_bf16) {
    if (W == 64) hipLaunchKernelGGL((k_up_twell<T, G, 64, uint16_t>), grid, dim3(G::NT), 0, s, x, w1t, b1, M, N, K, o);
    else hipLaunchKernelGGL((k_up_twell<T, G, 128, uint16_t>), grid, dim3(G::NT), 0, s, x, w1t, b1, M, N, K, o);
  } else {
    if (W == 64) hipLaunchKernelGGL((k_up_twell<T, G, 64, float>), grid, dim3(G::NT), 0, s, x, w1t, b1, M, N, K, o);
    else hipLaunchKernelGGL((k_up_twell<T, G, 128, float>), grid, dim3(G::NT), 0, s, x, w1t, b1, M, N, K, o);
  }
  return hipGetLastError();
}

static bool use_large(int M, int N) { return M >= 512 && N >= 1024; }

template <typename T>
static hipError_t launch_twell_dec(const T *x, const T *w1t, const float *b1, int M, int N, int K, const TwellOut &o,
                                   int W, hipStream_t s) {
  const dim3 grid(2 * ((N + TileD::BN - 1) / TileD::BN));
  if (o.val_bf16) {
    if (W == 64) hipLaunchKernelGGL((k_up_twell_dec<T, 64, uint16_t>), grid, dim3(128), 0, s, x, w1t, b1, M, N, K, o);
    else hipLaunchKernelGGL((k_up_twell_dec<T, 128, uint16_t>), grid, dim3(128), 0, s, x, w1t, b1, M, N, K, o);
  } else {
    if (W == 64) hipLaunchKernelGGL((k_up_twell_dec<T, 64, float>), grid, dim3(128), 0, s, x, w1t, b1, M, N, K, o);
    else hipLaunchKernelGGL((k_up_twell_dec<T, 128, float>), grid, dim3(128), 0, s, x, w1t, b1, M, N, K, o);
  }
  return hipGetLastError();
}

// After a stream kernel: the whole matrix (complete) or the TwELL alone, from the half sums.
template <int W, typename VT>
static void launch_dec_tail(const float *b1, int M, int N, const TwellOut &o, const TwellFinish &f, hipStream_t s) {
  if (f.complete)
    hipLaunchKernelGGL((k_dec_finish<W, VT>), dim3(M), dim3(1024), 0, s, o.dec_part, b1, M, N, o, f);
  else
    hipLaunchKernelGGL((k_dec_pack<W, VT>), dim3((M * o.n_t + 15) / 16), dim3(1024), 0, s, o.dec_part, b1, M, N, o);
}

// 1 to 16 bf16 tokens: the W1 stream (k_up_gemv_z for 1 or 2, k_up_mstream_z from 3) into the
// half sums of o.dec_part.
static void launch_stream_z(const uint16_t *x, const uint16_t *w1t, int M, int N, int K, const TwellOut &o,
                            hipStream_t s) {
  const dim3 grid(2 * ((N + kGemvUPW - 1) / kGemvUPW));
  if (M > kGemvMaxT) {
    if (K == 1024) hipLaunchKernelGGL((k_up_mstream_z<1>), grid, dim3(64), 0, s, x, nullptr, nullptr, M, w1t, N, K, o.dec_part, o.dec_ticket, o.ovf_bits, o.n_t, o.words);
    else if (K == 2048) hipLaunchKernelGGL((k_up_mstream_z<2>), grid, dim3(64), 0, s, x, nullptr, nullptr, M, w1t, N, K, o.dec_part, o.dec_ticket, o.ovf_bits, o.n_t, o.words);
    else hipLaunchKernelGGL((k_up_mstream_z<4>), grid, dim3(64), 0, s, x, nullptr, nullptr, M, w1t, N, K, o.dec_part, o.dec_ticket, o.ovf_bits, o.n_t, o.words);
  } else if (M == 1) {
    if (K == 1024) hipLaunchKernelGGL((k_up_gemv_z<1, 1>), grid, dim3(64), 0, s, x, nullptr, nullptr, M, w1t, N, K, o.dec_part, o.dec_ticket, o.ovf_bits, o.n_t, o.words);
    else if (K == 2048) hipLaunchKernelGGL((k_up_gemv_z<1, 2>), grid, dim3(64), 0, s, x, nullptr, nullptr, M, w1t, N, K, o.dec_part, o.dec_ticket, o.ovf_bits, o.n_t, o.words);
    else hipLaunchKernelGGL((k_up_gemv_z<1, 4>), grid, dim3(64), 0, s, x, nullptr, nullptr, M, w1t, N, K, o.dec_part, o.dec_ticket, o.ovf_bits, o.n_t, o.words);
  } else {
    if (K == 1024) hipLaunchKernelGGL((k_up_gemv_z<2, 1>), grid, dim3(64), 0, s, x, nullptr, nullptr, M, w1t, N, K, o.dec_part, o.dec_ticket, o.ovf_bits, o.n_t, o.words);
    else if (K == 2048) hipLaunchKernelGGL((k_up_gemv_z<2, 2>), grid, dim3(64), 0, s, x, nullptr, nullptr, M, w1t, N, K, o.dec_part, o.dec_ticket, o.ovf_bits, o.n_t, o.words);
    else hipLaunchKernelGGL((k_up_gemv_z<2, 4>), grid, dim3(64), 0, s, x, nullptr, nullptr, M, w1t, N, K, o.dec_part, o.dec_ticket, o.ovf_bits, o.n_t, o.words);
  }
}

// The stream, then the packing kernels.
static hipError_t launch_stream_twell(const uint16_t *x, const uint16_t *w1t, const float *b1, int M, int N, int K,
                                      const TwellOut &o, const TwellFinish &f, int W, hipStream_t s) {
  launch_stream_z(x, w1t, M, N, K, o, s);
  if (o.val_bf16) {
    if (W == 64) launch_dec_tail<64, uint16_t>(b1, M, N, o, f, s);
    else launch_dec_tail<128, uint16_t>(b1, M, N, o, f, s);
  } else {
    if (W == 64) launch_dec_tail<64, float>(b1, M, N, o, f, s);
    else launch_dec_tail<128, float>(b1, M, N, o, f, s);
  }
  return hipGetLastError();
}

template <int NK, int MM>
static hipError_t launch_mstream_dense_t(const uint16_t *x, const uint16_t *w1t, const float *b1, int M, int N, int K,
                                         const int32_t *arow, const int32_t *n_rows_dev, void *out, int out_bf16,
                                         int relu, uint8_t *idx, hipStream_t s) {
  const dim3 grid((N + kGemvUnits - 1) / kGemvUnits), blk(512);
  if (K == 1024)
    hipLaunchKernelGGL((k_up_mstream_dense<1, NK, MM>), grid, blk, 0, s, x, w1t, b1, M, N, K, arow, n_rows_dev, out,
                       out_bf16, relu, idx);
  else if (K == 2048)
    hipLaunchKernelGGL((k_up_mstream_dense<2, NK, MM>), grid, blk, 0, s, x, w1t, b1, M, N, K, arow, n_rows_dev, out,
                       out_bf16, relu, idx);
  else
    hipLaunchKernelGGL((k_up_mstream_dense<4, NK, MM>), grid, blk, 0, s, x, w1t, b1, M, N, K, arow, n_rows_dev, out,
                       out_bf16, relu, idx);
  return hipGetLastError();
}

template <int TT, int NK, int MM>
static void launch_gemv_dense_tt(const uint16_t *x, const uint16_t *w1t, const float *b1, int M, int N, int K,
                                 const int32_t *arow, const int32_t *n_rows_dev, void *out, int out_bf16, int relu,
                                 uint8_t *idx, hipStream_t s) {
  const dim3 grid((N + kGemvUnits - 1) / kGemvUnits), blk(512);
  if (K == 1024)
    hipLaunchKernelGGL((k_up_gemv_dense<TT, 1, NK, MM>), grid, blk, 0, s, x, w1t, b1, M, N, K, arow, n_rows_dev, out,
                       out_bf16, relu, idx);
  else if (K == 2048)
    hipLaunchKernelGGL((k_up_gemv_dense<TT, 2, NK, MM>), grid, blk, 0, s, x, w1t, b1, M, N, K, arow, n_rows_dev, out,
                       out_bf16, relu, idx);
  else
    hipLaunchKernelGGL((k_up_gemv_dense<TT, 4, NK, MM>), grid, blk, 0, s, x, w1t, b1, M, N, K, arow, n_rows_dev, out,
                       out_bf16, relu, idx);
}

template <int NK, int MM>
static hipError_t launch_gemv_dense_t(const uint16_t *x, const uint16_t *w1t, const float *b1, int M, int N, int K,
                                      int x_rows, const int32_t *arow, const int32_t *n_rows_dev, void *out,
                                      int out_bf16, int relu, uint8_t *idx, hipStream_t s) {
  if (x_rows <= 1) launch_gemv_dense_tt<1, NK, MM>(x, w1t, b1, M, N, K, arow, n_rows_dev, out, out_bf16, relu, idx, s);
  else launch_gemv_dense_tt<2, NK, MM>(x, w1t, b1, M, N, K, arow, n_rows_dev, out, out_bf16, relu, idx, s);
  return hipGetLastError();
}

bool up_stream_ok(int bf16, int M, int K) { return use_gemv(bf16, M, K) || use_mstream(bf16, M, K); }

hipError_t launch_up_stream(const void *x, const void *w1t, int M, int N, int K, const TwellOut &o, hipStream_t s) {
  if (!up_stream_ok(1, M, K) || !o.dec_part || (size_t)2 * M * N * 4 > o.dec_bytes) return hipErrorInvalidValue;
  launch_stream_z((const uint16_t *)x, (const uint16_t *)w1t, M, N, K, o, s);
  return hipGetLastError();
}

bool up_twell_completes(int bf16, int M, int K, const TwellFinish &f) {
  return f.complete && f.row_nnz && f.row_list && (use_gemv(bf16, M, K) || use_mstream(bf16, M, K));
}

hipError_t launch_up_twell(int bf16, const void *x, const void *w1t, const float *b1, int M, int N,
                           int K, const TwellOut &o, const TwellFinish &f, int W, hipStream_t s) {
  if ((bf16 ? use_decode<uint16_t>(M, K) || use_gemv(bf16, M, K) : use_decode<float>(M, K)) &&
      (!o.dec_part || !o.dec_ticket))
    return hipErrorInvalidValue;
  if (use_gemv(bf16, M, K) || use_mstream(bf16, M, K)) {
    if ((f.complete && (!f.ovf_n || !f.ovf_slot || (f.cap > 0 && (!f.ovf_rows || !f.ovf_dense)))) ||
        (size_t)2 * M * N * 4 > o.dec_bytes)
      return hipErrorInvalidValue;
    return launch_stream_twell((const uint16_t *)x, (const uint16_t *)w1t, b1, M, N, K, o, f, W, s);
  }
  if (bf16 && use_decode<uint16_t>(M, K))
    return launch_twell_dec<uint16_t>((const uint16_t *)x, (const uint16_t *)w1t, b1, M, N, K, o, W, s);
  if (!bf16 && use_decode<float>(M, K))
    return launch_twell_dec<float>((const float *)x, (const float *)w1t, b1, M, N, K, o, W, s);
  if (bf16) {
    if (use_large(M, N) && (TileL8::WN / W) * o.S <= 64)
      return launch_twell_t<uint16_t, TileL8>((const uint16_t *)x, (const uint16_t *)w1t, b1, M, N, K, o, W, s);
    if (use_large(M, N))
      return launch_twell_t<uint16_t, TileL>((const uint16_t *)x, (const uint16_t *)w1t, b1, M, N, K, o, W, s);
    return launch_twell_t<uint16_t, TileS>((const uint16_t *)x, (const uint16_t *)w1t, b1, M, N, K, o, W, s);
  }
  return launch_twell_t<float, TileSF>((const float *)x, (const float *)w1t, b1, M, N, K, o, W, s);
}

template <typename T, class G>
static hipError_t launch_dense_t(const T *x, const T *w1t, const float *b1, int M, int N, int K, int x_rows,
                                 const int32_t *arow, const int32_t *n_rows_dev, void *out, int out_bf16,
                                 int relu, hipStream_t s) {
  dim3 grid((N + G::BN - 1) / G::BN, (M + G::BM - 1) / G::BM);
  hipLaunchKernelGGL((k_up_dense<T, G>), grid, dim3(G::NT), 0, s, x, w1t, b1, M, N, K, x_rows, arow, n_rows_dev,
                     out, out_bf16, relu);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_dense_dec(const T *x, const T *w1t, const float *b1, int M, int N, int K, int x_rows,
                                   const int32_t *arow, const int32_t *n_rows_dev, void *out, int out_bf16, int relu,
                                   hipStream_t s) {
  const dim3 grid((N + TileDQ::BN - 1) / TileDQ::BN);
  hipLaunchKernelGGL((k_up_dense_dec<T>), grid, dim3(256), 0, s, x, w1t, b1, M, N, K, x_rows, arow, n_rows_dev, out,
                     out_bf16, relu);
  return hipGetLastError();
}

// The finish of at most 64 tokens after the decode tile GEMM (use_decode) in one launch, or
// hipErrorNotSupported where the recompute would take another kernel (then the caller launches
// the scan and the recompute separately).
hipError_t launch_finish_dec(int bf16, const TwellIn &h, const uint32_t *bits, int words, int32_t *ovf_n,
                             int32_t *ovf_rows, int32_t *ovf_slot, const void *x, const void *w1t, const float *b1,
                             int K, void *dense, hipStream_t s) {
  const int T = h.rows;
  if (T < 1 || T > 64 || words > 2 || use_gemv(bf16, T, K) || use_mstream(bf16, T, K) ||
      !(bf16 ? use_decode<uint16_t>(T, K) : use_decode<float>(T, K)))
    return hipErrorNotSupported;
  const int nlist = T;                                          // one row list per workgroup
  const int n_tiles = (h.cols + TileDQ::BN - 1) / TileDQ::BN;
  const dim3 grid(1 + nlist + n_tiles), blk(256);
  if (bf16) {
    if (h.val_bf16)
      hipLaunchKernelGGL((k_finish_dec<uint16_t, uint16_t>), grid, blk, 0, s, h, bits, words, ovf_n, ovf_rows, ovf_slot,
                         nlist, (const uint16_t *)x, (const uint16_t *)w1t, b1, K, dense, 1);
    else
      hipLaunchKernelGGL((k_finish_dec<uint16_t, float>), grid, blk, 0, s, h, bits, words, ovf_n, ovf_rows, ovf_slot,
                         nlist, (const uint16_t *)x, (const uint16_t *)w1t, b1, K, dense, 0);
  } else {
    if (h.val_bf16)
      hipLaunchKernelGGL((k_finish_dec<float, uint16_t>), grid, blk, 0, s, h, bits, words, ovf_n, ovf_rows, ovf_slot,
                         nlist, (const float *)x, (const float *)w1t, b1, K, dense, 1);
    else
      hipLaunchKernelGGL((k_finish_dec<float, float>), grid, blk, 0, s, h, bits, words, ovf_n, ovf_rows, ovf_slot,
                         nlist, (const float *)x, (const float *)w1t, b1, K, dense, 0);
  }
  return hipGetLastError();
}

// x_rows is the token count of the problem (for the overflow-row recompute it exceeds M): the
// K split is chosen by it, as in launch_up_twell, so both paths sum in the same order.
hipError_t launch_up_dense(int bf16, const void *x, const void *w1t, const float *b1, int M, int N, int K,
                           int x_rows, const int32_t *arow, const int32_t *n_rows_dev, void *out, int out_bf16,
                           int relu, hipStream_t s) {
  if (use_gemv(bf16, x_rows, K))
    return launch_gemv_dense_t<0, 0>((const uint16_t *)x, (const uint16_t *)w1t, b1, M, N, K, x_rows, arow, n_rows_dev,
                                     out, out_bf16, relu, nullptr, s);
  if (use_mstream(bf16, x_rows, K))
    return launch_mstream_dense_t<0, 0>((const uint16_t *)x, (const uint16_t *)w1t, b1, M, N, K, arow, n_rows_dev, out,
                                        out_bf16, relu, nullptr, s);
  if (bf16 && use_decode<uint16_t>(x_rows, K))
    return launch_dense_dec<uint16_t>((const uint16_t *)x, (const uint16_t *)w1t, b1, M, N, K, x_rows, arow,
                                      n_rows_dev, out, out_bf16, relu, s);
  if (!bf16 && use_decode<float>(x_rows, K))
    return launch_dense_dec<float>((const float *)x, (const float *)w1t, b1, M, N, K, x_rows, arow, n_rows_dev, out,
                                   out_bf16, relu, s);
  if (bf16) {
    if (use_large(M, N) && !arow)
      return launch_dense_t<uint16_t, TileL8>((const uint16_t *)x, (const uint16_t *)w1t, b1, M, N, K, x_rows, arow,
                                             n_rows_dev, out, out_bf16, relu, s);
    return launch_dense_t<uint16_t, TileS>((const uint16_t *)x, (const uint16_t *)w1t, b1, M, N, K, x_rows, arow,
                                           n_rows_dev, out, out_bf16, relu, s);
  }
  return launch_dense_t<float, TileSF>((const float *)x, (const float *)w1t, b1, M, N, K, x_rows, arow, n_rows_dev,
                                      out, out_bf16, relu, s);
}

// ------------------------------------------------------------------ up GEMM + N:M pruning

template <typename T, class G, int NK, int M>
static void launch_nm_one(const T *x, const T *w1t, const float *b1, int Mr, int N, int K, T *vals, uint8_t *idx,
                          hipStream_t s) {
  dim3 grid((N + G::BN - 1) / G::BN, (Mr + G::BM - 1) / G::BM);
  hipLaunchKernelGGL((k_up_nm<T, G, NK, M>), grid, dim3(G::NT), 0, s, x, w1t, b1, Mr, N, K, vals, idx);
}

template <typename T, class G>
static hipError_t launch_nm_t(const T *x, const T *w1t, const float *b1, int Mr, int N, int K, int n, int m,
                              T *vals, uint8_t *idx, hipStream_t s) {
  if (n == 2 && m == 4) launch_nm_one<T, G, 2, 4>(x, w1t, b1, Mr, N, K, vals, idx, s);
  else if (n == 4 && m == 8) launch_nm_one<T, G, 4, 8>(x, w1t, b1, Mr, N, K, vals, idx, s);
  else if (n == 8 && m == 16) launch_nm_one<T, G, 8, 16>(x, w1t, b1, Mr, N, K, vals, idx, s);
  else if (n == 16 && m == 32) launch_nm_one<T, G, 16, 32>(x, w1t, b1, Mr, N, K, vals, idx, s);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_nm_dec(const T *x, const T *w1t, const float *b1, int Mr, int N, int K, int n, int m,
                                T *vals, uint8_t *idx, hipStream_t s) {
  const dim3 grid((N + TileDQ::BN - 1) / TileDQ::BN), blk(256);
  if (n == 2 && m == 4) hipLaunchKernelGGL((k_up_nm_dec<T, 2, 4>), grid, blk, 0, s, x, w1t, b1, Mr, N, K, vals, idx);
  else if (n == 4 && m == 8) hipLaunchKernelGGL((k_up_nm_dec<T, 4, 8>), grid, blk, 0, s, x, w1t, b1, Mr, N, K, vals, idx);
  else if (n == 8 && m == 16) hipLaunchKernelGGL((k_up_nm_dec<T, 8, 16>), grid, blk, 0, s, x, w1t, b1, Mr, N, K, vals, idx);
  else if (n == 16 && m == 32) hipLaunchKernelGGL((k_up_nm_dec<T, 16, 32>), grid, blk, 0, s, x, w1t, b1, Mr, N, K, vals, idx);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

// The same kernel choice as launch_up_dense without gathered rows (x_rows = M), so the fused
// and the two-step results agree bit for bit.
hipError_t launch_up_nm(int bf16, const void *x, const void *w1t, const float *b1, int M, int N, int K, int n,
                        int m, void *vals, uint8_t *idx, hipStream_t s) {
  if (bf16) {
    const uint16_t *xb = (const uint16_t *)x, *wb = (const uint16_t *)w1t;
    uint16_t *vb = (uint16_t *)vals;
    if (use_gemv(bf16, M, K)) {
      if (n == 2 && m == 4) return launch_gemv_dense_t<2, 4>(xb, wb, b1, M, N, K, M, nullptr, nullptr, vb, 1, 1, idx, s);
      if (n == 4 && m == 8) return launch_gemv_dense_t<4, 8>(xb, wb, b1, M, N, K, M, nullptr, nullptr, vb, 1, 1, idx, s);
      if (n == 8 && m == 16) return launch_gemv_dense_t<8, 16>(xb, wb, b1, M, N, K, M, nullptr, nullptr, vb, 1, 1, idx, s);
      if (n == 16 && m == 32)
        return launch_gemv_dense_t<16, 32>(xb, wb, b1, M, N, K, M, nullptr, nullptr, vb, 1, 1, idx, s);
      return hipErrorInvalidValue;
    }
    if (use_mstream(bf16, M, K)) {
      if (n == 2 && m == 4) return launch_mstream_dense_t<2, 4>(xb, wb, b1, M, N, K, nullptr, nullptr, vb, 1, 1, idx, s);
      if (n == 4 && m == 8) return launch_mstream_dense_t<4, 8>(xb, wb, b1, M, N, K, nullptr, nullptr, vb, 1, 1, idx, s);
      if (n == 8 && m == 16) return launch_mstream_dense_t<8, 16>(xb, wb, b1, M, N, K, nullptr, nullptr, vb, 1, 1, idx, s);
      if (n == 16 && m == 32)
        return launch_mstream_dense_t<16, 32>(xb, wb, b1, M, N, K, nullptr, nullptr, vb, 1, 1, idx, s);
      return hipErrorInvalidValue;
    }
    if (use_decode<uint16_t>(M, K)) return launch_nm_dec<uint16_t>(xb, wb, b1, M, N, K, n, m, vb, idx, s);
    if (use_large(M, N)) return launch_nm_t<uint16_t, TileL8>(xb, wb, b1, M, N, K, n, m, vb, idx, s);
    return launch_nm_t<uint16_t, TileS>(xb, wb, b1, M, N, K, n, m, vb, idx, s);
  }
  const float *xf = (const float *)x, *wf = (const float *)w1t;
  float *vf = (float *)vals;
  if (use_decode<float>(M, K)) return launch_nm_dec<float>(xf, wf, b1, M, N, K, n, m, vf, idx, s);
  return launch_nm_t<float, TileSF>(xf, wf, b1, M, N, K, n, m, vf, idx, s);
}

}  // namespace tw
