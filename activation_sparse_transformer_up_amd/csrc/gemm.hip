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
// Operand staging: every K step moves 128 bytes of each operand row (64 bf16 or 32 fp32)
// = 8 chunks of 16 bytes, global -> registers -> LDS, double-buffered (one barrier per
// step). Chunk c of LDS row r is stored at position c ^ (r & 7) so that the 32 rows an
// MFMA operand read touches spread over the LDS banks.
//
// Accumulation order of one output element depends only on K and the fixed step order,
// not on the tile shape or the row's position, so every epilogue (TwELL, dense, backup
// rows) sees bit-identical z values.
#include "common.h"
#include "launch.h"

namespace tw {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <typename T> struct MfmaOps;

// bf16: one v_mfma_f32_32x32x16_bf16 per step; lanes 0-31 bring one 16-byte chunk
// (8 k values), lanes 32-63 the next one.
template <> struct MfmaOps<uint16_t> {
  static constexpr int KPT = 64;   // k values per 128-byte row
  static TW_DEV void step(f32x16_t &acc, u32x4_t a, u32x4_t b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  }
};

// fp32: a 16-byte chunk holds 4 k values; four v_mfma_f32_32x32x2_f32 consume them, lane
// half h bringing k = 4h + s in the s-th one (A and B use the same assignment).
template <> struct MfmaOps<float> {
  static constexpr int KPT = 32;
  static TW_DEV void step(f32x16_t &acc, u32x4_t a, u32x4_t b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
};

template <int BM_, int BN_, int WM_, int WN_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int NWM = BM / WM, NWN = BN / WN, NW = NWM * NWN, NT = NW * 64;
  static constexpr int MB = WM / 32, NB = WN / 32;
  static constexpr int CH_A = BM * 8 / NT, CH_B = BN * 8 / NT;   // 16-byte chunks / thread
  static constexpr int LDS_A = BM * 128, LDS_B = BN * 128;
  static constexpr int LDS_BYTES = 2 * (LDS_A + LDS_B);
  static_assert(CH_A >= 1 && CH_B >= 1 && (BM * 8) % NT == 0 && (BN * 8) % NT == 0, "tile");
};

// Large tiles for many tokens, small tiles for few. Waves are 128 columns wide in the
// large tile and the small one so that a 64- or 128-wide TwELL tile never straddles
// two waves.
typedef Tile<256, 256, 128, 128> TileL;
typedef Tile<64, 128, 32, 128> TileS;

// A operand row r of the tile reads global row arow[m0 + r] (if arow) or m0 + r; rows at or
// beyond a_rows are zero. B operand rows at or beyond b_rows are zero.
template <typename T, class G>
TW_DEV void mainloop(const T *__restrict__ A, const int32_t *__restrict__ arow, int a_rows,
                     const T *__restrict__ B, int b_rows, int K, int m0, int n0,
                     f32x16_t (&acc)[G::MB][G::NB], char *smem) {
  constexpr int EPC = 16 / sizeof(T);
  constexpr int KPT = MfmaOps<T>::KPT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / G::NWN, wn = wave % G::NWN;
  const int cth = tid & 7;                     // this thread's chunk column (NT % 8 == 0)

  const T *pa[G::CH_A];
  const T *pb[G::CH_B];
  int oa[G::CH_A], ob[G::CH_B];
  bool va[G::CH_A], vb[G::CH_B];
#pragma unroll
  for (int i = 0; i < G::CH_A; ++i) {
    const int q = tid + i * G::NT, r = q >> 3;
    const int gr = m0 + r;
    va[i] = gr < a_rows;
    const size_t row = va[i] ? (size_t)(arow ? arow[gr] : gr) : 0;
    pa[i] = A + row * (size_t)K + cth * EPC;
    oa[i] = r * 128 + ((cth ^ (r & 7)) << 4);
  }
#pragma unroll
  for (int i = 0; i < G::CH_B; ++i) {
    const int q = tid + i * G::NT, r = q >> 3;
    const int gr = n0 + r;
    vb[i] = gr < b_rows;
    pb[i] = B + (size_t)(vb[i] ? gr : 0) * (size_t)K + cth * EPC;
    ob[i] = r * 128 + ((cth ^ (r & 7)) << 4);
  }

  u32x4_t ra[G::CH_A], rb[G::CH_B];
  const int nk = (K + KPT - 1) / KPT;
  auto gload = [&](int kt) {
    const int k0 = kt * KPT;
    const bool kin = k0 + cth * EPC < K;
#pragma unroll
    for (int i = 0; i < G::CH_A; ++i)
      ra[i] = (va[i] && kin) ? *(const u32x4_t *)(pa[i] + k0) : u32x4_t{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < G::CH_B; ++i)
      rb[i] = (vb[i] && kin) ? *(const u32x4_t *)(pb[i] + k0) : u32x4_t{0, 0, 0, 0};
  };
  auto sstore = [&](int buf) {
    char *sa = smem + buf * (G::LDS_A + G::LDS_B);
    char *sb = sa + G::LDS_A;
#pragma unroll
    for (int i = 0; i < G::CH_A; ++i) *(u32x4_t *)(sa + oa[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < G::CH_B; ++i) *(u32x4_t *)(sb + ob[i]) = rb[i];
  };
  const int lr = lane & 31, lh = lane >> 5;
  auto compute = [&](int buf) {
    const char *sa = smem + buf * (G::LDS_A + G::LDS_B);
    const char *sb = sa + G::LDS_A;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = 2 * u + lh;
      u32x4_t a[G::MB], b[G::NB];
#pragma unroll
      for (int mb = 0; mb < G::MB; ++mb) {
        const int r = wm * G::WM + mb * 32 + lr;
        a[mb] = *(const u32x4_t *)(sa + r * 128 + ((c ^ (r & 7)) << 4));
      }
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb) {
        const int r = wn * G::WN + nb * 32 + lr;
        b[nb] = *(const u32x4_t *)(sb + r * 128 + ((c ^ (r & 7)) << 4));
      }
#pragma unroll
      for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb) MfmaOps<T>::step(acc[mb][nb], a[mb], b[nb]);
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) gload(kt + 1);
    compute(kt & 1);
    if (kt + 1 < nk) sstore((kt + 1) & 1);
    __syncthreads();
  }
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
template <class G, int W>
TW_DEV void epi_twell(f32x16_t (&acc)[G::MB][G::NB], const float *__restrict__ b1, int M, int N,
                      int m0, int n0, const TwellOut &o) {
  constexpr int BPT = W / 32;                   // 32-column blocks per TwELL tile
  constexpr int TPW = G::WN / W;                // TwELL tiles per wave
  static_assert(G::WN % W == 0, "a TwELL tile must sit inside one wave");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / G::NWN, wn = wave % G::NWN;
  const int lh = lane >> 5, li = lane & 31;
  const int row0 = m0 + wm * G::WM, col0 = n0 + wn * G::WN;
  const uint32_t below = (1u << li) - 1u;
  const int S = o.S;
  float bias[G::NB];
#pragma unroll
  for (int nb = 0; nb < G::NB; ++nb) {
    const int col = col0 + nb * 32 + li;
    bias[nb] = col < N ? b1[col] : 0.f;
  }
#pragma unroll
  for (int q = 0; q < TPW; ++q) {
    const int kt = col0 / W + q;
    if (kt * W >= N) break;
#pragma unroll
    for (int mb = 0; mb < G::MB; ++mb) {
      uint32_t ovf_word = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = row0 + mb * 32 + acc_row(r, lh);
        const bool rv = row < M;
        float v[BPT];
        uint32_t hm[BPT];
        int pre[BPT];
        int cnt = 0;
#pragma unroll
        for (int b = 0; b < BPT; ++b) {
          const int nb = q * BPT + b;
          const float z = acc[mb][nb][r] + bias[nb];
          v[b] = z;
          const uint64_t bal = ballot64(z > 0.f);
          hm[b] = lh ? (uint32_t)(bal >> 32) : (uint32_t)bal;
          pre[b] = cnt;
          cnt += __popc(hm[b]);
        }
        if (rv) {
          const size_t base = ((size_t)row * o.n_t + kt) * (size_t)S;
#pragma unroll
          for (int b = 0; b < BPT; ++b) {
            const int slot = pre[b] + __popc(hm[b] & below);
            if (v[b] > 0.f && slot < S) {
              const int col = kt * W + b * 32 + li;
              o.col_idx[base + slot] = col;
              if (o.val_bf16) ((uint16_t *)o.vals)[base + slot] = (uint16_t)f32_to_bf16(v[b]);
              else ((float *)o.vals)[base + slot] = v[b];
            }
          }
          for (int s = li; s < S; s += 32) {
            if (s >= cnt) {
              o.col_idx[base + s] = -1;
              if (o.val_bf16) ((uint16_t *)o.vals)[base + s] = 0;
              else ((float *)o.vals)[base + s] = 0.f;
            }
          }
          if (li == 0) o.counts[(size_t)row * o.n_t + kt] = cnt;
        }
        const uint64_t ob = ballot64(rv && cnt > S);
        const int bit = 8 * (r >> 2) + (r & 3);
        if (ob & 1ull) ovf_word |= 1u << bit;
        if ((ob >> 32) & 1ull) ovf_word |= 1u << (bit + 4);
      }
      const int w = (row0 + mb * 32) >> 5;
      if (lane == 0 && w < o.words) o.ovf_bits[(size_t)kt * o.words + w] = ovf_word;
    }
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

// ------------------------------------------------------------------------ kernels

template <typename T, class G, int W>
__global__ __launch_bounds__(G::NT) void k_up_twell(const T *__restrict__ x, const T *__restrict__ w1t,
                                                    const float *__restrict__ b1, int M, int N, int K,
                                                    TwellOut o) {
  __shared__ __attribute__((aligned(16))) char smem[G::LDS_BYTES];
  const int n0 = blockIdx.x * G::BN, m0 = blockIdx.y * G::BM;
  f32x16_t acc[G::MB][G::NB];
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb) acc[mb][nb] = f32x16_t{};
  mainloop<T, G>(x, nullptr, M, w1t, N, K, m0, n0, acc, smem);
  epi_twell<G, W>(acc, b1, M, N, m0, n0, o);
}

// Dense ReLU(x W1 + b1). With arow != NULL the A rows are gathered: tile row i reads x row
// arow[i] for i < min(*n_rows_dev, M) (the overflow rows of a TwELL), and writes out row i.
template <typename T, class G>
__global__ __launch_bounds__(G::NT) void k_up_dense(const T *__restrict__ x, const T *__restrict__ w1t,
                                                    const float *__restrict__ b1, int M, int N, int K,
                                                    const int32_t *__restrict__ arow,
                                                    const int32_t *__restrict__ n_rows_dev, void *out,
                                                    int out_bf16, int relu) {
  __shared__ __attribute__((aligned(16))) char smem[G::LDS_BYTES];
  const int n0 = blockIdx.x * G::BN, m0 = blockIdx.y * G::BM;
  int rows = M;
  if (n_rows_dev) rows = min(rows, *n_rows_dev);
  if (m0 >= rows) return;
  f32x16_t acc[G::MB][G::NB];
#pragma unroll
  for (int mb = 0; mb < G::MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb) acc[mb][nb] = f32x16_t{};
  mainloop<T, G>(x, arow, rows, w1t, N, K, m0, n0, acc, smem);
  epi_dense<G>(acc, b1, rows, N, m0, n0, out, out_bf16, relu);
}

// ------------------------------------------------------------------ host launchers

template <typename T, class G>
static hipError_t launch_twell_t(const T *x, const T *w1t, const float *b1, int M, int N, int K,
                                 const TwellOut &o, int W, hipStream_t s) {
  dim3 grid((N + G::BN - 1) / G::BN, (M + G::BM - 1) / G::BM);
  if (W == 64) hipLaunchKernelGGL((k_up_twell<T, G, 64>), grid, dim3(G::NT), 0, s, x, w1t, b1, M, N, K, o);
  else hipLaunchKernelGGL((k_up_twell<T, G, 128>), grid, dim3(G::NT), 0, s, x, w1t, b1, M, N, K, o);
  return hipGetLastError();
}

static bool use_large(int M, int N) { return M >= 512 && N >= 1024; }

hipError_t launch_up_twell(int bf16, const void *x, const void *w1t, const float *b1, int M, int N,
                           int K, const TwellOut &o, int W, hipStream_t s) {
  if (bf16) {
    if (use_large(M, N))
      return launch_twell_t<uint16_t, TileL>((const uint16_t *)x, (const uint16_t *)w1t, b1, M, N, K, o, W, s);
    return launch_twell_t<uint16_t, TileS>((const uint16_t *)x, (const uint16_t *)w1t, b1, M, N, K, o, W, s);
  }
  return launch_twell_t<float, TileS>((const float *)x, (const float *)w1t, b1, M, N, K, o, W, s);
}

template <typename T, class G>
static hipError_t launch_dense_t(const T *x, const T *w1t, const float *b1, int M, int N, int K,
                                 const int32_t *arow, const int32_t *n_rows_dev, void *out, int out_bf16,
                                 int relu, hipStream_t s) {
  dim3 grid((N + G::BN - 1) / G::BN, (M + G::BM - 1) / G::BM);
  hipLaunchKernelGGL((k_up_dense<T, G>), grid, dim3(G::NT), 0, s, x, w1t, b1, M, N, K, arow, n_rows_dev,
                     out, out_bf16, relu);
  return hipGetLastError();
}

hipError_t launch_up_dense(int bf16, const void *x, const void *w1t, const float *b1, int M, int N, int K,
                           const int32_t *arow, const int32_t *n_rows_dev, void *out, int out_bf16,
                           int relu, hipStream_t s) {
  if (bf16) {
    if (use_large(M, N) && !arow)
      return launch_dense_t<uint16_t, TileL>((const uint16_t *)x, (const uint16_t *)w1t, b1, M, N, K, arow,
                                             n_rows_dev, out, out_bf16, relu, s);
    return launch_dense_t<uint16_t, TileS>((const uint16_t *)x, (const uint16_t *)w1t, b1, M, N, K, arow,
                                           n_rows_dev, out, out_bf16, relu, s);
  }
  return launch_dense_t<float, TileS>((const float *)x, (const float *)w1t, b1, M, N, K, arow, n_rows_dev,
                                      out, out_bf16, relu, s);
}

}  // namespace tw
