// Gated feed-forward: the up projection over the gate's active units only.
//
// "Sparser, Faster, Lighter Transformer Language Models", section "2. Metodologia": the
// TwELL layout is produced by the dense product that computes the gate activations (block
// "Formato de Dados TwELL"), and the inference kernel iterates over the active units only,
// taking a dot product with the up weights and then multiplying-adding the unit's down row
// (block "Kernels de Inferência"). Here the dot products are a stage of their own between
// the gate's finish (row lists, overflow backup) and the down gather: for every entry
// (j, g) of a token's row list g <- g * (x[t] . w_up[j]), and the same for every nonzero
// of a dense backup row. The gather then sums (g u)_j w2[j].
//
// Few tokens (k_gate_dot): a wave takes ENT list entries at a time. Lane l holds 16-byte
// pieces l, l + 64, ... of x[t] (8 bf16 or 4 fp32 per piece), loads the same pieces of the
// ENT up rows before any arithmetic, and accumulates with v_dot2_f32_bf16 (bf16; two products
// per instruction, fp32 accumulation) or fp32 FMAs; the ENT sums are reduced across the wave
// and lane 0 rewrites the entries' values.
// Many tokens (k_gate_part + k_gate_sum): the products of all tokens read the whole of w_up
// from every XCD, so each XCD would fetch it from the shared last-level cache. As in the
// backward's SDDMM, the dot products are cut into 16-lane column chunks instead: chunk c runs
// on XCD c % 8, whose L2 then holds only its slices of w_up and x, and writes one partial per
// (entry, chunk) to the workspace; a second kernel adds the partials in chunk order.
#include "common.h"
#include "gather.h"
#include "launch.h"
#include "rows.h"
#include "stage.h"

namespace tw {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kGateEnt = 4;      // list entries per wave and round
constexpr int kGateDotEnt = 2;   // the same for k_gate_dot (measured at c3 T = 64)

template <typename XT> TW_DEV float dot16(uint4 a, uint4 b, float acc) {
  if constexpr (sizeof(XT) == 2) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.x), __builtin_bit_cast(bf16x2_t, b.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.y), __builtin_bit_cast(bf16x2_t, b.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.z), __builtin_bit_cast(bf16x2_t, b.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w), __builtin_bit_cast(bf16x2_t, b.w), acc, false);
  } else {
    acc = fmaf(__uint_as_float(a.x), __uint_as_float(b.x), acc);
    acc = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), acc);
    acc = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), acc);
    acc = fmaf(__uint_as_float(a.w), __uint_as_float(b.w), acc);
  }
  return acc;
}

// u[k] = x_row . wu[col[k]] for k < ENT (col[k] < 0: no entry, u = 0), summed over the wave.
// NP 16-byte pieces per lane are in flight at once (NP = 4 covers 2048 bf16 columns; fewer
// registers than needed for larger rows would cost occupancy for nothing at small d).
template <typename XT, int NP, int ENT = kGateEnt>
TW_DEV void wave_dots(const XT *__restrict__ xrow, const XT *__restrict__ wu, int d, const int (&col)[ENT],
                      float (&u)[ENT], int rows) {
  constexpr int EPL = 16 / sizeof(XT);
  const int lane = lane_id();
  const int npc = (d + 64 * EPL - 1) / (64 * EPL);
  const __amdgpu_buffer_rsrc_t rs = rows_rsrc(wu, rows_bytes<XT>(rows, d));
#pragma unroll
  for (int k = 0; k < ENT; ++k) u[k] = 0.f;
  for (int c0 = 0; c0 < npc; c0 += NP) {
    uint4 xv[NP], wv[ENT][NP];
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      const int i = ((c0 + q) * 64 + lane) * EPL;
      const bool ok = i < d;                                    // d is a multiple of EPL
      xv[q] = ok ? *(const uint4 *)(xrow + i) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int k = 0; k < ENT; ++k)
        wv[k][q] = (ok && col[k] >= 0) ? ld16<XT>(rs, (uint32_t)col[k] * (uint32_t)d + (uint32_t)i) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < NP; ++q)
#pragma unroll
      for (int k = 0; k < ENT; ++k) u[k] = dot16<XT>(xv[q], wv[k][q], u[k]);
  }
#pragma unroll
  for (int k = 0; k < ENT; ++k) u[k] = wave_sumf(u[k]);
}

// Row lists: workgroup (t, p) of 4 waves, numbered p * rows + t; wave w takes the entry
// groups p * 4 + w, p * 4 + w + 4 P, ... of ENT entries each (ENT = kGateDotEnt: two entries
// keep 2 NP row pieces per lane in flight, up to 16, and twice as many waves busy as four). Slot p of every token comes
// before slot p + 1 of any, so the workgroups that have entries (small p; P is sized for
// the longest possible list) are dispatched first and the empty ones last. Overflow rows
// are skipped (their backup row carries them).
template <typename XT, int NP, int ENT>
TW_DEV void gate_dot_wg(const TwellIn &h, const XT *__restrict__ x, const XT *__restrict__ wu, int d, int P, int b) {
  const int t = b % h.rows, p = b / h.rows;
  if (p >= P) return;
  // the overflow flag and the list length in one round trip, each entry's (column, gate)
  // pair in one load: the gate is kept for the final product instead of being re-read
  const int oslot = h.ovf_slot[t], nnz = list_len(h, h.row_nnz[t]);
  if (oslot >= 0) return;
  const int wave = threadIdx.x >> 6, lane = lane_id();
  uint2 *lst = h.row_list + (size_t)t * h.n_t * h.S;
  const XT *xrow = x + (size_t)t * d;
  for (int e0 = (p * 4 + wave) * ENT; e0 < nnz; e0 += P * 4 * ENT) {
    int col[ENT];
    float gv[ENT];
#pragma unroll
    for (int k = 0; k < ENT; ++k) {
      const uint2 en = e0 + k < nnz ? lst[e0 + k] : make_uint2(0xFFFFFFFFu, 0u);
      col[k] = (int)en.x;
      gv[k] = __uint_as_float(en.y);
    }
    float u[ENT];
    wave_dots<XT, NP, ENT>(xrow, wu, d, col, u, h.cols);
    if (lane == 0)
#pragma unroll
      for (int k = 0; k < ENT; ++k)
        if (col[k] >= 0) lst[e0 + k].y = __float_as_uint(gv[k] * u[k]);
  }
}

template <typename XT, int NP, int ENT>
__global__ __launch_bounds__(256) void k_gate_dot(TwellIn h, const XT *__restrict__ x, const XT *__restrict__ wu,
                                                  int d, int P) {
  gate_dot_wg<XT, NP, ENT>(h, x, wu, d, P, blockIdx.x);
}

// Backup rows (gate_backup_wave, in the launch of k_gate_dot_all below 512 tokens and of
// k_gate_sum_all from 512): wave (r0, blk) takes the 64-column block blk of the overflow rows r0,
// r0 + rstep, ... below min(ovf_n, cap); the block's nonzero gates are taken ENT at a time
// in ascending column order. The grid covers rstep = min(cap, kGateBackupRows) rows, not the
// whole capacity: the overflow count is only known on the device, and it is usually zero, so
// most of a capacity-sized grid would start only to exit.
constexpr int kGateBackupRows = 8;

template <typename XT, typename VT, int NP, int ENT>
TW_DEV void gate_backup_wave(const TwellIn &h, const XT *__restrict__ x, const XT *__restrict__ wu, int d, int rstep,
                             int wave_g) {
  const int nblk = (h.cols + 63) / 64;
  const int r0 = wave_g / nblk, blk = wave_g % nblk;
  if (r0 >= rstep) return;                                      // past the grid's rows
  const int nr = min(*h.ovf_n, h.cap);
  const int lane = lane_id();
  const int j = blk * 64 + lane;
  for (int r = r0; r < nr; r += rstep) {                        // wave-uniform
    const int t = h.ovf_rows[r];
    VT *row = (VT *)h.ovf_dense + (size_t)r * h.cols;
    const float g = j < h.cols ? Elem<VT>::load(row, j) : 0.f;
    uint64_t m = ballot64(g != 0.f);
    while (m) {
      int col[ENT];
#pragma unroll
      for (int k = 0; k < ENT; ++k) {
        col[k] = m ? blk * 64 + (int)__builtin_ctzll(m) : -1;
        m &= m ? m - 1 : 0;
      }
      float u[ENT];
      wave_dots<XT, NP, ENT>(x + (size_t)t * d, wu, d, col, u, h.cols);
#pragma unroll
      for (int k = 0; k < ENT; ++k) {
        const float gk = __shfl(g, col[k] & 63, 64);
        if (lane == 0 && col[k] >= 0) Elem<VT>::store(row, col[k], gk * u[k]);
      }
    }
  }
}


// k_gate_dot and the backup rows in one launch: workgroups 0 .. nA - 1 run k_gate_dot, the
// others the backup rows at k_gate_dot's shape (NP pieces per lane, ENT entries per round; the
// per-entry sums do not depend on either), so the backup needs no launch of its own when, as
// usual, no row overflowed.
template <typename XT, int NP, int ENT, typename VT>
__global__ __launch_bounds__(256) void k_gate_dot_all(TwellIn h, const XT *__restrict__ x, const XT *__restrict__ wu,
                                                      int d, int P, int nA, int rstep) {
  const int b = blockIdx.x;
  if (b < nA) gate_dot_wg<XT, NP, ENT>(h, x, wu, d, P, b);
  else gate_backup_wave<XT, VT, NP, ENT>(h, x, wu, d, rstep, (b - nA) * 4 + (threadIdx.x >> 6));
}

// part[c][t][e] = x[t][chunk c] . wu[col][chunk c] for the entries e of token t's row list
// (normal rows; a backup row has row_nnz < 0 and is done in k_gate_sum_all). Block b runs on
// XCD b % 8 with chunk b % 8 + 8 * ((b / 8) / ntb) and token block (b / 8) % ntb of 16
// tokens, one per 16-lane group; lane l holds 16 bytes of x[t]. Per round the group loads its
// next 16 pairs (coalesced), broadcasts the columns, issues the 16 up-row loads, and sums the
// 16 per-lane dot products across the group so that lane l stores entry l.
template <typename XT>
__global__ __launch_bounds__(256) void k_gate_part(TwellIn h, int d, int nchunk, int ntb, const XT *__restrict__ x,
                                                   const XT *__restrict__ wu, float *__restrict__ part) {
  constexpr int E = Vec16<XT>::N;
  constexpr int CW = 16 * E;
  const int b = blockIdx.x, xcd = b & 7, i = b >> 3;
  const int c = xcd + 8 * (i / ntb), tb = i % ntb;
  if (c >= nchunk) return;
  const int lane = lane_id(), g = lane >> 4, gl = lane & 15;
  const int t = tb * 16 + (threadIdx.x >> 6) * 4 + g;
  const int colo = c * CW + gl * E;
  const bool cv = colo < d;
  const __amdgpu_buffer_rsrc_t rs = rows_rsrc(wu, rows_bytes<XT>(h.cols, d));
  const size_t cap = (size_t)h.n_t * h.S;
  const int n = t < h.rows ? list_len(h, h.row_nnz[t]) : 0;
  int nw = max(n, __shfl_xor(n, 16, 64));
  nw = max(nw, __shfl_xor(nw, 32, 64));
  const int tt = t < h.rows ? t : 0;
  const uint4 a = (t < h.rows && cv) ? *(const uint4 *)(x + (size_t)tt * d + colo) : make_uint4(0, 0, 0, 0);
  const uint2 *lp = h.row_list + (size_t)tt * cap;
  float *out = part + ((size_t)c * h.rows + tt) * cap;
  int jn = gl < n ? (int)lp[gl].x : 0;
  // as in gather_list16: one 24-bit multiply-add per row piece, loads issued without a
  // per-lane branch (entries past the list and columns past the row read zeros through the
  // range check), rounds bounded by the wave's longest list (scalar branch)
  constexpr uint32_t OOB = 0x80000000u;
  const uint32_t rowb = (uint32_t)d * (uint32_t)sizeof(XT), colb = (uint32_t)colo * (uint32_t)sizeof(XT);
  for (int base = 0; base < nw; base += 16) {
    const int jq = jn;
    if (base + 16 < nw) jn = base + 16 + gl < n ? (int)lp[base + 16 + gl].x : 0;
    const int rem = nw - base;
    float v[16];
    auto round = [&](auto full_tag) {
      constexpr bool FULL = decltype(full_tag)::value;
      uint4 raw[16];
      static_for<16>([&](auto J) {
        constexpr int j = decltype(J)::value;
        if (!FULL && j >= rem) return;
        const uint32_t jj = row_bcast<j>((uint32_t)jq);
        const uint32_t off = (base + j < n && cv) ? __umul24(jj, rowb) + colb : OOB;
        const u32x4_t r = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0);
        raw[j] = make_uint4(r.x, r.y, r.z, r.w);
      });
      static_for<16>([&](auto J) {
        constexpr int j = decltype(J)::value;
        if (!FULL && j >= rem) {
          v[j] = 0.f;
          return;
        }
        v[j] = dot16<XT>(a, raw[j], 0.f);
      });
    };
    if (rem >= 16) round(std::true_type());
    else round(std::false_type());
    const float tot = group16_transpose_sum(v, gl);
    if (base + gl < n) out[base + gl] = tot;
  }
}

// Row list entry e of token t: g <- g * (sum over chunks c of part[c][t][e], in chunk order).
// One wave per token, lanes over the entries; each lane has the loads of 16 chunks in flight
// (clamped to valid addresses) before it adds them in order.
TW_DEV void gate_sum_wg(const TwellIn &h, int nchunk, const float *__restrict__ part, int b) {
  const int t = b * 4 + (threadIdx.x >> 6);
  if (t >= h.rows) return;
  const int n = list_len(h, h.row_nnz[t]);
  const size_t cap = (size_t)h.n_t * h.S, plane = (size_t)h.rows * cap;
  uint2 *lp = h.row_list + (size_t)t * cap;
  const float *pp = part + (size_t)t * cap;
  for (int e = lane_id(); e < n; e += 64) {
    float u = 0.f;
    for (int c0 = 0; c0 < nchunk; c0 += 16) {
      float v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) v[j] = pp[(size_t)min(c0 + j, nchunk - 1) * plane + e];
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (c0 + j < nchunk) u += v[j];
    }
    const uint2 q = lp[e];
    lp[e].y = __float_as_uint(__uint_as_float(q.y) * u);
  }
}

__global__ __launch_bounds__(256) void k_gate_sum(TwellIn h, int nchunk, const float *__restrict__ part) {
  gate_sum_wg(h, nchunk, part, blockIdx.x);
}

// k_gate_sum and the backup rows' products in one launch (many tokens): workgroups
// 0 .. nA - 1 add the partials, the others run the backup rows at k_gate_dot's shape (NP pieces
// per lane, ENT entries per round; the per-entry sums do not depend on either). The two touch
// disjoint data: list entries of normal rows, and the dense backup rows.
template <typename XT, int NP, int ENT, typename VT>
__global__ __launch_bounds__(256) void k_gate_sum_all(TwellIn h, int nchunk, const float *__restrict__ part,
                                                      const XT *__restrict__ x, const XT *__restrict__ wu, int d,
                                                      int nA, int rstep) {
  const int b = blockIdx.x;
  if (b < nA) gate_sum_wg(h, nchunk, part, b);
  else gate_backup_wave<XT, VT, NP, ENT>(h, x, wu, d, rstep, (b - nA) * 4 + (threadIdx.x >> 6));
}

// ------------------------------------------------------------ fused inference kernel
// "Kernels de Inferência": after the gate GEMM has written the TwELL of the gate, a single
// kernel walks each token's active units, takes the up dot product u = x[t] . w_up[j] and
// multiplies-adds (g u) w2[j] into y[t]. It runs in one launch and two kinds of work item:
//   up items (t, group of 4 tiles), claimed in batches from a work counter: for every active
//     slot (j, g) of the tiles, u = x[t] . w_up[j] and the pair (j, g u) is written to the
//     slot's place in row_list (read as [t][tile][S]); a tile holding more than S active
//     units lost units in its slots, so its gate pre-activations are recomputed
//     (x[t] . w_gate[j] + b[j], rounded to the value type as the TwELL stores it) and g u
//     (0 where inactive) goes to the token's dense row in the scratch. Each finished item
//     counts on its token;
//   down items (t, 512-column chunk), four waves of 128 columns: when every up item of token
//     t has finished, the token's pairs (from its slots and dense tiles, ascending column
//     order) are staged in LDS 256 at a time and the waves multiply-add the W2 row pieces.
// A workgroup takes down items only after the work counter has run past the last up item, so
// every up item it may wait for has been claimed by a running workgroup: no waiting depends
// on which workgroups are resident (no cooperative launch, no grid barrier).
// Values handed between work items (pairs, dense rows, counters) are written and read with
// agent-scope atomic accesses, which are coherent across the XCDs' L2 caches by themselves.
// Scratch: the decode workspace of the row-list scratch (free once the gate GEMM has ended):
// dense rows [T][f] fp32, and the state words at its end (fused_prepare).
constexpr int kFusedTilesPerItem = 1;
constexpr int kFusedUpBatch = 4;             // up items per claim (one per wave)
constexpr int kFusedGroups = 8;              // work counters: up items split in 8 ranges
constexpr uint64_t kFusedReady = 0x3C6EF372FE94F82Bull;
constexpr uint64_t kFusedInit = 0xA54FF53A5F1D36F1ull;

// State words: [0] readiness, [2] retired workgroups, [16 + 16 g] work counter of up-item range
// g (one 128-byte line each), [160 ..] per-token count of finished up items (uint32,
// kDecodeMaxT of them). The last workgroup to retire zeroes every counter and leaves [0] at
// kFusedReady. A readiness word holding anything else (a buffer this
// kernel never used) is claimed by one workgroup with a compare-and-swap; it zeroes the
// counters and publishes kFusedReady while the others wait for it (it is running, so the wait
// ends). Only a word that held kFusedInit or kFusedReady by chance before the first launch
// would mislead it (one chance in 2^63).
struct FusedState {
  uint64_t *w;
  TW_DEV uint32_t *done() const { return (uint32_t *)(w + 160); }
  TW_DEV uint64_t *ctr(int g) const { return w + 16 + 16 * g; }
};
constexpr int kFusedStateBytes = 160 * 8 + kDecodeMaxT * 4;

TW_DEV void fused_zero_counters(const FusedState &st, int T) {
  __hip_atomic_store(st.w + 2, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int g = 0; g < kFusedGroups; ++g) __hip_atomic_store(st.ctr(g), (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int i = 0; i < T; ++i) __hip_atomic_store(st.done() + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

TW_DEV void fused_prepare(const FusedState &st) {
  if (threadIdx.x == 0) {
    uint64_t r = __hip_atomic_load(st.w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (r != kFusedReady) {
      if (r != kFusedInit &&
          __hip_atomic_compare_exchange_strong(st.w, &r, kFusedInit, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT)) {
        fused_zero_counters(st, kDecodeMaxT);
        wait_vmcnt<0>();
        __hip_atomic_store(st.w, kFusedReady, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        while (__hip_atomic_load(st.w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != kFusedReady)
          __builtin_amdgcn_s_sleep(2);
      }
    }
  }
  __syncthreads();
}

TW_DEV uint64_t ld_coh64(const void *p) {
  return __hip_atomic_load((const uint64_t *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
TW_DEV float ld_cohf(const float *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// One up item by one wave: the active units of tiles [k0, k0 + 4) of token t.
template <typename XT, typename VT, int NP>
TW_DEV void fused_up_item(const TwellIn &h, const XT *__restrict__ x, const XT *__restrict__ wg,
                          const float *__restrict__ bg, const XT *__restrict__ wu, int d, float *__restrict__ dense,
                          int t, int k0) {
  const int lane = lane_id();
  const XT *xrow = x + (size_t)t * d;
  const VT *vals = (const VT *)h.vals;
  for (int k = k0; k < min(k0 + kFusedTilesPerItem, h.n_t); ++k) {
    const size_t sb = ((size_t)t * h.n_t + k) * h.S;
    const int c = h.counts[(size_t)t * h.n_t + k];
    if (c <= h.S) {
      for (int s0 = 0; s0 < c; s0 += kGateEnt) {
        int col[kGateEnt];
        float gv[kGateEnt];
#pragma unroll
        for (int q = 0; q < kGateEnt; ++q) {
          const bool ok = s0 + q < c;
          col[q] = ok ? h.col_idx[sb + s0 + q] : -1;
          gv[q] = ok ? Elem<VT>::load(vals, sb + s0 + q) : 0.f;
        }
        float u[kGateEnt];
        wave_dots<XT, NP>(xrow, wu, d, col, u, h.cols);
        if (lane == 0)
#pragma unroll
          for (int q = 0; q < kGateEnt; ++q)
            if (col[q] >= 0)
              __hip_atomic_store((uint64_t *)(h.row_list + sb + s0 + q),
                                 (uint64_t)(uint32_t)col[q] | ((uint64_t)__float_as_uint(gv[q] * u[q]) << 32),
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    } else {
      float *drow = dense + (size_t)t * h.cols;
      for (int j0 = k * h.W; j0 < (k + 1) * h.W; j0 += kGateEnt) {
        int col[kGateEnt];
#pragma unroll
        for (int q = 0; q < kGateEnt; ++q) col[q] = j0 + q;
        float z[kGateEnt];
        wave_dots<XT, NP>(xrow, wg, d, col, z, h.cols);
        int ucol[kGateEnt];
        float g[kGateEnt];
#pragma unroll
        for (int q = 0; q < kGateEnt; ++q) {
          const float zz = z[q] + bg[col[q]];
          g[q] = zz > 0.f ? Elem<VT>::load_rounded(zz) : 0.f;
          ucol[q] = g[q] != 0.f ? col[q] : -1;
        }
        float u[kGateEnt];
        wave_dots<XT, NP>(xrow, wu, d, ucol, u, h.cols);
        if (lane == 0)
#pragma unroll
          for (int q = 0; q < kGateEnt; ++q)
            __hip_atomic_store(drow + col[q], ucol[q] >= 0 ? g[q] * u[q] : 0.f, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

template <typename XT, typename VT, typename YT, int NP>
__global__ __launch_bounds__(256) void k_gated_fused(TwellIn h, const XT *__restrict__ x, const XT *__restrict__ wg,
                                                     const float *__restrict__ bg, const XT *__restrict__ wu,
                                                     const XT *__restrict__ w2, int d, YT *__restrict__ y,
                                                     float *__restrict__ dense, FusedState st) {
  constexpr int E = Vec16<XT>::N;
  constexpr int CW = 16 * E;                   // columns of one wave in a down item
  __shared__ int claim_s;
  __shared__ int pre_s[257];
  __shared__ uint2 lst_s[256];
  __shared__ int wsum_s[4];
  const int T = h.rows;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ngrp = (h.n_t + kFusedTilesPerItem - 1) / kFusedTilesPerItem;   // up items per token
  const int U = T * ngrp;
  fused_prepare(st);

  // up items: range g = [g U / 8, (g + 1) U / 8) has its own counter; a workgroup starts on
  // range blockIdx % 8 and moves on to the others when it runs dry, so it reaches the down
  // items only once every up item has been claimed
  for (int gi = 0; gi < kFusedGroups; ++gi) {
    const int g = (blockIdx.x + gi) % kFusedGroups;
    const int r0 = (int)((long long)U * g / kFusedGroups), r1 = (int)((long long)U * (g + 1) / kFusedGroups);
    for (;;) {
      if (tid == 0)
        claim_s = r0 + (int)__hip_atomic_fetch_add(st.ctr(g), (uint64_t)kFusedUpBatch, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      const int base = claim_s;
      __syncthreads();
      if (base >= r1) break;
      const int i = base + wave;
      if (i >= min(base + kFusedUpBatch, r1)) continue;
      const int t = i / ngrp, k0 = (i % ngrp) * kFusedTilesPerItem;
      fused_up_item<XT, VT, NP>(h, x, wg, bg, wu, d, dense, t, k0);
      wait_vmcnt<0>();                                          // this item's stores have completed
      if (lane == 0) __hip_atomic_fetch_add(st.done() + t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // down items (t, chunk of 4 * CW columns), statically spread over the workgroups
  const int nch = (d + 4 * CW - 1) / (4 * CW);
  const int g = lane >> 4, gl = lane & 15;
  const __amdgpu_buffer_rsrc_t rs = rows_rsrc(w2, rows_bytes<XT>(h.cols, d));
  for (int it = blockIdx.x; it < T * nch; it += gridDim.x) {
    const int t = it / nch, c = it % nch;
    const int colo = (c * 4 + wave) * CW + gl * E;
    const bool cv = colo < d;
    if (tid == 0)
      while (__hip_atomic_load(st.done() + t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < (uint32_t)ngrp)
        __builtin_amdgcn_s_sleep(1);
    // entries per tile: its stored slots, or all W columns of a recomputed (dense) tile
    int m = 0;
    if (tid < h.n_t) {
      const int cnt = h.counts[(size_t)t * h.n_t + tid];
      m = cnt <= h.S ? cnt : h.W;
    }
    int wt;
    const int ex = wave_excl_scan(m, &wt);
    if (lane == 0) wsum_s[wave] = wt;
    __syncthreads();                                           // also: the up items of t are done
    int wpre = 0, N = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      wpre += w < wave ? wsum_s[w] : 0;
      N += wsum_s[w];
    }
    pre_s[tid] = tid < h.n_t ? wpre + ex : N;                  // pre_s[k]: first entry of tile k
    if (tid == 0) pre_s[256] = N;
    __syncthreads();
    float acc[E];
#pragma unroll
    for (int q = 0; q < E; ++q) acc[q] = 0.f;
    for (int base = 0; base < N; base += 256) {
      const int e = base + tid;
      uint2 p = make_uint2(0, 0);
      if (e < N) {
        int lo = 0;                                            // last tile with pre_s <= e
#pragma unroll
        for (int step = 128; step > 0; step >>= 1)
          if (lo + step < h.n_t && pre_s[lo + step] <= e) lo += step;
        const int s = e - pre_s[lo];
        const size_t sb = ((size_t)t * h.n_t + lo) * h.S;
        if (h.counts[(size_t)t * h.n_t + lo] <= h.S) {
          const uint64_t en = ld_coh64(h.row_list + sb + s);
          p = make_uint2((uint32_t)en, (uint32_t)(en >> 32));
        } else {
          const int j = lo * h.W + s;
          p = make_uint2((uint32_t)j, __float_as_uint(ld_cohf(dense + (size_t)t * h.cols + j)));
        }
      }
      __syncthreads();                                         // the previous round's reads are done
      lst_s[tid] = p;
      __syncthreads();
      const int n = min(256, N - base);
      for (int e0 = 0; e0 < n; e0 += 64) {                     // group g takes entries e0 + g + 4 q
        uint4 raw[16];
        float vv[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int ee = e0 + g + 4 * q;
          vv[q] = 0.f;
          raw[q] = make_uint4(0, 0, 0, 0);
          if (ee < n) {
            const uint2 pp = lst_s[ee];
            vv[q] = __uint_as_float(pp.y);
            if (cv && vv[q] != 0.f) raw[q] = ld16<XT>(rs, pp.x * (uint32_t)d + (uint32_t)colo);
          }
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) fma16<XT, E>(acc, vv[q], raw[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < E; ++q) {
      acc[q] += __shfl_xor(acc[q], 16, 64);
      acc[q] += __shfl_xor(acc[q], 32, 64);
    }
    if (g == 0 && cv) store_out_nt<YT, E>(y, (size_t)t * d + colo, acc);
    __syncthreads();                                           // pre_s, lst_s reused by the next item
  }

  // retire; the last workgroup zeroes the counters for the next launch
  __syncthreads();
  if (tid == 0 &&
      __hip_atomic_fetch_add(st.w + 2, (uint64_t)1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1 == gridDim.x)
    fused_zero_counters(st, T);
}

template <typename XT, typename VT, typename YT>
static hipError_t fused_t(const TwellIn &h, const XT *x, const XT *wg, const float *bg, const XT *wu, const XT *w2,
                          int d, YT *y, float *dense, hipStream_t s) {
  // a workgroup per CU: enough down items to keep them busy at 64 tokens (8 per token at
  // d = 4096), and few enough that the work counter is not a point of contention
  const int nwg = 256;
  FusedState st;
  st.w = (uint64_t *)((char *)dense + dec_tiles(h.cols) * 2 * kDecHalfBytes - 2048);
  static_assert(kFusedStateBytes <= 2048, "fused state");
  hipLaunchKernelGGL((k_gated_fused<XT, VT, YT, 8>), dim3(nwg), dim3(256), 0, s, h, x, wg, bg, wu, w2, d, y, dense, st);
  return hipGetLastError();
}

hipError_t launch_gated_fused(const TwellIn &h, const void *x, const void *wg, const float *bg, const void *wu,
                              const void *w2, int bf16, int d, void *y, int y_bf16, float *dense, hipStream_t s) {
  if (h.rows == 0) return hipSuccess;
  if (bf16) {
    const uint16_t *X = (const uint16_t *)x, *G = (const uint16_t *)wg, *U = (const uint16_t *)wu,
                   *D = (const uint16_t *)w2;
    if (h.val_bf16) {
      if (y_bf16) return fused_t<uint16_t, uint16_t, uint16_t>(h, X, G, bg, U, D, d, (uint16_t *)y, dense, s);
      return fused_t<uint16_t, uint16_t, float>(h, X, G, bg, U, D, d, (float *)y, dense, s);
    }
    if (y_bf16) return fused_t<uint16_t, float, uint16_t>(h, X, G, bg, U, D, d, (uint16_t *)y, dense, s);
    return fused_t<uint16_t, float, float>(h, X, G, bg, U, D, d, (float *)y, dense, s);
  }
  const float *X = (const float *)x, *G = (const float *)wg, *U = (const float *)wu, *D = (const float *)w2;
  if (h.val_bf16) {
    if (y_bf16) return fused_t<float, uint16_t, uint16_t>(h, X, G, bg, U, D, d, (uint16_t *)y, dense, s);
    return fused_t<float, uint16_t, float>(h, X, G, bg, U, D, d, (float *)y, dense, s);
  }
  if (y_bf16) return fused_t<float, float, uint16_t>(h, X, G, bg, U, D, d, (uint16_t *)y, dense, s);
  return fused_t<float, float, float>(h, X, G, bg, U, D, d, (float *)y, dense, s);
}

static int gate_chunks(int d, int bf16) {
  const int cw = bf16 ? 128 : 64;
  return (d + cw - 1) / cw;
}

size_t gate_up_workspace_bytes(int T, int d, int n_t, int S, int bf16) {
  if (T < kGateChunkMinT) return 0;
  return (size_t)gate_chunks(d, bf16) * (size_t)T * (size_t)n_t * (size_t)S * 4;
}

hipError_t launch_gate_up(const TwellIn &h, const void *x, const void *wu, int bf16, int d, float *ws,
                          hipStream_t s) {
  if (h.rows == 0) return hipSuccess;
  if (h.rows >= kGateChunkMinT) {
    if (!ws) return hipErrorInvalidValue;
    const int nchunk = gate_chunks(d, bf16);
    const int ntb = (h.rows + 15) / 16;
    const dim3 grid((unsigned)(8 * (size_t)ntb * ((nchunk + 7) / 8))), rows4((h.rows + 3) / 4);
    const int rstep = min(h.cap, kGateBackupRows);
    const size_t nb = (size_t)rstep * ((h.cols + 63) / 64);
    const dim3 gridb((unsigned)((nb + 3) / 4));
    // the partial sums, then their sum with the backup rows' products in the same launch
    const int nA = (int)rows4.x;
    const dim3 gall((unsigned)(nA + gridb.x));
    if (bf16) {
      const uint16_t *xx = (const uint16_t *)x, *ww = (const uint16_t *)wu;
      hipLaunchKernelGGL((k_gate_part<uint16_t>), grid, dim3(256), 0, s, h, d, nchunk, ntb, xx, ww, ws);
      if (!nb) hipLaunchKernelGGL(k_gate_sum, rows4, dim3(256), 0, s, h, nchunk, ws);
      else if (d <= 2048) {
        if (h.val_bf16)
          hipLaunchKernelGGL((k_gate_sum_all<uint16_t, 4, kGateDotEnt, uint16_t>), gall, dim3(256), 0, s, h, nchunk, ws,
                             xx, ww, d, nA, rstep);
        else
          hipLaunchKernelGGL((k_gate_sum_all<uint16_t, 4, kGateDotEnt, float>), gall, dim3(256), 0, s, h, nchunk, ws, xx,
                             ww, d, nA, rstep);
      } else {
        if (h.val_bf16)
          hipLaunchKernelGGL((k_gate_sum_all<uint16_t, 8, kGateDotEnt, uint16_t>), gall, dim3(256), 0, s, h, nchunk, ws,
                             xx, ww, d, nA, rstep);
        else
          hipLaunchKernelGGL((k_gate_sum_all<uint16_t, 8, kGateDotEnt, float>), gall, dim3(256), 0, s, h, nchunk, ws, xx,
                             ww, d, nA, rstep);
      }
    } else {
      const float *xx = (const float *)x, *ww = (const float *)wu;
      hipLaunchKernelGGL((k_gate_part<float>), grid, dim3(256), 0, s, h, d, nchunk, ntb, xx, ww, ws);
      if (!nb) hipLaunchKernelGGL(k_gate_sum, rows4, dim3(256), 0, s, h, nchunk, ws);
      else if (d <= 1024) {
        if (h.val_bf16)
          hipLaunchKernelGGL((k_gate_sum_all<float, 4, kGateDotEnt, uint16_t>), gall, dim3(256), 0, s, h, nchunk, ws, xx,
                             ww, d, nA, rstep);
        else
          hipLaunchKernelGGL((k_gate_sum_all<float, 4, kGateDotEnt, float>), gall, dim3(256), 0, s, h, nchunk, ws, xx, ww,
                             d, nA, rstep);
      } else {
        if (h.val_bf16)
          hipLaunchKernelGGL((k_gate_sum_all<float, 8, kGateDotEnt, uint16_t>), gall, dim3(256), 0, s, h, nchunk, ws, xx,
                             ww, d, nA, rstep);
        else
          hipLaunchKernelGGL((k_gate_sum_all<float, 8, kGateDotEnt, float>), gall, dim3(256), 0, s, h, nchunk, ws, xx, ww,
                             d, nA, rstep);
      }
    }
    return hipGetLastError();
  }
  // enough workgroups to keep every CU busy at few tokens, without more entry groups per
  // token than a full list has
  const int groups = (h.n_t * h.S + 4 * kGateDotEnt - 1) / (4 * kGateDotEnt);
  const int P = max(1, min(groups, (2048 + h.rows - 1) / h.rows));
  const dim3 grid((unsigned)((size_t)h.rows * P));
  const int rstep = min(h.cap, kGateBackupRows);
  const size_t nb = (size_t)rstep * ((h.cols + 63) / 64);
  const dim3 gridb((unsigned)((nb + 3) / 4));
  const int nA = (int)grid.x;
  const dim3 gall((unsigned)(nA + gridb.x));
  if (bf16) {
    const uint16_t *xx = (const uint16_t *)x, *ww = (const uint16_t *)wu;
    if (!nb) {
      if (d <= 2048) hipLaunchKernelGGL((k_gate_dot<uint16_t, 4, kGateDotEnt>), grid, dim3(256), 0, s, h, xx, ww, d, P);
      else hipLaunchKernelGGL((k_gate_dot<uint16_t, 8, kGateDotEnt>), grid, dim3(256), 0, s, h, xx, ww, d, P);
    } else if (d <= 2048) {
      if (h.val_bf16)
        hipLaunchKernelGGL((k_gate_dot_all<uint16_t, 4, kGateDotEnt, uint16_t>), gall, dim3(256), 0, s, h, xx, ww, d, P,
                           nA, rstep);
      else
        hipLaunchKernelGGL((k_gate_dot_all<uint16_t, 4, kGateDotEnt, float>), gall, dim3(256), 0, s, h, xx, ww, d, P, nA,
                           rstep);
    } else {
      if (h.val_bf16)
        hipLaunchKernelGGL((k_gate_dot_all<uint16_t, 8, kGateDotEnt, uint16_t>), gall, dim3(256), 0, s, h, xx, ww, d, P,
                           nA, rstep);
      else
        hipLaunchKernelGGL((k_gate_dot_all<uint16_t, 8, kGateDotEnt, float>), gall, dim3(256), 0, s, h, xx, ww, d, P, nA,
                           rstep);
    }
  } else {
    const float *xx = (const float *)x, *ww = (const float *)wu;
    if (!nb) {
      if (d <= 1024) hipLaunchKernelGGL((k_gate_dot<float, 4, kGateDotEnt>), grid, dim3(256), 0, s, h, xx, ww, d, P);
      else hipLaunchKernelGGL((k_gate_dot<float, 8, kGateDotEnt>), grid, dim3(256), 0, s, h, xx, ww, d, P);
    } else if (d <= 1024) {
      if (h.val_bf16)
        hipLaunchKernelGGL((k_gate_dot_all<float, 4, kGateDotEnt, uint16_t>), gall, dim3(256), 0, s, h, xx, ww, d, P, nA,
                           rstep);
      else
        hipLaunchKernelGGL((k_gate_dot_all<float, 4, kGateDotEnt, float>), gall, dim3(256), 0, s, h, xx, ww, d, P, nA,
                           rstep);
    } else {
      if (h.val_bf16)
        hipLaunchKernelGGL((k_gate_dot_all<float, 8, kGateDotEnt, uint16_t>), gall, dim3(256), 0, s, h, xx, ww, d, P, nA,
                           rstep);
      else
        hipLaunchKernelGGL((k_gate_dot_all<float, 8, kGateDotEnt, float>), gall, dim3(256), 0, s, h, xx, ww, d, P, nA,
                           rstep);
    }
  }
  return hipGetLastError();
}

}  // namespace tw
