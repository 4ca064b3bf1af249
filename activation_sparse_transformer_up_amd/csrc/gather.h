// Shared core of the sparse row gathers: the forward down projection (rows of W2 selected
// by a token's active units), and the backward dx (rows of w1t) and dW (rows of dy and x
// selected by a unit's tokens).
//
//   out[r][c0 .. c0 + CW) = sum over the entries (i, v) of list r of v * M[i][c0 .. c0 + CW)
//
// Lists hold packed (row index, fp32 value bits) pairs. A 16-lane group owns one list and
// one column chunk: lane l covers 16 bytes (8 bf16 or 4 fp32 elements) of every selected
// row, so a chunk is 256 bytes of bf16 or fp32 rows and one vector load instruction of the
// wave fetches four rows of four lists. Per round a lane loads one pair of its group's list
// (coalesced), the sixteen pairs are broadcast inside the group with a DPP row broadcast,
// and all sixteen row loads are issued before the FMAs; the next round's pairs are loaded
// meanwhile. Accumulation is fp32 in list order.
#pragma once
#include <type_traits>

#include "common.h"

namespace tw {

// Lane J of this lane's 16-lane row (DPP row broadcast). Every lane's source exists, so no
// "old" value is needed (bound_ctrl), and the compiler emits no move before the broadcast.
template <int J> TW_DEV uint32_t row_bcast(uint32_t v) {
  static_assert(J >= 0 && J < 16, "row lane");
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x150 + J, 0xF, 0xF, true);
}

// acc[0..E) += v * the E elements in the 16 bytes raw (bf16 widened exactly to fp32).
template <typename WT, int E>
TW_DEV void fma16(float (&acc)[E], float v, uint4 raw) {
  float r[E];
  if constexpr (sizeof(WT) == 2) {
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      r[2 * q] = __uint_as_float(w[q] << 16);
      r[2 * q + 1] = __uint_as_float(w[q] & 0xFFFF0000u);
    }
  } else {
    r[0] = __uint_as_float(raw.x); r[1] = __uint_as_float(raw.y);
    r[2] = __uint_as_float(raw.z); r[3] = __uint_as_float(raw.w);
  }
#pragma unroll
  for (int q = 0; q < E; ++q) acc[q] = fmaf(v, r[q], acc[q]);
}

// The group's list p[0 .. n) against rows of M (row length d); this lane's columns start
// at col (cv: inside the row). nw = the largest n of the wave's four groups (the loop bound
// must be wave-uniform). Returns this lane's share of the sum of the list's values (lane l
// adds entries l, l + 16, ...).
template <typename WT>
TW_DEV float gather_list16(const uint2 *__restrict__ p, int n, int nw, const WT *__restrict__ M, int d, int col,
                           bool cv, float (&acc)[Vec16<WT>::N], uint32_t mbytes = 0x7FFFFFFFu) {
  constexpr int E = Vec16<WT>::N;
  constexpr uint32_t OOB = 0x80000000u;                      // beyond the range: reads zeros
  const int gl = lane_id() & 15;
  const __amdgpu_buffer_rsrc_t rs = rows_rsrc(M, mbytes);    // row pieces by buffer loads
  // byte offset of row i's piece: i * (row bytes) + this lane's column bytes, one 24-bit
  // multiply-add (row indices and row bytes are below 2^24, the operand below 2 GiB)
  const uint32_t rowb = (uint32_t)d * (uint32_t)sizeof(WT), colb = (uint32_t)col * (uint32_t)sizeof(WT);
  float vs = 0.f;
  uint2 pn = gl < n ? p[gl] : make_uint2(0, 0);
  for (int base = 0; base < nw; base += 16) {
    const uint2 q = pn;
    if (base + 16 < nw) pn = base + 16 + gl < n ? p[base + 16 + gl] : make_uint2(0, 0);
    vs += __uint_as_float(q.y);                 // zero for entries past n
    // Entries up to the wave's longest list in this round (rem, wave-uniform) are issued
    // without a per-lane branch: an entry past its own list (its pair, and so its value, is
    // zero) or a column past the row reads zeros through the range check. Entries past rem
    // are skipped by a scalar branch, loads and FMAs alike.
    const int rem = nw - base;
    auto round = [&](auto full_tag) {
      constexpr bool FULL = decltype(full_tag)::value;
      uint4 raw[16];
      float vv[16];
      static_for<16>([&](auto J) {
        constexpr int j = decltype(J)::value;
        if (!FULL && j >= rem) return;
        const uint32_t ij = row_bcast<j>(q.x), vj = row_bcast<j>(q.y);
        vv[j] = __uint_as_float(vj);
        const uint32_t off = (base + j < n && cv) ? __umul24(ij, rowb) + colb : OOB;
        const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0);
        raw[j] = make_uint4(v.x, v.y, v.z, v.w);
      });
      static_for<16>([&](auto J) {
        constexpr int j = decltype(J)::value;
        if (!FULL && j >= rem) return;
        fma16<WT, E>(acc, vv[j], raw[j]);
      });
    };
    if (rem >= 16) round(std::true_type());
    else round(std::false_type());
  }
  return vs;
}

// v[0..16) of the 16 lanes of a group summed across the group, one sum per lane: at step m
// (8, 4, 2, 1) a lane keeps the half of its remaining values selected by bit m of its lane
// index and adds the partner's (lane ^ m) copy of that half. Lane l ends with entry l.
TW_DEV float group16_transpose_sum(float (&v)[16], int gl) {
  static_for<4>([&](auto S) {
    constexpr int m = 8 >> decltype(S)::value, half = m;   // values left: 2 * m
    const bool hi = gl & m;
    static_for<half>([&](auto K) {
      constexpr int k = decltype(K)::value;
      const float keep = hi ? v[k + half] : v[k];
      const float send = hi ? v[k] : v[k + half];
      v[k] = keep + __shfl_xor(send, m, 64);
    });
  });
  return v[0];
}

// Sum over the 16 lanes of a group.
TW_DEV float group16_sum(float v) {
  v += __shfl_xor(v, 1, 64);
  v += __shfl_xor(v, 2, 64);
  v += __shfl_xor(v, 4, 64);
  v += __shfl_xor(v, 8, 64);
  return v;
}

}  // namespace tw
