// Device-side helpers shared by the gfx950 kernels of the TwELL FFN library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

#define TW_DEV __device__ __forceinline__

// f(std::integral_constant<int, 0>()), ..., f(std::integral_constant<int, N - 1>()): the
// index is a constant expression inside f, whatever the inliner and unroller do (register
// arrays indexed by it stay in registers).
template <typename F, int... J>
TW_DEV void static_for_impl(F &&f, std::integer_sequence<int, J...>) {
  (f(std::integral_constant<int, J>()), ...);
}
template <int N, typename F> TW_DEV void static_for(F &&f) {
  static_for_impl(f, std::make_integer_sequence<int, N>());
}

// bf16 is carried as its raw 16-bit pattern in memory.
TW_DEV float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16, round to nearest even (finite inputs).
TW_DEV uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

TW_DEV uint32_t lane_id() { return __lane_id(); }

// 64-bit wave ballot.
TW_DEV uint64_t ballot64(bool p) { return __ballot(p); }

// Number of set bits of `m` strictly below this lane (mbcnt).
TW_DEV uint32_t mbcnt64(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Exclusive prefix sum of v over the 64 lanes; *total receives the sum.
TW_DEV int wave_excl_scan(int v, int *total) {
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if ((int)lane_id() >= o) x += y;
  }
  *total = __shfl(x, 63, 64);
  return x - v;
}

TW_DEV int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

TW_DEV float wave_sumf(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Element access for the two storage types (uint16_t = bf16 bits, float = fp32).
template <typename T> struct Elem;
template <> struct Elem<float> {
  static TW_DEV float load(const float *p, size_t i) { return p[i]; }
  static TW_DEV void store(float *p, size_t i, float v) { p[i] = v; }
  static TW_DEV float load_rounded(float v) { return v; }     // v as this type stores it
};
template <> struct Elem<uint16_t> {
  static TW_DEV float load(const uint16_t *p, size_t i) { return bf16_to_f32(p[i]); }
  static TW_DEV void store(uint16_t *p, size_t i, float v) { p[i] = (uint16_t)f32_to_bf16(v); }
  static TW_DEV float load_rounded(float v) { return bf16_to_f32(f32_to_bf16(v)); }
};

// 16-byte vector of row elements, widened to fp32: 8 bf16 or 4 fp32.
template <typename T> struct Vec16;
template <> struct Vec16<uint16_t> {
  static constexpr int N = 8;
  static TW_DEV void load(const uint16_t *p, float (&o)[8]) {
    uint4 u = *(const uint4 *)p;
    o[0] = __uint_as_float(u.x << 16); o[1] = __uint_as_float(u.x & 0xFFFF0000u);
    o[2] = __uint_as_float(u.y << 16); o[3] = __uint_as_float(u.y & 0xFFFF0000u);
    o[4] = __uint_as_float(u.z << 16); o[5] = __uint_as_float(u.z & 0xFFFF0000u);
    o[6] = __uint_as_float(u.w << 16); o[7] = __uint_as_float(u.w & 0xFFFF0000u);
  }
};
template <> struct Vec16<float> {
  static constexpr int N = 4;
  static TW_DEV void load(const float *p, float (&o)[4]) {
    float4 u = *(const float4 *)p;
    o[0] = u.x; o[1] = u.y; o[2] = u.z; o[3] = u.w;
  }
};

// One lane's E consecutive fp32 results written as fp32 or bf16 (round to nearest even) with
// nontemporal 16-byte (or 8-byte) stores: outputs that the writing kernel never reads again
// should not displace the operand lines it keeps in L2. o must be a multiple of E.
template <typename YT, int E> TW_DEV void store_out_nt(YT *y, size_t o, const float (&a)[E]) {
  static_assert(E == 4 || E == 8, "vector width");
  if constexpr (std::is_same<YT, float>::value) {
#pragma unroll
    for (int q = 0; q < E; q += 4)
      __builtin_nontemporal_store(f32x4_t{a[q], a[q + 1], a[q + 2], a[q + 3]}, (f32x4_t *)(y + o + q));
  } else {
    uint32_t w[E / 2];
#pragma unroll
    for (int i = 0; i < E / 2; ++i) w[i] = f32_to_bf16(a[2 * i]) | (f32_to_bf16(a[2 * i + 1]) << 16);
    if constexpr (E == 8) {
      __builtin_nontemporal_store(u32x4_t{w[0], w[1], w[2], w[3]}, (u32x4_t *)(y + o));
    } else {
      typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
      __builtin_nontemporal_store(u32x2_t{w[0], w[1]}, (u32x2_t *)(y + o));
    }
  }
}

// Rows of a matrix read through a buffer resource: a scalar descriptor plus a 32-bit byte
// offset per lane (every operand is below 2 GiB). Offsets at or above `bytes` (default 2^31 - 1;
// e.g. from a negative index, or a row index read from a list that was never written) read as
// zeros.
TW_DEV __amdgpu_buffer_rsrc_t rows_rsrc(const void *p, uint32_t bytes = 0x7FFFFFFFu) {
  return __builtin_amdgcn_make_buffer_rsrc((void *)p, (short)0, (int)bytes, 0x00020000);
}
// Byte extent of a [rows][d] matrix of T for rows_rsrc (capped at 2^31 - 1).
template <typename T> TW_DEV uint32_t rows_bytes(int rows, int d) {
  const size_t b = (size_t)rows * (size_t)d * sizeof(T);
  return b < 0x7FFFFFFFu ? (uint32_t)b : 0x7FFFFFFFu;
}
template <typename WT> TW_DEV uint4 ld16(__amdgpu_buffer_rsrc_t rs, uint32_t elem) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(elem * (uint32_t)sizeof(WT)), 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
