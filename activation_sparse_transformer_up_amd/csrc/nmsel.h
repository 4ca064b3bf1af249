// N:M selection of one block of M activations, shared by the standalone pruning kernel and
// the up GEMM's N:M epilogue.
//
// "Motivating Next-Gen Accelerators with Flexible (N:M) Activation Sparsity ...", section
// "2. Metodologia" (criterion ACT): keep the N entries of largest magnitude in every block
// of M consecutive activations. Entry i is kept iff its rank
//   rank_i = #{k : |h_k| > |h_i|} + #{k < i : |h_k| == |h_i|}
// is below N (ties to the lower index). Magnitudes are compared as sign-cleared bit
// patterns, which is exact and monotone for finite values (+0 and -0 are equal).
#pragma once
#include "common.h"

namespace tw {

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

// keep[i] for the M raw bit patterns of one block (bf16 in the low 16 bits, or fp32).
// bf16: the ranks are those of the unique keys (magnitude << log2 M) | (M - 1 - i); every
// supported pattern keeps N = M / 2, and the N largest keys are found by sorting each half
// of the block (descending) and taking c_i = max(a_i, b_{N-1-i}), whose minimum is the
// N-th largest key. fp32 (31-bit magnitudes) counts the ranks directly.
template <int BYTES, int N, int M> TW_DEV void nm_keep(const uint32_t (&bits)[M], bool (&keep)[M]) {
  if constexpr (BYTES == 2) {
    static_assert(2 * N == M, "bf16 selection keeps half of each block");
    constexpr int LOGM = 31 - __builtin_clz(M);
    uint32_t key[M], a[N], b[N];
    static_for<M>([&](auto I) {
      constexpr int i = decltype(I)::value;
      key[i] = ((bits[i] & 0x7FFFu) << LOGM) | (uint32_t)(M - 1 - i);
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
      const uint32_t mi = bits[i] & 0x7FFFFFFFu;
      int rank = 0;
#pragma unroll
      for (int k = 0; k < M; ++k) {
        if (k == i) continue;
        const uint32_t mk = bits[k] & 0x7FFFFFFFu;
        rank += (k < i) ? (mk >= mi) : (mk > mi);
      }
      keep[i] = rank < N;
    }
  }
}

}  // namespace tw
