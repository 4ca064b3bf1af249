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

// Sorting network for L keys (L a power of two), descending: Batcher's odd-even merge sort
// (K. E. Batcher, "Sorting networks and their applications", 1968). It takes 5, 19 and 63
// compare-exchanges for 4, 8 and 16 keys, against 6, 24 and 80 for the bitonic network.
// Every index is a compile-time constant. Stage p merges sorted runs of length p into runs
// of 2p; within it, pass k compares i + j with i + j + k where both lie in one 2p-run.
template <int L> TW_DEV void oddeven_desc(uint32_t (&a)[L]) {
  static_for<31 - __builtin_clz(L)>([&](auto PS) {              // p = 1, 2, ..., L/2
    constexpr int p = 1 << decltype(PS)::value;
    static_for<decltype(PS)::value + 1>([&](auto KS) {           // k = p, p/2, ..., 1
      constexpr int k = p >> decltype(KS)::value;
      static_for<L>([&](auto JS) {                                // j = k mod p + 2k t
        constexpr int j = decltype(JS)::value;
        if constexpr (j >= k % p && (j - k % p) % (2 * k) == 0 && j + k < L) {
          static_for<k>([&](auto IS) {
            constexpr int lo = j + decltype(IS)::value, hi = lo + k;
            if constexpr (hi < L && lo / (2 * p) == hi / (2 * p)) {
              const uint32_t x = a[lo], y = a[hi];
              a[lo] = x > y ? x : y;
              a[hi] = x > y ? y : x;
            }
          });
        }
      });
    });
  });
}

// fp32: keep[i] for the M raw bit patterns of one block, by counting each entry's rank
// directly on the 31-bit magnitudes (M^2 comparisons; fp32 blocks are not the bandwidth-
// critical case).
template <int N, int M> TW_DEV void nm_keep32(const uint32_t (&bits)[M], bool (&keep)[M]) {
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

// bf16: the kept set of one block as a mask, bit 31 - i set iff entry i is kept (so
// count-leading-zeros walks the kept entries in ascending order). The keys are unique,
// (magnitude << log2 M) | (M - 1 - i), so their order is the rank order with ties to the
// lower index; every supported pattern keeps N = M / 2, and with both halves sorted c_i = max(a_i, b_{N-1-i}) (i < N) are exactly the N
// largest keys, and each names its entry in its low log2 M bits.
template <int N, int M> TW_DEV uint32_t nm_kept_mask(const uint32_t (&bits)[M]) {
  static_assert(2 * N == M, "bf16 selection keeps half of each block");
  constexpr int LOGM = 31 - __builtin_clz(M);
  uint32_t a[N], b[N];
  static_for<M>([&](auto I) {
    constexpr int i = decltype(I)::value;
    const uint32_t key = ((bits[i] & 0x7FFFu) << LOGM) | (uint32_t)(M - 1 - i);
    if constexpr (i < N) a[i] = key;
    else b[i - N] = key;
  });
  oddeven_desc<N>(a);
  oddeven_desc<N>(b);
  uint32_t mask = 0;
  static_for<N>([&](auto I) {
    constexpr int i = decltype(I)::value;
    const uint32_t c = a[i] > b[N - 1 - i] ? a[i] : b[N - 1 - i];
    mask |= 1u << (c & (uint32_t)(M - 1));                       // bit M - 1 - entry
  });
  return mask << (32 - M);
}

}  // namespace tw
