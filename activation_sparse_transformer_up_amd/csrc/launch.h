// Internal launchers shared between the kernel files and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tw {

// The up GEMM of at most kDecodeMaxT tokens splits each 128-column tile over two workgroups
// that meet in a workspace: two fp32 half sums of 64 x 128 per tile, then one 64-bit ticket
// per tile. It sits in the row-list scratch, after the lists. A ticket may hold any value
// before a launch (see dec_meet in gemm.hip); every launch leaves it zero.
constexpr int kDecodeMaxT = 64;
constexpr size_t kDecHalfBytes = 64 * 128 * 4;
inline size_t dec_tiles(int cols) { return (size_t)(cols + 127) / 128; }
inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }
inline size_t dec_ws_bytes(int cols) { return dec_tiles(cols) * 2 * kDecHalfBytes + align256(dec_tiles(cols) * 8); }

// Output side of a TwELL-producing kernel (see twell_matrix_t in include/twell.h).
struct TwellOut {
  int32_t *counts;
  int32_t *col_idx;
  void *vals;
  uint32_t *ovf_bits;
  float *dec_part;        // decode workspace (rows <= kDecodeMaxT): [tiles][2][64 x 128] fp32
  uint64_t *dec_ticket;   // [tiles]
  size_t dec_bytes;       // bytes of dec_part
  int n_t, S, words, val_bf16;
};

// The rest of a TwELL matrix, which the one- and two-token up projection completes when asked
// (complete): row lists (when row_nnz and row_list are given), overflow scan and dense backup
// rows [cap][cols].
struct TwellFinish {
  int32_t *row_nnz;
  uint2 *row_list;
  int32_t *ovf_n, *ovf_rows, *ovf_slot;
  void *ovf_dense;
  int cap;
  bool complete;
};

// Read side of a TwELL consumer.
struct TwellIn {
  const int32_t *counts;
  const int32_t *col_idx;
  const void *vals;
  const int32_t *ovf_slot;
  const void *ovf_dense;
  const int32_t *ovf_n;   // overflow rows found (may exceed cap)
  const int32_t *ovf_rows;
  int32_t *row_nnz;       // scratch: compact list length per row (-1: use the backup row)
  uint2 *row_list;        // scratch: [rows][n_t * S] (column, fp32 value bits)
  int rows, cols, n_t, S, W, val_bf16, cap;
};

// Length of row t's list as the gathers use it: row_nnz[t] clamped to [0, n_t S]. The lists
// are scratch that only the finish step writes; a matrix whose lists are stale or were never
// built then gives wrong sums, but no access outside its row of row_list.
__device__ __forceinline__ int list_len(const TwellIn &h, int nnz) { return min(max(nnz, 0), h.n_t * h.S); }

// gemm.hip
hipError_t launch_up_twell(int bf16, const void *x, const void *w1t, const float *b1, int M, int N, int K,
                           const TwellOut &o, const TwellFinish &f, int W, hipStream_t s);
// true if launch_up_twell of M tokens with f also completes the matrix (lists, overflow scan,
// backup rows): the finish step has nothing left to do
bool up_twell_completes(int bf16, int M, int K, const TwellFinish &f);
// 1 to 16 bf16 tokens: true if the up projection runs as a W1 stream that leaves the half sums
// in o.dec_part (launch_up_stream), which launch_dec_fused_down then turns into the TwELL, the
// overflow scan, the backup rows and y
bool up_stream_ok(int bf16, int M, int K);
hipError_t launch_up_stream(const void *x, const void *w1t, int M, int N, int K, const TwellOut &o, hipStream_t s);

// decode.hip: after launch_up_stream, the TwELL of the M <= 16 rows, the overflow scan, the
// backup rows and y = h W2 (bf16 W2 [N][d]) in one launch
hipError_t launch_dec_fused_down(const float *b1, int M, int N, const TwellOut &o, const TwellFinish &f, const void *w2,
                                 int d, void *y, int y_bf16, int W, hipStream_t s);
hipError_t launch_up_dense(int bf16, const void *x, const void *w1t, const float *b1, int M, int N, int K,
                           int x_rows, const int32_t *arow, const int32_t *n_rows_dev, void *out, int out_bf16, int relu,
                           hipStream_t s);
// h = ReLU(x W1 + b1) pruned to n:m in the GEMM epilogue (vals in the operand type)
hipError_t launch_up_nm(int bf16, const void *x, const void *w1t, const float *b1, int M, int N, int K, int n,
                        int m, void *vals, uint8_t *idx, hipStream_t s);

// pack.hip
hipError_t launch_pack(const void *h, int h_bf16, int R, int C, const TwellOut &o, int W, hipStream_t s);
hipError_t launch_ovf_scan(const uint32_t *bits, int n_t, int words, int R, int cap, int32_t *ovf_n,
                           int32_t *ovf_rows, int32_t *ovf_slot, hipStream_t s);
hipError_t launch_ovf_copy(const void *h, int h_bf16, int R, int C, const int32_t *ovf_n, const int32_t *ovf_rows,
                           int cap, void *dense, int dense_bf16, hipStream_t s);
hipError_t launch_set_int(int32_t *p, int v, hipStream_t s);
hipError_t launch_zero_i32(int32_t *p, int n, hipStream_t s);

#define TW_TRY_HIP(expr)                 \
  do {                                   \
    hipError_t e_ = (expr);              \
    if (e_ != hipSuccess) return e_;     \
  } while (0)

// rell.hip: the compact row-ELL (one tile per row) from a TwELL, and the row-nonzero histogram
hipError_t launch_to_row_ell(const TwellIn &src, const TwellOut &dst, int N, int cap, int32_t *ovf_n,
                             int32_t *ovf_rows, int32_t *ovf_slot, void *dense, hipStream_t s);
hipError_t launch_row_nnz_hist(const int32_t *counts, int rows, int n_t, int nbins, int32_t *hist, hipStream_t s);
// hist[0 .. W] <- histogram of the per-row maximum tile count
hipError_t launch_rowmax_hist(const int32_t *counts, int rows, int n_t, int W, int32_t *hist, hipStream_t s);

// bwd.hip
struct BwdArgs {
  TwellIn h;
  const void *x, *w1t, *w2, *dy;
  float l1;
  float *dx, *dw1t, *dw2, *db1;
  void *ws;
  size_t nz;              // entries the workspace holds (bwd_fit_entries)
  int d, bf16, cap;
};
size_t bwd_entry_capacity(int T, int f, int n_t, int S, int cap);
size_t bwd_workspace_bytes(int T, int d, int f, size_t NZ, int bf16);
size_t bwd_fit_entries(int T, int d, int f, size_t bytes, size_t NZmax, int bf16);
hipError_t launch_bwd(const BwdArgs &a, hipStream_t s);

// gated.hip
// From kGateChunkMinT tokens on the up products are chunked per XCD and need a workspace of
// gate_up_workspace_bytes (0 below that size).
constexpr int kGateChunkMinT = 512;
size_t gate_up_workspace_bytes(int T, int d, int n_t, int S, int bf16);
hipError_t launch_gate_up(const TwellIn &h, const void *x, const void *wu, int bf16, int d, float *ws,
                          hipStream_t s);

// One cooperative launch after the gate GEMM (rows <= kDecodeMaxT): row lists, up products,
// down products; dense: [rows][cols] fp32 scratch (the decode workspace of row_list).
hipError_t launch_gated_fused(const TwellIn &h, const void *x, const void *wg, const float *bg, const void *wu,
                              const void *w2, int bf16, int d, void *y, int y_bf16, float *dense, hipStream_t s);

// nm.hip
hipError_t launch_nm_prune(const void *h, int bf16, int T, int f, int n, int m, void *vals, uint8_t *idx,
                           hipStream_t s);
hipError_t launch_nm_down(const void *vals, const uint8_t *idx, int T, int f, int n, int m, const void *w2, int d,
                          void *y, int y_bf16, hipStream_t s);

// down.hip
hipError_t launch_twell_down(const TwellIn &h, const void *w2, int w_bf16, int d, void *y, int y_bf16,
                             bool build_lists, hipStream_t s);
// overflow scan + row lists in one launch (the finish step of the fused forward)
hipError_t launch_lists_scan(const TwellIn &h, const uint32_t *bits, int words, int32_t *ovf_n, int32_t *ovf_rows,
                             int32_t *ovf_slot, hipStream_t s);
// gemm.hip: the same finish plus the backup recompute in one launch, for at most 64 tokens on
// the decode tile GEMM; hipErrorNotSupported elsewhere
hipError_t launch_finish_dec(int bf16, const TwellIn &h, const uint32_t *bits, int words, int32_t *ovf_n,
                             int32_t *ovf_rows, int32_t *ovf_slot, const void *x, const void *w1t, const float *b1,
                             int K, void *dense, hipStream_t s);

}  // namespace tw
