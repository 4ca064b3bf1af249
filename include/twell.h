/*
 * twell.h — C ABI of the activation-sparse transformer feed-forward library (AMD gfx950).
 *
 * The layer is y = ReLU(x . W1 + b1) . W2 in which only the nonzero hidden activations
 * are stored and multiplied ("Sparser, Faster, Lighter Transformer Language Models",
 * section "1. O Problema", and section "2. Metodologia": "Formato de Dados TwELL",
 * "Kernels de Inferência", "Formato Híbrido para Treinamento", "Técnicas de Treinamento").
 * N:M activation pruning follows "Motivating Next-Gen Accelerators with Flexible (N:M)
 * Activation Sparsity ...", section "2. Metodologia" (magnitude criterion ACT).
 *
 * Conventions for every entry point:
 *   - Array pointers are DEVICE pointers (memory the caller allocated on the current HIP
 *     device), row-major, contiguous, 16-byte aligned. The caller owns every buffer; the
 *     library never allocates, frees or keeps a pointer after the call returns.
 *   - `stream` is a hipStream_t (NULL = the null stream). Work is enqueued on it and the
 *     call returns without synchronising (except twell_sync_status).
 *   - Arguments are validated before anything is enqueued; on an error nothing is written
 *     and a negative twell_status_t is returned. A failed launch returns TWELL_ERR_HIP.
 *   - Outputs must not alias inputs. Gradients are overwritten, not accumulated.
 *   - The library holds no mutable global state and is safe to call concurrently on
 *     different streams with different buffers.
 *   - Floating-point inputs must be finite; NaN/Inf are outside the contract.
 *
 * Layouts (T tokens, d = d_model, f = d_ff):
 *   x   [T][d]     token activations
 *   w1t [f][d]     row j = input weights of hidden unit j   (nn.Linear(d, f).weight)
 *   b1  [f]        fp32 bias
 *   w2  [f][d]     row j = output weights of hidden unit j  (nn.Linear(f, d).weight^T)
 *   y   [T][d]
 */
#ifndef TWELL_H
#define TWELL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TWELL_ABI_VERSION 4

typedef enum { TWELL_F32 = 0, TWELL_BF16 = 1 } twell_dtype_t;

typedef enum {
  TWELL_OK = 0,
  TWELL_ERR_ARG = -1,          /* null pointer, bad enum value, bad struct field          */
  TWELL_ERR_SHAPE = -2,        /* non-positive size, f % tile_w, slots out of range, ...   */
  TWELL_ERR_ALIGN = -3,        /* pointer not 16-byte aligned, or d % 8 != 0               */
  TWELL_ERR_WORKSPACE = -4,    /* workspace too small                                      */
  TWELL_ERR_OVF_CAPACITY = -5, /* (twell_sync_status only) more overflow rows than ovf_cap */
  TWELL_ERR_HIP = -6,          /* a HIP call or kernel launch failed                       */
  TWELL_ERR_UNSUPPORTED = -7   /* valid request this version does not implement           */
} twell_status_t;

/*
 * TwELL (Tile-wise ELLPACK) matrix with its row-level dense backup.
 *
 * "Formato de Dados TwELL": the columns of an R x C matrix are cut into tiles of tile_w
 * columns; for every (row, tile) the nonzero values and their column indices are stored
 * aligned inside that tile's slot block. "Formato Híbrido para Treinamento": rows with
 * too many nonzeros are routed to a dense backup matrix.
 *
 *   counts  [R][C/tile_w]           true nonzero count of the (row, tile); may exceed slots
 *   col_idx [R][C/tile_w][slots]    global column of the s-th nonzero, ascending; pad = -1
 *   vals    [R][C/tile_w][slots]    its value (val_dtype); pad = +0.0
 *   ovf_n   [1]                     true number of overflow rows (may exceed ovf_cap)
 *   ovf_rows[ovf_cap]               overflow rows in ascending order (first ovf_cap of them)
 *   ovf_slot[R]                     index into ovf_dense, or -1 (no overflow / no room)
 *   ovf_dense[ovf_cap][C]           the full row of each listed overflow row (val_dtype)
 *   ovf_bits[C/tile_w][ceil(R/32)]  library scratch (uint32 words), written and read
 *                                   inside one call; contents on return are unspecified
 *   row_nnz[R]                      library scratch: entries of each row's compact list
 *   row_list[R][C/tile_w * slots]   library scratch: compact (int32 column, fp32 value)
 *                                   pairs of each row, written by twell_up_finish and by
 *                                   twell_down before use; twell_row_list_bytes bytes.
 *                                   For R <= 64 it also holds the decode workspace of the
 *                                   up GEMM (after the lists): fp32 half sums of the K split
 *                                   and one 64-bit ticket per 128 columns. No part of
 *                                   row_list needs initialising: from 3 rows on, the two
 *                                   workgroups of a tile meet by swapping the ticket for
 *                                   their own tag constant, and any other previous value
 *                                   (an earlier call leaves zero) reads as "arrived first";
 *                                   with 1 or 2 rows the half sums are added by a later
 *                                   kernel of the same call. Calls that overlap on one h
 *                                   race.
 *
 * A row overflows iff some tile of it holds more than `slots` nonzeros. A (row, tile)
 * keeps its first min(count, slots) nonzeros in ascending column order. "Nonzero" is
 * "not +0 and not -0". The slots of an overflow row are still filled (first `slots` per
 * tile); consumers take such a row from ovf_dense. Rows that overflow beyond ovf_cap get
 * ovf_slot = -1 and their products are undefined; twell_sync_status reports the case.
 *
 * Supported: tile_w in {64, 128}; 1 <= slots <= min(tile_w, 64); ovf_cap >= 0 (ovf_rows
 * and ovf_dense may be NULL when ovf_cap == 0); val_dtype TWELL_F32 or TWELL_BF16.
 */
typedef struct {
  int32_t rows, cols, tile_w, slots, ovf_cap;
  int32_t val_dtype;
  int32_t *counts;
  int32_t *col_idx;
  void *vals;
  int32_t *ovf_n;
  int32_t *ovf_rows;
  int32_t *ovf_slot;
  void *ovf_dense;
  uint32_t *ovf_bits;
  int32_t *row_nnz;
  void *row_list;
} twell_matrix_t;

/* Returns TWELL_ABI_VERSION. */
int twell_abi_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char *twell_status_str(int status);

/* Number of uint32 words that twell_matrix_t.ovf_bits must hold. */
size_t twell_ovf_bits_words(int32_t rows, int32_t cols, int32_t tile_w);

/* Bytes that twell_matrix_t.row_list must hold: 8 bytes per slot of the matrix, plus, for
 * rows <= 64, the decode workspace (256-byte aligned after the lists; 64 KB per 128
 * columns, then 8 bytes of ticket per 128 columns rounded up to 256 bytes). */
size_t twell_row_list_bytes(int32_t rows, int32_t cols, int32_t tile_w, int32_t slots);

/*
 * twell_pack — dense h [R][C] (h_dtype) -> TwELL `out` (shape fields set by the caller).
 * The separate dense-to-sparse conversion that "Formato de Dados TwELL" describes as the
 * step the fused epilogue removes; kept as a building block and for testing. Values are
 * copied bit for bit (bf16 -> fp32 widening is exact; fp32 -> bf16 is refused).
 * Errors: TWELL_ERR_ARG (null), TWELL_ERR_SHAPE (C % tile_w, slots), TWELL_ERR_UNSUPPORTED.
 */
int twell_pack(const void *h, int32_t h_dtype, twell_matrix_t *out, void *stream);

/*
 * twell_ffn_fwd — y = ReLU(x . W1 + b1) . W2 with the hidden activations in TwELL.
 * "Formato de Dados TwELL": the up projection is a dense GEMM (MFMA) whose epilogue applies
 * the bias and ReLU and writes the TwELL slots directly; "Kernels de Inferência": the down
 * projection iterates over the active units only. The TwELL (h_out, shape fields and
 * buffers from the caller, rows = T, cols = d_ff) is left for the backward pass.
 * in_dtype: TWELL_F32 (x, w1t, w2 fp32) or TWELL_BF16 (bf16, fp32 accumulation).
 * y_dtype: TWELL_F32 or TWELL_BF16. T == 0 is allowed (only *ovf_n is written).
 * The row lists (row_nnz, row_list) are scratch: from 1 to 16 bf16 tokens with d_model 1024,
 * 2048 or 4096 the forward packs
 * the TwELL and gathers y in one kernel and leaves no lists in h; call twell_down (which
 * rebuilds them), not twell_fwd_down, on such an h.
 * Errors: TWELL_ERR_ARG, TWELL_ERR_SHAPE (d, d_ff <= 0, T < 0, d_ff % tile_w, h_out shape
 * mismatch), TWELL_ERR_ALIGN (d % 8), TWELL_ERR_UNSUPPORTED.
 */
int twell_ffn_fwd(const void *x, const void *w1t, const float *b1, const void *w2,
                  int32_t in_dtype, int32_t T, int32_t d_model, int32_t d_ff,
                  twell_matrix_t *h_out, void *y, int32_t y_dtype, void *stream);

/*
 * Stages of twell_ffn_fwd, callable one by one; run in this order on one stream they give
 * the TwELL twell_ffn_fwd gives, bit for bit, and y within the sum-order rounding (at the
 * decode sizes above twell_ffn_fwd runs its own fused kernels, elsewhere it enqueues exactly
 * these three):
 *   twell_up_gemm   — the up-projection MFMA GEMM with the fused bias + ReLU + TwELL
 *                     epilogue: writes counts, col_idx, vals and ovf_bits only.
 *   twell_up_finish — the overflow bookkeeping ("Formato Híbrido para Treinamento"): the
 *                     ordered overflow list, ovf_slot, *ovf_n, and ovf_dense recomputed by
 *                     the same GEMM for the listed rows; in the same launch as the
 *                     overflow scan it also fills the row lists (row_nnz, row_list) that
 *                     the down projection walks. Must follow twell_up_gemm on the same h.
 *                     After both, h is the complete TwELL of ReLU(x W1 + b1).
 * Same arguments, checks and errors as twell_ffn_fwd (twell_up_finish also needs row_nnz
 * and row_list; twell_up_gemm needs row_list when 0 < T <= 64, for the decode workspace,
 * else TWELL_ERR_ARG).
 *
 * Up to 64 tokens the GEMM sums K in four quarters, (q0 + q1) + (q2 + q3), and spreads each
 * 128-column tile over two workgroups (quarters 0-1 and 2-3) that meet in the decode
 * workspace of row_list; ffn_up_relu_dense sums the same quarters in the same order.
 */
int twell_up_gemm(const void *x, const void *w1t, const float *b1, int32_t in_dtype, int32_t T,
                  int32_t d_model, int32_t d_ff, twell_matrix_t *h, void *stream);
int twell_up_finish(const void *x, const void *w1t, const float *b1, int32_t in_dtype, int32_t T,
                    int32_t d_model, int32_t d_ff, twell_matrix_t *h, void *stream);

/*
 * twell_fwd_down — the last stage: twell_down without rebuilding the row lists, which
 * twell_up_finish left in h on the same stream. Arguments, checks and errors as twell_down.
 * Use twell_down for a TwELL from any other producer (twell_ffn_fwd included). Stale lists
 * give wrong sums but no access outside h's buffers (lengths are clamped to n_t S).
 */
int twell_fwd_down(const twell_matrix_t *h, const void *w2, int32_t w_dtype, int32_t d_model,
                   void *y, int32_t y_dtype, void *stream);

/*
 * twell_down — y[t] = sum over the nonzero h[t, j] of h[t, j] * w2[j] for an existing
 * TwELL h (rows = T, cols = d_ff; ovf_slot must be valid), fp32 accumulation.
 * "Kernels de Inferência": only the active units' rows of W2 are read.
 * Errors: TWELL_ERR_ARG (null, dtype), TWELL_ERR_SHAPE (d_model <= 0), TWELL_ERR_ALIGN
 * (d_model % 8, w2 or y not 16-byte aligned), TWELL_ERR_UNSUPPORTED (w2 or y of 2 GiB or
 * more: rows are addressed with 32-bit byte offsets).
 */
int twell_down(const twell_matrix_t *h, const void *w2, int32_t w_dtype, int32_t d_model,
               void *y, int32_t y_dtype, void *stream);

/*
 * Gated feed-forward ("Sparser, Faster, Lighter Transformer Language Models", section
 * "2. Metodologia", blocks "Formato de Dados TwELL" and "Kernels de Inferência"): the TwELL
 * holds the gate activations g = ReLU(x . Wg + bg), and only the active units take the up
 * projection u = x . Wu (no bias) before the down product:
 *   y = (g * u) . W2     (elementwise gate * up; rows of w_up_t as in w1t).
 *
 * twell_gate_up — the up stage: for every entry (j, g) of every row list in h, and every
 * nonzero of every stored dense backup row, g <- g * (x[t] . w_up_t[j]) (fp32 sum; bf16
 * products by v_dot2_f32_bf16). Call after twell_up_finish on the same h and stream (the
 * gate GEMM built the lists); then twell_fwd_down yields y. The TwELL slots (counts,
 * col_idx, vals) keep the gate; row_list values and ovf_dense rows hold g * u afterwards.
 * x [T][d_model] and w_up_t [d_ff][d_model] in in_dtype, 16-byte aligned; d_model a
 * multiple of 8. From 512 tokens on, the dot products of the row lists are cut into
 * per-XCD column chunks whose partial sums go to `workspace` (device, caller-owned, 16-byte
 * aligned, at least twell_gate_up_workspace_bytes; contents need not be initialised);
 * below 512 tokens no workspace is used (it may be NULL). Too small a workspace gives
 * TWELL_ERR_WORKSPACE before anything is enqueued; other errors as twell_ffn_fwd.
 */
size_t twell_gate_up_workspace_bytes(int32_t T, int32_t d_model, int32_t d_ff, int32_t in_dtype,
                                     const twell_matrix_t *h);
int twell_gate_up(twell_matrix_t *h, const void *x, const void *w_up_t, int32_t in_dtype,
                  int32_t T, int32_t d_model, int32_t d_ff, void *workspace, size_t workspace_bytes,
                  void *stream);

/*
 * twell_gated_ffn_fwd — the whole gated forward: twell_up_gemm and twell_up_finish on the
 * gate weights (w_gate_t, b_gate), twell_gate_up with w_up_t (and the workspace), then
 * twell_fwd_down with w2, in that order on the stream. Arguments, checks and errors as
 * twell_ffn_fwd plus w_up_t and the workspace of twell_gate_up.
 */
int twell_gated_ffn_fwd(const void *x, const void *w_gate_t, const float *b_gate, const void *w_up_t,
                        const void *w2, int32_t in_dtype, int32_t T, int32_t d_model, int32_t d_ff,
                        twell_matrix_t *h, void *y, int32_t y_dtype, void *workspace,
                        size_t workspace_bytes, void *stream);

/*
 * twell_gated_ffn_infer — the gated forward of twell_gated_ffn_fwd for inference at decode
 * sizes (0 <= T <= 64), as "Kernels de Inferência" describes it: after the gate GEMM (the
 * same kernel as twell_up_gemm, writing the gate's TwELL into h) ONE kernel iterates over
 * each token's active gate units, takes the up dot product u = x[t] . w_up_t[j] and
 * multiplies-adds (g u) w2[j] into y[t]; no intermediate goes through a separate launch.
 * A tile holding more than h->slots active units is recomputed inside that kernel (its gate
 * pre-activations x[t] . w_gate_t[j] + b_gate[j], rounded to the value type), its gated
 * products taken from a dense row of the scratch. So no hybrid backup is formed: ovf_n,
 * ovf_rows, ovf_slot and ovf_dense are not written (ovf_cap may be 0). h keeps the gate's
 * TwELL (counts, col_idx, vals); row_nnz and row_list are scratch and need no
 * initialisation. The down products of a token are summed in a fixed order (same bits on
 * every call). Calls that overlap on one h race. Arguments, layouts and errors as
 * twell_gated_ffn_fwd without the workspace; T > 64 or more than 256 tiles per row returns
 * TWELL_ERR_UNSUPPORTED (use twell_gated_ffn_fwd).
 */
int twell_gated_ffn_infer(const void *x, const void *w_gate_t, const float *b_gate, const void *w_up_t,
                          const void *w2, int32_t in_dtype, int32_t T, int32_t d_model, int32_t d_ff,
                          twell_matrix_t *h, void *y, int32_t y_dtype, void *stream);

/*
 * ffn_up_relu_dense — h = ReLU(x . W1 + b1) written densely ([T][d_ff], h_dtype = fp32 or
 * bf16). Same MFMA kernel and accumulation order as the fused TwELL path, so the fp32
 * output is bit-identical to the values the TwELL epilogue sees.
 */
int ffn_up_relu_dense(const void *x, const void *w1t, const float *b1, int32_t in_dtype,
                      int32_t T, int32_t d_model, int32_t d_ff, void *h, int32_t h_dtype,
                      void *stream);

/*
 * Workspace of twell_ffn_bwd. It grows with the number of entries it can hold, about
 * 36 + 4 * d_model / 128 bytes each (bf16; d_model / 64 column chunks for fp32: the SDDMM keeps
 * one partial dot product per entry and chunk so that every XCD reads only its own slices of
 * W2), plus 8 bytes per (32-token block, unit) and small per-token and per-unit arrays.
 *   twell_ffn_bwd_workspace_bytes      — room for every entry h can hold, T * (d_ff / tile_w)
 *                                        * slots + min(ovf_cap, T) * d_ff: always enough.
 *   twell_ffn_bwd_workspace_bytes_nnz  — room for nnz entries (at most that capacity): the
 *                                        stored entries of the call, i.e. the sum over rows of
 *                                        the row's nonzeros (slots in use, or the nonzeros of
 *                                        its backup row), which a caller knows from
 *                                        twell_row_nnz_histogram (sum of m * hist[m]).
 * 0 for invalid arguments. in_dtype as passed to twell_ffn_bwd.
 */
size_t twell_ffn_bwd_workspace_bytes(int32_t T, int32_t d_model, int32_t d_ff, int32_t in_dtype,
                                     const twell_matrix_t *h);
size_t twell_ffn_bwd_workspace_bytes_nnz(int32_t T, int32_t d_model, int32_t d_ff, int32_t in_dtype,
                                         const twell_matrix_t *h, int64_t nnz);

/*
 * twell_ffn_bwd — gradients of <dy, y> + l1_coef * sum(h) for the forward above.
 * "Formato Híbrido para Treinamento": the backward runs on the sparsity pattern stored in
 * the TwELL h (slots of normal rows, dense backup of overflow rows); "Técnicas de
 * Treinamento": the L1 penalty adds l1_coef on every active entry of dh.
 *   dz   = (dy . W2^T + l1_coef) on the pattern      (ReLU'(0) = 0)
 *   dx   = dz . w1t                 [T][d]  fp32
 *   dw1t = dz^T . x                 [f][d]  fp32
 *   dw2  = h^T . dy                 [f][d]  fp32
 *   db1  = sum_t dz                 [f]     fp32 (may be NULL)
 * x, w1t, w2, dy have in_dtype. Every overflow row needs a backup slot (*ovf_n <= ovf_cap):
 * a row beyond the capacity kept only its first slots per tile, so its gradients cannot be
 * formed, and then every output (dx, dw1t, dw2 and db1) is overwritten with quiet NaN on the
 * device, so the condition cannot pass unnoticed (twell_sync_status also reports it).
 * d_ff <= 16384 (a unit bit mask per 32-token block is built in LDS), else
 * TWELL_ERR_UNSUPPORTED. The workspace may be smaller than twell_ffn_bwd_workspace_bytes:
 * the call uses it for as many entries as fit, and if the call's entries do not fit (checked
 * on the device) every output is overwritten with quiet NaN; a workspace too small for even
 * zero entries gives TWELL_ERR_WORKSPACE before anything is enqueued. Contents need not be
 * initialised.
 */
int twell_ffn_bwd(const void *x, const void *w1t, const void *w2, int32_t in_dtype,
                  int32_t T, int32_t d_model, int32_t d_ff, const twell_matrix_t *h,
                  const void *dy, float l1_coef, float *dx, float *dw1t, float *dw2,
                  float *db1, void *workspace, size_t workspace_bytes, void *stream);

/*
 * twell_ffn_bwd_noalloc — twell_ffn_bwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc). The scratch is a fixed array of TWELL_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, held until the process ends; nothing is allocated or freed by the
 * call (the array's device address is looked up once per device, on the first call there).
 * Same arguments, kernels, results and errors as twell_ffn_bwd, except: a problem whose
 * twell_ffn_bwd_workspace_bytes exceeds TWELL_NOALLOC_SCRATCH_BYTES returns
 * TWELL_ERR_WORKSPACE before anything is enqueued, and TWELL_ERR_HIP if the scratch cannot be
 * located on the current device. Every call on one GPU shares that GPU's scratch: calls
 * that overlap in time on one GPU (different streams or threads) race and must be ordered by
 * the caller. The scratch needs no initialisation (the backward writes before it reads).
 */
#define TWELL_NOALLOC_SCRATCH_BYTES (64u << 20)
int twell_ffn_bwd_noalloc(const void *x, const void *w1t, const void *w2, int32_t in_dtype,
                          int32_t T, int32_t d_model, int32_t d_ff, const twell_matrix_t *h,
                          const void *dy, float l1_coef, float *dx, float *dw1t, float *dw2,
                          float *db1, void *stream);

/*
 * nm_prune — N:M activation pruning by magnitude ("Motivating Next-Gen Accelerators ...",
 * "2. Metodologia", criterion ACT): in every block of m consecutive entries of a row of
 * h [T][d_ff] keep the n of largest |h| (ties to the lower index), emitted in ascending
 * index order with their signed values.
 *   vals [T][d_ff/m][n]  dtype (bit-exact copies)
 *   idx  [T][d_ff/m][n]  uint8, index inside the block
 * Supported (n, m): (2,4), (4,8), (8,16), (16,32). dtype: TWELL_BF16 or TWELL_F32.
 */
int nm_prune(const void *h, int32_t dtype, int32_t T, int32_t d_ff, int32_t n, int32_t m,
             void *vals, uint8_t *idx, void *stream);

/*
 * ffn_up_relu_nm — the up projection with N:M pruning in its epilogue ("Motivating Next-Gen
 * Accelerators with Flexible (N:M) Activation Sparsity ...", "2. Metodologia", criterion
 * ACT, applied to h = ReLU(x . W1 + b1)). The dense h is never written: each workgroup
 * rounds its tile of h to in_dtype in LDS and prunes it there. The result is bit-identical
 * to nm_prune(n, m) applied to ffn_up_relu_dense(..., h_dtype = in_dtype):
 *   vals [T][d_ff/m][n]  in_dtype (the kept values of h, ascending index in the block)
 *   idx  [T][d_ff/m][n]  uint8
 * Arguments and checks as ffn_up_relu_dense and nm_prune: (n, m) in (2,4), (4,8), (8,16),
 * (16,32) and d_ff % m == 0, else TWELL_ERR_SHAPE; vals, idx 16-byte aligned.
 */
int ffn_up_relu_nm(const void *x, const void *w1t, const float *b1, int32_t in_dtype, int32_t T,
                   int32_t d_model, int32_t d_ff, int32_t n, int32_t m, void *vals, uint8_t *idx,
                   void *stream);

/*
 * nm_ffn_down — y = H_nm . W2 for N:M-packed activations (vals, idx from nm_prune, bf16).
 * gfx950's sparse matrix instructions take only a 2:4 structure (at most two nonzeros in
 * every four consecutive entries), which 8:16 and 16:32 blocks do not have, so each block is
 * expanded to dense bf16 in LDS and multiplied on MFMA; only the activation bytes shrink.
 * w2: [d_ff][d_model] bf16, row-major, the same down weight twell_down and twell_ffn_fwd
 * take, so one copy serves the TwELL and the N:M paths. y: [T][d_model], y_dtype fp32 or
 * bf16. (n, m) in (8,16), (16,32) (2:4 and 4:8 give TWELL_ERR_UNSUPPORTED); d_ff % 32 == 0
 * and d_model % 8 == 0, else TWELL_ERR_SHAPE; vals, idx, w2, y 16-byte aligned; w2 under
 * 2 GiB and d_ff < 2^23 (256 rows of packed values under 2 GiB), else
 * TWELL_ERR_UNSUPPORTED.
 */
int nm_ffn_down(const void *vals, const uint8_t *idx, int32_t dtype, int32_t T, int32_t d_ff,
                int32_t n, int32_t m, const void *w2, int32_t d_model, void *y,
                int32_t y_dtype, void *stream);

/*
 * Dynamic slot count ("Sparser, Faster, Lighter Transformer Language Models", "2. Metodologia",
 * block "Formato Híbrido para Treinamento": the compact width follows the data; rows beyond
 * it go to the dense backup). A training loop takes the histogram of one step's TwELL and
 * chooses the slot count of the next.
 *
 * twell_row_max_histogram — hist[m] = number of rows of h whose largest per-tile true count
 * is m, for m = 0 .. tile_w (hist: device int32 [tile_w + 1], overwritten; enqueued on
 * `stream`). Only h's shape fields and counts are read. For any S, sum over m > S of hist[m]
 * is the number of rows that overflow S slots.
 */
int twell_row_max_histogram(const twell_matrix_t *h, int32_t *hist, void *stream);

/*
 * twell_stash_bytes — bytes of a TwELL with `slots` slots and n_ovf backup rows as kept for
 * the backward: counts and ovf_slot (int32), col_idx (int32) and vals per slot, ovf_rows
 * (int32) and one backup row of vals per overflow row. 0 for invalid arguments.
 */
size_t twell_stash_bytes(int32_t rows, int32_t cols, int32_t tile_w, int32_t slots, int32_t n_ovf,
                         int32_t val_dtype);

/*
 * twell_choose_slots — host function; hist is a HOST copy of the histogram above. Returns the
 * slot count S in 1 .. min(tile_w, 64) with the smallest twell_stash_bytes among those whose
 * overflow rows fit ovf_cap (the smaller S on equal bytes), and stores its bytes in
 * *stash_bytes (may be NULL). TWELL_ERR_OVF_CAPACITY if no S fits; TWELL_ERR_ARG /
 * TWELL_ERR_SHAPE for invalid arguments.
 */
int twell_choose_slots(const int32_t *hist, int32_t tile_w, int32_t rows, int32_t cols, int32_t ovf_cap,
                       int32_t val_dtype, size_t *stash_bytes);

/*
 * The compact row-ELL of the hybrid training format ("Formato Híbrido para Treinamento": rows
 * with few nonzeros in a compact ELL whose width follows the data, the rest in a dense
 * backup). It is a twell_matrix_t whose single tile spans the row: tile_w == cols, slots = the
 * width N (1 <= N <= cols <= 16384), counts [R][1] = the row's nonzeros, col_idx / vals
 * [R][N] its first min(count, N) entries in ascending column order (pad -1, +0.0), and the
 * same ordered dense backup for the rows with more than N entries. twell_down,
 * twell_ffn_bwd (and _noalloc), twell_row_max_histogram, twell_row_nnz_histogram and
 * twell_sync_status take it; the GEMM producers and twell_pack make tile_w 64 or 128 only.
 *
 * twell_to_row_ell — the row-ELL `dst` (shape fields and buffers from the caller: rows and
 * cols of src, tile_w = cols, slots = N, ovf_cap, val_dtype; ovf_bits as
 * twell_ovf_bits_words) of a TwELL `src` whose backup bookkeeping is complete (after
 * twell_up_finish / twell_ffn_fwd or twell_pack). Values are copied bit for bit (bf16 ->
 * fp32 widening is exact; fp32 -> bf16 is refused). A src row beyond src's backup capacity
 * lost entries: then dst's *ovf_n is raised above dst's ovf_cap, so the capacity error
 * follows the data. Errors: TWELL_ERR_ARG, TWELL_ERR_SHAPE (dst not a row-ELL of src's
 * shape), TWELL_ERR_UNSUPPORTED.
 */
int twell_to_row_ell(const twell_matrix_t *src, twell_matrix_t *dst, void *stream);

/*
 * twell_row_nnz_histogram — hist[min(n_t, nbins - 1)] = number of rows t of h with n_t
 * nonzeros (the sum of the row's true tile counts, also for backup rows), nbins >= 2; hist:
 * device int32 [nbins], overwritten. sum over m of m * hist[m] (with nbins above the widest
 * row) is the number of entries the backward stores for h.
 */
int twell_row_nnz_histogram(const twell_matrix_t *h, int32_t *hist, int32_t nbins, void *stream);

/*
 * twell_choose_row_ell_width — host function; hist is a HOST copy of a row-nonzero histogram
 * (nbins >= 3). Returns the width N in 1 .. min(nbins - 2, cols) whose row-ELL has the
 * smallest twell_stash_bytes (tile_w = cols) among those whose rows with more than N entries
 * fit ovf_cap (the smaller N on equal bytes), its bytes in *stash_bytes (may be NULL).
 * TWELL_ERR_OVF_CAPACITY if none fits.
 */
int twell_choose_row_ell_width(const int32_t *hist, int32_t nbins, int32_t rows, int32_t cols,
                               int32_t ovf_cap, int32_t val_dtype, size_t *stash_bytes);

/*
 * twell_sync_status — waits for `stream`, then reads *ovf_n: TWELL_ERR_OVF_CAPACITY if it
 * exceeds ovf_cap, TWELL_OK otherwise (TWELL_ERR_HIP if the wait or copy fails).
 */
int twell_sync_status(const twell_matrix_t *h, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TWELL_H */
