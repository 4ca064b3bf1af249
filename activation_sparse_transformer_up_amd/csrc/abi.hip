// C ABI of the TwELL FFN library: argument validation, then launches on the caller's stream.
// Declarations, layouts and error contract: include/twell.h.
#include <string.h>

#include <mutex>

#include "../../include/twell.h"
#include "launch.h"

using namespace tw;

// Device scratch of twell_ffn_bwd_noalloc, for callers that cannot allocate: one copy per GPU
// (at its own address on each), held for the life of the process. In host code `scratch`
// names a host-side stand-in, not device memory: only the address hipGetSymbolAddress returns
// for the current device may be handed to kernels.
static __device__ __align__(256) char scratch[TWELL_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void *scratch_ptr[kMaxDevices];

// The current device's address of `scratch` (looked up once per device), or NULL on error.
void *scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

}  // namespace

namespace {

inline bool al16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
inline bool al4(const void *p) { return ((uintptr_t)p & 3u) == 0; }
inline bool dtype_ok(int32_t t) { return t == TWELL_F32 || t == TWELL_BF16; }
inline hipStream_t S(void *s) { return (hipStream_t)s; }
inline int hip_status(hipError_t e) { return e == hipSuccess ? TWELL_OK : TWELL_ERR_HIP; }

#define TW_TRY(expr)                               \
  do {                                             \
    hipError_t e_ = (expr);                        \
    if (e_ != hipSuccess) return TWELL_ERR_HIP;    \
  } while (0)

// A TwELL whose single tile spans the row: the compact row-ELL of the hybrid format.
inline bool is_row_ell(const twell_matrix_t *m) { return m->tile_w == m->cols && m->tile_w != 64 && m->tile_w != 128; }

// Shape and pointer checks of a TwELL struct used as output (writable) or input. row_ell:
// the consumer also takes the row-ELL form (tile_w == cols, 1 <= slots <= cols <= 16384).
int check_matrix(const twell_matrix_t *m, bool need_ovf_bits, bool need_rows = false, bool row_ell = false) {
  if (!m) return TWELL_ERR_ARG;
  if (!dtype_ok(m->val_dtype)) return TWELL_ERR_ARG;
  if (m->rows < 0 || m->cols <= 0 || m->ovf_cap < 0) return TWELL_ERR_SHAPE;
  if (row_ell && is_row_ell(m)) {
    if (m->cols > 16384) return TWELL_ERR_UNSUPPORTED;
    if (m->slots < 1 || m->slots > m->cols) return TWELL_ERR_SHAPE;
  } else {
    if (m->tile_w != 64 && m->tile_w != 128) return TWELL_ERR_UNSUPPORTED;
    if (m->cols % m->tile_w) return TWELL_ERR_SHAPE;
    if (m->slots < 1 || m->slots > m->tile_w || m->slots > 64) return TWELL_ERR_SHAPE;
  }
  if (!m->ovf_n) return TWELL_ERR_ARG;
  if (m->rows > 0) {
    if (!m->counts || !m->col_idx || !m->vals || !m->ovf_slot) return TWELL_ERR_ARG;
    if (need_ovf_bits && !m->ovf_bits) return TWELL_ERR_ARG;
    if (need_rows && (!m->row_nnz || !m->row_list)) return TWELL_ERR_ARG;
  }
  if (m->ovf_cap > 0 && (!m->ovf_rows || !m->ovf_dense)) return TWELL_ERR_ARG;
  if (!al4(m->counts) || !al4(m->col_idx) || !al4(m->vals) || !al4(m->ovf_n) || !al4(m->ovf_rows) ||
      !al4(m->ovf_slot) || !al4(m->ovf_bits) || !al16(m->ovf_dense) || !al4(m->row_nnz) || !al16(m->row_list))
    return TWELL_ERR_ALIGN;
  return TWELL_OK;
}

size_t list_bytes(int32_t rows, int32_t cols, int32_t tile_w, int32_t slots) {
  return (size_t)rows * (size_t)(cols / tile_w) * (size_t)slots * 8;
}

TwellOut out_of(const twell_matrix_t *m) {
  TwellOut o;
  o.counts = m->counts;
  o.col_idx = m->col_idx;
  o.vals = m->vals;
  o.ovf_bits = m->ovf_bits;
  o.dec_part = nullptr;
  o.dec_ticket = nullptr;
  o.dec_bytes = 0;
  if (m->row_list && m->rows <= kDecodeMaxT) {
    char *ws = (char *)m->row_list + align256(list_bytes(m->rows, m->cols, m->tile_w, m->slots));
    o.dec_part = (float *)ws;
    o.dec_ticket = (uint64_t *)(ws + dec_tiles(m->cols) * 2 * kDecHalfBytes);
    o.dec_bytes = dec_tiles(m->cols) * 2 * kDecHalfBytes;
  }
  o.n_t = m->cols / m->tile_w;
  o.S = m->slots;
  o.words = (m->rows + 31) / 32;
  o.val_bf16 = m->val_dtype == TWELL_BF16;
  return o;
}

TwellFinish finish_of(twell_matrix_t *m, bool complete) {
  TwellFinish f;
  f.complete = complete;
  f.row_nnz = m->row_nnz;
  f.row_list = (uint2 *)m->row_list;
  f.ovf_n = m->ovf_n;
  f.ovf_rows = m->ovf_rows;
  f.ovf_slot = m->ovf_slot;
  f.ovf_dense = m->ovf_dense;
  f.cap = m->ovf_cap;
  return f;
}

TwellIn in_of(const twell_matrix_t *m) {
  TwellIn h;
  h.counts = m->counts;
  h.col_idx = m->col_idx;
  h.vals = m->vals;
  h.ovf_slot = m->ovf_slot;
  h.ovf_dense = m->ovf_dense;
  h.ovf_n = m->ovf_n;
  h.ovf_rows = m->ovf_rows;
  h.cap = m->ovf_cap;
  h.row_nnz = m->row_nnz;
  h.row_list = (uint2 *)m->row_list;
  h.rows = m->rows;
  h.cols = m->cols;
  h.n_t = m->cols / m->tile_w;
  h.S = m->slots;
  h.W = m->tile_w;
  h.val_bf16 = m->val_dtype == TWELL_BF16;
  return h;
}

}  // namespace

extern "C" {

int twell_abi_version(void) { return TWELL_ABI_VERSION; }

const char *twell_status_str(int status) {
  switch (status) {
    case TWELL_OK: return "TWELL_OK";
    case TWELL_ERR_ARG: return "TWELL_ERR_ARG: null pointer or invalid enum/struct field";
    case TWELL_ERR_SHAPE: return "TWELL_ERR_SHAPE: invalid or inconsistent sizes";
    case TWELL_ERR_ALIGN: return "TWELL_ERR_ALIGN: misaligned pointer or d_model % 8 != 0";
    case TWELL_ERR_WORKSPACE: return "TWELL_ERR_WORKSPACE: workspace too small";
    case TWELL_ERR_OVF_CAPACITY: return "TWELL_ERR_OVF_CAPACITY: more overflow rows than ovf_cap";
    case TWELL_ERR_HIP: return "TWELL_ERR_HIP: HIP runtime or launch failure";
    case TWELL_ERR_UNSUPPORTED: return "TWELL_ERR_UNSUPPORTED: valid request not implemented";
    default: return "TWELL_UNKNOWN_STATUS";
  }
}

size_t twell_ovf_bits_words(int32_t rows, int32_t cols, int32_t tile_w) {
  if (rows < 0 || cols <= 0 || tile_w <= 0) return 0;
  return (size_t)(cols / tile_w) * (size_t)((rows + 31) / 32);
}

size_t twell_row_list_bytes(int32_t rows, int32_t cols, int32_t tile_w, int32_t slots) {
  if (rows < 0 || cols <= 0 || tile_w <= 0 || slots <= 0) return 0;
  const size_t lists = list_bytes(rows, cols, tile_w, slots);
  return rows <= kDecodeMaxT ? align256(lists) + dec_ws_bytes(cols) : lists;
}

int twell_pack(const void *h, int32_t h_dtype, twell_matrix_t *out, void *stream) {
  if (!h || !out) return TWELL_ERR_ARG;
  if (!dtype_ok(h_dtype)) return TWELL_ERR_ARG;
  int st = check_matrix(out, true);
  if (st) return st;
  if (h_dtype == TWELL_F32 && out->val_dtype == TWELL_BF16) return TWELL_ERR_UNSUPPORTED;
  if (!al16(h)) return TWELL_ERR_ALIGN;
  const int R = out->rows, C = out->cols;
  if (R == 0) return hip_status(launch_set_int(out->ovf_n, 0, S(stream)));
  const TwellOut o = out_of(out);
  TW_TRY(launch_pack(h, h_dtype == TWELL_BF16, R, C, o, out->tile_w, S(stream)));
  TW_TRY(launch_ovf_scan(out->ovf_bits, o.n_t, o.words, R, out->ovf_cap, out->ovf_n, out->ovf_rows,
                         out->ovf_slot, S(stream)));
  TW_TRY(launch_ovf_copy(h, h_dtype == TWELL_BF16, R, C, out->ovf_n, out->ovf_rows, out->ovf_cap,
                         out->ovf_dense, out->val_dtype == TWELL_BF16, S(stream)));
  return TWELL_OK;
}

static int check_ffn_args(const void *x, const void *w1t, const void *w2, int32_t in_dtype, int32_t T,
                          int32_t d, int32_t f) {
  if (!w1t || (T > 0 && !x)) return TWELL_ERR_ARG;
  if (!dtype_ok(in_dtype)) return TWELL_ERR_ARG;
  if (T < 0 || d <= 0 || f <= 0) return TWELL_ERR_SHAPE;
  if (d % 8) return TWELL_ERR_ALIGN;
  if (!al16(x) || !al16(w1t) || (w2 && !al16(w2))) return TWELL_ERR_ALIGN;
  // the GEMM addresses each operand with 32-bit byte offsets
  const size_t es = in_dtype == TWELL_BF16 ? 2 : 4;
  if ((size_t)T * d * es >= ((size_t)1 << 31) || (size_t)f * d * es >= ((size_t)1 << 31)) return TWELL_ERR_UNSUPPORTED;
  return TWELL_OK;
}

static int check_up_args(const void *x, const void *w1t, const float *b1, int32_t in_dtype, int32_t T,
                         int32_t d_model, int32_t d_ff, const twell_matrix_t *h) {
  if (!b1 || !h) return TWELL_ERR_ARG;
  int st = check_ffn_args(x, w1t, nullptr, in_dtype, T, d_model, d_ff);
  if (st) return st;
  st = check_matrix(h, true);
  if (st) return st;
  if (h->rows != T || h->cols != d_ff) return TWELL_ERR_SHAPE;
  if (T > 0 && T <= kDecodeMaxT && !h->row_list) return TWELL_ERR_ARG;   // decode workspace
  if (!al4(b1)) return TWELL_ERR_ALIGN;
  return TWELL_OK;
}

// complete: let the GEMM stage also build the lists, the overflow scan and the backup rows
// where it can do that itself (one or two tokens; see gemm_completes)
static int up_gemm(const void *x, const void *w1t, const float *b1, int32_t in_dtype, int32_t T, int32_t d_model,
                   int32_t d_ff, twell_matrix_t *h, hipStream_t s, bool complete = false) {
  if (T == 0) return TWELL_OK;
  TW_TRY(launch_up_twell(in_dtype == TWELL_BF16, x, w1t, b1, T, d_ff, d_model, out_of(h), finish_of(h, complete),
                         h->tile_w, s));
  return TWELL_OK;
}

// true if up_gemm(..., complete = true) completes the matrix (lists, overflow scan, backup
// rows): then up_finish has nothing left to do
static bool gemm_completes(int32_t in_dtype, int32_t T, int32_t d_model, twell_matrix_t *h) {
  return T > 0 && up_twell_completes(in_dtype == TWELL_BF16, T, d_model, finish_of(h, true));
}

static int up_finish(const void *x, const void *w1t, const float *b1, int32_t in_dtype, int32_t T,
                     int32_t d_model, int32_t d_ff, twell_matrix_t *h, hipStream_t s) {
  if (T == 0) return hip_status(launch_set_int(h->ovf_n, 0, s));
  const TwellOut o = out_of(h);
  const hipError_t fe = launch_finish_dec(in_dtype == TWELL_BF16, in_of(h), h->ovf_bits, o.words, h->ovf_n,
                                          h->ovf_rows, h->ovf_slot, x, w1t, b1, d_model, h->ovf_dense, s);
  if (fe == hipSuccess) return TWELL_OK;
  if (fe != hipErrorNotSupported) return hip_status(fe);
  TW_TRY(launch_lists_scan(in_of(h), h->ovf_bits, o.words, h->ovf_n, h->ovf_rows, h->ovf_slot, s));
  if (h->ovf_cap > 0) {
    const int M = h->ovf_cap < T ? h->ovf_cap : T;
    TW_TRY(launch_up_dense(in_dtype == TWELL_BF16, x, w1t, b1, M, d_ff, d_model, T, h->ovf_rows, h->ovf_n,
                           h->ovf_dense, h->val_dtype == TWELL_BF16, 1, s));
  }
  return TWELL_OK;
}

int twell_up_gemm(const void *x, const void *w1t, const float *b1, int32_t in_dtype, int32_t T,
                  int32_t d_model, int32_t d_ff, twell_matrix_t *h, void *stream) {
  int st = check_up_args(x, w1t, b1, in_dtype, T, d_model, d_ff, h);
  if (st) return st;
  return up_gemm(x, w1t, b1, in_dtype, T, d_model, d_ff, h, S(stream));
}

int twell_up_finish(const void *x, const void *w1t, const float *b1, int32_t in_dtype, int32_t T,
                    int32_t d_model, int32_t d_ff, twell_matrix_t *h, void *stream) {
  int st = check_up_args(x, w1t, b1, in_dtype, T, d_model, d_ff, h);
  if (st) return st;
  st = check_matrix(h, true, true);
  if (st) return st;
  return up_finish(x, w1t, b1, in_dtype, T, d_model, d_ff, h, S(stream));
}

int twell_ffn_fwd(const void *x, const void *w1t, const float *b1, const void *w2, int32_t in_dtype,
                  int32_t T, int32_t d_model, int32_t d_ff, twell_matrix_t *h, void *y, int32_t y_dtype,
                  void *stream) {
  if (!w2 || (T > 0 && !y)) return TWELL_ERR_ARG;
  if (!dtype_ok(y_dtype)) return TWELL_ERR_ARG;
  int st = check_up_args(x, w1t, b1, in_dtype, T, d_model, d_ff, h);
  if (st) return st;
  st = check_matrix(h, true, true);
  if (st) return st;
  if (!al16(w2) || !al16(y)) return TWELL_ERR_ALIGN;
  hipStream_t s = S(stream);
  if (T > 0 && in_dtype == TWELL_BF16 && up_stream_ok(1, T, d_model)) {
    // up to 16 tokens: the W1 stream, then the TwELL, the overflow scan and y in one launch
    const TwellOut o = out_of(h);
    TW_TRY(launch_up_stream(x, w1t, T, d_ff, d_model, o, s));
    TW_TRY(launch_dec_fused_down(b1, T, d_ff, o, finish_of(h, true), w2, d_model, y, y_dtype == TWELL_BF16, h->tile_w,
                                 s));
    return TWELL_OK;
  }
  st = up_gemm(x, w1t, b1, in_dtype, T, d_model, d_ff, h, s, true);
  if (st) return st;
  if (!gemm_completes(in_dtype, T, d_model, h)) st = up_finish(x, w1t, b1, in_dtype, T, d_model, d_ff, h, s);
  if (st || T == 0) return st;
  TW_TRY(launch_twell_down(in_of(h), w2, in_dtype == TWELL_BF16, d_model, y, y_dtype == TWELL_BF16, false, s));
  return TWELL_OK;
}

static int down_args(const twell_matrix_t *h, const void *w2, int32_t w_dtype, int32_t d_model, const void *y,
                     int32_t y_dtype, bool row_ell = false) {
  if (!h || !w2 || !y) return TWELL_ERR_ARG;
  if (!dtype_ok(w_dtype) || !dtype_ok(y_dtype)) return TWELL_ERR_ARG;
  int st = check_matrix(h, false, true, row_ell);
  if (st) return st;
  if (d_model <= 0) return TWELL_ERR_SHAPE;
  if (d_model % 8) return TWELL_ERR_ALIGN;
  if (!al16(w2) || !al16(y)) return TWELL_ERR_ALIGN;
  // the gathers address W2 rows (and y) with 32-bit byte offsets
  const size_t wb = w_dtype == TWELL_BF16 ? 2 : 4, yb = y_dtype == TWELL_BF16 ? 2 : 4;
  if ((size_t)h->cols * d_model * wb >= ((size_t)1 << 31) || (size_t)h->rows * d_model * yb >= ((size_t)1 << 31))
    return TWELL_ERR_UNSUPPORTED;
  return TWELL_OK;
}

int twell_fwd_down(const twell_matrix_t *h, const void *w2, int32_t w_dtype, int32_t d_model, void *y,
                   int32_t y_dtype, void *stream) {
  int st = down_args(h, w2, w_dtype, d_model, y, y_dtype);
  if (st) return st;
  if (h->rows == 0) return TWELL_OK;
  TW_TRY(launch_twell_down(in_of(h), w2, w_dtype == TWELL_BF16, d_model, y, y_dtype == TWELL_BF16, false,
                           S(stream)));
  return TWELL_OK;
}

int twell_down(const twell_matrix_t *h, const void *w2, int32_t w_dtype, int32_t d_model, void *y,
               int32_t y_dtype, void *stream) {
  int st = down_args(h, w2, w_dtype, d_model, y, y_dtype, true);
  if (st) return st;
  if (h->rows == 0) return TWELL_OK;
  TW_TRY(launch_twell_down(in_of(h), w2, w_dtype == TWELL_BF16, d_model, y, y_dtype == TWELL_BF16, true,
                           S(stream)));
  return TWELL_OK;
}

size_t twell_gate_up_workspace_bytes(int32_t T, int32_t d_model, int32_t d_ff, int32_t in_dtype,
                                     const twell_matrix_t *h) {
  if (!h || T < 0 || d_model <= 0 || d_ff <= 0 || h->tile_w <= 0 || h->slots <= 0) return 0;
  if (!dtype_ok(in_dtype)) return 0;
  return gate_up_workspace_bytes(T, d_model, d_ff / h->tile_w, h->slots, in_dtype == TWELL_BF16);
}

// The workspace the up products need for this h (checked before anything is enqueued).
static int gate_ws_check(const twell_matrix_t *h, int32_t in_dtype, int32_t d_model, const void *ws,
                         size_t ws_bytes) {
  const size_t need = gate_up_workspace_bytes(h->rows, d_model, h->cols / h->tile_w, h->slots, in_dtype == TWELL_BF16);
  if (need == 0) return TWELL_OK;
  if (!ws || ws_bytes < need) return TWELL_ERR_WORKSPACE;
  if (!al16(ws)) return TWELL_ERR_ALIGN;
  return TWELL_OK;
}

int twell_gate_up(twell_matrix_t *h, const void *x, const void *w_up_t, int32_t in_dtype, int32_t T,
                  int32_t d_model, int32_t d_ff, void *workspace, size_t workspace_bytes, void *stream) {
  if (!h) return TWELL_ERR_ARG;
  int st = check_ffn_args(x, w_up_t, nullptr, in_dtype, T, d_model, d_ff);
  if (st) return st;
  st = check_matrix(h, false, true);
  if (st) return st;
  if (h->rows != T || h->cols != d_ff) return TWELL_ERR_SHAPE;
  st = gate_ws_check(h, in_dtype, d_model, workspace, workspace_bytes);
  if (st) return st;
  if (T == 0) return TWELL_OK;
  TW_TRY(launch_gate_up(in_of(h), x, w_up_t, in_dtype == TWELL_BF16, d_model, (float *)workspace, S(stream)));
  return TWELL_OK;
}

int twell_gated_ffn_fwd(const void *x, const void *w_gate_t, const float *b_gate, const void *w_up_t,
                        const void *w2, int32_t in_dtype, int32_t T, int32_t d_model, int32_t d_ff,
                        twell_matrix_t *h, void *y, int32_t y_dtype, void *workspace, size_t workspace_bytes,
                        void *stream) {
  if (!w2 || !w_up_t || (T > 0 && !y)) return TWELL_ERR_ARG;
  if (!dtype_ok(y_dtype)) return TWELL_ERR_ARG;
  int st = check_up_args(x, w_gate_t, b_gate, in_dtype, T, d_model, d_ff, h);
  if (st) return st;
  st = check_matrix(h, true, true);
  if (st) return st;
  if (!al16(w2) || !al16(y) || !al16(w_up_t)) return TWELL_ERR_ALIGN;
  st = gate_ws_check(h, in_dtype, d_model, workspace, workspace_bytes);
  if (st) return st;
  hipStream_t s = S(stream);
  st = up_gemm(x, w_gate_t, b_gate, in_dtype, T, d_model, d_ff, h, s, true);
  if (st) return st;
  if (!gemm_completes(in_dtype, T, d_model, h)) st = up_finish(x, w_gate_t, b_gate, in_dtype, T, d_model, d_ff, h, s);
  if (st || T == 0) return st;
  TW_TRY(launch_gate_up(in_of(h), x, w_up_t, in_dtype == TWELL_BF16, d_model, (float *)workspace, s));
  TW_TRY(launch_twell_down(in_of(h), w2, in_dtype == TWELL_BF16, d_model, y, y_dtype == TWELL_BF16, false, s));
  return TWELL_OK;
}

int twell_gated_ffn_infer(const void *x, const void *w_gate_t, const float *b_gate, const void *w_up_t,
                          const void *w2, int32_t in_dtype, int32_t T, int32_t d_model, int32_t d_ff,
                          twell_matrix_t *h, void *y, int32_t y_dtype, void *stream) {
  if (!w2 || !w_up_t || (T > 0 && !y)) return TWELL_ERR_ARG;
  if (!dtype_ok(y_dtype)) return TWELL_ERR_ARG;
  int st = check_up_args(x, w_gate_t, b_gate, in_dtype, T, d_model, d_ff, h);
  if (st) return st;
  st = check_matrix(h, true, true);
  if (st) return st;
  if (!al16(w2) || !al16(y) || !al16(w_up_t)) return TWELL_ERR_ALIGN;
  if (T > kDecodeMaxT || d_ff / h->tile_w > 256) return TWELL_ERR_UNSUPPORTED;
  if (T == 0) return TWELL_OK;
  hipStream_t s = S(stream);
  st = up_gemm(x, w_gate_t, b_gate, in_dtype, T, d_model, d_ff, h, s);
  if (st) return st;
  const TwellOut o = out_of(h);           // o.dec_part: the dense scratch rows [T][d_ff] fp32
  TW_TRY(launch_gated_fused(in_of(h), x, w_gate_t, b_gate, w_up_t, w2, in_dtype == TWELL_BF16, d_model, y,
                            y_dtype == TWELL_BF16, o.dec_part, s));
  return TWELL_OK;
}

int ffn_up_relu_dense(const void *x, const void *w1t, const float *b1, int32_t in_dtype, int32_t T,
                      int32_t d_model, int32_t d_ff, void *h, int32_t h_dtype, void *stream) {
  if (!b1 || (T > 0 && !h)) return TWELL_ERR_ARG;
  if (!dtype_ok(h_dtype)) return TWELL_ERR_ARG;
  int st = check_ffn_args(x, w1t, nullptr, in_dtype, T, d_model, d_ff);
  if (st) return st;
  if (!al16(h) || !al4(b1)) return TWELL_ERR_ALIGN;
  if (T == 0) return TWELL_OK;
  TW_TRY(launch_up_dense(in_dtype == TWELL_BF16, x, w1t, b1, T, d_ff, d_model, T, nullptr, nullptr, h,
                         h_dtype == TWELL_BF16, 1, S(stream)));
  return TWELL_OK;
}

size_t twell_ffn_bwd_workspace_bytes(int32_t T, int32_t d_model, int32_t d_ff, int32_t in_dtype,
                                     const twell_matrix_t *h) {
  if (!h || T < 0 || d_model <= 0 || d_ff <= 0 || h->tile_w <= 0 || h->slots <= 0 || h->ovf_cap < 0) return 0;
  if (!dtype_ok(in_dtype)) return 0;
  const size_t nz = bwd_entry_capacity(T, d_ff, d_ff / h->tile_w, h->slots, h->ovf_cap);
  return bwd_workspace_bytes(T, d_model, d_ff, nz, in_dtype == TWELL_BF16);
}

size_t twell_ffn_bwd_workspace_bytes_nnz(int32_t T, int32_t d_model, int32_t d_ff, int32_t in_dtype,
                                         const twell_matrix_t *h, int64_t nnz) {
  if (!h || T < 0 || d_model <= 0 || d_ff <= 0 || h->tile_w <= 0 || h->slots <= 0 || h->ovf_cap < 0 || nnz < 0)
    return 0;
  if (!dtype_ok(in_dtype)) return 0;
  const size_t cap = bwd_entry_capacity(T, d_ff, d_ff / h->tile_w, h->slots, h->ovf_cap);
  return bwd_workspace_bytes(T, d_model, d_ff, (size_t)nnz < cap ? (size_t)nnz : cap, in_dtype == TWELL_BF16);
}

int twell_ffn_bwd(const void *x, const void *w1t, const void *w2, int32_t in_dtype, int32_t T,
                  int32_t d_model, int32_t d_ff, const twell_matrix_t *h, const void *dy, float l1_coef,
                  float *dx, float *dw1t, float *dw2, float *db1, void *workspace, size_t workspace_bytes,
                  void *stream) {
  if (!h || !w2 || !dw1t || !dw2 || !workspace) return TWELL_ERR_ARG;
  if (T > 0 && (!dy || !dx)) return TWELL_ERR_ARG;
  int st = check_ffn_args(x, w1t, w2, in_dtype, T, d_model, d_ff);
  if (st) return st;
  st = check_matrix(h, false, false, true);
  if (st) return st;
  if (h->rows != T || h->cols != d_ff) return TWELL_ERR_SHAPE;
  if (!al16(dy) || !al16(dx) || !al16(dw1t) || !al16(dw2) || !al4(db1) || !al16(workspace)) return TWELL_ERR_ALIGN;
  // unit masks of a 32-token block live in LDS (4 bytes per unit)
  if (d_ff > 16384) return TWELL_ERR_UNSUPPORTED;
  // the workspace holds `nz` entries (all of h's capacity if it is that large); whether the
  // call's actual entries fit is checked on the device
  const size_t cap = bwd_entry_capacity(T, d_ff, d_ff / h->tile_w, h->slots, h->ovf_cap);
  const size_t nz = bwd_fit_entries(T, d_model, d_ff, workspace_bytes, cap, in_dtype == TWELL_BF16);
  if (nz == SIZE_MAX) return TWELL_ERR_WORKSPACE;
  BwdArgs a;
  a.nz = nz;
  a.h = in_of(h);
  a.x = x; a.w1t = w1t; a.w2 = w2; a.dy = dy;
  a.l1 = l1_coef;
  a.dx = dx; a.dw1t = dw1t; a.dw2 = dw2; a.db1 = db1;
  a.ws = workspace;
  a.d = d_model;
  a.bf16 = in_dtype == TWELL_BF16;
  a.cap = h->ovf_cap;
  TW_TRY(launch_bwd(a, S(stream)));
  return TWELL_OK;
}

int twell_ffn_bwd_noalloc(const void *x, const void *w1t, const void *w2, int32_t in_dtype, int32_t T,
                          int32_t d_model, int32_t d_ff, const twell_matrix_t *h, const void *dy, float l1_coef,
                          float *dx, float *dw1t, float *dw2, float *db1, void *stream) {
  if (!h) return TWELL_ERR_ARG;
  // the size check comes first, so that a problem beyond the fixed scratch is refused before
  // any device lookup
  if (T >= 0 && d_model > 0 && d_ff > 0 && dtype_ok(in_dtype) && h->tile_w > 0 && h->slots > 0 && h->ovf_cap >= 0 &&
      twell_ffn_bwd_workspace_bytes(T, d_model, d_ff, in_dtype, h) > (size_t)TWELL_NOALLOC_SCRATCH_BYTES)
    return TWELL_ERR_WORKSPACE;
  void *ws = scratch_on_current_device();
  if (!ws) return TWELL_ERR_HIP;
  return twell_ffn_bwd(x, w1t, w2, in_dtype, T, d_model, d_ff, h, dy, l1_coef, dx, dw1t, dw2, db1, ws,
                       (size_t)TWELL_NOALLOC_SCRATCH_BYTES, stream);
}

int nm_prune(const void *h, int32_t dtype, int32_t T, int32_t d_ff, int32_t n, int32_t m, void *vals,
             uint8_t *idx, void *stream) {
  if ((T > 0 && (!h || !vals || !idx))) return TWELL_ERR_ARG;
  if (!dtype_ok(dtype)) return TWELL_ERR_ARG;
  if (T < 0 || d_ff <= 0) return TWELL_ERR_SHAPE;
  if (!((n == 2 && m == 4) || (n == 4 && m == 8) || (n == 8 && m == 16) || (n == 16 && m == 32)))
    return TWELL_ERR_SHAPE;
  if (d_ff % m) return TWELL_ERR_SHAPE;
  if (!al16(h) || !al16(vals) || !al16(idx)) return TWELL_ERR_ALIGN;
  TW_TRY(launch_nm_prune(h, dtype == TWELL_BF16, T, d_ff, n, m, vals, idx, S(stream)));
  return TWELL_OK;
}

int ffn_up_relu_nm(const void *x, const void *w1t, const float *b1, int32_t in_dtype, int32_t T, int32_t d_model,
                   int32_t d_ff, int32_t n, int32_t m, void *vals, uint8_t *idx, void *stream) {
  if (!b1 || (T > 0 && (!vals || !idx))) return TWELL_ERR_ARG;
  int st = check_ffn_args(x, w1t, nullptr, in_dtype, T, d_model, d_ff);
  if (st) return st;
  if (!((n == 2 && m == 4) || (n == 4 && m == 8) || (n == 8 && m == 16) || (n == 16 && m == 32)))
    return TWELL_ERR_SHAPE;
  if (d_ff % m) return TWELL_ERR_SHAPE;
  if (!al4(b1) || !al16(vals) || !al16(idx)) return TWELL_ERR_ALIGN;
  if (T == 0) return TWELL_OK;
  TW_TRY(launch_up_nm(in_dtype == TWELL_BF16, x, w1t, b1, T, d_ff, d_model, n, m, vals, idx, S(stream)));
  return TWELL_OK;
}

int nm_ffn_down(const void *vals, const uint8_t *idx, int32_t dtype, int32_t T, int32_t d_ff, int32_t n,
                int32_t m, const void *w2, int32_t d_model, void *y, int32_t y_dtype, void *stream) {
  if (!w2 || (T > 0 && (!vals || !idx || !y))) return TWELL_ERR_ARG;
  if (!dtype_ok(dtype) || !dtype_ok(y_dtype)) return TWELL_ERR_ARG;
  if (T < 0 || d_ff <= 0 || d_model <= 0) return TWELL_ERR_SHAPE;
  if (!((n == 8 && m == 16) || (n == 16 && m == 32))) {
    if ((n == 2 && m == 4) || (n == 4 && m == 8)) return TWELL_ERR_UNSUPPORTED;
    return TWELL_ERR_SHAPE;
  }
  if (dtype != TWELL_BF16) return TWELL_ERR_UNSUPPORTED;
  if (d_ff % 32 || d_model % 8) return TWELL_ERR_SHAPE;
  if (!al16(vals) || !al16(idx) || !al16(w2) || !al16(y)) return TWELL_ERR_ALIGN;
  if ((size_t)d_model * d_ff * 2 >= ((size_t)1 << 31) || d_ff >= (1 << 23)) return TWELL_ERR_UNSUPPORTED;
  TW_TRY(launch_nm_down(vals, idx, T, d_ff, n, m, w2, d_model, y, y_dtype == TWELL_BF16, S(stream)));
  return TWELL_OK;
}

int twell_row_max_histogram(const twell_matrix_t *h, int32_t *hist, void *stream) {
  if (!hist) return TWELL_ERR_ARG;
  int st = check_matrix(h, false, false, true);
  if (st) return st;
  if (!al4(hist)) return TWELL_ERR_ALIGN;
  TW_TRY(launch_rowmax_hist(h->counts, h->rows, h->cols / h->tile_w, h->tile_w, hist, S(stream)));
  return TWELL_OK;
}

size_t twell_stash_bytes(int32_t rows, int32_t cols, int32_t tile_w, int32_t slots, int32_t n_ovf,
                         int32_t val_dtype) {
  if (rows < 0 || cols <= 0 || tile_w <= 0 || cols % tile_w || slots <= 0 || n_ovf < 0 || !dtype_ok(val_dtype))
    return 0;
  const size_t vb = val_dtype == TWELL_BF16 ? 2 : 4;
  const size_t cells = (size_t)rows * (size_t)(cols / tile_w);
  return cells * 4 + cells * (size_t)slots * (4 + vb) + (size_t)rows * 4 + (size_t)n_ovf * (4 + (size_t)cols * vb);
}

int twell_choose_slots(const int32_t *hist, int32_t tile_w, int32_t rows, int32_t cols, int32_t ovf_cap,
                       int32_t val_dtype, size_t *stash_bytes) {
  if (!hist || !dtype_ok(val_dtype)) return TWELL_ERR_ARG;
  if ((tile_w != 64 && tile_w != 128) || rows < 0 || cols <= 0 || cols % tile_w || ovf_cap < 0)
    return TWELL_ERR_SHAPE;
  int best = TWELL_ERR_OVF_CAPACITY;
  size_t best_bytes = 0;
  const int smax = tile_w < 64 ? tile_w : 64;
  for (int S = 1; S <= smax; ++S) {
    long long n_ovf = 0;
    for (int m = S + 1; m <= tile_w; ++m) n_ovf += hist[m];
    if (n_ovf > ovf_cap) continue;
    const size_t b = twell_stash_bytes(rows, cols, tile_w, S, (int32_t)n_ovf, val_dtype);
    if (best < 0 || b < best_bytes) {
      best = S;
      best_bytes = b;
    }
  }
  if (stash_bytes) *stash_bytes = best > 0 ? best_bytes : 0;
  return best;
}

int twell_row_nnz_histogram(const twell_matrix_t *h, int32_t *hist, int32_t nbins, void *stream) {
  if (!hist) return TWELL_ERR_ARG;
  int st = check_matrix(h, false, false, true);
  if (st) return st;
  if (nbins < 2) return TWELL_ERR_SHAPE;
  if (!al4(hist)) return TWELL_ERR_ALIGN;
  TW_TRY(launch_row_nnz_hist(h->counts, h->rows, h->cols / h->tile_w, nbins, hist, S(stream)));
  return TWELL_OK;
}

int twell_choose_row_ell_width(const int32_t *hist, int32_t nbins, int32_t rows, int32_t cols, int32_t ovf_cap,
                               int32_t val_dtype, size_t *stash_bytes) {
  if (!hist || !dtype_ok(val_dtype)) return TWELL_ERR_ARG;
  if (nbins < 3 || rows < 0 || cols <= 0 || ovf_cap < 0) return TWELL_ERR_SHAPE;
  // rows with more than N entries overflow; the last bin holds every row of nbins - 1 or more
  int best = TWELL_ERR_OVF_CAPACITY;
  size_t best_bytes = 0;
  long long above = 0;
  for (int m = 0; m < nbins; ++m) above += hist[m];
  const int nmax = nbins - 2 < cols ? nbins - 2 : cols;
  for (int N = 0; N <= nmax; ++N) {
    above -= hist[N];                          // rows with more than N entries
    if (N < 1 || above > ovf_cap) continue;
    const size_t b = twell_stash_bytes(rows, cols, cols, N, (int32_t)above, val_dtype);
    if (best < 0 || b < best_bytes) {
      best = N;
      best_bytes = b;
    }
  }
  if (stash_bytes) *stash_bytes = best > 0 ? best_bytes : 0;
  return best;
}

int twell_to_row_ell(const twell_matrix_t *src, twell_matrix_t *dst, void *stream) {
  int st = check_matrix(src, false);
  if (st) return st;
  st = check_matrix(dst, true, false, true);
  if (st) return st;
  if (dst->rows != src->rows || dst->cols != src->cols || dst->tile_w != dst->cols) return TWELL_ERR_SHAPE;
  if (src->val_dtype == TWELL_F32 && dst->val_dtype == TWELL_BF16) return TWELL_ERR_UNSUPPORTED;
  if (dst->cols > 16384) return TWELL_ERR_UNSUPPORTED;
  TW_TRY(launch_to_row_ell(in_of(src), out_of(dst), dst->slots, dst->ovf_cap, dst->ovf_n, dst->ovf_rows, dst->ovf_slot,
                           dst->ovf_dense, S(stream)));
  return TWELL_OK;
}

int twell_sync_status(const twell_matrix_t *h, void *stream) {
  if (!h || !h->ovf_n) return TWELL_ERR_ARG;
  if (hipStreamSynchronize(S(stream)) != hipSuccess) return TWELL_ERR_HIP;
  int32_t n = 0;
  if (hipMemcpy(&n, h->ovf_n, sizeof(n), hipMemcpyDeviceToHost) != hipSuccess) return TWELL_ERR_HIP;
  return n > h->ovf_cap ? TWELL_ERR_OVF_CAPACITY : TWELL_OK;
}

}  // extern "C"
