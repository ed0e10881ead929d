// The C ABI of libquip: argument validation on the host (before anything is
// enqueued), dispatch to the kernels, status strings and per-thread messages.
#include <cmath>
#include <cstring>
#include <string>

#include "common.h"

namespace quip {

// implemented in the other translation units
quip_status hessian_accumulate(const float* X, int64_t N, int64_t n, int64_t ldx, float* H,
                               int64_t ldh, bool accumulate, float* P, size_t P_floats,
                               hipStream_t s);
quip_status hessian_finalize(float* H, int64_t n, int64_t ldh, int64_t N_total, float alpha,
                             double* scratch, hipStream_t s);
quip_status kron_apply(const float* A, float* out, int64_t rows, int64_t cols, int64_t ld,
                       const float* F1, int64_t p, const float* F2, int64_t q, bool left,
                       bool inverse, void* ws, size_t ws_bytes, hipStream_t s);
size_t kron_workspace_bytes(int64_t rows, int64_t cols);
quip_status ldl_factor(const float* H, int64_t n, int64_t ldh, int g, float* U, float* D,
                       int32_t* info, void* ws, size_t ws_bytes, hipStream_t s);
size_t ldl_workspace_bytes(int64_t n);
void timing_enable(bool on);
quip_status timing_reset();
quip_status timing_report(std::string& out);
quip_status ldlq_run(const float* W, int64_t m, int64_t n, int64_t ldw, const float* U,
                     const float* D, int g, int64_t B, const quip_quantizer& q, float* scales,
                     void* codes, float* What, const float* codebook, double* row_loss,
                     double* loss, void* ws, size_t ws_bytes, hipStream_t s);
size_t ldlq_workspace_bytes(int64_t m, int64_t n, int g, int64_t B, const quip_quantizer& q);
quip_status scales_run(const float* W, int64_t m, int64_t n, int64_t ldw, const quip_quantizer& q,
                       float* scales, void* mse_out, const float* codebook, void* ws,
                       size_t ws_bytes, hipStream_t s);
size_t scales_workspace_bytes(int64_t m, int64_t n, const quip_quantizer& q);
size_t loss_workspace_bytes(int64_t m, int64_t n);
quip_status proxy_loss(const float* W, const float* What, int64_t m, int64_t n, int64_t ld,
                       const float* H, int64_t ldh, double* loss, void* ws, size_t ws_bytes,
                       hipStream_t s);

namespace {
thread_local std::string g_last_error;
}

void set_error(const std::string& msg) { g_last_error = msg; }
const char* last_error_cstr() { return g_last_error.c_str(); }
void clear_error() { g_last_error.clear(); }

quip_status fail(quip_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

quip_status launch_check(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(QUIP_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return QUIP_OK;
}

}  // namespace quip

using namespace quip;

namespace {

quip_status check_ws(void* ws, size_t have, size_t need, const char* who) {
  if (need == 0) return QUIP_OK;
  if (!ws) return fail(QUIP_ERR_WORKSPACE, std::string(who) + ": workspace is null");
  if (reinterpret_cast<uintptr_t>(ws) & 255)
    return fail(QUIP_ERR_WORKSPACE, std::string(who) + ": workspace must be 256-byte aligned");
  if (have < need)
    return fail(QUIP_ERR_WORKSPACE, std::string(who) + ": workspace too small (need " +
                                        std::to_string(need) + " bytes)");
  return QUIP_OK;
}

quip_status check_matrix(const void* p, int64_t rows, int64_t cols, int64_t ld, const char* who,
                         const char* name) {
  if (!p) return fail(QUIP_ERR_ARG, std::string(who) + ": " + name + " is null");
  if (rows <= 0 || cols <= 0)
    return fail(QUIP_ERR_ARG, std::string(who) + ": " + name + " must have positive sizes");
  if (ld < cols)
    return fail(QUIP_ERR_ARG, std::string(who) + ": leading dimension of " + name +
                                  " is smaller than its number of columns");
  return QUIP_OK;
}

quip_status check_quantizer(const quip_quantizer* q, int64_t n, const float* codebook,
                            const char* who) {
  if (!q) return fail(QUIP_ERR_ARG, std::string(who) + ": quantizer is null");
  if (q->n_cand < 2 || q->n_cand > 64)
    return fail(QUIP_ERR_ARG, std::string(who) + ": n_cand must be in [2, 64]");
  if (q->scale_mode != QUIP_SCALE_COMPUTE && q->scale_mode != QUIP_SCALE_GIVEN)
    return fail(QUIP_ERR_ARG, std::string(who) + ": bad scale_mode");
  if (q->kind == QUIP_Q_UNIFORM) {
    if (q->bits < 1) return fail(QUIP_ERR_ARG, std::string(who) + ": bits must be >= 1");
    if (q->bits > 8)
      return fail(QUIP_ERR_UNSUPPORTED, std::string(who) + ": more than 8 bits per weight");
    return QUIP_OK;
  }
  if (q->kind == QUIP_Q_E8) {
    if (q->bits != 2) return fail(QUIP_ERR_ARG, std::string(who) + ": the E8 codebook is 2 bits per weight");
    if (!codebook) return fail(QUIP_ERR_ARG, std::string(who) + ": E8 needs the codebook");
    if (n % 8) return fail(QUIP_ERR_SHAPE, std::string(who) + ": E8 needs n % 8 == 0");
    return QUIP_OK;
  }
  return fail(QUIP_ERR_ARG, std::string(who) + ": bad quantizer kind");
}

quip_status rht_validate(const float* A, float* out, int64_t rows, int64_t cols, int64_t ld,
                         const float* signs, int side, const char* who) {
  QUIP_TRY(check_matrix(A, rows, cols, ld, who, "A"));
  if (!out) return fail(QUIP_ERR_ARG, std::string(who) + ": out is null");
  if (!signs) return fail(QUIP_ERR_ARG, std::string(who) + ": signs is null");
  if (!aligned16(signs)) return fail(QUIP_ERR_ARG, std::string(who) + ": signs must be 16-byte aligned");
  if (side != QUIP_LEFT && side != QUIP_RIGHT) return fail(QUIP_ERR_ARG, std::string(who) + ": bad side");
  int64_t d = side == QUIP_LEFT ? rows : cols;
  if (!is_pow2(d) || d < 2 || d > 16384)
    return fail(QUIP_ERR_SHAPE, std::string(who) + ": transform length must be a power of two in [2, 16384]");
  return QUIP_OK;
}

quip_status rht_dispatch(const float* A, float* out, int64_t rows, int64_t cols, int64_t ld,
                         const float* signs, int side, bool inverse, hipStream_t s) {
  if (side == QUIP_RIGHT) return rht_rows(A, out, rows, cols, ld, signs, inverse, s);
  return rht_cols(A, out, rows, cols, ld, signs, inverse, s);
}

}  // namespace

extern "C" {

int32_t quip_version(void) { return 1 * 10000 + 0 * 100 + 0; }

const char* quip_status_string(quip_status st) {
  switch (st) {
    case QUIP_OK: return "QUIP_OK";
    case QUIP_ERR_ARG: return "QUIP_ERR_ARG";
    case QUIP_ERR_SHAPE: return "QUIP_ERR_SHAPE";
    case QUIP_ERR_NOT_PD: return "QUIP_ERR_NOT_PD";
    case QUIP_ERR_HIP: return "QUIP_ERR_HIP";
    case QUIP_ERR_UNSUPPORTED: return "QUIP_ERR_UNSUPPORTED";
    case QUIP_ERR_WORKSPACE: return "QUIP_ERR_WORKSPACE";
  }
  return "QUIP_ERR_UNKNOWN";
}

const char* quip_last_error(void) { return last_error_cstr(); }

quip_status quip_hessian_workspace(int64_t N, int64_t n, size_t* bytes) {
  clear_error();
  if (!bytes) return fail(QUIP_ERR_ARG, "quip_hessian_workspace: null pointer");
  if (N < 0 || n <= 0) return fail(QUIP_ERR_ARG, "quip_hessian_workspace: need N >= 0 and n > 0");
  *bytes = N > 0 ? gemm_upper_tail_floats(n, N) * sizeof(float) : 0;
  return QUIP_OK;
}

quip_status quip_hessian(const float* X, int64_t N, int64_t n, int64_t ldx, float* H, int64_t ldh,
                         int accumulate, void* ws, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  if (N < 0 || n <= 0) return fail(QUIP_ERR_ARG, "quip_hessian: need N >= 0 and n > 0");
  if (N > 0) QUIP_TRY(check_matrix(X, N, n, ldx, "quip_hessian", "X"));
  QUIP_TRY(check_matrix(H, n, n, ldh, "quip_hessian", "H"));
  if (ws && (reinterpret_cast<uintptr_t>(ws) & 15))
    return fail(QUIP_ERR_ARG, "quip_hessian: workspace must be 16-byte aligned");
  return hessian_accumulate(X, N, n, ldx, H, ldh, accumulate != 0, static_cast<float*>(ws),
                            ws ? ws_bytes / sizeof(float) : 0, stream);
}

quip_status quip_hessian_finalize(float* H, int64_t n, int64_t ldh, int64_t N_total, float alpha,
                                  void* ws, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  QUIP_TRY(check_matrix(H, n, n, ldh, "quip_hessian_finalize", "H"));
  if (N_total <= 0) return fail(QUIP_ERR_ARG, "quip_hessian_finalize: N_total must be positive");
  if (!(alpha >= 0.f) || !std::isfinite(alpha))
    return fail(QUIP_ERR_ARG, "quip_hessian_finalize: alpha must be finite and >= 0");
  QUIP_TRY(check_ws(ws, ws_bytes, 256, "quip_hessian_finalize"));
  return hessian_finalize(H, n, ldh, N_total, alpha, static_cast<double*>(ws), stream);
}

quip_status quip_rht(const float* A, float* out, int64_t rows, int64_t cols, int64_t ld,
                     const float* signs, quip_side side, hipStream_t stream) {
  clear_error();
  QUIP_TRY(rht_validate(A, out, rows, cols, ld, signs, side, "quip_rht"));
  return rht_dispatch(A, out, rows, cols, ld, signs, side, false, stream);
}

quip_status quip_rht_inv(const float* A, float* out, int64_t rows, int64_t cols, int64_t ld,
                         const float* signs, quip_side side, hipStream_t stream) {
  clear_error();
  QUIP_TRY(rht_validate(A, out, rows, cols, ld, signs, side, "quip_rht_inv"));
  return rht_dispatch(A, out, rows, cols, ld, signs, side, true, stream);
}

quip_status quip_rht2(const float* A, float* out, int64_t rows, int64_t cols, int64_t ld,
                      const float* signs_left, const float* signs_right, hipStream_t stream) {
  clear_error();
  QUIP_TRY(rht_validate(A, out, rows, cols, ld, signs_left, QUIP_LEFT, "quip_rht2"));
  QUIP_TRY(rht_validate(A, out, rows, cols, ld, signs_right, QUIP_RIGHT, "quip_rht2"));
  QUIP_TRY(rht_rows(A, out, rows, cols, ld, signs_right, false, stream, /*last_pass=*/false));
  return rht_cols(out, out, rows, cols, ld, signs_left, false, stream);
}

quip_status quip_rht2_inv(const float* A, float* out, int64_t rows, int64_t cols, int64_t ld,
                          const float* signs_left, const float* signs_right, hipStream_t stream) {
  clear_error();
  QUIP_TRY(rht_validate(A, out, rows, cols, ld, signs_left, QUIP_LEFT, "quip_rht2_inv"));
  QUIP_TRY(rht_validate(A, out, rows, cols, ld, signs_right, QUIP_RIGHT, "quip_rht2_inv"));
  QUIP_TRY(rht_cols(A, out, rows, cols, ld, signs_left, true, stream));
  return rht_rows(out, out, rows, cols, ld, signs_right, true, stream);
}

quip_status quip_kron_orth_workspace(int64_t rows, int64_t cols, size_t* bytes) {
  clear_error();
  if (!bytes) return fail(QUIP_ERR_ARG, "quip_kron_orth_workspace: bytes is null");
  if (rows <= 0 || cols <= 0) return fail(QUIP_ERR_ARG, "quip_kron_orth_workspace: sizes must be positive");
  *bytes = kron_workspace_bytes(rows, cols);
  return QUIP_OK;
}

static quip_status kron_common(const float* A, float* out, int64_t rows, int64_t cols, int64_t ld,
                               const float* F1, int64_t p, const float* F2, int64_t q,
                               quip_side side, void* ws, size_t ws_bytes, bool inverse,
                               hipStream_t stream, const char* who) {
  clear_error();
  QUIP_TRY(check_matrix(A, rows, cols, ld, who, "A"));
  if (!out || !F1 || !F2) return fail(QUIP_ERR_ARG, std::string(who) + ": null pointer");
  if (side != QUIP_LEFT && side != QUIP_RIGHT) return fail(QUIP_ERR_ARG, std::string(who) + ": bad side");
  if (p < 1 || q < 1) return fail(QUIP_ERR_SHAPE, std::string(who) + ": factor sizes must be >= 1");
  const int64_t d = side == QUIP_LEFT ? rows : cols;
  if (p * q != d) return fail(QUIP_ERR_SHAPE, std::string(who) + ": p*q must equal the transformed dimension");
  if (side == QUIP_RIGHT && rows > 65535 && ld != cols)
    return fail(QUIP_ERR_UNSUPPORTED, std::string(who) + ": more than 65535 rows needs ld == cols");
  if (side == QUIP_LEFT && (p > 65535 || q > 65535))
    return fail(QUIP_ERR_UNSUPPORTED, std::string(who) + ": factor larger than 65535");
  QUIP_TRY(check_ws(ws, ws_bytes, kron_workspace_bytes(rows, cols), who));
  return kron_apply(A, out, rows, cols, ld, F1, p, F2, q, side == QUIP_LEFT, inverse, ws, ws_bytes,
                    stream);
}

quip_status quip_kron_orth(const float* A, float* out, int64_t rows, int64_t cols, int64_t ld,
                           const float* F1, int64_t p, const float* F2, int64_t q, quip_side side,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
  return kron_common(A, out, rows, cols, ld, F1, p, F2, q, side, ws, ws_bytes, false, stream,
                     "quip_kron_orth");
}

quip_status quip_kron_orth_inv(const float* A, float* out, int64_t rows, int64_t cols, int64_t ld,
                               const float* F1, int64_t p, const float* F2, int64_t q,
                               quip_side side, void* ws, size_t ws_bytes, hipStream_t stream) {
  return kron_common(A, out, rows, cols, ld, F1, p, F2, q, side, ws, ws_bytes, true, stream,
                     "quip_kron_orth_inv");
}

quip_status quip_ldl_workspace(int64_t n, int64_t g, size_t* bytes) {
  clear_error();
  if (!bytes) return fail(QUIP_ERR_ARG, "quip_ldl_workspace: bytes is null");
  if (g != 1 && g != 8) return fail(QUIP_ERR_ARG, "quip_ldl_workspace: g must be 1 or 8");
  if (n <= 0 || n % g) return fail(QUIP_ERR_SHAPE, "quip_ldl_workspace: need n > 0 and n % g == 0");
  *bytes = ldl_workspace_bytes(n);
  return QUIP_OK;
}

quip_status quip_ldl(const float* H, int64_t n, int64_t ldh, int64_t g, float* U, float* D,
                     int32_t* info, void* ws, size_t ws_bytes, hipStream_t stream) {
  clear_error();
  if (g != 1 && g != 8) return fail(QUIP_ERR_ARG, "quip_ldl: g must be 1 or 8");
  if (n <= 0 || n % g) return fail(QUIP_ERR_SHAPE, "quip_ldl: need n > 0 and n % g == 0");
  QUIP_TRY(check_matrix(H, n, n, ldh, "quip_ldl", "H"));
  if (!U || !D || !info) return fail(QUIP_ERR_ARG, "quip_ldl: null output pointer");
  QUIP_TRY(check_ws(ws, ws_bytes, ldl_workspace_bytes(n), "quip_ldl"));
  return ldl_factor(H, n, ldh, int(g), U, D, info, ws, ws_bytes, stream);
}

quip_status quip_scales_workspace(int64_t m, int64_t n, const quip_quantizer* q, size_t* bytes) {
  clear_error();
  if (!bytes || !q) return fail(QUIP_ERR_ARG, "quip_scales_workspace: null pointer");
  if (m <= 0 || n <= 0) return fail(QUIP_ERR_ARG, "quip_scales_workspace: sizes must be positive");
  *bytes = scales_workspace_bytes(m, n, *q);
  return QUIP_OK;
}

quip_status quip_scales(const float* W, int64_t m, int64_t n, int64_t ldw, const quip_quantizer* q,
                        float* scales, void* mse_out, const float* codebook, void* ws,
                        size_t ws_bytes, hipStream_t stream) {
  clear_error();
  QUIP_TRY(check_matrix(W, m, n, ldw, "quip_scales", "W"));
  QUIP_TRY(check_quantizer(q, n, codebook, "quip_scales"));
  if (!scales) return fail(QUIP_ERR_ARG, "quip_scales: scales is null");
  QUIP_TRY(check_ws(ws, ws_bytes, scales_workspace_bytes(m, n, *q), "quip_scales"));
  return scales_run(W, m, n, ldw, *q, scales, mse_out, codebook, ws, ws_bytes, stream);
}

quip_status quip_ldlq_workspace(int64_t m, int64_t n, int64_t g, int64_t B,
                                const quip_quantizer* q, size_t* bytes) {
  clear_error();
  if (!bytes || !q) return fail(QUIP_ERR_ARG, "quip_ldlq_workspace: null pointer");
  if (m <= 0 || n <= 0 || B <= 0) return fail(QUIP_ERR_ARG, "quip_ldlq_workspace: sizes must be positive");
  *bytes = ldlq_workspace_bytes(m, n, int(g), B, *q);
  return QUIP_OK;
}

quip_status quip_ldlq(const float* W, int64_t m, int64_t n, int64_t ldw, const float* U,
                      const float* D, int64_t g, int64_t B, const quip_quantizer* q,
                      float* scales, void* codes, float* What, const float* codebook,
                      double* row_loss, double* loss, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  clear_error();
  QUIP_TRY(check_matrix(W, m, n, ldw, "quip_ldlq", "W"));
  QUIP_TRY(check_quantizer(q, n, codebook, "quip_ldlq"));
  if (!U || !scales || !codes) return fail(QUIP_ERR_ARG, "quip_ldlq: null pointer");
  if (g != 1 && g != 8) return fail(QUIP_ERR_ARG, "quip_ldlq: g must be 1 or 8");
  if ((q->kind == QUIP_Q_UNIFORM) != (g == 1))
    return fail(QUIP_ERR_ARG, "quip_ldlq: the scalar grid needs g = 1 and the E8 codebook g = 8");
  if (n % g) return fail(QUIP_ERR_SHAPE, "quip_ldlq: n must be a multiple of g");
  if (B < 8 || B > 4096 || B % g) return fail(QUIP_ERR_SHAPE, "quip_ldlq: B must be a multiple of g in [8, 4096]");
  if ((q->kind == QUIP_Q_E8 || row_loss || loss) && !D) return fail(QUIP_ERR_ARG, "quip_ldlq: D is null");
  QUIP_TRY(check_ws(ws, ws_bytes, ldlq_workspace_bytes(m, n, int(g), B, *q), "quip_ldlq"));
  return ldlq_run(W, m, n, ldw, U, D, int(g), B, *q, scales, codes, What, codebook, row_loss, loss,
                  ws, ws_bytes, stream);
}

quip_status quip_pack_codes(const uint8_t* codes, int64_t m, int64_t n, int64_t ldc, int32_t bits,
                            uint8_t* packed, hipStream_t stream) {
  clear_error();
  QUIP_TRY(check_matrix(codes, m, n, ldc, "quip_pack_codes", "codes"));
  if (!packed) return fail(QUIP_ERR_ARG, "quip_pack_codes: packed is null");
  if (bits < 1 || bits > 8) return fail(QUIP_ERR_ARG, "quip_pack_codes: bits must be in [1, 8]");
  return pack_codes(codes, m, n, ldc, bits, packed, stream);
}

quip_status quip_packed_row_bytes(int64_t n, int32_t bits, int64_t* bytes) {
  clear_error();
  if (!bytes) return fail(QUIP_ERR_ARG, "quip_packed_row_bytes: bytes is null");
  if (n <= 0) return fail(QUIP_ERR_ARG, "quip_packed_row_bytes: n must be positive");
  if (bits < 1 || bits > 8) return fail(QUIP_ERR_ARG, "quip_packed_row_bytes: bits must be in [1, 8]");
  *bytes = (n * code_container_bits(bits) + 7) / 8;
  return QUIP_OK;
}

quip_status quip_qmatvec_rht_workspace(int64_t m, int64_t n, size_t* bytes) {
  clear_error();
  if (!bytes) return fail(QUIP_ERR_ARG, "quip_qmatvec_rht_workspace: bytes is null");
  if (m <= 0 || n <= 0) return fail(QUIP_ERR_ARG, "quip_qmatvec_rht_workspace: sizes must be positive");
  *bytes = qmatvec_workspace_bytes(m, n);
  return QUIP_OK;
}

quip_status quip_qmatvec_rht(const uint8_t* packed, int64_t m, int64_t n, int32_t bits,
                             const float* scales, const float* signs_left,
                             const float* signs_right, const float* x, float* y, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  clear_error();
  const char* who = "quip_qmatvec_rht";
  if (!packed || !scales || !signs_left || !signs_right || !x || !y)
    return fail(QUIP_ERR_ARG, std::string(who) + ": null pointer");
  if (bits < 1 || bits > 8) return fail(QUIP_ERR_ARG, std::string(who) + ": bits must be in [1, 8]");
  if (!is_pow2(m) || m < 2 || m > 16384)
    return fail(QUIP_ERR_SHAPE, std::string(who) + ": m must be a power of two in [2, 16384]");
  if (!is_pow2(n) || n < 1024 || n > 16384)
    return fail(QUIP_ERR_SHAPE, std::string(who) + ": n must be a power of two in [1024, 16384]");
  if (!aligned16(packed) || !aligned16(x) || !aligned16(y) || !aligned16(signs_left) ||
      !aligned16(signs_right))
    return fail(QUIP_ERR_ARG, std::string(who) + ": packed, x, y and the signs must be 16-byte aligned");
  QUIP_TRY(check_ws(ws, ws_bytes, qmatvec_workspace_bytes(m, n), who));
  return qmatvec_rht(packed, m, n, bits, scales, signs_left, signs_right, x, y, ws, ws_bytes,
                     stream);
}

quip_status quip_qmatvec_rht_noalloc(const uint8_t* packed, int64_t m, int64_t n, int32_t bits,
                                     const float* scales, const float* signs_left,
                                     const float* signs_right, const float* x, float* y,
                                     hipStream_t stream) {
  clear_error();
  const char* who = "quip_qmatvec_rht_noalloc";
  if (!packed || !scales || !signs_left || !signs_right || !x || !y)
    return fail(QUIP_ERR_ARG, std::string(who) + ": null pointer");
  if (bits < 1 || bits > 8) return fail(QUIP_ERR_ARG, std::string(who) + ": bits must be in [1, 8]");
  if (!is_pow2(m) || m < 2 || m > 16384)
    return fail(QUIP_ERR_SHAPE, std::string(who) + ": m must be a power of two in [2, 16384]");
  if (!is_pow2(n) || n < 1024 || n > 16384)
    return fail(QUIP_ERR_SHAPE, std::string(who) + ": n must be a power of two in [1024, 16384]");
  if (!aligned16(packed) || !aligned16(x) || !aligned16(y) || !aligned16(signs_left) ||
      !aligned16(signs_right))
    return fail(QUIP_ERR_ARG, std::string(who) + ": packed, x, y and the signs must be 16-byte aligned");
  return qmatvec_rht_noalloc(packed, m, n, bits, scales, signs_left, signs_right, x, y, stream);
}

quip_status quip_permute(const float* A, int64_t lda, float* out, int64_t ldo, int64_t rows,
                         int64_t cols, const int32_t* row_index, const int32_t* col_index,
                         int32_t scatter, hipStream_t stream) {
  clear_error();
  const char* who = "quip_permute";
  if (rows < 0 || cols < 0) return fail(QUIP_ERR_ARG, std::string(who) + ": negative size");
  if (scatter != 0 && scatter != 1) return fail(QUIP_ERR_ARG, std::string(who) + ": scatter must be 0 or 1");
  if (rows == 0 || cols == 0) return QUIP_OK;
  if (!A || !out) return fail(QUIP_ERR_ARG, std::string(who) + ": null matrix");
  if (lda < cols || ldo < cols)
    return fail(QUIP_ERR_ARG, std::string(who) + ": leading dimension smaller than cols");
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(A), o0 = reinterpret_cast<uintptr_t>(out);
  const uintptr_t a1 = a0 + sizeof(float) * size_t((rows - 1) * lda + cols);
  const uintptr_t o1 = o0 + sizeof(float) * size_t((rows - 1) * ldo + cols);
  if (a0 < o1 && o0 < a1) return fail(QUIP_ERR_ARG, std::string(who) + ": A and out overlap");
  if (col_index && cols > permute_max_cols())
    return fail(QUIP_ERR_SHAPE, std::string(who) + ": at most 32768 columns with a column index");
  return permute(A, lda, out, ldo, rows, cols, row_index, col_index, scatter != 0, stream);
}

quip_status quip_peak_copy(const float* src, float* dst, int64_t count, hipStream_t stream) {
  clear_error();
  const char* who = "quip_peak_copy";
  if (count < 0) return fail(QUIP_ERR_ARG, std::string(who) + ": negative count");
  if (count == 0) return QUIP_OK;
  if (!src || !dst) return fail(QUIP_ERR_ARG, std::string(who) + ": null pointer");
  if (!aligned16(src) || !aligned16(dst))
    return fail(QUIP_ERR_ARG, std::string(who) + ": src and dst must be 16-byte aligned");
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  const uintptr_t bytes = sizeof(float) * uintptr_t(count);
  if (s0 < d0 + bytes && d0 < s0 + bytes) return fail(QUIP_ERR_ARG, std::string(who) + ": src and dst overlap");
  return peak_copy(src, dst, count, stream);
}

quip_status quip_peak_compute(int32_t kind, int64_t iters, float* out, double* flops,
                              hipStream_t stream) {
  clear_error();
  const char* who = "quip_peak_compute";
  if (kind < 0 || kind > 2) return fail(QUIP_ERR_ARG, std::string(who) + ": kind must be 0, 1 or 2");
  if (iters <= 0) return fail(QUIP_ERR_ARG, std::string(who) + ": iters must be positive");
  if (!out) return fail(QUIP_ERR_ARG, std::string(who) + ": out is null");
  return peak_compute(kind, iters, out, flops, stream);
}

quip_status quip_diag_order_workspace(int64_t n, size_t* bytes) {
  clear_error();
  if (!bytes) return fail(QUIP_ERR_ARG, "quip_diag_order_workspace: bytes is null");
  if (n <= 0) return fail(QUIP_ERR_ARG, "quip_diag_order_workspace: n must be positive");
  *bytes = diag_order_workspace_bytes(n);
  return QUIP_OK;
}

quip_status quip_diag_order(const float* H, int64_t n, int64_t ldh, int32_t* order, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  clear_error();
  QUIP_TRY(check_matrix(H, n, n, ldh, "quip_diag_order", "H"));
  if (!order) return fail(QUIP_ERR_ARG, "quip_diag_order: order is null");
  QUIP_TRY(check_ws(ws, ws_bytes, diag_order_workspace_bytes(n), "quip_diag_order"));
  return diag_order(H, n, ldh, order, ws, ws_bytes, stream);
}

quip_status quip_tcq_workspace(int64_t rows, int64_t T, int32_t L, size_t* bytes) {
  clear_error();
  if (!bytes) return fail(QUIP_ERR_ARG, "quip_tcq_workspace: bytes is null");
  if (rows <= 0 || T <= 0) return fail(QUIP_ERR_ARG, "quip_tcq_workspace: sizes must be positive");
  if (L < 4 || L > 15) return fail(QUIP_ERR_UNSUPPORTED, "quip_tcq_workspace: L must be in [4, 15]");
  *bytes = tcq_workspace_bytes(rows, T, L);
  return QUIP_OK;
}

quip_status quip_tcq_quantize(const float* X, int64_t rows, int64_t T, int64_t ldx, int32_t L,
                              int32_t k, float scale, uint16_t* states, int64_t lds, float* Xhat,
                              int64_t ldq, float* cost, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  clear_error();
  const char* who = "quip_tcq_quantize";
  QUIP_TRY(check_matrix(X, rows, T, ldx, who, "X"));
  if (!states || !cost) return fail(QUIP_ERR_ARG, std::string(who) + ": states or cost is null");
  if (lds < T || (Xhat && ldq < T))
    return fail(QUIP_ERR_ARG, std::string(who) + ": leading dimension smaller than T");
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(QUIP_ERR_ARG, std::string(who) + ": scale must be finite and positive");
  if (k != 2) return fail(QUIP_ERR_UNSUPPORTED, std::string(who) + ": k must be 2");
  if (L < 4 || L > 15) return fail(QUIP_ERR_UNSUPPORTED, std::string(who) + ": L must be in [4, 15]");
  QUIP_TRY(check_ws(ws, ws_bytes, tcq_workspace_bytes(rows, T, L), who));
  return tcq_quantize(X, rows, T, ldx, L, scale, states, lds, Xhat, ldq, cost, ws, ws_bytes, stream);
}

quip_status quip_proxy_loss_workspace(int64_t m, int64_t n, size_t* bytes) {
  clear_error();
  if (!bytes) return fail(QUIP_ERR_ARG, "quip_proxy_loss_workspace: bytes is null");
  if (m <= 0 || n <= 0) return fail(QUIP_ERR_ARG, "quip_proxy_loss_workspace: sizes must be positive");
  *bytes = loss_workspace_bytes(m, n);
  return QUIP_OK;
}

quip_status quip_proxy_loss(const float* W, const float* What, int64_t m, int64_t n, int64_t ld,
                            const float* H, int64_t ldh, double* loss_dev, void* ws,
                            size_t ws_bytes, hipStream_t stream) {
  clear_error();
  QUIP_TRY(check_matrix(W, m, n, ld, "quip_proxy_loss", "W"));
  QUIP_TRY(check_matrix(What, m, n, ld, "quip_proxy_loss", "What"));
  QUIP_TRY(check_matrix(H, n, n, ldh, "quip_proxy_loss", "H"));
  if (!loss_dev) return fail(QUIP_ERR_ARG, "quip_proxy_loss: loss is null");
  QUIP_TRY(check_ws(ws, ws_bytes, loss_workspace_bytes(m, n), "quip_proxy_loss"));
  return proxy_loss(W, What, m, n, ld, H, ldh, loss_dev, ws, ws_bytes, stream);
}

quip_status quip_timing_enable(int on) {
  clear_error();
  timing_enable(on != 0);
  return QUIP_OK;
}

quip_status quip_timing_reset(void) {
  clear_error();
  return timing_reset();
}

quip_status quip_timing_report(char* buf, size_t len, size_t* needed) {
  clear_error();
  std::string out;
  const quip_status st = timing_report(out);
  if (needed) *needed = out.size() + 1;
  if (buf && len > 0) {
    const size_t k = out.size() < len - 1 ? out.size() : len - 1;
    std::memcpy(buf, out.data(), k);
    buf[k] = 0;
  }
  return st;
}

quip_status quip_e8_codebook(float* host_out) {
  clear_error();
  if (!host_out) return fail(QUIP_ERR_ARG, "quip_e8_codebook: host_out is null");
  e8_build_codebook(host_out);
  return QUIP_OK;
}

}  // extern "C"
