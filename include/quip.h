/*
 * quip.h -- C ABI of libquip, the QuIP-family layer-quantization pass for
 * AMD Instinct MI355X (gfx950).
 *
 * The pass: proxy Hessian H = X^T X / N, damping, incoherence processing
 * (random-sign Hadamard transform or Kronecker product of two orthogonal
 * factors on each side), LDL factorization H = (I+U) D (I+U)^T, per-row or
 * global quantizer scale, LDLQ / BlockLDLQ rounding onto a scalar grid or an
 * E8-lattice codebook, post-processing and the proxy loss.
 *
 * Sources, cited by title and section:
 *   [QuIP]  "QuIP: 2-Bit Quantization of Large Language Models With
 *           Guarantees" (Chee, Cai, Kuleshov, De Sa, 2023).
 *   [QuIP#] "QuIP#: Even Better LLM Quantization with Hadamard Incoherence
 *           and Lattice Codebooks" (Tseng et al., 2024), abstract.
 *   [QTIP]  "QTIP: Quantization with Trellises and Incoherence Processing",
 *           summary page, "Builds on" (BlockLDLQ).
 *
 * Conventions shared by every entry point:
 *   - Array arguments are DEVICE pointers unless the name says host. Matrices
 *     are float32, row-major, with an explicit leading dimension (elements)
 *     that must be >= the number of columns.
 *   - The caller owns all memory: inputs, outputs and workspace. Workspace
 *     sizes come from the quip_*_workspace queries; a workspace must be 256-byte
 *     aligned. The library allocates no device memory and keeps no global
 *     mutable state other than the optional per-kernel timing registry
 *     (quip_timing_*, off by default) and the static scratch array of
 *     quip_qmatvec_rht_noalloc; calls on different streams are independent
 *     (except overlapping calls of quip_qmatvec_rht_noalloc on one GPU).
 *   - Every call only enqueues work on `stream` (asynchronous) and returns at
 *     once. Argument and shape errors are detected on the host before any
 *     launch, and then nothing is enqueued. A failure found on the device (a
 *     non-positive pivot) is written to a caller-provided int32 device word
 *     following LAPACK's `info` convention.
 *   - No C++ exception crosses the ABI. quip_status_string() names a status;
 *     quip_last_error() gives the calling thread's last message.
 */
#ifndef QUIP_H
#define QUIP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QUIP_OK = 0,
  QUIP_ERR_ARG = 1,         /* null pointer, bad leading dimension, bad enum */
  QUIP_ERR_SHAPE = 2,       /* sizes that the operation does not accept */
  QUIP_ERR_NOT_PD = 3,      /* reported through `info`, never returned by a launch */
  QUIP_ERR_HIP = 4,         /* a HIP runtime call failed */
  QUIP_ERR_UNSUPPORTED = 5, /* a valid request this build does not implement */
  QUIP_ERR_WORKSPACE = 6    /* workspace missing, too small or misaligned */
} quip_status;

typedef enum {
  QUIP_LEFT = 0,  /* transform mixes rows:    out = Q A       */
  QUIP_RIGHT = 1  /* transform mixes columns: out = A Q^T     */
} quip_side;

typedef enum {
  QUIP_Q_UNIFORM = 0, /* 2^bits-level midrise grid, one scale per row */
  QUIP_Q_E8 = 1       /* E8 codebook of 65536 points, g = 8, one global scale */
} quip_qkind;

typedef enum {
  QUIP_SCALE_COMPUTE = 0, /* search the scale(s) and write them to `scales` */
  QUIP_SCALE_GIVEN = 1    /* read the scale(s) from `scales` */
} quip_scale_mode;

typedef struct {
  int32_t kind;       /* quip_qkind */
  int32_t bits;       /* QUIP_Q_UNIFORM: 1..8 (2^bits levels); QUIP_Q_E8: must be 2 */
  int32_t n_cand;     /* number of scale candidates searched, 2..64 (32 by default) */
  int32_t scale_mode; /* quip_scale_mode */
} quip_quantizer;

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int32_t quip_version(void);
/* Static string naming a status. */
const char* quip_status_string(quip_status st);
/* The calling thread's last error message ("" after a successful call). */
const char* quip_last_error(void);

/*
 * quip_hessian -- H (+)= X^T X   ([QuIP] "Adaptive Rounding Step": the proxy
 * Hessian is the second moment of the layer inputs).
 *   X: N x n calibration rows (one input vector per row), leading dim ldx.
 *   H: n x n output, leading dim ldh, written in full symmetric storage.
 *   accumulate: 0 overwrites H with X^T X, 1 adds X^T X to H (stream X in
 *   chunks of rows and call quip_hessian_finalize once with the total N).
 *   N may be 0 (H is zeroed, or left as is when accumulating).
 *   ws: optional (may be NULL) 16-byte aligned device workspace of
 *   quip_hessian_workspace() bytes (0 bytes when none is needed). With it,
 *   the output tiles that would otherwise run alone in a last round of
 *   work-groups are split along N and their pieces summed in a fixed order:
 *   the result is deterministic either way, and bitwise the same for every
 *   call with the same sizes and workspace choice.
 * Errors: QUIP_ERR_ARG (null pointer, ldx < n, ldh < n, n <= 0, N < 0,
 *   misaligned ws).
 */
quip_status quip_hessian_workspace(int64_t N, int64_t n, size_t* bytes);
quip_status quip_hessian(const float* X, int64_t N, int64_t n, int64_t ldx, float* H,
                         int64_t ldh, int accumulate, void* ws, size_t ws_bytes,
                         hipStream_t stream);

/*
 * quip_hessian_finalize -- H <- H / N_total + alpha * mean(diag(H / N_total)) * I
 *   ([QuIP] "Experiments / Methods": damping for numerical stability).
 *   In place on the n x n matrix H (leading dim ldh). alpha >= 0.
 *   ws: device workspace of at least 256 bytes (holds partial traces).
 * Errors: QUIP_ERR_ARG (null H, N_total <= 0, alpha < 0 or not finite),
 *   QUIP_ERR_WORKSPACE.
 */
quip_status quip_hessian_finalize(float* H, int64_t n, int64_t ldh, int64_t N_total, float alpha,
                                  void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * quip_rht / quip_rht_inv -- randomized Hadamard transform ([QuIP#] abstract;
 * the orthogonal multiplications of [QuIP] "Incoherence Processing").
 *   With d = rows (LEFT) or cols (RIGHT), S = diag(signs) and
 *   Q = H_d S / sqrt(d), H_d the natural-order Sylvester Hadamard matrix:
 *     quip_rht:     LEFT out = Q A,     RIGHT out = A Q^T
 *     quip_rht_inv: LEFT out = Q^T A,   RIGHT out = A Q
 *   A, out: rows x cols, same leading dim ld; out == A (in place) allowed,
 *   other overlap is not. signs: d floats, each +1 or -1, 16-byte aligned.
 * Errors: QUIP_ERR_ARG (null pointer, ld < cols, bad side, misaligned signs);
 *   QUIP_ERR_SHAPE (d not a power of two, or d > 16384, or d < 2).
 */
quip_status quip_rht(const float* A, float* out, int64_t rows, int64_t cols, int64_t ld,
                     const float* signs, quip_side side, hipStream_t stream);
quip_status quip_rht_inv(const float* A, float* out, int64_t rows, int64_t cols, int64_t ld,
                         const float* signs, quip_side side, hipStream_t stream);

/*
 * quip_rht2 -- both sides at once: out = Q_L A Q_R^T (signs_left: rows floats,
 * signs_right: cols floats), same result as quip_rht LEFT after quip_rht RIGHT.
 * quip_rht2_inv gives Q_L^T A Q_R. out == A allowed.
 * Errors: as quip_rht for each side.
 */
quip_status quip_rht2(const float* A, float* out, int64_t rows, int64_t cols, int64_t ld,
                      const float* signs_left, const float* signs_right, hipStream_t stream);
quip_status quip_rht2_inv(const float* A, float* out, int64_t rows, int64_t cols, int64_t ld,
                          const float* signs_left, const float* signs_right, hipStream_t stream);

/*
 * quip_kron_orth / quip_kron_orth_inv -- multiplication by Q = F1 (x) F2,
 * the Kronecker product of two orthogonal factors ([QuIP] "Introduction" and
 * "Conclusion": pre- and post-processing by a Kronecker product of random
 * orthogonal matrices). Row-major index i = a*q + b.
 *     quip_kron_orth:     LEFT out = Q A,     RIGHT out = A Q^T
 *     quip_kron_orth_inv: LEFT out = Q^T A,   RIGHT out = A Q
 *   F1: p x p row-major (device), F2: q x q row-major (device); p*q must equal
 *   rows (LEFT) or cols (RIGHT). A, out: rows x cols, leading dim ld; out may
 *   equal A. ws: device workspace of quip_kron_orth_workspace() bytes.
 * Errors: QUIP_ERR_ARG, QUIP_ERR_SHAPE (p*q mismatch, p or q < 1),
 *   QUIP_ERR_WORKSPACE.
 */
quip_status quip_kron_orth_workspace(int64_t rows, int64_t cols, size_t* bytes);
quip_status quip_kron_orth(const float* A, float* out, int64_t rows, int64_t cols, int64_t ld,
                           const float* F1, int64_t p, const float* F2, int64_t q, quip_side side,
                           void* ws, size_t ws_bytes, hipStream_t stream);
quip_status quip_kron_orth_inv(const float* A, float* out, int64_t rows, int64_t cols, int64_t ld,
                               const float* F1, int64_t p, const float* F2, int64_t q,
                               quip_side side, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * quip_ldl -- H = (I + U) D (I + U)^T with U strictly upper triangular
 * (g = 1) or strictly block-upper with g x g blocks (g = 8), D diagonal or
 * block diagonal. The factor LDLQ feeds back through ([QuIP] "Adaptive
 * Rounding Step"; block form for BlockLDLQ, [QTIP] "Builds on").
 *   H: n x n symmetric, leading dim ldh; only the upper triangle is read.
 *   U: n x n output (leading dim n); every entry on or below the diagonal
 *      (on or below the diagonal blocks for g = 8) is written as 0.
 *   D: output, n floats (g = 1) or n/8 row-major 8x8 blocks (g = 8).
 *   info: one int32 device word; 0 on success, else 1 + the index of the
 *      first pivot (first column of the first block) found not positive
 *      definite, processing from the last column down; U and D are then
 *      undefined.
 *   ws: device workspace of quip_ldl_workspace() bytes.
 * Errors: QUIP_ERR_ARG (null pointer, ldh < n, g not 1 or 8),
 *   QUIP_ERR_SHAPE (n <= 0, n % g != 0), QUIP_ERR_WORKSPACE.
 */
quip_status quip_ldl_workspace(int64_t n, int64_t g, size_t* bytes);
quip_status quip_ldl(const float* H, int64_t n, int64_t ldh, int64_t g, float* U, float* D,
                     int32_t* info, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * quip_scales -- the quantizer scale(s) without rounding.
 *   UNIFORM: scales[r] for every row r of W: the step among n_cand candidates
 *     s_c = s_max * 16^(-c/(n_cand-1)), s_max = max_j |W_rj| / ((L-1)/2),
 *     minimizing the row's nearest-rounding squared error (ties to the smaller
 *     c; an all-zero row gets 1).
 *   E8: scales[0] = global scale among 0.5 * 4^(c/(n_cand-1)) minimizing the
 *     nearest-codeword squared error of all 8-vectors of the row-normalized
 *     W; scales[1 + r] = root-mean-square of row r (1 for an all-zero row).
 *   W: m x n, leading dim ldw. codebook: 65536 x 8 device floats for E8,
 *   else NULL; any order works, and quip_e8_codebook's order (whose full
 *   shells hold each point's negation in reverse order, checked on the device
 *   every call) lets the search take one member of each pair {c, -c}. mse_out: optional (may be NULL) device output of the squared
 *   error per candidate: m x n_cand (UNIFORM) or n_cand (E8), float64 for E8,
 *   float32 for UNIFORM.
 * Errors: QUIP_ERR_ARG, QUIP_ERR_SHAPE (n % 8 != 0 for E8), QUIP_ERR_WORKSPACE.
 */
quip_status quip_scales_workspace(int64_t m, int64_t n, const quip_quantizer* q, size_t* bytes);
quip_status quip_scales(const float* W, int64_t m, int64_t n, int64_t ldw, const quip_quantizer* q,
                        float* scales, void* mse_out, const float* codebook, void* ws,
                        size_t ws_bytes, hipStream_t stream);

/*
 * quip_ldlq -- LDLQ / BlockLDLQ rounding: columns (groups of g columns) in
 * natural order, W^_K = Q(W_K + (W - W^)_{:,<K} U_{<K,K}) ([QuIP] "Adaptive
 * Rounding Step" and "Conclusion": rounding with linear feedback through the
 * LDL factor; [QTIP] "Builds on": BlockLDLQ). Lazily blocked: B columns are
 * swept at a time and the rest of the matrix is updated once per block.
 *   W: m x n incoherence-processed weights, leading dim ldw (read only).
 *   U, D: from quip_ldl with the same g (D is read for g = 8 and for the
 *     loss outputs).
 *   B: lazy block size, a multiple of g, 8..4096.
 *   q: quantizer (UNIFORM needs g = 1; E8 needs g = 8).
 *   scales: as quip_scales; written when q->scale_mode is COMPUTE, read when
 *     GIVEN (E8: the caller supplies the global scale and the row RMS).
 *   codes: UNIFORM: uint8 m x n (row-major, leading dim n), the grid index
 *     0..2^bits-1 of every weight. E8: uint16 m x (n/8), the codebook index
 *     of every 8-vector.
 *   What: optional (may be NULL) m x n output (leading dim n) of the
 *     quantized weights in the same (incoherent) domain as W; for E8 rows are
 *     scaled back by their RMS.
 *   codebook: 65536 x 8 device floats for E8, else NULL. Codes index this
 *     array; any order works, and quip_e8_codebook's order searches faster
 *     (one member of each pair {c, -c} of its full shells; see quip_scales).
 *   row_loss, loss: optional (may be NULL) device float64 outputs, m values
 *     and one value: the proxy loss tr((W^ - W) H (W^ - W)^T) ([QuIP]
 *     "Introduction") per row and summed, in W's domain, for the H whose
 *     factors U, D are passed. It is taken from the rounding itself: with
 *     H = (I + U) D (I + U)^T, column K of (W - W^)(I + U) is the pre-rounding
 *     target P_K minus W^_K, so the loss is sum_K (P_K - W^_K) D_K
 *     (P_K - W^_K)^T, O(mn) instead of O(mn^2). Requires D.
 *   ws: device workspace of quip_ldlq_workspace() bytes.
 * Errors: QUIP_ERR_ARG, QUIP_ERR_SHAPE (n % g, B % g, B range),
 *   QUIP_ERR_WORKSPACE, QUIP_ERR_UNSUPPORTED (bits > 8).
 */
quip_status quip_ldlq_workspace(int64_t m, int64_t n, int64_t g, int64_t B,
                                const quip_quantizer* q, size_t* bytes);
quip_status quip_ldlq(const float* W, int64_t m, int64_t n, int64_t ldw, const float* U,
                      const float* D, int64_t g, int64_t B, const quip_quantizer* q,
                      float* scales, void* codes, float* What, const float* codebook,
                      double* row_loss, double* loss, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/*
 * quip_proxy_loss -- loss = tr((W^ - W) H (W^ - W)^T) ([QuIP] "Introduction":
 * the proxy objective), accumulated in float64.
 *   W, What: m x n, both with leading dim ld. H: n x n symmetric, leading
 *   dim ldh; only its upper triangle is read.
 *   loss_dev: one device double, overwritten.
 *   ws: device workspace of quip_proxy_loss_workspace() bytes.
 * Errors: QUIP_ERR_ARG, QUIP_ERR_WORKSPACE.
 */
quip_status quip_proxy_loss_workspace(int64_t m, int64_t n, size_t* bytes);
quip_status quip_proxy_loss(const float* W, const float* What, int64_t m, int64_t n, int64_t ld,
                            const float* H, int64_t ldh, double* loss_dev, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/*
 * Kernel timing (measurement support; not a step of the method). While
 * enabled, every kernel the library launches carries two HIP events that its
 * own dispatch stamps with the kernel's start and end (hipExtLaunchKernel;
 * no extra work on the stream), filed under its kernel family (GEMMs by
 * call site: "gemm:hessian", "gemm:ldl_inner", "gemm:ldl_outer",
 * "gemm:ldlq_inner", "gemm:ldlq_outer", "gemm:kron", "gemm:proxy_loss").
 * Process-wide, off by default.
 *   quip_timing_enable(on): 1 on, 0 off.
 *   quip_timing_reset(): waits for recorded events, then clears all sums.
 *   quip_timing_report(buf, len, needed): waits for recorded events, adds them
 *     to the sums and writes one text line "name launches total_ms flops
 *     bytes" per family into buf (NUL-terminated, truncated to len), where
 *     flops and bytes are the summed algorithmic work of the launches (useful
 *     floating-point operations, compulsory global-memory bytes; 0 where not
 *     modelled); *needed receives the full size. buf may be NULL to query the
 *     size.
 * Errors: QUIP_ERR_HIP (an event could not be waited on).
 */
quip_status quip_timing_enable(int on);
quip_status quip_timing_reset(void);
quip_status quip_timing_report(char* buf, size_t len, size_t* needed);

/*
 * quip_pack_codes -- packs the per-weight codes of the scalar grid (as
 * quip_ldlq writes them) for inference: row by row, code j of a row occupies
 * bits [(j w) mod 8, (j w) mod 8 + w) of byte (j w) / 8 of that row, least
 * significant bits first, with w = 2, 4 or 8 the smallest container that
 * holds `bits` (no code straddles a byte); a row takes
 * quip_packed_row_bytes(n, bits) bytes and the rows follow each other without
 * padding.
 *   codes: m x n uint8 (device), leading dim ldc; values below 2^bits (higher
 *     bits are dropped).
 *   packed: m x quip_packed_row_bytes(n, bits) bytes (device, caller-owned).
 * Errors: QUIP_ERR_ARG (null pointer, sizes, ldc < n, bits outside 1..8).
 */
quip_status quip_packed_row_bytes(int64_t n, int32_t bits, int64_t* bytes);
quip_status quip_pack_codes(const uint8_t* codes, int64_t m, int64_t n, int64_t ldc, int32_t bits,
                            uint8_t* packed, hipStream_t stream);

/*
 * quip_qmatvec_rht -- product of the quantized layer with a full-precision
 * vector at inference: the quantized-matrix full-precision-vector product with
 * the incoherence transforms applied around it ([QuIP] "Experiments",
 * "Throughput Comparison"), with random-sign Hadamard sides ([QuIP#]
 * abstract). With W^~[r][j] = scales[r] (code[r][j] - (2^bits - 1)/2) and
 * Q_L = H_m diag(signs_left)/sqrt(m), Q_R = H_n diag(signs_right)/sqrt(n) (the
 * transforms of quip_rht), it computes y = Q_L^T W^~ Q_R x, the layer W^ =
 * Q_L^T W^~ Q_R in the original basis times x, without forming W^.
 *   packed: m x quip_packed_row_bytes(n, bits) bytes from quip_pack_codes.
 *   scales: m floats (the grid step of every row, as quip_ldlq uses them).
 *   signs_left: m floats, signs_right: n floats (+1 / -1), as passed to
 *     quip_rht for the two sides of W.
 *   x: n floats in; y: m floats out (device). m: a power of two in
 *     [2, 16384]; n: a power of two in [1024, 16384]. packed, x, y and the
 *     signs 16-byte aligned.
 *   ws: device workspace of quip_qmatvec_rht_workspace() bytes.
 * Errors: QUIP_ERR_ARG, QUIP_ERR_SHAPE (m, n), QUIP_ERR_WORKSPACE.
 */
quip_status quip_qmatvec_rht_workspace(int64_t m, int64_t n, size_t* bytes);
quip_status quip_qmatvec_rht(const uint8_t* packed, int64_t m, int64_t n, int32_t bits,
                             const float* scales, const float* signs_left,
                             const float* signs_right, const float* x, float* y, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/*
 * quip_qmatvec_rht_noalloc -- quip_qmatvec_rht without a workspace, for callers
 * that cannot allocate device memory or pass a workspace (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation). Same
 * arguments, kernels and result as quip_qmatvec_rht (bit for bit); its scratch
 * (the transformed vector, the transform's intermediate and the per-slice
 * partial sums) lives in a static device array of 4 MiB inside the library,
 * one copy per GPU, held until the process ends. Allocates nothing (no
 * hipMalloc, no library allocation); the first call on a device looks the
 * array's device address up once (hipGetSymbolAddress).
 *   Every call on one GPU shares that GPU's array: calls that overlap in time
 *   on one GPU (different streams, or host threads on the same device) race
 *   and give undefined results; serialize them. The array keeps the last
 *   call's contents; every word a call reads it writes first.
 * Errors: as quip_qmatvec_rht (QUIP_ERR_ARG, QUIP_ERR_SHAPE; the accepted
 *   shapes, m and n up to 16384, need at most 2.1 MiB of the 4 MiB, and a
 *   product needing more is refused with QUIP_ERR_SHAPE); QUIP_ERR_HIP if the
 *   array's address cannot be obtained.
 */
quip_status quip_qmatvec_rht_noalloc(const uint8_t* packed, int64_t m, int64_t n, int32_t bits,
                                     const float* scales, const float* signs_left,
                                     const float* signs_right, const float* x, float* y,
                                     hipStream_t stream);

/*
 * quip_permute -- moves the rows and columns of a matrix by index vectors:
 * the permutation step inside the fast orthogonal multiplication ([QuIP]
 * "Further Ablation", Table 5: the side transform becomes Q = K P, the
 * coordinates permuted before they are mixed) and LDLQ-RG's re-ordering of the
 * weights ([QuIP] "Experiments / Methods").
 *   scatter = 0 (gather): out[i][j] = A[row_index[i]][col_index[j]], i.e.
 *     out = P_r A P_c^T with (P_p x)_i = x_{p(i)}.
 *   scatter = 1: out[row_index[i]][col_index[j]] = A[i][j], i.e.
 *     out = P_r^T A P_c (the inverse of the gather with the same vectors).
 *   A, out: rows x cols float32 (device), leading dims lda, ldo >= cols; they
 *     must not overlap (no in-place use).
 *   row_index: rows int32 (device) or NULL (identity); col_index: cols int32
 *     (device) or NULL (identity). The vectors should be permutations of
 *     0..rows-1 and 0..cols-1; they are not checked on the host. Gather: an
 *     index outside the matrix yields NaN. Scatter: an entry with such an index
 *     is dropped, and entries of out that no index reaches are unspecified.
 *     No access leaves the matrices either way.
 * Errors: QUIP_ERR_ARG (null pointer with a non-empty matrix, negative sizes,
 * leading dimension < cols, overlapping A and out, scatter not 0 or 1),
 * QUIP_ERR_SHAPE (cols > 32768 with a column index: the row is staged in LDS).
 */
quip_status quip_permute(const float* A, int64_t lda, float* out, int64_t ldo, int64_t rows,
                         int64_t cols, const int32_t* row_index, const int32_t* col_index,
                         int32_t scatter, hipStream_t stream);

/*
 * quip_diag_order -- LDLQ-RG's quantization order ([QuIP] "Experiments /
 * Methods": the weights re-ordered by diag(H)): order[k] is the column
 * quantized k-th, the columns taken by decreasing H[j][j], equal values by
 * increasing j (NaN after every number; +0 and -0 equal). Deterministic.
 *   H: n x n float32 (device), leading dim ldh >= n; only the diagonal is read.
 *   order: n int32 (device).
 *   ws: quip_diag_order_workspace(n) bytes, 256-byte aligned.
 * Errors: QUIP_ERR_ARG (null pointer, n <= 0, ldh < n), QUIP_ERR_WORKSPACE.
 */
quip_status quip_diag_order_workspace(int64_t n, size_t* bytes);
quip_status quip_diag_order(const float* H, int64_t n, int64_t ldh, int32_t* order, void* ws,
                            size_t ws_bytes, hipStream_t stream);

/*
 * quip_tcq_quantize -- trellis-coded quantization with a bitshift trellis
 * ([QTIP] summary page, Approach): each row x_0..x_{T-1} of X becomes the
 * state sequence s_0..s_{T-1} of an L-bit shift register that takes k new
 * bits per step (s_t = (s_{t-1} << k | b_t) mod 2^L, so the stream is
 * s_0 followed by k bits per later weight: k + (L - k)/T bits per weight),
 * minimizing sum_t (x_t - c(s_t))^2 exactly (Viterbi; ties to the lowest
 * predecessor, then the lowest final state; the first state is free, no
 * tail-biting). c is a computed pseudorandom Gaussian code (the page names
 * such codes without a formula; this one is a reading): h = (1664525 s +
 * 1013904223) mod 2^32, c(s) = fma(sum of the four bytes of h, alpha, beta)
 * in float32, with alpha = float32(scale / sqrt(21845)) and beta =
 * float32(-510 scale / sqrt(21845)).
 *   X: rows x T float32 (device), leading dim ldx >= T.
 *   L: state bits, 4..15 (the 2^L costs of a row are held in one LDS buffer);
 *   k: bits per step, 2.
 *   scale: finite, > 0 (the values are scale times a unit-variance code).
 *   states: rows x T uint16 (device), leading dim lds >= T.
 *   Xhat: rows x T float32 (device) with leading dim ldq >= T, or NULL:
 *     c(states).
 *   cost: rows float32 (device): the minimum of each row (float32 sums).
 *   ws: quip_tcq_workspace(rows, T, L) bytes, 256-byte aligned (2-bit
 *     back-pointers of up to 2048 rows at a time).
 * Errors: QUIP_ERR_ARG (null pointer, sizes, leading dimensions, scale),
 * QUIP_ERR_UNSUPPORTED (k != 2, L outside 4..15), QUIP_ERR_WORKSPACE.
 */
quip_status quip_tcq_workspace(int64_t rows, int64_t T, int32_t L, size_t* bytes);
quip_status quip_tcq_quantize(const float* X, int64_t rows, int64_t T, int64_t ldx, int32_t L,
                              int32_t k, float scale, uint16_t* states, int64_t lds, float* Xhat,
                              int64_t ldq, float* cost, void* ws, size_t ws_bytes,
                              hipStream_t stream);

/*
 * Attainable-rate probes: measurement aids beside the method, not part of it.
 * The roofline fractions are quoted against the chip's published peaks; these
 * two calls measure what plain, dependency-free work attains on the device at
 * hand, with the same launch path (and the same timing registry) as the
 * library's kernels.
 *
 * quip_peak_copy -- dst[i] = src[i] for 0 <= i < count: 8 count bytes of HBM
 * traffic (16 work-groups per CU looping over the array, four 16-byte
 * non-temporal loads per thread and round before its four stores).
 *   src, dst: count float32 (device), 16-byte aligned, not overlapping.
 * Errors: QUIP_ERR_ARG (negative count, null or misaligned pointer, overlap).
 *
 * quip_peak_compute -- `iters` rounds of independent instructions on four
 * work-groups of 256 threads per CU (four waves per SIMD):
 *   kind 0: fp32 matrix cores, v_mfma_f32_32x32x2_f32, four accumulators per
 *     wave (4096 flops per instruction);
 *   kind 1: f16 matrix cores with fp32 accumulation, v_mfma_f32_32x32x16_f16,
 *     four accumulators per wave (32768 flops per instruction);
 *   kind 2: fp32 vector FMAs, eight chains per lane (2 flops each; one FMA
 *     per lane and instruction, as everywhere in this library).
 *   out: 1 float32 (device); written only if the result equals an improbable
 *     value (the write keeps the work alive), so its content is unspecified.
 *   flops: host double receiving the launch's flop count, or NULL.
 * Errors: QUIP_ERR_ARG (kind not 0..2, iters <= 0, null out).
 */
quip_status quip_peak_copy(const float* src, float* dst, int64_t count, hipStream_t stream);
quip_status quip_peak_compute(int32_t kind, int64_t iters, float* out, double* flops,
                              hipStream_t stream);

/*
 * quip_e8_codebook -- fills HOST memory with the 65536 smallest-norm points of
 * the E8 lattice (D8 together with D8 + 1/2) ordered by squared norm, then by
 * coordinates ascending with the first coordinate most significant; 65536 x 8
 * floats, row-major ([QuIP#] abstract: E8-lattice codebooks).
 * Errors: QUIP_ERR_ARG (null pointer).
 */
quip_status quip_e8_codebook(float* host_out);

#ifdef __cplusplus
}
#endif

#endif /* QUIP_H */
