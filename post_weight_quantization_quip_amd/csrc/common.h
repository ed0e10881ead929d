// Internal helpers shared by the libquip translation units (gfx950 only).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "quip.h"

namespace quip {

// ---------------------------------------------------------------- errors

void set_error(const std::string& msg);
void clear_error();
const char* last_error_cstr();

struct Status {
  quip_status st;
  Status(quip_status s = QUIP_OK) : st(s) {}
  operator quip_status() const { return st; }
  bool ok() const { return st == QUIP_OK; }
};

quip_status fail(quip_status st, const std::string& msg);

#define QUIP_HIP(call)                                                              \
  do {                                                                              \
    hipError_t e_ = (call);                                                         \
    if (e_ != hipSuccess)                                                           \
      return ::quip::fail(QUIP_ERR_HIP, std::string(#call) + ": " + hipGetErrorString(e_)); \
  } while (0)

#define QUIP_TRY(expr)                   \
  do {                                   \
    quip_status s_ = (expr);             \
    if (s_ != QUIP_OK) return s_;        \
  } while (0)

// Checks the last launch on this thread.
quip_status launch_check(const char* what);

// ---------------------------------------------------------------- kernel timing

// While timing is on (quip_timing_enable), every launch is bracketed by two
// HIP events on its stream, filed under `name` (timing.cpp).
// The launch lambda receives a start / stop event pair (null when timing is
// off) and launches with QUIP_KERNEL, which hands the pair to the dispatch
// itself (hipExtLaunchKernelGGL): the events carry the kernel's own start and
// end times, with no extra packets on the stream. `flops` and `bytes` are the
// launch's algorithmic work (useful floating-point operations, compulsory
// global-memory bytes), summed with the times.
bool timing_on();
bool timing_begin(const char* name, double flops, double bytes, hipEvent_t* start,
                  hipEvent_t* stop);

#define QUIP_KERNEL(kernel, grid, block, shmem, stream, ...) \
  hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, ev_start_, ev_stop_, 0, __VA_ARGS__)

template <typename F>
quip_status timed_launch(const char* name, hipStream_t s, F&& launch, double flops = 0.0,
                         double bytes = 0.0) {
  (void)s;
  hipEvent_t a = nullptr, b = nullptr;
  if (timing_on() && !timing_begin(name, flops, bytes, &a, &b)) a = b = nullptr;
  launch(a, b);
  return launch_check(name);
}

// ---------------------------------------------------------------- workspace

// Carves 256-byte aligned sub-buffers out of a caller workspace. With a null
// base it only measures.
struct Carver {
  char* base;
  size_t cap;
  size_t used = 0;
  Carver(void* b, size_t c) : base(static_cast<char*>(b)), cap(c) {}
  template <typename T>
  T* take(size_t count) {
    size_t off = (used + 255) & ~size_t(255);
    used = off + count * sizeof(T);
    return base ? reinterpret_cast<T*>(base + off) : nullptr;
  }
  bool fits() const { return used <= cap; }
};

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }
inline bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
inline int ilog2(int64_t v) {
  int l = 0;
  while ((int64_t(1) << l) < v) ++l;
  return l;
}
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------- device helpers

// Work-group ids are dealt round-robin to the 8 XCDs (each with its own L2).
// Remap the hardware id so that consecutive logical tiles land on the same XCD.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int nx = 8;
  int per = total / nx, rem = total % nx;
  int x = bid % nx, local = bid / nx;
  int start = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
  return start + local;
}

// ---------------------------------------------------------------- inference (qmatvec.hip)

int code_container_bits(int bits);
quip_status pack_codes(const uint8_t* codes, int64_t m, int64_t n, int64_t ldc, int bits,
                       uint8_t* packed, hipStream_t s);
size_t qmatvec_workspace_bytes(int64_t m, int64_t n);
quip_status qmatvec_rht(const uint8_t* packed, int64_t m, int64_t n, int bits, const float* scales,
                        const float* signs_left, const float* signs_right, const float* x,
                        float* y, void* ws, size_t ws_bytes, hipStream_t s);
// The same product with its scratch in a static device array (no workspace).
size_t qmatvec_scratch_bytes();
quip_status qmatvec_rht_noalloc(const uint8_t* packed, int64_t m, int64_t n, int bits,
                                const float* scales, const float* signs_left,
                                const float* signs_right, const float* x, float* y,
                                hipStream_t s);

// ---------------------------------------------------------------- permutations (permute.hip)

int64_t permute_max_cols();
quip_status permute(const float* A, int64_t lda, float* out, int64_t ldo, int64_t rows,
                    int64_t cols, const int32_t* ridx, const int32_t* cidx, bool scatter,
                    hipStream_t s);
size_t diag_order_workspace_bytes(int64_t n);
quip_status diag_order(const float* H, int64_t n, int64_t ldh, int32_t* order, void* ws,
                       size_t ws_bytes, hipStream_t s);

// ---------------------------------------------------------------- trellis (tcq.hip)

// attainable-rate probes (peak.hip)
quip_status peak_copy(const float* src, float* dst, int64_t count, hipStream_t s);
quip_status peak_compute(int kind, int64_t iters, float* out, double* flops, hipStream_t s);

size_t tcq_workspace_bytes(int64_t rows, int64_t T, int L);
quip_status tcq_quantize(const float* X, int64_t rows, int64_t T, int64_t ldx, int L, float scale,
                         uint16_t* states, int64_t lds, float* xhat, int64_t ldq, float* cost,
                         void* ws, size_t ws_bytes, hipStream_t s);

// ---------------------------------------------------------------- GEMM (gemm.hip)

enum GemmEpi {
  EPI_STORE = 0,  // C_out = alpha * op(A) op(B) + beta * C_in
  EPI_DOT = 1,    // *dot += sum(alpha * op(A) op(B) .* E)  (float64 accumulate)
  EPI_SPLIT = 2,  // like STORE, columns >= split go to C2 (ldc2) at column - split
  EPI_DOT_SYM = 3 // like DOT with B symmetric (K == N): only B's upper triangle is read,
                  // off-diagonal entries count twice, so output column j sums k <= j only
};

struct GemmArgs {
  int64_t M = 0, N = 0, K = 0;
  const float* A = nullptr;  // !transA: A[m*lda + k]; transA: A[k*lda + m]
  int64_t lda = 0, strideA = 0;
  const float* B = nullptr;  // !transB: B[k*ldb + n]; transB: B[n*ldb + k]
  int64_t ldb = 0, strideB = 0;
  float* C = nullptr;
  int64_t ldc = 0, strideC = 0;
  const float* Cin = nullptr;  // beta source (defaults to C)
  int64_t ldcin = 0, strideCin = 0;
  float alpha = 1.f, beta = 0.f;
  int batch = 1;
  bool transA = false, transB = false;
  bool upper_tiles = false;  // only output tiles with tile_row <= tile_col (M == N)
  bool mirror = false;       // upper_tiles: also write the transpose below the diagonal
  int epi = EPI_STORE;
  const float* E = nullptr;  // EPI_DOT operand, E[m*lde + n]
  int64_t lde = 0;
  double* dot = nullptr;
  int64_t split = 0;  // EPI_SPLIT
  float* C2 = nullptr;
  int64_t ldc2 = 0;
  // upper_tiles + EPI_STORE: when the tile count does not fill the last round
  // of work-groups, the leftover tiles are split along K into pieces written
  // to P (float count P_floats) and summed in a fixed order (deterministic).
  float* P = nullptr;
  size_t P_floats = 0;
  const char* tag = "gemm";  // name under which launches are timed
  // internal: tiles [tile0, tile0 + grid / kpieces) of the grid, K in pieces of kchunk
  int tile0 = 0;
  int kpieces = 1;
  int64_t kchunk = 0;
};

// Partial-tile workspace (floats) that gemm() uses for the leftover tiles of
// the Hessian's upper-tile product X^T X (X: K x n); 0 when there are none.
int device_cus();
size_t gemm_upper_tail_floats(int64_t n, int64_t K);

quip_status gemm(const GemmArgs& a, hipStream_t stream);

// ---------------------------------------------------------------- misc kernels (misc.hip)

quip_status fill_f32(float* p, int64_t count, float v, hipStream_t stream);
// zeros in row i, columns [0, bs floor(i / bs)) of an n x n matrix, and in
// *word when word is not null
quip_status fill_lower_blocks(float* p, int64_t n, int64_t ld, int64_t bs, int32_t* word,
                              hipStream_t stream);
quip_status fill_matrix(float* p, int64_t rows, int64_t cols, int64_t ld, float v,
                        hipStream_t stream);
quip_status sub_matrix(const float* a, const float* b, float* out, int64_t rows, int64_t cols,
                       int64_t lda, int64_t ldb, int64_t ldo, hipStream_t stream);  // out = a - b
quip_status fill_f64(double* p, int64_t count, double v, hipStream_t stream);
quip_status copy_matrix(const float* src, int64_t lds, float* dst, int64_t ldd, int64_t rows,
                        int64_t cols, hipStream_t stream);

// ---------------------------------------------------------------- RHT (rht.hip)

// last_pass: no other pass of the same transform reads `out` next (its rows
// are then written with non-temporal stores)
quip_status rht_rows(const float* A, float* out, int64_t rows, int64_t cols, int64_t ld,
                     const float* signs, bool inverse, hipStream_t stream, bool last_pass = true);
quip_status rht_cols(const float* A, float* out, int64_t rows, int64_t cols, int64_t ld,
                     const float* signs, bool inverse, hipStream_t stream);

// ---------------------------------------------------------------- E8 (e8.cpp)

void e8_build_codebook(float* host_out);

}  // namespace quip
