// Small element-wise kernels (fills, copies, differences). Fills are kernels,
// not hipMemsetAsync, so that a stream capture of the pass records only
// kernel nodes.
#include "common.h"

namespace quip {
namespace {

__global__ void fill_f32_kernel(float* p, int64_t count, float v) {
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (; i < count; i += stride) p[i] = v;
}

__global__ void fill_f64_kernel(double* p, int64_t count, double v) {
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (; i < count; i += stride) p[i] = v;
}

// 2-D kernels: one work-group row-chunk per (row, 1024-column strip).
__global__ void fill_matrix_kernel(float* p, int64_t rows, int64_t cols, int64_t ld, float v) {
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y)
    for (int64_t c = int64_t(blockIdx.x) * 1024 + threadIdx.x; c < cols;
         c += int64_t(gridDim.x) * 1024)
    p[r * ld + c] = v;
}

__global__ void sub_matrix_kernel(const float* a, const float* b, float* out, int64_t rows,
                                  int64_t cols, int64_t lda, int64_t ldb, int64_t ldo) {
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y)
    for (int64_t c = int64_t(blockIdx.x) * 1024 + threadIdx.x; c < cols;
         c += int64_t(gridDim.x) * 1024)
    out[r * ldo + c] = a[r * lda + c] - b[r * ldb + c];
}

__global__ void copy_matrix_kernel(const float* s, int64_t lds, float* d, int64_t ldd,
                                   int64_t rows, int64_t cols) {
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y)
    for (int64_t c = int64_t(blockIdx.x) * 1024 + threadIdx.x; c < cols;
         c += int64_t(gridDim.x) * 1024)
    d[r * ldd + c] = s[r * lds + c];
}

// Row i of an n x n matrix: zeros in the columns [0, bs floor(i / bs)), the
// part left of its diagonal block. One work-group per row; float4 stores when
// the rows are 16-byte aligned.
__global__ __launch_bounds__(256) void fill_lower_blocks_kernel(float* p, int64_t n, int64_t ld,
                                                                int64_t bs, bool vec,
                                                                int32_t* word) {
  const int64_t i = blockIdx.x;
  if (word && i == 0 && threadIdx.x == 0) *word = 0;
  const int64_t cnt = bs * (i / bs);
  float* row = p + i * ld;
  if (vec) {
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int64_t c = 4 * int64_t(threadIdx.x); c < cnt; c += 1024)
      *reinterpret_cast<float4*>(row + c) = z;
  } else {
    for (int64_t c = threadIdx.x; c < cnt; c += 256) row[c] = 0.f;
  }
}

dim3 grid2d(int64_t rows, int64_t cols) {
  int64_t gx = cdiv(cols, 1024);
  if (gx > 64) gx = 64;
  return dim3(unsigned(gx < 1 ? 1 : gx), unsigned(rows < 65535 ? rows : 65535));
}

}  // namespace

quip_status fill_lower_blocks(float* p, int64_t n, int64_t ld, int64_t bs, int32_t* word,
                              hipStream_t s) {
  if (n <= 0) return QUIP_OK;
  const bool vec = ld % 4 == 0 && bs % 4 == 0 && (reinterpret_cast<uintptr_t>(p) & 15) == 0;
  return timed_launch("fill_lower_blocks", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL(fill_lower_blocks_kernel, dim3(unsigned(n)), dim3(256), 0, s, p, n, ld, bs, vec,
                word);
  });
}

quip_status fill_f32(float* p, int64_t count, float v, hipStream_t s) {
  if (count <= 0) return QUIP_OK;
  int64_t blocks = cdiv(count, 256);
  if (blocks > 8192) blocks = 8192;
  return timed_launch("fill_f32", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL(fill_f32_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, p, count, v);
  });
}

quip_status fill_f64(double* p, int64_t count, double v, hipStream_t s) {
  if (count <= 0) return QUIP_OK;
  int64_t blocks = cdiv(count, 256);
  if (blocks > 8192) blocks = 8192;
  return timed_launch("fill_f64", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL(fill_f64_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, p, count, v);
  });
}

quip_status fill_matrix(float* p, int64_t rows, int64_t cols, int64_t ld, float v, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return QUIP_OK;
  if (ld == cols) return fill_f32(p, rows * cols, v, s);
  return timed_launch("fill_matrix", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL(fill_matrix_kernel, grid2d(rows, cols), dim3(1024), 0, s, p, rows, cols, ld, v);
  });
}

quip_status sub_matrix(const float* a, const float* b, float* out, int64_t rows, int64_t cols,
                       int64_t lda, int64_t ldb, int64_t ldo, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return QUIP_OK;
  return timed_launch("sub_matrix", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL(sub_matrix_kernel, grid2d(rows, cols), dim3(1024), 0, s, a, b, out, rows,
                       cols, lda, ldb, ldo);
  });
}

quip_status copy_matrix(const float* src, int64_t lds, float* dst, int64_t ldd, int64_t rows,
                        int64_t cols, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return QUIP_OK;
  return timed_launch("copy_matrix", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL(copy_matrix_kernel, grid2d(rows, cols), dim3(1024), 0, s, src, lds, dst, ldd,
                       rows, cols);
  });
}

}  // namespace quip
