// Proxy Hessian H = X^T X (QuIP, "Adaptive Rounding Step": the second moment
// of the layer inputs) as a symmetric rank-N update on the fp32 matrix cores:
// only output tiles on or above the diagonal are computed, and each is also
// written to its mirror position. The tiles that would run alone in a last
// round of work-groups are split along N (the calibration rows) into pieces
// summed in a fixed order, when the caller passes the workspace for them. Damping (QuIP, "Experiments / Methods"):
// H <- H / N + alpha * mean(diag(H / N)) * I.
#include "common.h"

namespace quip {
namespace {

// Partial traces: work-group p of TRACE_PARTS sums the diagonal entries of
// its contiguous slice of rows and writes out[p] (the finalize sums the parts
// in a fixed order).
constexpr int TRACE_PARTS = 32;
static_assert(TRACE_PARTS * sizeof(double) <= 256, "the parts fit the finalize's 256-byte workspace");
__global__ __launch_bounds__(256) void trace_kernel(const float* H, int64_t n, int64_t ldh,
                                                    double* out) {
  __shared__ double part[4];
  const int64_t per = (n + TRACE_PARTS - 1) / TRACE_PARTS;
  const int64_t i0 = int64_t(blockIdx.x) * per;
  const int64_t i1 = (i0 + per < n) ? i0 + per : n;
  double s = 0.0;
  for (int64_t i = i0 + threadIdx.x; i < i1; i += blockDim.x) s += double(H[i * ldh + i]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_down(s, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = (part[0] + part[1]) + (part[2] + part[3]);
}

__global__ __launch_bounds__(256) void finalize_kernel(float* H, int64_t n, int64_t ldh,
                                                       const double* trace_parts,
                                                       double inv_n_total, double alpha, bool vec) {
  double trace = 0.0;
#pragma unroll
  for (int p = 0; p < TRACE_PARTS; ++p) trace += trace_parts[p];
  const float shift = float(alpha * trace * inv_n_total / double(n));
  const float scale = float(inv_n_total);
  const int64_t r = blockIdx.x;
  float* row = H + r * ldh;
  if (vec) {
    for (int64_t c = int64_t(threadIdx.x) * 4; c < n; c += 1024) {
      float4 v = *reinterpret_cast<const float4*>(row + c);
      v = make_float4(v.x * scale, v.y * scale, v.z * scale, v.w * scale);
      if (r == c + 0) v.x += shift;
      if (r == c + 1) v.y += shift;
      if (r == c + 2) v.z += shift;
      if (r == c + 3) v.w += shift;
      *reinterpret_cast<float4*>(row + c) = v;
    }
  } else {
    for (int64_t c = threadIdx.x; c < n; c += 256) {
      float v = row[c] * scale;
      if (r == c) v += shift;
      row[c] = v;
    }
  }
}

}  // namespace

quip_status hessian_accumulate(const float* X, int64_t N, int64_t n, int64_t ldx, float* H,
                               int64_t ldh, bool accumulate, float* P, size_t P_floats,
                               hipStream_t s) {
  if (N == 0) {
    if (!accumulate) return fill_matrix(H, n, n, ldh, 0.f, s);
    return QUIP_OK;
  }
  GemmArgs g;
  g.M = n;
  g.N = n;
  g.K = N;
  g.A = X;  // op(A)[i][t] = X[t][i]
  g.lda = ldx;
  g.transA = true;
  g.B = X;  // op(B)[t][j] = X[t][j]
  g.ldb = ldx;
  g.transB = false;
  g.C = H;
  g.ldc = ldh;
  g.alpha = 1.f;
  g.beta = accumulate ? 1.f : 0.f;
  g.upper_tiles = true;
  g.mirror = true;
  g.tag = "gemm:hessian";
  g.P = P;  // leftover tiles split along K when the workspace holds their pieces
  g.P_floats = P_floats;
  return gemm(g, s);
}

quip_status hessian_finalize(float* H, int64_t n, int64_t ldh, int64_t N_total, float alpha,
                             double* scratch, hipStream_t s) {
  QUIP_TRY(timed_launch("trace_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL(trace_kernel, dim3(TRACE_PARTS), dim3(256), 0, s, H, n, ldh, scratch);
  }));
  const bool vec = aligned16(H) && ldh % 4 == 0 && n % 4 == 0;
  return timed_launch("finalize_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL(finalize_kernel, dim3(unsigned(n)), dim3(256), 0, s, H, n, ldh, scratch,
                1.0 / double(N_total), double(alpha), vec);
  }, 2.0 * double(n) * double(n), 8.0 * double(n) * double(n));
}

}  // namespace quip
