// Attainable-rate probes. They are measurement aids, not part of the method:
// the roofline fractions divide by the chip's published peaks, and these
// loops show what a launch of plain, dependency-free work attains on the card
// at hand (an HBM copy, the fp32 and f16 matrix cores, fp32 vector FMAs).
//
// Every probe writes nothing unless its result equals an improbable value, so
// the compiler keeps the work and the launch stays a pure rate measurement.
#include "common.h"

namespace quip {
namespace {

constexpr int PEAK_THREADS = 256;
constexpr int PEAK_GROUPS_PER_CU = 4;  // four waves on every SIMD
constexpr int F32_CHAINS = 4;          // independent 32x32x2 accumulators per wave
constexpr int F16_CHAINS = 4;          // independent 32x32x16 accumulators per wave
constexpr int VALU_CHAINS = 8;         // independent FMA chains per lane

typedef float peak_f32x16 __attribute__((ext_vector_type(16)));
typedef float peak_f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 peak_f16x8 __attribute__((ext_vector_type(8)));

constexpr float IMPROBABLE = -1.2345678e-30f;

// Four 16-byte chunks per thread and round, loads before stores, with the
// non-temporal hint (the data is touched once); the scalar tail covers the
// last count mod 4 floats.
constexpr int COPY_UNROLL = 4;

__global__ __launch_bounds__(PEAK_THREADS) void peak_copy_kernel(const float* __restrict__ src,
                                                                 float* __restrict__ dst,
                                                                 int64_t count) {
  const int64_t n4 = count / 4;
  const peak_f32x4* s4 = reinterpret_cast<const peak_f32x4*>(src);
  peak_f32x4* d4 = reinterpret_cast<peak_f32x4*>(dst);
  const int64_t stride = int64_t(gridDim.x) * PEAK_THREADS * COPY_UNROLL;
  int64_t i = int64_t(blockIdx.x) * PEAK_THREADS * COPY_UNROLL + threadIdx.x;
  for (; i + PEAK_THREADS * (COPY_UNROLL - 1) < n4; i += stride) {
    peak_f32x4 v[COPY_UNROLL];
#pragma unroll
    for (int u = 0; u < COPY_UNROLL; ++u) v[u] = __builtin_nontemporal_load(s4 + i + PEAK_THREADS * u);
#pragma unroll
    for (int u = 0; u < COPY_UNROLL; ++u) __builtin_nontemporal_store(v[u], d4 + i + PEAK_THREADS * u);
  }
  // the round that does not fit whole: its chunks one by one
  for (; i < n4; i += PEAK_THREADS) d4[i] = s4[i];
  const int64_t t = int64_t(blockIdx.x) * PEAK_THREADS + threadIdx.x;
  if (t < count - 4 * n4) dst[4 * n4 + t] = src[4 * n4 + t];
}

// fp32 matrix cores: v_mfma_f32_32x32x2_f32, 4096 flops per instruction.
__global__ __launch_bounds__(PEAK_THREADS) void peak_mfma_f32_kernel(int64_t iters, float seed,
                                                                     float* out) {
  peak_f32x16 acc[F32_CHAINS];
#pragma unroll
  for (int c = 0; c < F32_CHAINS; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[c][j] = 0.f;
  const float a = seed * float(threadIdx.x + 1), b = seed * 0.5f;
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < F32_CHAINS; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < F32_CHAINS; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[c][j];
  if (s == IMPROBABLE) out[0] = s;
}

// f16 matrix cores: v_mfma_f32_32x32x16_f16, 32768 flops per instruction
// (the 16x16x32 form needs about 16 independent accumulators per wave to come
// near the same rate).
__global__ __launch_bounds__(PEAK_THREADS) void peak_mfma_f16_kernel(int64_t iters, float seed,
                                                                     float* out) {
  peak_f32x16 acc[F16_CHAINS];
#pragma unroll
  for (int c = 0; c < F16_CHAINS; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[c][j] = 0.f;
  peak_f16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = _Float16(seed * float(threadIdx.x + j));
    b[j] = _Float16(seed * float(j + 1));
  }
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < F16_CHAINS; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < F16_CHAINS; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[c][j];
  if (s == IMPROBABLE) out[0] = s;
}

// fp32 vector FMAs (one per lane and instruction: packed fp32 is not used in
// this library), 2 flops each.
__global__ __launch_bounds__(PEAK_THREADS) void peak_valu_f32_kernel(int64_t iters, float seed,
                                                                     float* out) {
  float x[VALU_CHAINS];
#pragma unroll
  for (int c = 0; c < VALU_CHAINS; ++c) x[c] = seed * float(threadIdx.x + c);
  const float m = 1.f - seed, a = seed;
  for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < VALU_CHAINS; ++c) x[c] = fmaf(x[c], m, a);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < VALU_CHAINS; ++c) s += x[c];
  if (s == IMPROBABLE) out[0] = s;
}

int peak_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  return cus;
}

}  // namespace

quip_status peak_copy(const float* src, float* dst, int64_t count, hipStream_t s) {
  if (count == 0) return QUIP_OK;
  const dim3 grid(unsigned(16 * peak_cus()));
  return timed_launch("peak_copy_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL(peak_copy_kernel, grid, dim3(PEAK_THREADS), 0, s, src, dst, count);
  }, 0.0, 8.0 * double(count));
}

quip_status peak_compute(int kind, int64_t iters, float* out, double* flops, hipStream_t s) {
  const int64_t groups = int64_t(PEAK_GROUPS_PER_CU) * peak_cus();
  const int64_t waves = groups * (PEAK_THREADS / 64);
  const dim3 grid{unsigned(groups)}, block{unsigned(PEAK_THREADS)};
  const float seed = 1.0f / 1024.0f;
  double f = 0.0;
  quip_status st = QUIP_OK;
  switch (kind) {
    case 0:
      f = double(waves) * double(iters) * F32_CHAINS * (32.0 * 32.0 * 2.0 * 2.0);
      st = timed_launch("peak_mfma_f32_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
        QUIP_KERNEL(peak_mfma_f32_kernel, grid, block, 0, s, iters, seed, out);
      }, f, 0.0);
      break;
    case 1:
      f = double(waves) * double(iters) * F16_CHAINS * (32.0 * 32.0 * 16.0 * 2.0);
      st = timed_launch("peak_mfma_f16_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
        QUIP_KERNEL(peak_mfma_f16_kernel, grid, block, 0, s, iters, seed, out);
      }, f, 0.0);
      break;
    default:
      f = double(groups) * PEAK_THREADS * double(iters) * VALU_CHAINS * 2.0;
      st = timed_launch("peak_valu_f32_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
        QUIP_KERNEL(peak_valu_f32_kernel, grid, block, 0, s, iters, seed, out);
      }, f, 0.0);
      break;
  }
  if (flops) *flops = f;
  return st;
}

}  // namespace quip
