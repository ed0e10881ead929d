// Inference with the quantized layer: y = Q_L^T W^~ Q_R x, the quantized
// matrix times a full-precision vector with the incoherence transforms applied
// around it ([QuIP] "Experiments", "Throughput Comparison"; random-sign
// Hadamard sides as in [QuIP#] abstract). W^~ is held as packed b-bit codes
// and a step per row: W^~[r][j] = s_r (code - (L-1)/2).
//
// Packed format (pack_codes_kernel): row by row, code j of a row in bits
// [(j w) mod 8, + w) of byte (j w) / 8, w = 2, 4 or 8 the container width
// (the smallest that holds b bits, so that no code straddles a byte).
//
// The product runs in three launches: x' = Q_R x (the row RHT on one row),
// y' = W^~ x' (qmatvec_kernel), y = Q_L^T y' (the inverse row RHT on one
// row). qmatvec_kernel is bound by the packed codes it streams and by the
// VALU work of unpacking them: each thread owns CPT consecutive columns of a
// row (n / CPT threads per row, CPT <= 64 so x' stays in registers), reads its
// codes as 32-bit words and unpacks four at a time (a shift, a mask of one
// code per byte, four byte-to-float conversions), and subtracts the grid
// offset once through the sum of its x'. Four rows per thread per iteration;
// the per-row sums are reduced across lanes with shuffles and across waves
// through LDS.
#include "common.h"

namespace quip {
namespace {

template <int W>
__global__ __launch_bounds__(256) void pack_codes_kernel(const uint8_t* __restrict__ codes,
                                                         int64_t m, int64_t n, int64_t ldc,
                                                         uint8_t* __restrict__ packed,
                                                         int64_t rowbytes) {
  constexpr int PER = 8 / W;
  const int64_t b = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (b >= rowbytes) return;
  for (int64_t r = blockIdx.y; r < m; r += gridDim.y) {
    uint32_t v = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int64_t j = b * PER + i;
      if (j < n) v |= uint32_t(codes[r * ldc + j] & ((1u << W) - 1u)) << (i * W);
    }
    packed[r * rowbytes + b] = uint8_t(v);
  }
}

constexpr int QMV_RB = 4;  // rows per row-group and iteration

// y'[r] = s_r sum_j (code_j - cen) x'_j for the rows of a persistent
// work-group. T = n / CPT threads per row (64, 128 or 256).
template <int W, int CPT>
__global__ __launch_bounds__(256) void qmatvec_kernel(const uint8_t* __restrict__ packed,
                                                      int64_t m, int64_t n,
                                                      const float* __restrict__ scales,
                                                      const float* __restrict__ xp, float cen,
                                                      float* __restrict__ yp) {
  constexpr int NW = CPT * W / 32;  // 32-bit words of codes per thread and row
  constexpr int CPW = 32 / W;       // codes per word
  constexpr int CPB = 8 / W;        // codes per byte
  static_assert(NW >= 1 && CPT % 4 == 0, "thread chunk");
  __shared__ float red[4][QMV_RB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = int(n / CPT);  // threads per row: 64, 128 or 256
  const int groups = 256 / T;  // row-groups per work-group
  const int g = tid / T, p = tid % T;
  const int wpr = T / 64;      // waves per row
  const int64_t rowbytes = n * W / 8;

  float x[CPT];
  float xs = 0.f;
#pragma unroll
  for (int v = 0; v < CPT / 4; ++v) {
    const float4 t = *reinterpret_cast<const float4*>(xp + int64_t(p) * CPT + 4 * v);
    x[4 * v + 0] = t.x;
    x[4 * v + 1] = t.y;
    x[4 * v + 2] = t.z;
    x[4 * v + 3] = t.w;
    xs += (t.x + t.y) + (t.z + t.w);
  }
  const float off = cen * xs;  // this thread's share of the grid offset

  const int64_t per_iter = int64_t(groups) * QMV_RB;
  for (int64_t base = int64_t(blockIdx.x) * per_iter; base < m; base += int64_t(gridDim.x) * per_iter) {
    float part[QMV_RB];
#pragma unroll
    for (int q = 0; q < QMV_RB; ++q) {
      const int64_t r = base + int64_t(g) * QMV_RB + q;
      float acc = 0.f;
      if (r < m) {
        const uint32_t* src =
            reinterpret_cast<const uint32_t*>(packed + r * rowbytes + int64_t(p) * (CPT * W / 8));
        uint32_t wd[NW];
#pragma unroll
        for (int i = 0; i < NW; ++i) wd[i] = src[i];
#pragma unroll
        for (int i = 0; i < NW; ++i) {
#pragma unroll
          for (int sh = 0; sh < 8; sh += W) {
            const uint32_t t = (wd[i] >> sh) & (0x01010101u * ((1u << W) - 1u));
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const float c = float((t >> (8 * k)) & 0xFFu);
              acc = fmaf(c, x[i * CPW + k * CPB + sh / W], acc);
            }
          }
        }
        acc -= off;
      }
      part[q] = acc;
    }
    // sums over the T threads of each row: lanes, then the waves of the row
#pragma unroll
    for (int q = 0; q < QMV_RB; ++q) {
      float v = part[q];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
      part[q] = v;
    }
    if (lane == 0) {
#pragma unroll
      for (int q = 0; q < QMV_RB; ++q) red[wave][q] = part[q];
    }
    __syncthreads();
    if (tid < groups * QMV_RB) {
      const int gg = tid / QMV_RB, q = tid % QMV_RB;
      const int64_t r = base + int64_t(gg) * QMV_RB + q;
      if (r < m) {
        float v = 0.f;
        for (int w = 0; w < wpr; ++w) v += red[gg * wpr + w][q];
        yp[r] = scales[r] * v;
      }
    }
    __syncthreads();
  }
}

template <int W>
quip_status qmatvec_t(const uint8_t* packed, int64_t m, int64_t n, const float* scales,
                      const float* xp, float cen, float* yp, hipStream_t s) {
  const int cpt = n >= 4096 ? 64 : int(n / 64);
  const int T = int(n / cpt);
  const int64_t per_iter = int64_t(256 / T) * QMV_RB;
  int64_t nwg = cdiv(m, per_iter);
  if (nwg > 2048) nwg = 2048;
  const dim3 grid{unsigned(nwg)};
  const double bytes = double(m) * double(n) * W / 8.0 + 4.0 * double(n + 2 * m);
  const double flops = 2.0 * double(m) * double(n);
  return timed_launch("qmatvec_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    switch (cpt) {
#define CASE(C)                                                                           \
  case C:                                                                                 \
    QUIP_KERNEL((qmatvec_kernel<W, C>), grid, dim3(256), 0, s, packed, m, n, scales, xp, cen, yp); \
    break;
      CASE(16) CASE(32) CASE(64)
#undef CASE
    }
  }, flops, bytes);
}

}  // namespace

int code_container_bits(int bits) { return bits <= 2 ? 2 : (bits <= 4 ? 4 : 8); }

quip_status pack_codes(const uint8_t* codes, int64_t m, int64_t n, int64_t ldc, int bits,
                       uint8_t* packed, hipStream_t s) {
  const int w = code_container_bits(bits);
  const int64_t rowbytes = cdiv(n * w, 8);
  const dim3 grid{unsigned(cdiv(rowbytes, 256)), unsigned(m < 65535 ? m : 65535)};
  return timed_launch("pack_codes_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    if (w == 2)
      QUIP_KERNEL((pack_codes_kernel<2>), grid, dim3(256), 0, s, codes, m, n, ldc, packed, rowbytes);
    else if (w == 4)
      QUIP_KERNEL((pack_codes_kernel<4>), grid, dim3(256), 0, s, codes, m, n, ldc, packed, rowbytes);
    else
      QUIP_KERNEL((pack_codes_kernel<8>), grid, dim3(256), 0, s, codes, m, n, ldc, packed, rowbytes);
  }, 0.0, double(m) * double(n) + double(m) * double(rowbytes));
}

size_t qmatvec_workspace_bytes(int64_t m, int64_t n) {
  Carver c(nullptr, 0);
  c.take<float>(size_t(n));  // x'
  c.take<float>(size_t(m));  // y'
  return c.used;
}

quip_status qmatvec_rht(const uint8_t* packed, int64_t m, int64_t n, int bits, const float* scales,
                        const float* signs_left, const float* signs_right, const float* x,
                        float* y, void* ws, size_t ws_bytes, hipStream_t s) {
  Carver c(ws, ws_bytes);
  float* xp = c.take<float>(size_t(n));
  float* yp = c.take<float>(size_t(m));
  if (!c.fits()) return fail(QUIP_ERR_WORKSPACE, "quip_qmatvec_rht: workspace too small");
  const float cen = 0.5f * float((1 << bits) - 1);
  QUIP_TRY(rht_rows(x, xp, 1, n, n, signs_right, false, s));  // x' = Q_R x
  const int w = code_container_bits(bits);
  if (w == 2) QUIP_TRY(qmatvec_t<2>(packed, m, n, scales, xp, cen, yp, s));
  else if (w == 4) QUIP_TRY(qmatvec_t<4>(packed, m, n, scales, xp, cen, yp, s));
  else QUIP_TRY(qmatvec_t<8>(packed, m, n, scales, xp, cen, yp, s));
  return rht_rows(yp, y, 1, m, m, signs_left, true, s);  // y = Q_L^T y'
}

}  // namespace quip
