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
// The product runs in five launches: x' = Q_R x in two passes of
// qmv_vec_fwht_kernel (H_n = H_n1 (x) H_n2: transforms of the contiguous chunks,
// then of the strided columns, one short transform per wave), per-slice partial
// sums of W^~ x' (qmv_mfma_kernel), and y = Q_L^T y' in two more passes, the
// first of which forms y' (the sum of the slices times the row step).
//
// qmv_mfma_kernel puts the dot products on the matrix cores
// (v_mfma_f32_16x16x32_f16), so the vector ALUs only unpack codes. A code c
// of w bits becomes an exact half-precision value with one shift and one
// and-or per pair of codes: OR-ing it into the mantissa of 1.0 gives
// 1 + c 2^-p (p = 2, 4, 8 for w = 2, 4, 8). For w = 4 and 8 a packed half
// subtraction then centres it, (c - (L-1)/2) 2^-p exactly; for w = 2 the
// offset is removed once per block through the sum of x' instead (one VALU op
// per code). x' enters as two half-precision columns, x' = hi + lo (about 22
// bits), so the products are exact and the matrix cores accumulate in float32.
//
// Layout: a work-group is one wave and owns a slice of 256 KS columns (KS = 1
// for n below 2048, else 2). Lane (r, h) of the wave (r = lane
// mod 16 the row of the 16-row tile, h = lane / 16) reads one contiguous run of
// 64 KS codes of its row (KS w / 2 loads of 16 bytes; the four runs of a row
// are one contiguous 256 KS-code segment), which feeds 8 KS MFMA steps: the
// k order inside an MFMA is a permutation of the run. The x' operand (hi in the
// even columns, lo in the odd ones) is written in that order by the last pass
// of the transform of x, loaded once per wave (16 bytes per step and lane) and
// kept in registers while the wave walks its row tiles. The steps of a tile
// feed QMV_CHAINS independent accumulators, added at the end (one dependent
// chain of these products would be bound by the instruction's latency).
// The two used accumulator columns are added with one lane swap and each
// slice writes one partial per row; the first pass of the inverse transform
// sums the slices in a fixed order (deterministic; no atomics, no barriers).
#include <mutex>
#include <string>

#include "common.h"

// Size of the allocation-free product's scratch: the workspace of the largest
// product the entry points accept (m = n = 16384: 2.1 MiB) with room to spare.
#define QMV_SCRATCH_BYTES (4u << 20)
#define QMV_MAX_DEVICES 64

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

typedef _Float16 qmv_half2 __attribute__((ext_vector_type(2)));
typedef _Float16 qmv_half8 __attribute__((ext_vector_type(8)));
typedef float qmv_float4 __attribute__((ext_vector_type(4)));
constexpr int QMV_CHAINS = 4;  // independent accumulators per tile

// Position, within a lane's run of codes, of the code in MFMA step s, slot j
// (j = 2v + t: A register v, half t), matching qmv_unpack.
template <int W>
__device__ __forceinline__ int qmv_code_index(int s, int j) {
  const int v = j >> 1, t = j & 1;
  if (W == 2) return 16 * (s >> 1) + 4 * (s & 1) + v + 8 * t;  // pairs (c, c + 8) of a word
  if (W == 4) return 8 * s + v + 4 * t;                          // pairs (c, c + 4) of a word
  return 4 * (2 * s + (v >> 1)) + (v & 1) + 2 * t;               // pairs (c, c + 2) of a word
}

// The inverse of qmv_code_index: step s and slot j of run position r.
template <int W>
__device__ __forceinline__ void qmv_slot_of(int r, int& s, int& j) {
  if (W == 2) {
    const int rem = r & 15, t = rem >> 3, e = (rem & 7) >> 2, v = rem & 3;
    s = 2 * (r >> 4) + e;
    j = 2 * v + t;
  } else if (W == 4) {
    const int rem = r & 7, t = rem >> 2, v = rem & 3;
    s = r >> 3;
    j = 2 * v + t;
  } else {
    const int rem = r & 7, v = 2 * (rem >> 2) + (rem & 1), t = (rem >> 1) & 1;
    s = r >> 3;
    j = 2 * v + t;
  }
}

// A operand of step s: four registers of two halves each, 1 + c 2^-p (W = 2)
// or (c - cen) 2^-p (W = 4, 8), from the lane's code words q.
// (a & m) | o in one instruction. A vector instruction here may read one
// scalar register, so m comes from a scalar and o from a vector register
// (the compiler otherwise splits the pair into an and and an or).
__device__ __forceinline__ uint32_t qmv_and_or(uint32_t a, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(m), "v"(o));
  return r;
}

// kmask selects the two codes' bits after the shift (0x03000300, 0x03C003C0
// or 0x03FC03FC for W = 2, 4, 8; a kernel argument, so a scalar) and kone is
// 1.0 in both halves (0x3C003C00, held in a vector register): each pair of
// codes costs one shift and one v_and_or_b32.
template <int W>
__device__ __forceinline__ qmv_half8 qmv_unpack(const uint32_t* q, int s, qmv_half2 sub,
                                                uint32_t kmask, uint32_t kone) {
  uint32_t r[4];
  if (W == 2) {
    const uint32_t w = q[s >> 1];
    const int e = s & 1;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int j = 4 * e + v;  // codes j and j + 8 of the word
      const uint32_t sh = j <= 4 ? (w << (8 - 2 * j)) : (w >> (2 * j - 8));
      r[v] = qmv_and_or(sh, kmask, kone);
    }
  } else if (W == 4) {
    const uint32_t w = q[s];
    r[0] = qmv_and_or(w << 6, kmask, kone);
    r[1] = qmv_and_or(w << 2, kmask, kone);
    r[2] = qmv_and_or(w >> 2, kmask, kone);
    r[3] = qmv_and_or(w >> 6, kmask, kone);
  } else {
    const uint32_t w0 = q[2 * s], w1 = q[2 * s + 1];
    r[0] = qmv_and_or(w0 << 2, kmask, kone);
    r[1] = qmv_and_or(w0 >> 6, kmask, kone);
    r[2] = qmv_and_or(w1 << 2, kmask, kone);
    r[3] = qmv_and_or(w1 >> 6, kmask, kone);
  }
  qmv_half8 a;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    qmv_half2 h2 = __builtin_bit_cast(qmv_half2, r[v]);
    if (W != 2) h2 = h2 - sub;  // exact: (1 + c 2^-p) - (1 + cen 2^-p)
    a[2 * v] = h2[0];
    a[2 * v + 1] = h2[1];
  }
  return a;
}

// part[blockIdx.y][r] = sum over the wave's slice of 256 KS columns of
// (code - cen) x'_j, for the rows r of the wave's tiles. One wave per
// work-group: the slice's x' operand stays in registers while the wave walks
// its row tiles, and every slice writes its own partials (no barriers).
template <int W, int KS, int PF>
__global__ __launch_bounds__(64) void qmv_mfma_kernel(const uint8_t* __restrict__ packed,
                                                      int64_t m, int64_t n,
                                                      const _Float16* __restrict__ xop,
                                                      float cen, float* __restrict__ part,
                                                      uint32_t kmask, uint32_t kone) {
  constexpr int STEPS = 8 * KS;        // MFMA steps per tile (8 codes per lane and step)
  constexpr int RUN = 64 * KS;         // codes in a lane's run
  constexpr int NQ = KS * W / 2;       // 16-byte loads per lane and tile
  constexpr float P2 = W == 2 ? 4.f : (W == 4 ? 16.f : 256.f);  // 2^p

  const int lane = threadIdx.x;
  const int c = lane & 15, h = lane >> 4;
  const int64_t rowbytes = n * W / 8;
  const int64_t run0 = int64_t(blockIdx.y) * (4 * RUN) + int64_t(h) * RUN;

  // x' operand: hi in the even columns, lo in the odd ones, already in the
  // slot order of the steps (written by the last pass of the transform of x:
  // [slice][h][hi, lo][step][8 halves]). Only columns 0 and 1 of the product
  // are read; the other columns only feed accumulator columns never used.
  const uint4* xo = reinterpret_cast<const uint4*>(xop) +
                    ((int64_t(blockIdx.y) * 4 + h) * 2 + (c & 1)) * STEPS;
  qmv_half8 B[STEPS];
  float xs = 0.f;  // this lane's halves, summed
#pragma unroll
  for (int s = 0; s < STEPS; ++s) {
    B[s] = __builtin_bit_cast(qmv_half8, xo[s]);
#pragma unroll
    for (int j = 0; j < 8; ++j) xs += float(B[s][j]);
  }
  // the slice's sum of x' as the halves represent it (for the W = 2 offset):
  // hi + lo from a lane pair, then the four runs of the lane groups h
  xs += __shfl_xor(xs, 1, 64);
  xs += __shfl_xor(xs, 16, 64);
  xs += __shfl_xor(xs, 32, 64);
  const qmv_half2 sub = {_Float16(1.f + cen / P2), _Float16(1.f + cen / P2)};
  float* const out = part + int64_t(blockIdx.y) * m;

  // code words of the tiles in flight: a ring of PF tiles per lane, refilled
  // with the tile PF strides ahead as soon as a slot is consumed
  const uint8_t* const base = packed + run0 * W / 8;
  auto load = [&](uint32_t* q, int64_t t) {
    const int64_t row = t * 16 + c;
    if (row < m) {
      const uint4* src = reinterpret_cast<const uint4*>(base + row * rowbytes);
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        const uint4 v = src[i];
        q[4 * i] = v.x;
        q[4 * i + 1] = v.y;
        q[4 * i + 2] = v.z;
        q[4 * i + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4 * NQ; ++i) q[i] = 0u;
    }
  };
  const int64_t g = gridDim.x;
  uint32_t ring[PF][4 * NQ];
#pragma unroll
  for (int k = 0; k < PF; ++k) load(ring[k], int64_t(blockIdx.x) + k * g);

  for (int64_t t = blockIdx.x; t * 16 < m;) {
#pragma unroll
    for (int k = 0; k < PF; ++k) {
      if (t * 16 < m) {
        // QMV_CHAINS independent accumulators (step s feeds chain s mod
        // QMV_CHAINS): one dependent chain of 16x16x32 products is bound by
        // the instruction's latency, not by the matrix cores' rate
        qmv_float4 Dc[QMV_CHAINS];
#pragma unroll
        for (int q = 0; q < QMV_CHAINS; ++q) Dc[q] = qmv_float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < STEPS; ++s)
          Dc[s % QMV_CHAINS] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              qmv_unpack<W>(ring[k], s, sub, kmask, kone), B[s], Dc[s % QMV_CHAINS], 0, 0, 0);
        qmv_float4 D = Dc[0];
#pragma unroll
        for (int q = 1; q < QMV_CHAINS; ++q) D += Dc[q];
        load(ring[k], t + PF * g);
        // lane (c, h) holds rows 4h..4h+3 of column c: add columns 0 and 1
#pragma unroll
        for (int i = 0; i < 4; ++i) D[i] += __shfl_xor(D[i], 1, 64);
        const int64_t r0 = t * 16 + 4 * h;
        if (c == 0 && r0 < m) {
          float4 v;
          v.x = W == 2 ? P2 * D[0] - (P2 + cen) * xs : P2 * D[0];
          v.y = W == 2 ? P2 * D[1] - (P2 + cen) * xs : P2 * D[1];
          v.z = W == 2 ? P2 * D[2] - (P2 + cen) * xs : P2 * D[2];
          v.w = W == 2 ? P2 * D[3] - (P2 + cen) * xs : P2 * D[3];
          if (r0 + 4 <= m) {
            *reinterpret_cast<float4*>(out + r0) = v;
          } else {  // m < 4 (a power of two: 2)
            out[r0] = v.x;
            if (r0 + 1 < m) out[r0 + 1] = v.y;
          }
        }
        t += g;
      }
    }
  }
}

// One transform of length L <= 128 per wave for a vector of length n = n1 n2
// seen as an n1 x n2 row-major matrix (index i = a n2 + b): the natural-order
// Sylvester matrix is H_n = H_n1 (x) H_n2, so H_n v is H_n2 on every row (the
// contiguous chunks, pass 0) followed by H_n1 on every column (stride n2,
// pass 1). Lane l holds elements u = l and u = l + 64 of its transform; the
// butterflies on bits 0..5 of u go through lane shuffles. Options by pass:
//   pass 0: in[i] times pre[i] (the random signs of the forward transform),
//           or, with part given, in[i] = scales[i] * sum_b part[b][i] (the
//           product's partial sums; the finish of the inverse transform);
//   pass 1: times scale, then times post[i] (the signs of the inverse).
template <int W>
__device__ __forceinline__ void qmv_put_operand(_Float16* xop, int64_t i, int ks, float x) {
  const int64_t run = 64 * ks, slice = i / (4 * run);
  const int h = int((i % (4 * run)) / run), r = int(i % run);
  int st, j;
  qmv_slot_of<W>(r, st, j);
  const _Float16 hi = _Float16(x), lo = _Float16(x - float(hi));
  _Float16* base = xop + ((slice * 4 + h) * 2) * (8 * ks * 8) + st * 8 + j;
  base[0] = hi;           // [slice][h][0][st][j]
  base[8 * ks * 8] = lo;  // [slice][h][1][st][j]
}

__global__ __launch_bounds__(64) void qmv_vec_fwht_kernel(
    const float* __restrict__ in, float* __restrict__ out, int pass, int L, int64_t n2,
    const float* __restrict__ pre, const float* __restrict__ part, int nblk, int64_t m,
    const float* __restrict__ scales, const float* __restrict__ post, float scale,
    _Float16* __restrict__ xop, int w, int ks) {
  const int lane = threadIdx.x;
  const int64_t t = blockIdx.x;
  const int64_t base = pass == 0 ? t * L : t;      // first element of this transform
  const int64_t step = pass == 0 ? 1 : n2;         // distance between its elements
  float v[2] = {0.f, 0.f};
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int u = lane + 64 * k;
    if (u < L) {
      const int64_t i = base + int64_t(u) * step;
      float x;
      if (part) {
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;  // nblk is a multiple of 4
        for (int b = 0; b < nblk; b += 4) {
          a0 += part[int64_t(b) * m + i];
          a1 += part[int64_t(b + 1) * m + i];
          a2 += part[int64_t(b + 2) * m + i];
          a3 += part[int64_t(b + 3) * m + i];
        }
        x = scales[i] * ((a0 + a1) + (a2 + a3));
      } else {
        x = in[i];
      }
      if (pre) x *= pre[i];
      v[k] = x;
    }
  }
  if (L == 128) {  // bit 6 of u: within the lane
    const float a = v[0], b = v[1];
    v[0] = a + b;
    v[1] = a - b;
  }
  for (int j = 1; j < 64 && j < L; j <<= 1) {  // bits 0..5 of u: across lanes
    const bool upper = (lane & j) != 0;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const float o = __shfl_xor(v[k], j, 64);
      v[k] = upper ? o - v[k] : v[k] + o;
    }
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int u = lane + 64 * k;
    if (u < L) {
      const int64_t i = base + int64_t(u) * step;
      float x = v[k] * scale;
      if (post) x *= post[i];
      if (out) out[i] = x;
      if (xop) {  // the product's operand layout (hi and lo halves, slot order)
        if (w == 2) qmv_put_operand<2>(xop, i, ks, x);
        else if (w == 4) qmv_put_operand<4>(xop, i, ks, x);
        else qmv_put_operand<8>(xop, i, ks, x);
      }
    }
  }
}

// n = n1 n2 with n2 = 2^ceil(k/2) <= 128 (n <= 16384)
inline int64_t vec_n2(int64_t n) { return int64_t(1) << ((ilog2(n) + 1) / 2); }

quip_status vec_fwht_pass(const float* in, float* out, int pass, int64_t n, const float* pre,
                          const float* part, int nblk, const float* scales, const float* post,
                          float scale, hipStream_t s, _Float16* xop = nullptr, int w = 2,
                          int ks = 1) {
  const int64_t n2 = vec_n2(n), n1 = n / n2;
  const int L = int(pass == 0 ? n2 : n1);
  const int64_t count = pass == 0 ? n1 : n2;
  const double bytes = 8.0 * double(n) + (part ? 4.0 * double(nblk) * double(n) : 0.0);
  return timed_launch("qmv_vec_fwht_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL(qmv_vec_fwht_kernel, dim3(unsigned(count)), dim3(64), 0, s, in, out, pass, L, n2,
                pre, part, nblk, n, scales, post, scale, xop, w, ks);
  }, double(n) * double(ilog2(L)), bytes);
}

constexpr int QMV_PF = 3;  // tiles in flight per wave
int qmv_ks(int64_t n) { return n >= 2048 ? 2 : 1; }
int64_t qmv_blocks(int64_t n) { return n / (256 * qmv_ks(n)); }  // column slices, one per wave

template <int W>
quip_status qmv_mfma_t(const uint8_t* packed, int64_t m, int64_t n, const _Float16* xop,
                       float cen, float* part, hipStream_t s) {
  const int64_t nblk = qmv_blocks(n);
  const int64_t tiles = cdiv(m, 16);
  // as many one-wave work-groups as are resident at once, split over the
  // column slices; each walks its share of the row tiles
  const void* kfn = qmv_ks(n) == 2 ? reinterpret_cast<const void*>(&qmv_mfma_kernel<W, 2, QMV_PF>)
                                   : reinterpret_cast<const void*>(&qmv_mfma_kernel<W, 1, QMV_PF>);
  int per_cu = 0, dev = 0, cus = 0;
  int64_t resident = 4096;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kfn, 64, 0) == hipSuccess &&
      hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      per_cu > 0 && cus > 0)
    resident = int64_t(per_cu) * cus;
  int64_t gx = resident / nblk;
  if (gx < 1) gx = 1;
  if (gx > tiles) gx = tiles;
  const dim3 grid{unsigned(gx), unsigned(nblk)};
  const uint32_t kmask = W == 2 ? 0x03000300u : (W == 4 ? 0x03C003C0u : 0x03FC03FCu);
  const uint32_t kone = 0x3C003C00u;  // 1.0 in both halves
  const double bytes = double(m) * double(n) * W / 8.0 + 4.0 * double(n) + 4.0 * double(nblk) * double(m);
  const double flops = 2.0 * double(m) * double(n);
  return timed_launch("qmatvec_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    if (qmv_ks(n) == 2)
      QUIP_KERNEL((qmv_mfma_kernel<W, 2, QMV_PF>), grid, dim3(64), 0, s, packed, m, n, xop, cen,
                  part, kmask, kone);
    else
      QUIP_KERNEL((qmv_mfma_kernel<W, 1, QMV_PF>), grid, dim3(64), 0, s, packed, m, n, xop, cen,
                  part, kmask, kone);
  }, flops, bytes);
}

// Scratch of the allocation-free variant of the product: partial sums, the
// transformed vector and the transform's intermediate live in this array
// instead of a caller workspace. One copy per GPU, held until the process
// ends. Host code never passes the array's name to a kernel (on the host it is
// a stand-in, not a device address): it uses the address hipGetSymbolAddress
// gives for the current device.
static __device__ __align__(256) unsigned char scratch[QMV_SCRATCH_BYTES];

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
  c.take<_Float16>(size_t(2 * n));             // x' as the product's operand (hi, lo)
  c.take<float>(size_t(m > n ? m : n));        // between the two passes of a transform
  c.take<float>(size_t(qmv_blocks(n) * m));    // per-slice partial sums
  return c.used;
}

quip_status qmatvec_rht(const uint8_t* packed, int64_t m, int64_t n, int bits, const float* scales,
                        const float* signs_left, const float* signs_right, const float* x,
                        float* y, void* ws, size_t ws_bytes, hipStream_t s) {
  Carver c(ws, ws_bytes);
  _Float16* xop = c.take<_Float16>(size_t(2 * n));
  float* tmp = c.take<float>(size_t(m > n ? m : n));
  float* part = c.take<float>(size_t(qmv_blocks(n) * m));
  if (!c.fits()) return fail(QUIP_ERR_WORKSPACE, "quip_qmatvec_rht: workspace too small");
  const float cen = 0.5f * float((1 << bits) - 1);
  // x' = Q_R x = H_n diag(signs_right) x / sqrt(n): two passes, signs first
  QUIP_TRY(vec_fwht_pass(x, tmp, 0, n, signs_right, nullptr, 0, nullptr, nullptr, 1.f, s));
  const int w = code_container_bits(bits);
  QUIP_TRY(vec_fwht_pass(tmp, nullptr, 1, n, nullptr, nullptr, 0, nullptr, nullptr,
                         1.0f / sqrtf(float(n)), s, xop, w, qmv_ks(n)));
  if (w == 2) QUIP_TRY(qmv_mfma_t<2>(packed, m, n, xop, cen, part, s));
  else if (w == 4) QUIP_TRY(qmv_mfma_t<4>(packed, m, n, xop, cen, part, s));
  else QUIP_TRY(qmv_mfma_t<8>(packed, m, n, xop, cen, part, s));
  // y = Q_L^T y' = diag(signs_left) H_m y' / sqrt(m), with y' = scales * (sum of
  // the slices' partials) formed in the first pass
  const int nblk = int(qmv_blocks(n));
  QUIP_TRY(vec_fwht_pass(nullptr, tmp, 0, m, nullptr, part, nblk, scales, nullptr, 1.f, s));
  return vec_fwht_pass(tmp, y, 1, m, nullptr, nullptr, 0, nullptr, signs_left,
                       1.0f / sqrtf(float(m)), s);
}

size_t qmatvec_scratch_bytes() { return QMV_SCRATCH_BYTES; }

// Device address of `scratch` on the current device, looked up once per device.
static quip_status scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[QMV_MAX_DEVICES] = {};
  int dev = 0;
  QUIP_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= QMV_MAX_DEVICES)
    return fail(QUIP_ERR_UNSUPPORTED, "quip_qmatvec_rht_noalloc: device index out of range");
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    QUIP_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return fail(QUIP_ERR_HIP, "quip_qmatvec_rht_noalloc: no address for the scratch array");
    addr[dev] = p;
  }
  *out = addr[dev];
  return QUIP_OK;
}

quip_status qmatvec_rht_noalloc(const uint8_t* packed, int64_t m, int64_t n, int bits,
                                const float* scales, const float* signs_left,
                                const float* signs_right, const float* x, float* y,
                                hipStream_t s) {
  const size_t need = qmatvec_workspace_bytes(m, n);
  if (need > QMV_SCRATCH_BYTES)
    return fail(QUIP_ERR_SHAPE, "quip_qmatvec_rht_noalloc: the product of this size needs " +
                                    std::to_string(need) + " bytes of scratch, more than the " +
                                    std::to_string(size_t(QMV_SCRATCH_BYTES)) + " it has");
  void* ws = nullptr;
  QUIP_TRY(scratch_address(&ws));
  // every scratch word the product reads is written earlier in the same call,
  // so nothing needs clearing between calls
  return qmatvec_rht(packed, m, n, bits, scales, signs_left, signs_right, x, y, ws,
                     QMV_SCRATCH_BYTES, s);
}

}  // namespace quip
