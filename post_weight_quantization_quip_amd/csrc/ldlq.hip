// LDLQ / BlockLDLQ rounding (QuIP, "Adaptive Rounding Step" and
// "Conclusion": W^ = Q(W + (W - W^) U) with U from H = (I+U) D (I+U)^T;
// BlockLDLQ with 8-column groups and the E8 codebook of QuIP#'s abstract, as
// named on the QTIP page under "Builds on").
//
// Schedule (lazy blocking; the rounding decisions are the unblocked ones):
//   F = 0
//   for each block of B columns [j0, j0 + B):
//     sweep the block column by column (group by group), each pre-rounding
//     value being  W_k + F_k + sum_{i in block, i < k} E_i U_ik,  E = W - W^
//     F[:, j0+B:] += E_block U[j0:j0+B, j0+B:]        (matrix cores)
//
// Scalar grid sweep: one wave holds 16 rows; each row is spread over a quad of
// 4 lanes, lane g owning the 4-column chunks {16t + 4g .. 16t + 4g + 3}. The
// owner of column k rounds it, the error goes to the quad's other lanes with
// one DPP quad_perm broadcast, and every lane updates its later columns with
// the row of U held in LDS (laid out so that each lane's columns are
// contiguous).
//
// E8 groups: the pre-rounding 8-vectors of all rows are searched against the
// 65536 codewords as a distance contraction on the matrix cores
// (codewords x rows, K = 8), with the per-row argmin kept as a packed
// (order-preserving distance bits, index) 64-bit key and atomicMin.
#include <type_traits>

#include <utility>

#include "common.h"

namespace quip {

quip_status ldlq_run(const float* W, int64_t m, int64_t n, int64_t ldw, const float* U,
                     const float* D, int g, int64_t B, const quip_quantizer& q, float* scales,
                     void* codes, float* What, const float* codebook, double* row_loss,
                     double* loss, void* ws, size_t ws_bytes, hipStream_t s);
size_t ldlq_workspace_bytes(int64_t m, int64_t n, int g, int64_t B, const quip_quantizer& q);
quip_status scales_run(const float* W, int64_t m, int64_t n, int64_t ldw, const quip_quantizer& q,
                       float* scales, void* mse_out, const float* codebook, void* ws,
                       size_t ws_bytes, hipStream_t s);
size_t scales_workspace_bytes(int64_t m, int64_t n, const quip_quantizer& q);

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float quad_bcast(float v, int src) {
  // quad_perm [src, src, src, src]
  const int ctrl = src * 0x55;
  int r;
  switch (ctrl) {
    case 0x00: r = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x00, 0xF, 0xF, false); break;
    case 0x55: r = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x55, 0xF, 0xF, false); break;
    case 0xAA: r = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xAA, 0xF, 0xF, false); break;
    default: r = __builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xFF, 0xF, 0xF, false); break;
  }
  return __int_as_float(r);
}

// ------------------------------------------------------------------ scale search (grid)

template <int NC>
__global__ __launch_bounds__(256) void grid_scale_kernel(const float* __restrict__ W, int64_t m,
                                                         int64_t n, int64_t ldw, int L, int ncand,
                                                         const float* __restrict__ factors,
                                                         float* __restrict__ scales,
                                                         float* __restrict__ mse_out) {
  __shared__ float red[4][NC];
  __shared__ float smax_sh;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x;
  const float* w = W + row * ldw;

  float amax = 0.f;
  for (int64_t j = tid; j < n; j += 256) amax = fmaxf(amax, fabsf(w[j]));
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if (lane == 0) red[wave][0] = amax;
  __syncthreads();
  if (tid == 0) smax_sh = fmaxf(fmaxf(red[0][0], red[1][0]), fmaxf(red[2][0], red[3][0]));
  __syncthreads();
  const float gmax = smax_sh;
  if (gmax == 0.f) {
    if (tid == 0) scales[row] = 1.f;
    if (mse_out)
      for (int c = tid; c < ncand; c += 256) mse_out[row * ncand + c] = 0.f;
    return;
  }
  // Error in units of the candidate step: t = x / s + (L-1)/2 (one fma),
  // code k = clamp(round(t), 0, L-1), e / s = t - k (exact for in-range codes,
  // Sterbenz); the sum over the row is scaled by s^2 once at the end. Round
  // half to even differs from floor(t + 1/2) only at exact ties, where both
  // codes leave |e / s| = 1/2.
  const float cen = (L - 1) * 0.5f, hi = float(L - 1);
  const float smax = gmax / cen;
  float sc[NC], inv[NC], acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    sc[c] = smax * factors[c < ncand ? c : 0];
    inv[c] = 1.f / sc[c];
    acc[c] = 0.f;
  }
  for (int64_t j = tid; j < n; j += 256) {
    const float x = w[j];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const float t = fmaf(x, inv[c], cen);
      const float k = __builtin_amdgcn_fmed3f(rintf(t), 0.f, hi);
      const float e = t - k;
      acc[c] = fmaf(e, e, acc[c]);
    }
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) acc[c] *= sc[c] * sc[c];
  __syncthreads();
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float v = acc[c];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0) red[wave][c] = v;
  }
  __syncthreads();
  if (tid == 0) {
    int best = 0;
    float bv = 0.f;
    for (int c = 0; c < ncand; ++c) {
      float v = (red[0][c] + red[1][c]) + (red[2][c] + red[3][c]);
      if (mse_out) mse_out[row * ncand + c] = v;
      if (c == 0 || v < bv) {
        bv = v;
        best = c;
      }
    }
    scales[row] = smax * factors[best];
  }
}

// Compile-time loop: f(std::integral_constant<int, I>) for I = 0 .. N-1.
template <typename F, int... I>
__device__ __forceinline__ void static_for_(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_(f, std::make_integer_sequence<int, N>{});
}

// Value of lane J of this lane's 16-lane row (DPP row_newbcast).
template <int J>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + J, 0xF, 0xF, false));
}

// ------------------------------------------------------------------ scalar LDLQ sweep

// Scalar LDLQ sweep of one block of B columns for 16 rows per work-group.
//
// 4 waves x 4 rows; each row is one 16-lane DPP row of its wave, and lane j of
// the row owns column 16 tk + j of the current 16-column chunk tk. Every lane
// evaluates the rounding on its own target; the owner's error of column kk is
// sent to the row with one DPP row_newbcast and every lane adds its share of
// the feedback (rank-1, one FMA; U is zero on and below the diagonal, so the
// columns already rounded are left alone). After a chunk, each lane adds the
// chunk's rank-16 feedback to one accumulator per later chunk; those live in
// registers, shifted down by one chunk per step so that every register index
// is static. U's rows are staged transposed in LDS (row c = column c of U) in
// a two-chunk ring, one 16-row chunk ahead of their use, so that a lane's 16
// coefficients of a chunk are four float4 reads and the LDS footprint does not
// grow with B.
template <int B>
__global__ __launch_bounds__(256) void ldlq_sweep_kernel(
    const float* __restrict__ W, int64_t ldw, const float* __restrict__ F, int64_t ldf, bool useF,
    const float* __restrict__ U, int64_t ldu, const float* __restrict__ scales, int L, int64_t m,
    int64_t s0, int bw, uint8_t* __restrict__ codes, int64_t ldcode, float* __restrict__ What,
    int64_t ldwh, float* __restrict__ Eb, int64_t lde, const float* __restrict__ Dg,
    double* __restrict__ rowloss, bool vec) {
  constexpr int NT = B / 16;  // 16-column chunks
  constexpr int UP = 36;      // two 16-row chunks of U (a ring) and a pad, per column
  extern __shared__ __align__(16) float sm[];
  float* Ut = sm;            // [B][UP]: column c of U's rows of the current and next chunk
  float* Ds = sm + B * UP;   // [B]: D of the block (proxy loss)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int j = lane & 15;  // column of the chunk owned by this lane
  const int64_t row = int64_t(blockIdx.x) * 16 + (tid >> 4);
  const bool live = row < m;

  // U's rows are staged chunk by chunk: rows [16 t, 16 t + 16) are loaded
  // (coalesced) while chunk t - 1 is processed and written transposed into a
  // two-chunk ring (k mod 32), with the float4 slot swizzled by c so that the
  // writes spread over the banks:
  //   Ut[c * UP + 4 * (((k / 4) & 7) ^ ((c / 4) & 7)) + k % 4] = U[s0 + k][s0 + c]
  constexpr int RV = 16 * (B / 4);                 // float4 of one row chunk
  constexpr int NV = (RV + 255) / 256;             // per thread
  const bool fastU = vec && bw == B;
  auto load_rows = [&](int t, float4 (&v)[NV]) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = tid + 256 * i;
      const int k = 16 * t + e / (B / 4), c4 = (e % (B / 4)) * 4;
      v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (e >= RV) continue;
      const float* src = U + (s0 + k) * ldu + s0 + c4;
      if (fastU) {
        v[i] = *reinterpret_cast<const float4*>(src);
      } else if (k < bw) {
        if (c4 + 0 < bw) v[i].x = src[0];
        if (c4 + 1 < bw) v[i].y = src[1];
        if (c4 + 2 < bw) v[i].z = src[2];
        if (c4 + 3 < bw) v[i].w = src[3];
      }
    }
  };
  auto store_rows = [&](int t, const float4 (&v)[NV]) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int e = tid + 256 * i;
      if (e >= RV) continue;
      const int k = 16 * t + e / (B / 4), c4 = (e % (B / 4)) * 4;
      const float vv[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int c = c4 + x;
        Ut[c * UP + 4 * (((k >> 2) & 7) ^ ((c >> 2) & 7)) + (k & 3)] = vv[x];
      }
    }
  };
  float4 upre[NV];
  load_rows(0, upre);
  {
    // Warm this XCD's L2 with U's block: work-groups are dealt round-robin to
    // the 8 XCDs, and every group reads the whole block, so each takes its
    // share of the rows of the block once here; the chunk loads then hit L2.
    const int per_xcd = int((gridDim.x + 7) / 8);
    const int share = (B + per_xcd - 1) / per_xcd;  // rows per work-group
    const int r0 = int(blockIdx.x / 8) * share;
    const int e = tid;  // one float4 per thread
    const int k = r0 + e / (B / 4), c4 = (e % (B / 4)) * 4;
    if (e < share * (B / 4) && k < bw && k < r0 + share) {
      const float* src = U + (s0 + k) * ldu + s0 + c4;
      const float v = *src;  // one float per 16 bytes touches the line
      if (v != v && tid > 4096) Ds[0] = v;  // never taken: keeps the load
    }
  }
  store_rows(0, upre);
  if (rowloss) {
    for (int i = tid; i < B; i += 256) Ds[i] = i < bw ? Dg[s0 + i] : 0.f;
  }
  // accumulators: `acc` for the current chunk, ar[i] for chunk tk + 1 + i
  float acc = 0.f, ar[NT > 1 ? NT - 1 : 1];
#pragma unroll
  for (int i = 0; i < NT - 1; ++i) ar[i] = 0.f;
  if (useF && live) {
    if (j < bw) acc = F[row * ldf + s0 + j];
#pragma unroll
    for (int i = 0; i < NT - 1; ++i) {
      const int c = 16 * (i + 1) + j;
      if (c < bw) ar[i] = F[row * ldf + s0 + c];
    }
  }
  __syncthreads();

  const float s = live ? scales[row] : 1.f;
  const float inv = 1.f / s;
  const float half = L * 0.5f, cen = (L - 1) * 0.5f, hi = float(L - 1);
  // proxy loss of this row: with H = (I + U) D (I + U)^T and E = W - W^, the
  // column j of E (I + U) is the target p_j minus its rounded value, so
  // tr(E H E^T) = sum_j D_j (p_j - q_j)^2 over the columns this lane owns
  double lsum = 0.0;

  float wnext = (live && j < bw) ? W[row * ldw + s0 + j] : 0.f;
  for (int tk = 0; tk < NT; ++tk) {
    if (16 * tk >= bw) break;
    const int c = 16 * tk + j;  // this lane's column in the block
    const bool own = live && c < bw;
    const float w = wnext;
    if (tk + 1 < NT) {
      const int cn = c + 16;
      wnext = (live && cn < bw) ? W[row * ldw + s0 + cn] : 0.f;
    }
    // the chunk's 16 coefficients U[16 tk + kk][c] of this lane's column
    if (tk + 1 < NT) load_rows(tk + 1, upre);  // next chunk's rows, stored after this chunk
    float u16[16];
    {
      const float4* up = reinterpret_cast<const float4*>(Ut + c * UP);
      const int sw = (c >> 2) & 7;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float4 x = up[((4 * tk + v) & 7) ^ sw];
        u16[4 * v + 0] = x.x;
        u16[4 * v + 1] = x.y;
        u16[4 * v + 2] = x.z;
        u16[4 * v + 3] = x.w;
      }
    }
    float e16[16];
    // One pass over the 16 columns of the chunk; returns this lane's
    // accumulator as it stood at its own column (it does not change after: the
    // remaining coefficients lie below the diagonal and are zero), so the
    // owner's rounding is redone once afterwards with the same arithmetic.
    // EXACT = false rounds with p * (1/s); when an owner lane lands within 1e-4
    // of a decision boundary, where p * (1/s) and the IEEE quotient p / s might
    // differ, the chunk is redone with EXACT = true. The error sent to the row
    // is w - q with q = (k - c) * s, each rounded once (no contraction), the
    // same values the outputs store.
    auto pass = [&](auto exact_tag) -> float {
      constexpr bool EXACT = decltype(exact_tag)::value;
      float a = acc;
      static_for<16>([&](auto KI) {
        constexpr int kk = decltype(KI)::value;
        const float p = w + a;
        float y;
        if constexpr (EXACT) {
          y = p / s + half;
        } else {
          y = fmaf(p, inv, half);
        }
        const float kf = __builtin_amdgcn_fmed3f(floorf(y), 0.f, hi);
        const float ev = __fsub_rn(w, __fmul_rn(kf - cen, s));
        const float eb = row_bcast<kk>(ev);
        e16[kk] = eb;
        a = fmaf(eb, u16[kk], a);  // zero coefficient on and below the diagonal
      });
      return a;
    };
    float af = pass(std::false_type{});
    float p = w + af;
    float y = fmaf(p, inv, half);
    {
      const float fr = y - floorf(y);
      const bool near = own && ((fr < 1e-4f) | (fr > 0.9999f));
      if (__builtin_amdgcn_ballot_w64(near)) {
        af = pass(std::true_type{});
        p = w + af;
        y = p / s + half;
      }
    }
    const float kf = __builtin_amdgcn_fmed3f(floorf(y), 0.f, hi);
    const float q = __fmul_rn(kf - cen, s);
    const float err = __fsub_rn(w, q);
    const float res = p - q;
    const uint32_t code = uint32_t(kf);
    // outputs of this chunk: one column per lane
    if (own) {
      codes[row * ldcode + s0 + c] = uint8_t(code);
      if (What) What[row * ldwh + s0 + c] = q;
      Eb[row * lde + c] = err;
      if (rowloss) {
        const double r = res;
        lsum += double(Ds[c]) * (r * r);
      }
    }
    // rank-16 update of the later chunks, then shift them down by one
#pragma unroll
    for (int i = 0; i < NT - 1; ++i) {
      if (i < NT - 1 - tk) {
        const int cc = c + 16 * (i + 1);
        const float4* up = reinterpret_cast<const float4*>(Ut + cc * UP);
        const int sw = (cc >> 2) & 7;
        float t = ar[i];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float4 x = up[((4 * tk + v) & 7) ^ sw];
          t = fmaf(e16[4 * v + 0], x.x, t);
          t = fmaf(e16[4 * v + 1], x.y, t);
          t = fmaf(e16[4 * v + 2], x.z, t);
          t = fmaf(e16[4 * v + 3], x.w, t);
        }
        ar[i] = t;
      }
    }
    if (NT > 1) {
      acc = ar[0];
#pragma unroll
      for (int i = 0; i + 1 < NT - 1; ++i) ar[i] = ar[i + 1];
    }
    if (tk + 1 < NT) {  // rows of the next chunk, into the other half of the ring
      store_rows(tk + 1, upre);
      __syncthreads();
    }
  }
  if (rowloss) {
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) lsum += __shfl_xor(lsum, off, 64);
    if (live && j == 0) rowloss[row] += lsum;  // one work-group per row per launch
  }
}

// ------------------------------------------------------------------ E8

__device__ __forceinline__ uint32_t ordered_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Row RMS and the normalized copy Wn = W / rms (rms given or computed).
__global__ __launch_bounds__(256) void rownorm_kernel(const float* W, int64_t n, int64_t ldw,
                                                      float* Wn, float* rms_io, bool compute) {
  __shared__ double part[4];
  __shared__ float rms_sh;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const float* w = W + row * ldw;
  if (compute) {
    double acc = 0.0;
    for (int64_t j = tid; j < n; j += 256) acc += double(w[j]) * double(w[j]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc += __shfl_down(acc, off, 64);
    if ((tid & 63) == 0) part[tid >> 6] = acc;
    __syncthreads();
    if (tid == 0) {
      double ms = (part[0] + part[1] + part[2] + part[3]) / double(n);
      float r = float(sqrt(ms));
      if (!(r > 0.f)) r = 1.f;
      rms_io[row] = r;
      rms_sh = r;
    }
    __syncthreads();
  } else {
    if (tid == 0) rms_sh = rms_io[row];
    __syncthreads();
  }
  const float r = rms_sh;
  for (int64_t j = tid; j < n; j += 256) Wn[row * n + j] = w[j] / r;
}

__global__ void e8_norms_kernel(const float* C, float* c2, _Float16* c16) {
  int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= 65536) return;
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    s = fmaf(C[i * 8 + k], C[i * 8 + k], s);
    c16[i * 8 + k] = _Float16(C[i * 8 + k]);
  }
  c2[i] = s;
}

// Squared error of the nearest codeword, summed over all 8-vectors, for every
// candidate scale. One wave: 32 vectors x all codewords; lanes 0-31 and 32-63
// see the same vectors and different codeword rows of each 32x32 block.
typedef _Float16 e8_half8 __attribute__((ext_vector_type(8)));

// The dot products <y, c> of 32 vectors with a 32-codeword tile in one
// v_mfma_f32_32x32x16_f16: A holds each codeword twice along k (codewords are
// exact in half precision), B holds y rounded to half (k < 8) and the half
// rounding of the remainder (k >= 8), so the product is <c, hi + lo> with
// hi + lo within about 2^-22 of y, accumulated in float32. Lane (j, g) with
// j = lane mod 32 gives codeword row j of A (the same 8 halves for g = 0, 1)
// and column j of B (hi for g = 0, lo for g = 1), and receives the dots of
// vector j with codewords 8 (r / 4) + 4 g + r mod 4 of the tile (r < 16).
__device__ __forceinline__ e8_half8 e8_split_operand(const float* y8, int g) {
  e8_half8 b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const _Float16 hi = _Float16(y8[k]);
    b[k] = g == 0 ? hi : _Float16(y8[k] - float(hi));
  }
  return b;
}

// Squared error of the nearest codeword, summed over all 8-vectors, for every
// candidate scale. One wave: 32 vectors x all codewords.
template <int NC>
__global__ __launch_bounds__(256) void e8_scale_kernel(const float* __restrict__ Y, int64_t nvec,
                                                       const _Float16* __restrict__ C16,
                                                       const float* __restrict__ c2,
                                                       const float* __restrict__ cand, int ncand,
                                                       double* __restrict__ sse) {
  __shared__ double red[NC];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid < NC) red[tid] = 0.0;
  __syncthreads();
  const int64_t v0 = (int64_t(blockIdx.x) * 4 + wave) * 32;
  const int j = lane & 31, kh = lane >> 5;
  const int64_t vj = v0 + j;
  const bool live = vj < nvec;
  float y8[8];
  float y2 = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    y8[k] = live ? Y[vj * 8 + k] : 0.f;
    y2 = fmaf(y8[k], y8[k], y2);
  }
  const e8_half8 yb = e8_split_operand(y8, kh);
  float sc[NC], best[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    sc[c] = cand[c < ncand ? c : 0];
    best[c] = 3.4e38f;
  }
  // For every scale s the distance term is s n_i - 2 <y, c_i> with n_i = |c_i|^2.
  // Over codewords of one norm it is smallest at the largest dot product, and
  // fma(s, n, -2 x) does not increase with x, so each lane keeps the largest
  // dot of the current run of equal norms and folds it into the 32 minima
  // when the norm changes: the minima equal those over every codeword taken
  // one by one, for any codebook order (sorted by norm, as quip_e8_codebook
  // returns it, there are seven runs and almost every tile takes one max per
  // value).
  float run_n = c2[0], run_max = -3.4e38f;
  auto fold = [&]() {
#pragma unroll
    for (int c = 0; c < NC; ++c) best[c] = fminf(best[c], fmaf(sc[c], run_n, -2.f * run_max));
  };
  // tiles go in pairs (two independent products, so one tile's maxima overlap
  // the other's product); the next pair's codewords (as 8 halves) and norms
  // are loaded one pair ahead
  auto tile = [&](const f32x16& acc, float cn) {
    if (__all(cn == run_n)) {  // the whole tile continues the run
#pragma unroll
      for (int r = 0; r < 16; ++r) run_max = fmaxf(run_max, acc[r]);
    } else {  // a run ends inside this tile
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float n2 = __shfl(cn, 8 * (r / 4) + 4 * kh + (r % 4), 64);
        if (n2 != run_n) {
          fold();
          run_n = n2;
          run_max = -3.4e38f;
        }
        run_max = fmaxf(run_max, acc[r]);
      }
    }
  };
  const uint4* C4 = reinterpret_cast<const uint4*>(C16);
  uint4 na = C4[j], nb = C4[32 + j];
  float nca = c2[j], ncb = c2[32 + j];
  for (int cw0 = 0; cw0 < 65536; cw0 += 64) {
    const uint4 wa = na, wb = nb;
    const float ca = nca, cb = ncb;
    if (cw0 + 64 < 65536) {
      na = C4[cw0 + 64 + j];
      nb = C4[cw0 + 96 + j];
      nca = c2[cw0 + 64 + j];
      ncb = c2[cw0 + 96 + j];
    }
    f32x16 aa, ab;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      aa[r] = 0.f;
      ab[r] = 0.f;
    }
    aa = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(e8_half8, wa), yb, aa, 0, 0, 0);
    ab = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(e8_half8, wb), yb, ab, 0, 0, 0);
    tile(aa, ca);
    tile(ab, cb);
  }
  fold();
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    float other = __shfl_xor(best[c], 32, 64);
    float b = fminf(best[c], other);
    double e = live && kh == 0 ? double(y2) + double(sc[c]) * double(b) : 0.0;
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) e += __shfl_xor(e, off, 64);
    if (lane == 0 && c < ncand) atomicAdd(&red[c], e);
  }
  __syncthreads();
  if (tid < ncand && tid < NC) atomicAdd(&sse[tid], red[tid]);
}

// Pre-rounding vectors of one group step of BlockLDLQ, once per step:
// y[row][k] = Wn[row][c0 + k] + F[row][c0 + k] + sum_{c < nprev} E[row][c] U[s0 + c][c0 + k]
// (the in-block feedback of the block's earlier groups). 16 lanes per row
// split the sum over c and add their partial sums with lane shuffles.
__global__ __launch_bounds__(256) void e8_prerounding_kernel(
    const float* __restrict__ Wn, int64_t n, const float* __restrict__ F, bool useF,
    const float* __restrict__ Eb, int64_t lde, int nprev, const float* __restrict__ U,
    int64_t c0, int64_t s0, int64_t m, float* __restrict__ y8) {
  const int sub = threadIdx.x & 15;
  const int64_t row = int64_t(blockIdx.x) * 16 + (threadIdx.x >> 4);
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  if (row < m) {
    for (int c = sub; c < nprev; c += 16) {
      const float e = Eb[row * lde + c];
      const float* u = U + (s0 + c) * n + c0;
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = fmaf(e, u[k], acc[k]);
    }
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] += __shfl_xor(acc[k], o, 64);
  }
  if (row < m && sub < 8) {
    float v = acc[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) v = sub == k ? acc[k] : v;
    float y = Wn[row * n + c0 + sub] + v;
    if (useF) y += F[row * n + c0 + sub];
    y8[row * 8 + sub] = y;
  }
}

// One group step of BlockLDLQ: the nearest scaled codeword to each row's
// pre-rounding vector over a chunk of codewords (4 waves split the chunk;
// atomicMin of a packed (distance, index) key per row). The dot products come
// from the split half-precision product of e8_scale_kernel; the distance term
// s n_i - 2 <y, c_i> is smallest, over a run of equal norms, at the largest
// dot, so each lane keeps that dot (and its first index) per run and compares
// runs by distance; ties go to the lower index.
__global__ __launch_bounds__(256) void e8_argmin_kernel(
    const float* __restrict__ y8g, const _Float16* __restrict__ C16, const float* __restrict__ c2,
    const float* __restrict__ sp, int64_t m, int chunk, unsigned long long* __restrict__ keys) {
  __shared__ unsigned long long ksh[4][32];
  const float s = *sp;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t r0 = int64_t(blockIdx.x) * 32;
  const int j = lane & 31, kh = lane >> 5;
  float y8[8];
  {
    const int64_t row = r0 + j;
#pragma unroll
    for (int k = 0; k < 8; ++k) y8[k] = row < m ? y8g[row * 8 + k] : 0.f;
  }
  const e8_half8 yb = e8_split_operand(y8, kh);
  const int cbeg = blockIdx.y * chunk + wave * (chunk / 4);
  const int cend = cbeg + chunk / 4;
  float bestv = 3.4e38f;
  int besti = cbeg;  // always a valid codeword, even if every distance is NaN
  float run_n = c2[cbeg], run_max = -3.4e38f;
  int run_i = cbeg;
  auto fold = [&]() {
    const float v = fmaf(s, run_n, -2.f * run_max);
    if (v < bestv) {  // runs are visited in increasing index within a lane
      bestv = v;
      besti = run_i;
    }
  };
  // tiles in pairs, as in e8_scale_kernel
  auto tile = [&](const f32x16& acc, float cn, int cw0) {
    if (__all(cn == run_n)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = cw0 + 8 * (r / 4) + 4 * kh + (r % 4);
        const bool gt = acc[r] > run_max;
        run_max = gt ? acc[r] : run_max;
        run_i = gt ? i : run_i;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = cw0 + 8 * (r / 4) + 4 * kh + (r % 4);
        const float n2 = __shfl(cn, 8 * (r / 4) + 4 * kh + (r % 4), 64);
        if (n2 != run_n) {
          fold();
          run_n = n2;
          run_max = -3.4e38f;
          run_i = i;
        }
        const bool gt = acc[r] > run_max;
        run_max = gt ? acc[r] : run_max;
        run_i = gt ? i : run_i;
      }
    }
  };
  const uint4* C4 = reinterpret_cast<const uint4*>(C16);
  uint4 na = C4[cbeg + j], nb = C4[cbeg + 32 + j];
  float nca = c2[cbeg + j], ncb = c2[cbeg + 32 + j];
  for (int cw0 = cbeg; cw0 < cend; cw0 += 64) {  // chunk / 4 is a multiple of 64
    const uint4 wa = na, wb = nb;
    const float ca = nca, cb = ncb;
    if (cw0 + 64 < cend) {
      na = C4[cw0 + 64 + j];
      nb = C4[cw0 + 96 + j];
      nca = c2[cw0 + 64 + j];
      ncb = c2[cw0 + 96 + j];
    }
    f32x16 aa, ab;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      aa[r] = 0.f;
      ab[r] = 0.f;
    }
    aa = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(e8_half8, wa), yb, aa, 0, 0, 0);
    ab = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(e8_half8, wb), yb, ab, 0, 0, 0);
    tile(aa, ca, cw0);
    tile(ab, cb, cw0 + 32);
  }
  fold();
  unsigned long long key = (unsigned long long)ordered_bits(bestv) << 32 | uint32_t(besti);
  unsigned long long other = __shfl_xor(key, 32, 64);
  key = key < other ? key : other;
  if (kh == 0) ksh[wave][j] = key;
  __syncthreads();
  if (tid < 32) {
    unsigned long long k2 = ksh[0][tid];
    for (int wv = 1; wv < 4; ++wv) k2 = ksh[wv][tid] < k2 ? ksh[wv][tid] : k2;
    if (r0 + tid < m) atomicMin(&keys[r0 + tid], k2);
  }
}

// Finish a group step: codes, quantized values, errors; reset the keys. With
// rowloss, also the group's proxy-loss term rms^2 (y - q) D_g (y - q)^T, y the
// pre-rounding vector (normalized domain) of e8_prerounding_kernel.
__global__ void e8_finish_kernel(const float* __restrict__ Wn, int64_t n, const float* __restrict__ C,
                                 const float* __restrict__ sp, const float* __restrict__ rms,
                                 int64_t c0, int64_t m,
                                 unsigned long long* __restrict__ keys, uint16_t* __restrict__ codes,
                                 int64_t ldcode, float* __restrict__ What, float* __restrict__ Eb,
                                 int64_t lde, int ecol, const float* __restrict__ y8,
                                 const float* __restrict__ Dg, double* __restrict__ rowloss) {
  const int64_t row = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (row >= m) return;
  const float s = *sp;
  const uint32_t code = uint32_t(keys[row] & 0xFFFFull);
  keys[row] = ~0ull;
  codes[row * ldcode + c0 / 8] = uint16_t(code);
  const float r = rms[row];
  double res[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float qv = s * C[code * 8 + k];
    if (rowloss) res[k] = double(y8[row * 8 + k]) - double(qv);
    Eb[row * lde + ecol + k] = Wn[row * n + c0 + k] - qv;
    if (What) What[row * n + c0 + k] = r * qv;
  }
  if (rowloss) {
    double acc = 0.0;
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      double t = 0.0;
#pragma unroll
      for (int b = 0; b < 8; ++b) t += double(Dg[(c0 + a) * 8 + b]) * res[b];
      acc += res[a] * t;
    }
    rowloss[row] += double(r) * double(r) * acc;
  }
}

// loss = sum of the row losses, in a fixed order (one work-group).
__global__ __launch_bounds__(256) void sum_rows_kernel(const double* __restrict__ rowloss,
                                                       int64_t m, double* __restrict__ out) {
  __shared__ double part[256];
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < m; i += 256) acc += rowloss[i];
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (int(threadIdx.x) < h) part[threadIdx.x] += part[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = part[0];
}

__global__ void fill_u64_kernel(unsigned long long* p, int64_t count, unsigned long long v) {
  int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i < count) p[i] = v;
}

__global__ void e8_pick_scale_kernel(const double* sse, const float* cand, int ncand,
                                     float* scales) {
  if (threadIdx.x != 0) return;
  int best = 0;
  for (int c = 1; c < ncand; ++c)
    if (sse[c] < sse[best]) best = c;
  scales[0] = cand[best];
}

// ------------------------------------------------------------------ host helpers

void host_grid_factors(int ncand, float* out) {
  for (int c = 0; c < ncand; ++c) out[c] = float(pow(16.0, -double(c) / double(ncand - 1)));
}
void host_e8_candidates(int ncand, float* out) {
  for (int c = 0; c < ncand; ++c) out[c] = float(0.5 * pow(4.0, double(c) / double(ncand - 1)));
}

quip_status finish_loss(const double* rl, int64_t m, double* loss, hipStream_t s) {
  if (!loss) return QUIP_OK;
  return timed_launch("sum_rows_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL(sum_rows_kernel, dim3(1), dim3(256), 0, s, rl, m, loss);
  });
}

struct E8Ws {
  float* Wn;
  float* F;
  float* Eb;
  unsigned long long* keys;
  float* c2;
  _Float16* c16;  // the codebook in half precision (exact: multiples of 1/2 up to 3.5)
  float* cand;
  double* sse;
};

quip_status grid_scales(const float* W, int64_t m, int64_t n, int64_t ldw, int L, int ncand,
                        float* factors_dev, float* scales, float* mse, hipStream_t s) {
  // work: every candidate step rounds every weight of the row once
  const double gfl = double(m) * double(n) * double(ncand) * 6.0;
  const double gby = 4.0 * double(m) * double(n) + 4.0 * double(m);
  return timed_launch("grid_scale_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    if (ncand <= 32)
      QUIP_KERNEL((grid_scale_kernel<32>), dim3(unsigned(m)), dim3(256), 0, s, W, m, n, ldw, L,
                         ncand, factors_dev, scales, mse);
    else
      QUIP_KERNEL((grid_scale_kernel<64>), dim3(unsigned(m)), dim3(256), 0, s, W, m, n, ldw, L,
                         ncand, factors_dev, scales, mse);
  }, gfl, gby);
}

quip_status e8_scales(const float* Wn, int64_t m, int64_t n, const float* C, const E8Ws& e,
                      int ncand, float* scales, double* sse_out, hipStream_t s) {
  QUIP_TRY(fill_f64(e.sse, 64, 0.0, s));
  const int64_t nvec = m * (n / 8);
  dim3 grid(unsigned(cdiv(nvec, 128)));
  QUIP_TRY(timed_launch("e8_scale_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    if (ncand <= 32)
      QUIP_KERNEL((e8_scale_kernel<32>), grid, dim3(256), 0, s, Wn, nvec, e.c16, e.c2, e.cand,
                         ncand, e.sse);
    else
      QUIP_KERNEL((e8_scale_kernel<64>), grid, dim3(256), 0, s, Wn, nvec, e.c16, e.c2, e.cand,
                         ncand, e.sse);
  }, 16.0 * 65536.0 * double(nvec), 32.0 * double(nvec)));  // <y, c> for every vector and codeword
  QUIP_TRY(timed_launch("e8_pick_scale_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL(e8_pick_scale_kernel, dim3(1), dim3(64), 0, s, e.sse, e.cand, ncand, scales);
  }));
  if (sse_out) QUIP_HIP(hipMemcpyAsync(sse_out, e.sse, sizeof(double) * ncand, hipMemcpyDeviceToDevice, s));
  return QUIP_OK;
}

template <int B>
quip_status sweep_t(const float* W, int64_t ldw, const float* F, int64_t ldf, bool useF,
                    const float* U, int64_t ldu, const float* scales, int L, int64_t m, int64_t s0,
                    int bw, uint8_t* codes, int64_t ldc, float* What, int64_t ldwh, float* Eb,
                    int64_t lde, const float* D, double* rowloss, hipStream_t s) {
  const size_t shmem = (size_t(B) * 36 + B) * sizeof(float);
  if (shmem > 65536)
    QUIP_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(&ldlq_sweep_kernel<B>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, int(shmem)));
  // float4 paths need 16-byte alignment of every row start and of the block start
  const bool vec = aligned16(W) && aligned16(F) && aligned16(U) && aligned16(Eb) &&
                   (What == nullptr || aligned16(What)) &&
                   ((reinterpret_cast<uintptr_t>(codes) & 3) == 0) && ldw % 4 == 0 &&
                   ldf % 4 == 0 && ldu % 4 == 0 && ldc % 4 == 0 && ldwh % 4 == 0 &&
                   lde % 4 == 0 && s0 % 4 == 0;
  // work: per row the in-block feedback (bw (bw - 1) flops) and the rounding;
  // reads W, F and the U block, writes codes, W^ and the errors
  const double md = double(m), bd = double(bw);
  const double flops = md * (bd * (bd - 1.0) + 6.0 * bd);
  const double bytes = md * bd * (4.0 + (useF ? 4.0 : 0.0) + 1.0 + (What ? 4.0 : 0.0) + 4.0) +
                       4.0 * bd * bd + (rowloss ? 16.0 * md : 0.0);
  return timed_launch("ldlq_sweep_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL((ldlq_sweep_kernel<B>), dim3(unsigned(cdiv(m, 16))), dim3(256), shmem, s, W, ldw,
                       F, ldf, useF, U, ldu, scales, L, m, s0, bw, codes, ldc, What, ldwh, Eb, lde,
                       D, rowloss, vec);
  }, flops, bytes);
}

quip_status sweep(int b, const float* W, int64_t ldw, const float* F, int64_t ldf, bool useF,
                  const float* U, int64_t ldu, const float* scales, int L, int64_t m, int64_t s0,
                  int bw, uint8_t* codes, int64_t ldc, float* What, int64_t ldwh, float* Eb,
                  int64_t lde, const float* D, double* rowloss, hipStream_t s) {
  switch (b) {
    case 32: return sweep_t<32>(W, ldw, F, ldf, useF, U, ldu, scales, L, m, s0, bw, codes, ldc, What, ldwh, Eb, lde, D, rowloss, s);
    case 64: return sweep_t<64>(W, ldw, F, ldf, useF, U, ldu, scales, L, m, s0, bw, codes, ldc, What, ldwh, Eb, lde, D, rowloss, s);
    case 128: return sweep_t<128>(W, ldw, F, ldf, useF, U, ldu, scales, L, m, s0, bw, codes, ldc, What, ldwh, Eb, lde, D, rowloss, s);
    case 256: return sweep_t<256>(W, ldw, F, ldf, useF, U, ldu, scales, L, m, s0, bw, codes, ldc, What, ldwh, Eb, lde, D, rowloss, s);
  }
  return fail(QUIP_ERR_UNSUPPORTED, "ldlq: inner block size");
}

// F[:, c0:c1] (+)= Eb[:, e0:e0+K] U[r0:r0+K, c0:c1]
quip_status feedback_gemm(const float* Eb, int64_t lde, int64_t e0, int64_t K, const float* U,
                          int64_t n, int64_t r0, int64_t c0, int64_t c1, float* F, int64_t m,
                          bool accumulate, const char* tag, hipStream_t s) {
  if (c1 <= c0 || K <= 0) return QUIP_OK;
  GemmArgs a;
  a.M = m;
  a.N = c1 - c0;
  a.K = K;
  a.A = Eb + e0;
  a.lda = lde;
  a.B = U + r0 * n + c0;
  a.ldb = n;
  a.C = F + c0;
  a.ldc = n;
  a.alpha = 1.f;
  a.beta = accumulate ? 1.f : 0.f;
  a.tag = tag;
  return gemm(a, s);
}

}  // namespace

size_t scales_workspace_bytes(int64_t m, int64_t n, const quip_quantizer& q) {
  Carver c(nullptr, 0);
  c.take<float>(64);  // candidate factors
  if (q.kind == QUIP_Q_E8) {
    c.take<float>(size_t(m) * n);  // Wn
    c.take<float>(65536);          // |c|^2
    c.take<_Float16>(65536 * 8);   // the codebook in half precision
    c.take<double>(64);            // sse
  }
  return c.used;
}

quip_status scales_run(const float* W, int64_t m, int64_t n, int64_t ldw, const quip_quantizer& q,
                       float* scales, void* mse_out, const float* codebook, void* ws,
                       size_t ws_bytes, hipStream_t s) {
  Carver c(ws, ws_bytes);
  float* fac = c.take<float>(64);
  float hostf[64];
  if (q.kind == QUIP_Q_UNIFORM) {
    if (!c.fits()) return fail(QUIP_ERR_WORKSPACE, "quip_scales: workspace too small");
    host_grid_factors(q.n_cand, hostf);
    QUIP_HIP(hipMemcpyAsync(fac, hostf, sizeof(float) * q.n_cand, hipMemcpyHostToDevice, s));
    return grid_scales(W, m, n, ldw, 1 << q.bits, q.n_cand, fac, scales,
                       static_cast<float*>(mse_out), s);
  }
  E8Ws e{};
  e.Wn = c.take<float>(size_t(m) * n);
  e.c2 = c.take<float>(65536);
  e.c16 = c.take<_Float16>(65536 * 8);
  e.sse = c.take<double>(64);
  e.cand = fac;
  if (!c.fits()) return fail(QUIP_ERR_WORKSPACE, "quip_scales: workspace too small");
  host_e8_candidates(q.n_cand, hostf);
  QUIP_HIP(hipMemcpyAsync(fac, hostf, sizeof(float) * q.n_cand, hipMemcpyHostToDevice, s));
  QUIP_TRY(timed_launch("rownorm_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL(rownorm_kernel, dim3(unsigned(m)), dim3(256), 0, s, W, n, ldw, e.Wn, scales + 1,
                       true);
  }));
  QUIP_TRY(timed_launch("e8_norms_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL(e8_norms_kernel, dim3(256), dim3(256), 0, s, codebook, e.c2, e.c16);
  }));
  return e8_scales(e.Wn, m, n, codebook, e, q.n_cand, scales, static_cast<double*>(mse_out), s);
}

// Trailing-update batch of the scalar sweep: the lazily updated block of B
// columns is swept in sub-blocks of at most 128 columns (the sweep kernel), the
// rest of each 512-column batch is updated after every sub-block, and the rest
// of the matrix once per batch (one K = 512 product instead of four K = 128
// ones: a quarter of the read-modify-write traffic of F).
static int64_t outer_block(int64_t n, int g, int64_t B) {
  if (g != 1) return B;
  int64_t bo = B >= 512 ? B : B * (512 / B);
  return bo < n ? bo : n;
}

size_t ldlq_workspace_bytes(int64_t m, int64_t n, int g, int64_t B, const quip_quantizer& q) {
  Carver c(nullptr, 0);
  c.take<float>(64);
  c.take<float>(size_t(m) * n);  // F
  c.take<float>(size_t(m) * outer_block(n, g, B));  // Eb
  c.take<double>(size_t(m));                         // per-row proxy loss
  if (q.kind == QUIP_Q_E8) {
    c.take<float>(size_t(m) * n);  // Wn
    c.take<unsigned long long>(size_t(m));
    c.take<float>(size_t(m) * 8);  // pre-rounding vectors of a group step
    c.take<float>(65536);
    c.take<_Float16>(65536 * 8);
    c.take<double>(64);
  }
  (void)g;
  return c.used;
}

quip_status ldlq_run(const float* W, int64_t m, int64_t n, int64_t ldw, const float* U,
                     const float* D, int g, int64_t B, const quip_quantizer& q, float* scales,
                     void* codes, float* What, const float* codebook, double* row_loss,
                     double* loss, void* ws, size_t ws_bytes, hipStream_t s) {
  Carver c(ws, ws_bytes);
  float* fac = c.take<float>(64);
  float* F = c.take<float>(size_t(m) * n);
  const int64_t Bo = outer_block(n, g, B);
  float* Eb = c.take<float>(size_t(m) * Bo);
  double* rl_ws = c.take<double>(size_t(m));
  float hostf[64];
  // per-row proxy loss: the caller's buffer, or the workspace when only the total is wanted
  double* rl = row_loss ? row_loss : (loss ? rl_ws : nullptr);
  if (rl && c.fits()) QUIP_TRY(fill_f64(rl, m, 0.0, s));

  if (q.kind == QUIP_Q_UNIFORM) {
    if (!c.fits()) return fail(QUIP_ERR_WORKSPACE, "quip_ldlq: workspace too small");
    const int L = 1 << q.bits;
    if (q.scale_mode == QUIP_SCALE_COMPUTE) {
      host_grid_factors(q.n_cand, hostf);
      QUIP_HIP(hipMemcpyAsync(fac, hostf, sizeof(float) * q.n_cand, hipMemcpyHostToDevice, s));
      QUIP_TRY(grid_scales(W, m, n, ldw, L, q.n_cand, fac, scales, nullptr, s));
    }
    const int bi = B >= 256 ? 256 : (B >= 128 ? 128 : (B >= 64 ? 64 : 32));
    uint8_t* cd = static_cast<uint8_t*>(codes);
    for (int64_t j0 = 0; j0 < n; j0 += Bo) {
      const int64_t bo = (n - j0 < Bo) ? n - j0 : Bo;
      for (int64_t s0 = j0; s0 < j0 + bo; s0 += bi) {
        const int bw = int((j0 + bo - s0) < bi ? (j0 + bo - s0) : bi);
        QUIP_TRY(sweep(bi, W, ldw, F, n, s0 > 0, U, n, scales, L, m, s0, bw, cd, n, What, n,
                       Eb + (s0 - j0), Bo, D, rl, s));
        // rest of this batch
        QUIP_TRY(feedback_gemm(Eb, Bo, s0 - j0, bw, U, n, s0, s0 + bw, j0 + bo, F, m,
                               !(j0 == 0 && s0 == 0), "gemm:ldlq_inner", s));
      }
      QUIP_TRY(feedback_gemm(Eb, Bo, 0, bo, U, n, j0, j0 + bo, n, F, m, j0 > 0, "gemm:ldlq_outer", s));
    }
    return finish_loss(rl, m, loss, s);
  }

  // ---- E8, g = 8
  E8Ws e{};
  e.Wn = c.take<float>(size_t(m) * n);
  e.keys = c.take<unsigned long long>(size_t(m));
  float* y8 = c.take<float>(size_t(m) * 8);
  e.c2 = c.take<float>(65536);
  e.c16 = c.take<_Float16>(65536 * 8);
  e.sse = c.take<double>(64);
  e.cand = fac;
  e.F = F;
  e.Eb = Eb;
  if (!c.fits()) return fail(QUIP_ERR_WORKSPACE, "quip_ldlq: workspace too small");
  const bool compute = q.scale_mode == QUIP_SCALE_COMPUTE;
  QUIP_TRY(timed_launch("rownorm_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL(rownorm_kernel, dim3(unsigned(m)), dim3(256), 0, s, W, n, ldw, e.Wn, scales + 1,
                       compute);
  }));
  QUIP_TRY(timed_launch("e8_norms_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL(e8_norms_kernel, dim3(256), dim3(256), 0, s, codebook, e.c2, e.c16);
  }));
  if (compute) {
    host_e8_candidates(q.n_cand, hostf);
    QUIP_HIP(hipMemcpyAsync(fac, hostf, sizeof(float) * q.n_cand, hipMemcpyHostToDevice, s));
    QUIP_TRY(e8_scales(e.Wn, m, n, codebook, e, q.n_cand, scales, nullptr, s));
  }
  // the global scale stays on the device (scales[0]); the step kernels read it there
  const float* sglob = scales;
  QUIP_TRY(timed_launch("fill_u64_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL(fill_u64_kernel, dim3(unsigned(cdiv(m, 256))), dim3(256), 0, s, e.keys, m, ~0ull);
  }));
  uint16_t* cd = static_cast<uint16_t*>(codes);
  const int chunk = 4096;
  for (int64_t j0 = 0; j0 < n; j0 += B) {
    const int64_t bo = (n - j0 < B) ? n - j0 : B;
    for (int64_t c0 = j0; c0 < j0 + bo; c0 += 8) {
      const int nprev = int(c0 - j0);
      QUIP_TRY(timed_launch("e8_prerounding_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
        QUIP_KERNEL(e8_prerounding_kernel, dim3(unsigned(cdiv(m, 16))), dim3(256), 0, s, e.Wn, n, F,
                    j0 > 0, Eb, B, nprev, U, c0, j0, m, y8);
      }, 16.0 * double(m) * double(nprev), 4.0 * double(m) * (double(nprev) + 24.0)));
      dim3 grid(unsigned(cdiv(m, 32)), unsigned(65536 / chunk));
      QUIP_TRY(timed_launch("e8_argmin_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
        QUIP_KERNEL(e8_argmin_kernel, grid, dim3(256), 0, s, y8, e.c16, e.c2, sglob, m, chunk,
                    e.keys);
      }, 16.0 * 65536.0 * double(m), 32.0 * double(m) + 8.0 * double(m) * 8.0));
      QUIP_TRY(timed_launch("e8_finish_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
        QUIP_KERNEL(e8_finish_kernel, dim3(unsigned(cdiv(m, 256))), dim3(256), 0, s, e.Wn, n,
                           codebook, sglob, scales + 1, c0, m, e.keys, cd, n / 8, What, Eb, B,
                           nprev, y8, D, rl);
      }));
    }
    QUIP_TRY(feedback_gemm(Eb, B, 0, bo, U, n, j0, j0 + bo, n, F, m, j0 > 0, "gemm:ldlq_outer", s));
  }
  return finish_loss(rl, m, loss, s);
}

}  // namespace quip
