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
// Scalar grid sweep: a work-group of 4 waves holds 16 rows; each row is one
// 16-lane DPP row of its wave, and lane j owns column 16 t + j of the current
// 16-column chunk t. Every lane evaluates the rounding of its own target; the
// error of column kk reaches the whole row with one DPP row_newbcast from its
// owner, and each lane adds its share of the feedback with U's coefficients
// staged transposed in LDS one chunk ahead.
//
// E8 groups: the pre-rounding 8-vectors of all rows are searched against the
// 65536 codewords as a dot-product contraction on the matrix cores
// (codewords x rows; each vector as two half-precision parts, K = 16), with
// the per-row result kept as a packed (order-preserving distance bits,
// reference) 64-bit key and atomicMin; the last work-group of each row block
// resolves the codes and finishes the step.
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
//
// Feedback of the earlier sub-blocks of the same batch (left-looking): the
// columns [kb0, s0) with kb0 = s0 - kfold were rounded by earlier launches,
// their errors are in Ef (same rows, leading dimension lde), and their share
// of this block's targets, G = Ef[:, 0:kfold] U[kb0:s0, s0:s0+bw], is formed
// here on the matrix cores before the sweep starts and added to the
// accumulators (the rest of the matrix receives it through the batch's outer
// product). F holds the earlier batches' feedback when useF.
template <int B, bool VEC>
__device__ __forceinline__ void sweep_fold(const float* __restrict__ Ef, int64_t lde,
                                           const float* __restrict__ U, int64_t ldu, int64_t s0,
                                           int kfold, int bw, int64_t row0, int64_t m,
                                           float* __restrict__ Gs);

template <int B, bool FOLD>
__global__ __launch_bounds__(256) void ldlq_sweep_kernel(
    const float* __restrict__ W, int64_t ldw, const float* __restrict__ F, int64_t ldf, bool useF,
    const float* __restrict__ U, int64_t ldu, const float* __restrict__ scales, int L, int64_t m,
    int64_t s0, int bw, uint8_t* __restrict__ codes, int64_t ldcode, float* __restrict__ What,
    int64_t ldwh, float* __restrict__ Eb, int64_t lde, const float* __restrict__ Dg,
    double* __restrict__ rowloss, bool vec, const float* __restrict__ Ef, int kfold) {
  constexpr int NT = B / 16;  // 16-column chunks
  constexpr int UP = 36;      // two 16-row chunks of U (a ring) and a pad, per column
  constexpr int GLD = B + 4;  // row length of the fold's result tile
  extern __shared__ __align__(16) float sm[];
  float* Ut = sm;            // [B][UP]: column c of U's rows of the current and next chunk
  float* Ds = sm + B * UP;   // [B]: D of the block (proxy loss)
  float* Gs = Ds + B;        // [16][GLD]: the fold's feedback for the 16 rows

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
  if (FOLD && kfold > 0) {
    if (vec)
      sweep_fold<B, true>(Ef, lde, U, ldu, s0, kfold, bw, int64_t(blockIdx.x) * 16, m, Gs);
    else
      sweep_fold<B, false>(Ef, lde, U, ldu, s0, kfold, bw, int64_t(blockIdx.x) * 16, m, Gs);
    __syncthreads();
    const float* g = Gs + (tid >> 4) * GLD;
    if (j < bw) acc += g[j];
#pragma unroll
    for (int i = 0; i < NT - 1; ++i) {
      const int c = 16 * (i + 1) + j;
      if (c < bw) ar[i] += g[c];
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
    // owner's rounding is redone once afterwards. EXACT = false rounds with
    // a * (1/s) + (w * (1/s) + L/2), the part that does not depend on the
    // feedback formed before the chain; when an owner lane lands within 1e-4
    // of a decision boundary, where that and the IEEE quotient (w + a) / s
    // might differ, the chunk is redone with EXACT = true, so every code sent
    // is the one the outputs store. The error sent to the row is
    // (w + c s) - k s (one fma on the precomputed w + c s), the value the
    // outputs store.
    const float wh = fmaf(w, inv, half), wcs = fmaf(cen, s, w);
    auto pass = [&](auto exact_tag) -> float {
      constexpr bool EXACT = decltype(exact_tag)::value;
      float a = acc;
      static_for<16>([&](auto KI) {
        constexpr int kk = decltype(KI)::value;
        float y;
        if constexpr (EXACT) {
          y = (w + a) / s + half;
        } else {
          y = fmaf(a, inv, wh);
        }
        const float kf = __builtin_amdgcn_fmed3f(floorf(y), 0.f, hi);
        const float ev = fmaf(-s, kf, wcs);
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
    const float err = fmaf(-s, kf, wcs);
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
    // rank-16 update of the NR = NT - 1 - tk later chunks, then shift them
    // down by one. NR is made a compile-time count so that the NR chains go
    // interleaved (one LDS read of every chain, then four fmas of every chain,
    // per float4 of coefficients); each chain keeps its own order of fmas.
    auto rank_update = [&](auto nr_tag) {
      constexpr int NR = decltype(nr_tag)::value;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float4 x[NR];
        static_for<NR>([&](auto I) {
          constexpr int i = decltype(I)::value;
          const int cc = c + 16 * (i + 1);
          const float4* up = reinterpret_cast<const float4*>(Ut + cc * UP);
          x[i] = up[((4 * tk + v) & 7) ^ ((cc >> 2) & 7)];
        });
        static_for<NR>([&](auto I) {
          constexpr int i = decltype(I)::value;
          float t = ar[i];
          t = fmaf(e16[4 * v + 0], x[i].x, t);
          t = fmaf(e16[4 * v + 1], x[i].y, t);
          t = fmaf(e16[4 * v + 2], x[i].z, t);
          t = fmaf(e16[4 * v + 3], x[i].w, t);
          ar[i] = t;
        });
      }
    };
    static_for<NT>([&](auto K) {
      constexpr int NR = decltype(K)::value;
      if constexpr (NR > 0) {
        if (NR == NT - 1 - tk) rank_update(std::integral_constant<int, NR>{});
      }
    });
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
    // one work-group per row per launch; the sweep at column 0 starts the sum
    if (live && j == 0) rowloss[row] = (s0 == 0 ? 0.0 : rowloss[row]) + lsum;
  }
}

typedef float sw_f32x4 __attribute__((ext_vector_type(4)));

// G[r][c] = sum_k Ef[row0 + r][k] U[s0 - kfold + k][s0 + c] for the 16 rows
// of the work-group, written to Gs[r][c] (row length B + 4); columns c >= bw
// and rows past m hold values of clamped addresses that the caller ignores.
// v_mfma_f32_16x16x4f32 on 16 x 16 tiles, tile t of the block on wave t % 4:
// lane (i, h) = (lane % 16, lane / 16) supplies A[i][k] and B[k][i] for the k
// of its quarter h, and holds D[4 h + r][i] in element r. A 16-wide k step is
// one float4 of Ef per lane (quarter h takes k = 4 h .. 4 h + 3, one per
// instruction) and four U values per tile; four steps are in flight. kfold is
// a multiple of 32.
template <int B, bool VEC>
__device__ __forceinline__ void sweep_fold(const float* __restrict__ Ef, int64_t lde,
                                           const float* __restrict__ U, int64_t ldu, int64_t s0,
                                           int kfold, int bw, int64_t row0, int64_t m,
                                           float* __restrict__ Gs) {
  constexpr int CT = B / 16;         // 16-column tiles of the block
  constexpr int TW = (CT + 3) / 4;   // tiles per wave
  constexpr int GLD = B + 4;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, h = lane >> 4;
  // tile tt of this wave exists (known at compile time unless B = 32)
  auto has = [&](int tt) { return CT >= 4 * (tt + 1) || wave + 4 * tt < CT; };
  const float* ea = Ef + (row0 + li < m ? row0 + li : 0) * lde + 4 * h;
  const float* ub[TW];
#pragma unroll
  for (int tt = 0; tt < TW; ++tt) {
    const int col = 16 * (wave + 4 * tt) + li;
    ub[tt] = U + (s0 - kfold + 4 * h) * ldu + s0 + (col < bw ? col : 0);
  }
  sw_f32x4 acc[TW];
#pragma unroll
  for (int tt = 0; tt < TW; ++tt) acc[tt] = sw_f32x4{0.f, 0.f, 0.f, 0.f};

  struct Ops {
    float a[4];
    float b[TW][4];
  };
  auto load = [&](int kb, Ops& o) {
    if constexpr (VEC) {
      const float4 v = *reinterpret_cast<const float4*>(ea + kb);
      o.a[0] = v.x;
      o.a[1] = v.y;
      o.a[2] = v.z;
      o.a[3] = v.w;
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) o.a[t] = ea[kb + t];
    }
#pragma unroll
    for (int tt = 0; tt < TW; ++tt) {
      if (has(tt)) {
#pragma unroll
        for (int t = 0; t < 4; ++t) o.b[tt][t] = ub[tt][int64_t(kb + t) * ldu];
      }
    }
  };
  auto mma = [&](const Ops& o) {
#pragma unroll
    for (int tt = 0; tt < TW; ++tt) {
      if (has(tt)) {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[tt] = __builtin_amdgcn_mfma_f32_16x16x4f32(o.a[t], o.b[tt][t], acc[tt], 0, 0, 0);
      }
    }
  };
  // loads are never skipped (a step past the end reloads the last one), so
  // the loop body has no branch around a load and four steps stay in flight
  auto kc = [&](int k) { return k < kfold ? k : kfold - 16; };
  Ops o0, o1, o2, o3;
  load(0, o0);
  load(16, o1);
  load(kc(32), o2);
  load(kc(48), o3);
  // (the scheduling barriers keep this order: otherwise the compiler sinks
  // the loads next to their use and only one step is in flight)
  for (int kb = 0; kb < kfold; kb += 64) {
    mma(o0);
    __builtin_amdgcn_sched_barrier(0);
    load(kc(kb + 64), o0);
    __builtin_amdgcn_sched_barrier(0);
    mma(o1);
    __builtin_amdgcn_sched_barrier(0);
    load(kc(kb + 80), o1);
    __builtin_amdgcn_sched_barrier(0);
    if (kb + 32 < kfold) {
      mma(o2);
      mma(o3);
    }
    __builtin_amdgcn_sched_barrier(0);
    load(kc(kb + 96), o2);
    load(kc(kb + 112), o3);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int tt = 0; tt < TW; ++tt) {
    if (has(tt)) {
#pragma unroll
      for (int r = 0; r < 4; ++r) Gs[(4 * h + r) * GLD + 16 * (wave + 4 * tt) + li] = acc[tt][r];
    }
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

// The search kernels load the codewords of the next two pairs of 32-codeword
// tiles ahead of their use, also past their last pair (up to three pairs past
// it); the half-precision copy and the norms carry E8_PAD more rows (copies of
// the first codewords) so those loads stay inside the buffers. Their products
// are never used.
constexpr int E8_PAD = 256;
constexpr int E8_ROWS = 65536 + E8_PAD;

__global__ void e8_norms_kernel(const float* C, float* c2, _Float16* c16) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= E8_ROWS) return;
  const int src = i & 65535;
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    s = fmaf(C[src * 8 + k], C[src * 8 + k], s);
    c16[i * 8 + k] = _Float16(C[src * 8 + k]);
  }
  c2[i] = s;
}

// The lattice is symmetric: -c is a lattice point of the same norm as c. In
// the codebook of quip_e8_codebook (squared norm, then coordinates in
// increasing order) each full shell of squared norm 2, 4, 6, 8 and 10,
// [E8_SH_A[r], E8_SH_A[r] + E8_SH_S[r]), holds the negation of its i-th point
// at position a + S - 1 - i (negation reverses the coordinate order). A search
// over one member of each such pair, with |<y, c>| in place of <y, c>, finds the
// same minima: over {c, -c}, s |c|^2 - 2 <y, +-c> is smallest at the sign of
// <y, c>. The search layout holds the first halves of the five shells (the
// symmetric region, E8_SYM_CW entries with padding) and then the zero vector and
// the partial shell of squared norm 12 as they are (the plain region). For any
// other codebook the pairing check fails and the kernels search the codebook
// as given.
__constant__ int E8_SH_A[5] = {1, 241, 2401, 9121, 26641};
__constant__ int E8_SH_S[5] = {240, 2160, 6720, 17520, 30240};
__constant__ int E8_SH_OFF[6] = {0, 120, 1200, 4560, 13320, 28440};
constexpr int E8_SYM_HALF = 28440;                          // first halves of the five shells
constexpr int E8_SYM_CW = 28480;                            // padded to whole pairs (445)
constexpr int E8_PLAIN_CW = 1 + (65536 - 56881);            // zero vector + the partial shell
constexpr int E8_LAYOUT_CW = E8_SYM_CW + 8704;              // plain region padded (136 pairs)
static_assert(E8_PLAIN_CW <= 8704, "plain region");

// One thread per entry of the symmetric search layout: its codeword (half
// precision) and norm, the codebook index it stands for and that of its
// negation. Padding repeats the region's last entry. bad is set if a pair of
// the symmetric region is not c, -c, or a codeword is not exact in half
// precision.
__global__ void e8_layout_kernel(const float* __restrict__ C, _Float16* __restrict__ c16,
                                 float* __restrict__ c2, uint32_t* __restrict__ orig,
                                 uint32_t* __restrict__ neg, int* __restrict__ bad) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E8_LAYOUT_CW) return;
  int i, partner;
  if (e < E8_SYM_CW) {
    const int h = e < E8_SYM_HALF ? e : E8_SYM_HALF - 1;
    int r = 0;
#pragma unroll
    for (int q = 1; q < 5; ++q) r = h >= E8_SH_OFF[q] ? q : r;
    i = E8_SH_A[r] + (h - E8_SH_OFF[r]);
    partner = 2 * E8_SH_A[r] + E8_SH_S[r] - 1 - i;
  } else {
    const int q0 = e - E8_SYM_CW;
    const int q = q0 < E8_PLAIN_CW ? q0 : E8_PLAIN_CW - 1;
    i = q == 0 ? 0 : 56880 + q;
    partner = i;
  }
  float v[8];
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    v[k] = C[i * 8 + k];
    s = fmaf(v[k], v[k], s);
    c16[e * 8 + k] = _Float16(v[k]);
  }
  c2[e] = s;
  orig[e] = uint32_t(i);
  neg[e] = uint32_t(partner);
  // the pairing, and codewords exact in half precision (the finish takes
  // the winner's coordinates from the half copy)
  bool ok = true;
#pragma unroll
  for (int k = 0; k < 8; ++k) ok = ok && (float(_Float16(v[k])) == v[k]);
  if (e < E8_SYM_HALF) {
#pragma unroll
    for (int k = 0; k < 8; ++k) ok = ok && (C[partner * 8 + k] == -v[k]);
  }
  if (!ok) atomicOr(bad, 1);
}

// The codebook as the search kernels see it: the symmetric layout when its
// pairing check passed, else the codebook as given (identity map).
struct E8Book {
  const _Float16* c16p;  // as given: 65536 codewords (+ E8_PAD) in half precision
  const float* c2p;
  const _Float16* c16s;  // the symmetric layout
  const float* c2s;
  const uint32_t* orig;
  const uint32_t* neg;
  const int* bad;
};

struct E8View {
  const uint4* cw;        // codewords as 8 halves, one uint4 each
  const float* nm;        // norms
  const uint32_t* orig;   // null: identity
  const uint32_t* neg;
  int sym_pairs;          // pairs [0, sym_pairs) search one member per {c, -c}
  int pairs;              // pairs in all
};

__device__ __forceinline__ E8View e8_view(const E8Book& b) {
  const bool sym = __builtin_amdgcn_readfirstlane(*b.bad) == 0;
  E8View v;
  v.cw = reinterpret_cast<const uint4*>(sym ? b.c16s : b.c16p);
  v.nm = sym ? b.c2s : b.c2p;
  v.orig = sym ? b.orig : nullptr;
  v.neg = sym ? b.neg : nullptr;
  v.sym_pairs = sym ? E8_SYM_CW / 64 : 0;
  v.pairs = sym ? E8_LAYOUT_CW / 64 : 1024;
  return v;
}

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

// The largest of the 16 values of an accumulator tile (of their magnitudes
// with ABS) and x (max3 tree; the magnitudes are operand modifiers).
template <bool ABS>
__device__ __forceinline__ float e8_max16(const f32x16& a, float x) {
  auto v = [&](int r) { return ABS ? fabsf(a[r]) : a[r]; };
  const float t0 = fmaxf(fmaxf(v(0), v(1)), v(2));
  const float t1 = fmaxf(fmaxf(v(3), v(4)), v(5));
  const float t2 = fmaxf(fmaxf(v(6), v(7)), v(8));
  const float t3 = fmaxf(fmaxf(v(9), v(10)), v(11));
  const float t4 = fmaxf(fmaxf(v(12), v(13)), v(14));
  const float u0 = fmaxf(fmaxf(t0, t1), t2);
  const float u1 = fmaxf(fmaxf(t3, t4), v(15));
  return fmaxf(fmaxf(u0, u1), x);
}

// One pair of 32-codeword tiles against the 32 vectors of a wave (split-half
// products, see e8_split_operand).
__device__ __forceinline__ void e8_pair_products(const uint4& wa, const uint4& wb,
                                                 const e8_half8& yb, f32x16& aa, f32x16& ab) {
  f32x16 z;
#pragma unroll
  for (int r = 0; r < 16; ++r) z[r] = 0.f;
  aa = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(e8_half8, wa), yb, z, 0, 0, 0);
  ab = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(e8_half8, wb), yb, z, 0, 0, 0);
}

// The pairs [pb, pe) of 32-codeword tiles of a search view against a wave's 32
// vectors: tile(acc, cn, t) for every tile, in order (acc: the lane's 16 dot
// products, cn: the norm of the lane's codeword row j, t: the tile's first
// entry). The products of the next pair are issued before the current pair's
// tiles are taken, so the matrix cores run while the vector ALUs reduce; the
// codewords (as 8 halves) and norms are loaded two pairs ahead, up to three
// pairs past pe (inside the buffers' padding). Two pairs per iteration, so the
// products of the two pairs in flight keep their registers (aa, ab and xa, xb
// swap roles) instead of being copied.
template <typename Tile>
__device__ __forceinline__ void e8_pairs(const uint4* cw, const float* nm, int pb, int pe, int j,
                                         const e8_half8& yb, Tile&& tile) {
  if (pb >= pe) return;
  const uint4* cp = cw + pb * 64;  // the current pair (the same address in every lane)
  const float* np = nm + pb * 64;
  f32x16 aa, ab, xa, xb;
  e8_pair_products(cp[j], cp[32 + j], yb, aa, ab);
  float ca = np[j], cb = np[32 + j], xca, xcb;
  uint4 na = cp[64 + j], nb = cp[96 + j];
  float nca = np[64 + j], ncb = np[96 + j];
  for (int p = pb; p < pe; p += 2) {
    e8_pair_products(na, nb, yb, xa, xb);  // pair p + 1
    xca = nca;
    xcb = ncb;
    cp += 64;
    np += 64;
    na = cp[64 + j];  // pair p + 2
    nb = cp[96 + j];
    nca = np[64 + j];
    ncb = np[96 + j];
    tile(aa, ca, p * 64);
    tile(ab, cb, p * 64 + 32);
    e8_pair_products(na, nb, yb, aa, ab);  // pair p + 2
    ca = nca;
    cb = ncb;
    cp += 64;
    np += 64;
    na = cp[64 + j];  // pair p + 3
    nb = cp[96 + j];
    nca = np[64 + j];
    ncb = np[96 + j];
    if (p + 1 < pe) {
      tile(xa, xca, (p + 1) * 64);
      tile(xb, xcb, (p + 1) * 64 + 32);
    }
  }
}

// Squared error of the nearest codeword, summed over all 8-vectors, for every
// candidate scale. One wave: 32 vectors x all codewords.
// Each work-group writes its NC partial sums to part[blockIdx.x * NC + c]
// (waves added in a fixed order); e8_sse_reduce_kernel adds the work-groups'
// partials in a fixed order, so the table, and the scale picked from it, are
// the same on every run.
template <int NC>
__global__ __launch_bounds__(256) void e8_scale_kernel(const float* __restrict__ Y, int64_t nvec,
                                                       E8Book book,
                                                       const float* __restrict__ cand, int ncand,
                                                       double* __restrict__ part) {
  __shared__ double red[4][NC];
  __shared__ float sc[NC];
  // best[c * 256 + tid]: the lane's minimum for candidate c, in LDS (written
  // only when a run ends), so the loop carries no per-candidate state
  extern __shared__ float best[];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  if (tid < NC) sc[tid] = cand[tid < ncand ? tid : 0];
#pragma unroll
  for (int c = 0; c < NC; ++c) best[c * 256 + tid] = 3.4e38f;
  __syncthreads();
  // For every scale s the distance term is s n_i - 2 <y, c_i> with n_i = |c_i|^2.
  // Over codewords of one norm it is smallest at the largest dot product, and
  // fma(s, n, -2 x) does not increase with x, so each lane keeps the largest
  // dot of the current run of equal norms and folds it into the 32 minima
  // when the norm changes: the minima equal those over every codeword taken
  // one by one, for any codebook order (in the symmetric layout there are
  // seven runs and almost every tile takes one max per value). In the
  // symmetric region the dot's magnitude stands for the pair {c, -c}.
  const E8View v = e8_view(book);
  float run_n = v.nm[0], run_max = -3.4e38f;
  auto fold = [&]() {
#pragma unroll
    for (int c = 0; c < NC; ++c)
      best[c * 256 + tid] = fminf(best[c * 256 + tid], fmaf(sc[c], run_n, -2.f * run_max));
  };
  auto tile_of = [&](auto abs_tag) {
    constexpr bool ABS = decltype(abs_tag)::value;
    return [&](const f32x16& acc, float cn, int) {
      if (__all(cn == run_n)) {  // the whole tile continues the run
        run_max = e8_max16<ABS>(acc, run_max);
      } else {  // a run ends inside this tile
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float n2 = __shfl(cn, 8 * (r / 4) + 4 * kh + (r % 4), 64);
          if (n2 != run_n) {
            fold();
            run_n = n2;
            run_max = -3.4e38f;
          }
          run_max = fmaxf(run_max, ABS ? fabsf(acc[r]) : acc[r]);
        }
      }
    };
  };
  e8_pairs(v.cw, v.nm, 0, v.sym_pairs, j, yb, tile_of(std::true_type{}));
  e8_pairs(v.cw, v.nm, v.sym_pairs, v.pairs, j, yb, tile_of(std::false_type{}));
  fold();
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const float mine = best[c * 256 + tid];
    const float other = __shfl_xor(mine, 32, 64);
    const float b = fminf(mine, other);
    double e = live && kh == 0 ? double(y2) + double(sc[c]) * double(b) : 0.0;
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) e += __shfl_xor(e, off, 64);
    if (lane == 0) red[wave][c] = e;
  }
  __syncthreads();
  if (tid < NC) {
    part[int64_t(blockIdx.x) * NC + tid] =
        tid < ncand ? (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]) : 0.0;
  }
}

// sse[c] = sum over the nblk work-groups of part[b * NC + c], one work-group per
// candidate, in a fixed order (strided partial sums, then a tree).
template <int NC>
__global__ __launch_bounds__(256) void e8_sse_reduce_kernel(const double* __restrict__ part,
                                                            int64_t nblk,
                                                            double* __restrict__ sse) {
  __shared__ double t[256];
  const int c = blockIdx.x;
  double acc = 0.0;
  for (int64_t b = threadIdx.x; b < nblk; b += 256) acc += part[b * NC + c];
  t[threadIdx.x] = acc;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (int(threadIdx.x) < h) t[threadIdx.x] += t[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) sse[c] = t[0];
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

// Finish a group step for one row: code, quantized values, errors. With
// rowloss, also the group's proxy-loss term rms^2 (y - q) D_g (y - q)^T, y the
// pre-rounding vector (normalized domain) of e8_prerounding_kernel.
struct E8Finish {
  const float* Wn;
  int64_t n;
  const float* C;
  const float* rms;
  int64_t c0;
  uint16_t* codes;
  int64_t ldcode;
  float* What;
  float* Eb;
  int64_t lde;
  int ecol;
  const float* y8;
  const float* Dg;
  double* rowloss;
  // the next group step of the same block, when there is one: its
  // pre-rounding vectors (as e8_prerounding_kernel forms them) go to ynext
  float* ynext;
  const float* F;  // null: no outer-block feedback yet
  const float* U;
  int64_t s0;      // first column of the block
};

// Low word of a search key: an entry of the search view, with E8_NEG when
// the entry's negation is meant, or (E8_TILE set) one half of a 32-entry tile
// (tile base | half) whose 16 entries, all of one norm, hold the best dot
// product (its magnitude, in the symmetric region) that the search saw.
constexpr uint32_t E8_TILE = 0x80000000u;
constexpr uint32_t E8_NEG = 0x20000000u;

// The coordinates of search entry e (negated with neg): from the half copy
// when the view is the symmetric layout (whose codewords the layout kernel
// checked to be exact in half precision), else from the codebook as given.
__device__ __forceinline__ void e8_coords(const E8Finish& f, const E8View& v, uint32_t e, bool neg,
                                          float* c) {
  if (v.orig) {
    const e8_half8 h = __builtin_bit_cast(e8_half8, v.cw[e]);
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = neg ? -float(h[k]) : float(h[k]);
  } else {
#pragma unroll
    for (int k = 0; k < 8; ++k) c[k] = f.C[e * 8 + k];
  }
}

// Finishes a group step for the row of this lane's group of eight (sub = 0..7):
// the codeword its key names, the code, W^, the errors, the loss term and,
// when there is a next group in the block, its pre-rounding vector. Loads that
// do not depend on the key are issued first, so their latency overlaps the
// key's exchange.
//
// The key: an entry as it stands (E8_NEG: its negation); for a tile half, the
// largest float32 dot <y, c> over its 16 entries (one norm: the largest dot is
// the nearest), or in the symmetric region the largest |<y, c>| and the member
// of {c, -c} its sign gives (c for a zero dot); the lower entry on ties. Lane
// sub takes two entries of the tile half and the eight agree by shuffles.
//
// Loss term: lane sub forms res_sub (D_g res)_sub; the eight lanes' terms are
// added by shuffles in a fixed order. Next pre-rounding vector (as
// e8_prerounding_kernel forms it): Wn + sum over the block's groups so far of
// E U, + F; lane sub takes the block's columns c = sub mod 8 for all eight
// dimensions, and the eight partial vectors are added by shuffles.
__device__ __forceinline__ void e8_finish(const E8Finish& f, const E8View& v, float s,
                                          unsigned long long* __restrict__ keys, int64_t row,
                                          int sub, int lane) {
  // ---- independent of the key
  unsigned long long rk = 0ull;
  if (sub == 0) rk = atomicExch(&keys[row], ~0ull);
  float y[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) y[k] = f.y8[row * 8 + k];
  const float r = f.rms[row];
  const float wn = f.Wn[row * f.n + f.c0 + sub];
  float dg[8];
  if (f.rowloss) {
#pragma unroll
    for (int b = 0; b < 8; ++b) dg[b] = f.Dg[(f.c0 + sub) * 8 + b];
  }
  const int64_t cn = f.c0 + 8;  // the next group's first column
  const int nprev = f.ecol;     // the block's columns before this group
  float acc[8], ucur[8];
  float wnx = 0.f, fx = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  if (f.ynext) {
    wnx = f.Wn[row * f.n + cn + sub];
    if (f.F) fx = f.F[row * f.n + cn + sub];
    const float* uc = f.U + (f.s0 + nprev + sub) * f.n + cn;  // this group's column nprev + sub
#pragma unroll
    for (int k = 0; k < 8; ++k) ucur[k] = uc[k];
    // the earlier groups' columns, four at a time, loads before products
    for (int c0 = sub; c0 < nprev; c0 += 32) {
      float e[4], u[4][8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = c0 + 8 * q;
        const bool ok = c < nprev;
        const int cc = ok ? c : sub;
        e[q] = ok ? f.Eb[row * f.lde + cc] : 0.f;
        const float* ur = f.U + (f.s0 + cc) * f.n + cn;
#pragma unroll
        for (int k = 0; k < 8; ++k) u[q][k] = ur[k];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int k = 0; k < 8; ++k) acc[k] = fmaf(e[q], u[q][k], acc[k]);
    }
  }
  // ---- the key: the entry, its sign, its coordinates
  rk = __shfl(rk, lane & ~7, 64);
  const uint32_t ref = uint32_t(rk & 0xFFFFFFFFull);
  uint32_t e;
  bool negate;
  float cw[8];
  if (!(ref & E8_TILE)) {
    e = ref & ~E8_NEG;
    negate = (ref & E8_NEG) != 0;
    e8_coords(f, v, e, negate, cw);
  } else {
    const uint32_t base = ref & 0x7FFFFFE0u, kh = ref & 1u;
    const bool sym = base < uint32_t(v.sym_pairs) * 64u;
    // this lane's two entries of the tile half: places r = 2 sub and 2 sub + 1
    // (adjacent entries); both loads are issued before either is used
    const uint32_t i0 = base + 8 * ((2 * sub) / 4) + 4 * kh + (2 * sub) % 4, i1 = i0 + 1;
    float a0[8], a1[8];
    if (v.orig) {
      const e8_half8 h0 = __builtin_bit_cast(e8_half8, v.cw[i0]);
      const e8_half8 h1 = __builtin_bit_cast(e8_half8, v.cw[i1]);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        a0[k] = float(h0[k]);
        a1[k] = float(h1[k]);
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        a0[k] = f.C[i0 * 8 + k];
        a1[k] = f.C[i1 * 8 + k];
      }
    }
    float d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      d0 = fmaf(a0[k], y[k], d0);
      d1 = fmaf(a1[k], y[k], d1);
    }
    // the sign rides in the low bit of the entry: entries are compared with it
    // cleared
    uint32_t t0 = i0 << 1, t1 = i1 << 1;
    if (sym) {
      t0 |= d0 < 0.f ? 1u : 0u;
      t1 |= d1 < 0.f ? 1u : 0u;
      d0 = fabsf(d0);
      d1 = fabsf(d1);
    }
    if (d0 != d0) d0 = -INFINITY;  // a NaN dot ranks last, the same in every lane
    if (d1 != d1) d1 = -INFINITY;
    float bv = d0;
    uint32_t bi = t0;
    if (d1 > bv) {
      bv = d1;
      bi = t1;
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      const float ov = __shfl_xor(bv, o, 8);
      const uint32_t oi = __shfl_xor(bi, o, 8);
      if (ov > bv || (ov == bv && (oi >> 1) < (bi >> 1))) {
        bv = ov;
        bi = oi;
      }
    }
    e = bi >> 1;
    negate = (bi & 1u) != 0;
    // the winner's coordinates from the lane that loaded them
    const uint32_t off = e - base - 4 * kh;         // 8 (r / 4) + r mod 4
    const int rw = int(4 * (off / 8) + (off % 8));  // the winner's place r in 0..15
    const int src = (lane & ~7) + rw / 2;
    const bool second = (rw & 1) != 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float c = __shfl(second ? a1[k] : a0[k], src, 64);
      cw[k] = negate ? -c : c;
    }
  }
  const uint32_t code = !v.orig ? e : (negate ? v.neg[e] : v.orig[e]);
  // ---- outputs
  if (sub == 0) f.codes[row * f.ldcode + f.c0 / 8] = uint16_t(code);
  float mycw = cw[0];
#pragma unroll
  for (int k = 1; k < 8; ++k) mycw = sub == k ? cw[k] : mycw;
  const float qs = s * mycw;
  const float err = wn - qs;
  f.Eb[row * f.lde + f.ecol + sub] = err;
  if (f.What) f.What[row * f.n + f.c0 + sub] = r * qs;
  if (f.rowloss) {
    double t = 0.0;
#pragma unroll
    for (int b = 0; b < 8; ++b) t += double(dg[b]) * (double(y[b]) - double(s * cw[b]));
    double al = (double(y[sub]) - double(qs)) * t;
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) al += __shfl_xor(al, o, 8);
    if (sub == 0) f.rowloss[row] += double(r) * double(r) * al;
  }
  if (f.ynext) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = fmaf(err, ucur[k], acc[k]);
#pragma unroll
    for (int o = 4; o > 0; o >>= 1) {
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] += __shfl_xor(acc[k], o, 8);
    }
    float vv = acc[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) vv = sub == k ? acc[k] : vv;
    float yv = wnx + vv;
    if (f.F) yv += fx;
    f.ynext[row * 8 + sub] = yv;
  }
}

// One group step of BlockLDLQ: the nearest scaled codeword to each row's
// pre-rounding vector. A work-group takes 32 rows; its 4 waves and the
// gridDim.y work-groups of those rows split the tile pairs of the search view
// evenly (gridDim.y <= 256), and the per-row results meet in an atomicMin of a
// packed (distance, reference) key. The dot products come from the split
// half-precision product of e8_scale_kernel; the distance term s n_i - 2 <y, c_i>
// is smallest, over a run of equal norms, at the largest dot (in the symmetric
// region: the largest magnitude, for the pair {c, -c}), so each lane keeps that
// dot per run, and where it was, and compares runs by distance. Inside a tile
// of one norm a lane takes only the tile's largest dot (one max3 tree) and
// remembers the tile; the codeword in it is found once per row, by the
// finisher (e8_finish). Where a run ends inside a tile, the lane goes through
// the tile's dots one by one and keeps exact entries. Ties go to the lower
// entry within a lane and to the lower reference between lanes.
struct E8Shared {
  unsigned long long ksh[4][32];
  float bestv[256];
  uint32_t bestref[256];
  unsigned last;
};

// Returns (the same in every thread) whether this work-group finished the
// step: the one whose count, added to `cnt`, reaches `target`.
__device__ __forceinline__ bool e8_step(E8Shared& sh, const E8View& v, float s, int64_t m,
                                        unsigned long long* __restrict__ keys,
                                        unsigned* __restrict__ cnt, unsigned target,
                                        const E8Finish& fin) {
  float* bestv_sh = sh.bestv;
  uint32_t* bestref_sh = sh.bestref;
  const float* y8g = fin.y8;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t r0 = int64_t(blockIdx.x) * 32;
  const int j = lane & 31, kh = lane >> 5;
  float y8[8];
  {
    const int64_t row = r0 + j;
#pragma unroll
    for (int k = 0; k < 8; ++k) y8[k] = row < m ? y8g[row * 8 + k] : 0.f;
  }
  const e8_half8 yb = e8_split_operand(y8, kh);
  const int nw = int(gridDim.y) * 4, gw = int(blockIdx.y) * 4 + wave;
  const int p0 = gw * v.pairs / nw, p1 = (gw + 1) * v.pairs / nw;  // this wave's pairs
  // The lane's best run so far lives in LDS (written only when a run ends),
  // so the loop carries only the current run. Inside the loop a reference is a
  // tile base (this lane's half implied) or an exact entry tagged with
  // E8_EXACT (and E8_NEG); it becomes a key's low word at the end.
  constexpr uint32_t E8_EXACT = 0x40000000u;
  bestv_sh[tid] = 3.4e38f;
  bestref_sh[tid] = uint32_t(p0 * 64) | E8_EXACT;  // valid even if every distance is NaN
  float run_n = v.nm[p0 * 64], run_max = -3.4e38f;
  uint32_t run_ref = uint32_t(p0 * 64) | E8_EXACT;
  auto fold = [&]() {
    const float d = fmaf(s, run_n, -2.f * run_max);
    if (d < bestv_sh[tid]) {  // runs are visited in increasing entry order within a lane
      bestv_sh[tid] = d;
      bestref_sh[tid] = run_ref;
    }
  };
  auto tile_of = [&](auto abs_tag) {
    constexpr bool ABS = decltype(abs_tag)::value;
    return [&](const f32x16& acc, float cn, int t) {
      if (__all(cn == run_n)) {  // the whole tile continues the run
        const float mx = e8_max16<ABS>(acc, run_max);
        run_ref = mx > run_max ? uint32_t(t) : run_ref;
        run_max = mx;
      } else {  // a run ends inside this tile
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int i = t + 8 * (r / 4) + 4 * kh + (r % 4);
          const float n2 = __shfl(cn, 8 * (r / 4) + 4 * kh + (r % 4), 64);
          if (n2 != run_n) {
            fold();
            run_n = n2;
            run_max = -3.4e38f;
          }
          const float x = ABS ? fabsf(acc[r]) : acc[r];
          const bool gt = x > run_max;
          run_max = gt ? x : run_max;
          const uint32_t sg = (ABS && acc[r] < 0.f) ? E8_NEG : 0u;
          run_ref = gt ? (uint32_t(i) | E8_EXACT | sg) : run_ref;
        }
      }
    };
  };
  e8_pairs(v.cw, v.nm, p0, p1 < v.sym_pairs ? p1 : v.sym_pairs, j, yb, tile_of(std::true_type{}));
  e8_pairs(v.cw, v.nm, p0 > v.sym_pairs ? p0 : v.sym_pairs, p1, j, yb, tile_of(std::false_type{}));
  fold();
  const uint32_t ref = bestref_sh[tid];
  const uint32_t low = (ref & E8_EXACT) ? (ref ^ E8_EXACT) : (E8_TILE | ref | uint32_t(kh));
  unsigned long long key = (unsigned long long)ordered_bits(bestv_sh[tid]) << 32 | low;
  unsigned long long other = __shfl_xor(key, 32, 64);
  key = key < other ? key : other;
  if (kh == 0) sh.ksh[wave][j] = key;
  __syncthreads();
  if (tid < 32) {
    unsigned long long k2 = sh.ksh[0][tid];
    for (int wv = 1; wv < 4; ++wv) k2 = sh.ksh[wv][tid] < k2 ? sh.ksh[wv][tid] : k2;
    if (r0 + tid < m) atomicMin(&keys[r0 + tid], k2);
  }
  // The last of the gridDim.y work-groups of these 32 rows to get here
  // finishes the step for them (a counter per row block; no group waits).
  // The keys are only touched by atomics: each group waits until its own
  // atomicMin operations are complete before it counts, and the finisher takes
  // each key with an atomic exchange (a read-modify-write sees the latest
  // value), which also resets it for the next use. No cache-wide fence is
  // needed (and none is taken: they would flush the L2 holding the codebook).
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) sh.last = atomicAdd(cnt, 1u) == target - 1u ? 1u : 0u;
  __syncthreads();
  if (!sh.last) return false;
  {
    const int sub = tid & 7;
    const int64_t row = r0 + (tid >> 3);
    if (row < m) {  // the same for the eight lanes of a row
      e8_finish(fin, v, s, keys, row, sub, lane);
    }
  }
  return true;
}

// One group step per launch.
__global__ __launch_bounds__(256) void e8_argmin_kernel(E8Book book, const float* __restrict__ sp,
                                                        int64_t m,
                                                        unsigned long long* __restrict__ keys,
                                                        unsigned* __restrict__ done, E8Finish fin) {
  __shared__ E8Shared sh;
  const E8View v = e8_view(book);
  if (e8_step(sh, v, *sp, m, keys, &done[blockIdx.x], gridDim.y, fin) &&
      threadIdx.x == 0)
    done[blockIdx.x] = 0u;
}

// loss = sum of the row losses, in a fixed order (one work-group).
// Sum of the per-row losses: 1024 threads, each a strided slice, then wave
// sums by shuffles and the 16 wave sums added in a fixed order.
__global__ __launch_bounds__(1024) void sum_rows_kernel(const double* __restrict__ rowloss,
                                                        int64_t m, double* __restrict__ out) {
  __shared__ double part[16];
  double acc = 0.0;
  for (int64_t i = threadIdx.x; i < m; i += 1024) acc += rowloss[i];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
#pragma unroll
    for (int w = 0; w < 16; ++w) t += part[w];
    *out = t;
  }
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
    QUIP_KERNEL(sum_rows_kernel, dim3(1), dim3(1024), 0, s, rl, m, loss);
  });
}

struct E8Ws {
  float* Wn;
  float* F;
  float* Eb;
  unsigned long long* keys;
  float* c2;
  _Float16* c16;  // the codebook in half precision (exact: multiples of 1/2 up to 3.5)
  float* c2s;     // the symmetric search layout (e8_layout_kernel)
  _Float16* c16s;
  uint32_t* orig;
  uint32_t* neg;
  int* bad;
  float* cand;
  double* sse;
  double* part;  // per-work-group partial sums of the scale search
  E8Book book() const { return E8Book{c16, c2, c16s, c2s, orig, neg, bad}; }
};

// Codebook-side buffers of the E8 search, carved in this order.
void e8_take_book(Carver& c, E8Ws& e) {
  e.c2 = c.take<float>(E8_ROWS);
  e.c16 = c.take<_Float16>(size_t(E8_ROWS) * 8);
  e.c2s = c.take<float>(E8_ROWS);
  e.c16s = c.take<_Float16>(size_t(E8_ROWS) * 8);
  e.orig = c.take<uint32_t>(E8_ROWS);
  e.neg = c.take<uint32_t>(E8_ROWS);
  e.bad = c.take<int>(16);
}

// Both views of the codebook: as given, and the symmetric layout with its
// pairing check.
quip_status e8_prepare_book(const float* codebook, const E8Ws& e, hipStream_t s) {
  QUIP_TRY(timed_launch("e8_norms_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL(e8_norms_kernel, dim3(unsigned(cdiv(E8_ROWS, 256))), dim3(256), 0, s, codebook,
                e.c2, e.c16);
  }));
  QUIP_TRY(fill_f32(reinterpret_cast<float*>(e.bad), 1, 0.f, s));  // bad <- 0 (bit pattern)
  return timed_launch("e8_layout_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL(e8_layout_kernel, dim3(unsigned(cdiv(E8_LAYOUT_CW, 256))), dim3(256), 0, s,
                codebook, e.c16s, e.c2s, e.orig, e.neg, e.bad);
  });
}

// Work-groups per 32-row block of a group step's search (gridDim.y of
// e8_argmin_kernel). The total search work does not depend on the split; the
// launch's fixed part (first loads after the kernel boundary, the key exchange,
// the finish) does, per work-group. Measured on 256 CUs with n = 256 (µs per
// step, argmin plus the pre-rounding launch where it is separate): m = 1024:
// 8 splits 13.7 (16: 14.0, 4: 16.2); m = 4096: 4 splits 19.4 (8: 20.5, 3:
// 24.0); m = 8192: 4 splits 27.3 (2: 29.4); m = 16384: 2 splits 46.2 (4: 48.9,
// 1: 51.1). Two work-groups per CU, at least two and at most eight splits,
// comes within 8% of the best at every size.
int e8_argmin_split(int64_t m) {
  const int64_t rb = cdiv(m, 32);
  const int64_t y = cdiv(2 * int64_t(device_cus()), rb);
  return int(y < 2 ? 2 : (y > 8 ? 8 : y));
}

// Work-groups of the E8 scale search (128 vectors each) and their partial sums.
int64_t e8_scale_blocks(int64_t m, int64_t n) { return cdiv(m * (n / 8), 128); }
size_t e8_partial_count(int64_t m, int64_t n) { return size_t(e8_scale_blocks(m, n)) * 64; }

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
  const int64_t nvec = m * (n / 8);
  const int64_t nblk = e8_scale_blocks(m, n);
  const dim3 grid{unsigned(nblk)};
  const size_t sh32 = sizeof(float) * 32 * 256, sh64 = sizeof(float) * 64 * 256;
  if (ncand > 32)
    QUIP_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(&e8_scale_kernel<64>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, int(sh64)));
  QUIP_TRY(timed_launch("e8_scale_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    if (ncand <= 32)
      QUIP_KERNEL((e8_scale_kernel<32>), grid, dim3(256), sh32, s, Wn, nvec, e.book(), e.cand,
                         ncand, e.part);
    else
      QUIP_KERNEL((e8_scale_kernel<64>), grid, dim3(256), sh64, s, Wn, nvec, e.book(), e.cand,
                         ncand, e.part);
  }, 16.0 * 65536.0 * double(nvec), 32.0 * double(nvec)));  // <y, c> for every vector and codeword
  QUIP_TRY(timed_launch("e8_sse_reduce_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    if (ncand <= 32)
      QUIP_KERNEL((e8_sse_reduce_kernel<32>), dim3(unsigned(ncand)), dim3(256), 0, s, e.part,
                  nblk, e.sse);
    else
      QUIP_KERNEL((e8_sse_reduce_kernel<64>), dim3(unsigned(ncand)), dim3(256), 0, s, e.part,
                  nblk, e.sse);
  }));
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
                    int64_t lde, const float* D, double* rowloss, const float* Ef, int kfold,
                    hipStream_t s) {
  // the fold in its own instantiation, with its result tile: the kernel
  // without it keeps its registers and LDS (occupancy of the many-row layers)
  const bool fold = kfold > 0;
  const void* fn = fold ? reinterpret_cast<const void*>(&ldlq_sweep_kernel<B, true>)
                        : reinterpret_cast<const void*>(&ldlq_sweep_kernel<B, false>);
  const size_t shmem = (size_t(B) * 36 + B + (fold ? 16 * (B + 4) : 0)) * sizeof(float);
  if (shmem > 65536)
    QUIP_HIP(hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(shmem)));
  // float4 paths need 16-byte alignment of every row start and of the block start
  const bool vec = aligned16(W) && aligned16(F) && aligned16(U) && aligned16(Eb) && aligned16(Ef) &&
                   (What == nullptr || aligned16(What)) &&
                   ((reinterpret_cast<uintptr_t>(codes) & 3) == 0) && ldw % 4 == 0 &&
                   ldf % 4 == 0 && ldu % 4 == 0 && ldc % 4 == 0 && ldwh % 4 == 0 &&
                   lde % 4 == 0 && s0 % 4 == 0;
  // work: per row the batch's earlier feedback (2 kfold bw flops), the
  // in-block feedback (bw (bw - 1) flops) and the rounding; reads W, F, the
  // earlier errors and the U block and the rows above it, writes codes, W^
  // and the errors
  const double md = double(m), bd = double(bw), kd = double(kfold);
  const double flops = md * (2.0 * kd * bd + bd * (bd - 1.0) + 6.0 * bd);
  const double bytes = md * bd * (4.0 + (useF ? 4.0 : 0.0) + 1.0 + (What ? 4.0 : 0.0) + 4.0) +
                       4.0 * bd * bd + 4.0 * kd * (md + bd) + (rowloss ? 16.0 * md : 0.0);
  return timed_launch("ldlq_sweep_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    if (fold)
      QUIP_KERNEL((ldlq_sweep_kernel<B, true>), dim3(unsigned(cdiv(m, 16))), dim3(256), shmem, s,
                  W, ldw, F, ldf, useF, U, ldu, scales, L, m, s0, bw, codes, ldc, What, ldwh, Eb,
                  lde, D, rowloss, vec, Ef, kfold);
    else
      QUIP_KERNEL((ldlq_sweep_kernel<B, false>), dim3(unsigned(cdiv(m, 16))), dim3(256), shmem, s,
                  W, ldw, F, ldf, useF, U, ldu, scales, L, m, s0, bw, codes, ldc, What, ldwh, Eb,
                  lde, D, rowloss, vec, Ef, kfold);
  }, flops, bytes);
}

quip_status sweep(int b, const float* W, int64_t ldw, const float* F, int64_t ldf, bool useF,
                  const float* U, int64_t ldu, const float* scales, int L, int64_t m, int64_t s0,
                  int bw, uint8_t* codes, int64_t ldc, float* What, int64_t ldwh, float* Eb,
                  int64_t lde, const float* D, double* rowloss, const float* Ef, int kfold,
                  hipStream_t s) {
  switch (b) {
    case 32: return sweep_t<32>(W, ldw, F, ldf, useF, U, ldu, scales, L, m, s0, bw, codes, ldc, What, ldwh, Eb, lde, D, rowloss, Ef, kfold, s);
    case 64: return sweep_t<64>(W, ldw, F, ldf, useF, U, ldu, scales, L, m, s0, bw, codes, ldc, What, ldwh, Eb, lde, D, rowloss, Ef, kfold, s);
    case 128: return sweep_t<128>(W, ldw, F, ldf, useF, U, ldu, scales, L, m, s0, bw, codes, ldc, What, ldwh, Eb, lde, D, rowloss, Ef, kfold, s);
    case 256: return sweep_t<256>(W, ldw, F, ldf, useF, U, ldu, scales, L, m, s0, bw, codes, ldc, What, ldwh, Eb, lde, D, rowloss, Ef, kfold, s);
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
    E8Ws e{};
    e8_take_book(c, e);            // the codebook's half-precision views
    c.take<double>(64);            // sse
    c.take<double>(e8_partial_count(m, n));  // per-work-group partial sums
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
  e8_take_book(c, e);
  e.sse = c.take<double>(64);
  e.part = c.take<double>(e8_partial_count(m, n));
  e.cand = fac;
  if (!c.fits()) return fail(QUIP_ERR_WORKSPACE, "quip_scales: workspace too small");
  host_e8_candidates(q.n_cand, hostf);
  QUIP_HIP(hipMemcpyAsync(fac, hostf, sizeof(float) * q.n_cand, hipMemcpyHostToDevice, s));
  QUIP_TRY(timed_launch("rownorm_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL(rownorm_kernel, dim3(unsigned(m)), dim3(256), 0, s, W, n, ldw, e.Wn, scales + 1,
                       true);
  }));
  QUIP_TRY(e8_prepare_book(codebook, e, s));
  return e8_scales(e.Wn, m, n, codebook, e, q.n_cand, scales, static_cast<double*>(mse_out), s);
}

// Trailing-update batch of the scalar sweep: the lazily updated block of B
// columns is swept in sub-blocks of at most 256 columns (the sweep kernel);
// each sub-block receives the feedback of the batch's earlier sub-blocks
// (inside the sweep launch, left-looking on the matrix cores, when the rows
// fit one work-group per CU; else from a product after each sub-block), and
// the rest of the matrix is updated once per batch of 512 columns (one
// K = 512 product instead of four K = 128 ones: a quarter of the
// read-modify-write traffic of F), 1024 above n = 4096 (half the passes over F
// again: 8192 x 28672 layer LDLQ 66.7 -> 64.0 ms; 28672 x 8192: 22.4 -> 21.6
// ms; 4096 x 11008: 6.72 -> 6.40 ms).
static int64_t outer_block(int64_t n, int g, int64_t B) {
  if (g != 1) return B;
  const int64_t t = n > 4096 ? 1024 : 512;
  int64_t bo = B >= t ? B : B * (t / B);
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
    c.take<float>(size_t(m) * 8);  // pre-rounding vectors of two group steps
    c.take<float>(size_t(m) * 8);
    c.take<unsigned>(size_t(cdiv(m, 32)));  // per row block: groups done
    E8Ws e{};
    e8_take_book(c, e);
    c.take<double>(64);
    c.take<double>(e8_partial_count(m, n));
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
  // the grid path's first sweep starts every row's sum itself
  if (rl && c.fits() && (q.kind != QUIP_Q_UNIFORM || n == 0)) QUIP_TRY(fill_f64(rl, m, 0.0, s));

  if (q.kind == QUIP_Q_UNIFORM) {
    if (!c.fits()) return fail(QUIP_ERR_WORKSPACE, "quip_ldlq: workspace too small");
    const int L = 1 << q.bits;
    if (q.scale_mode == QUIP_SCALE_COMPUTE) {
      host_grid_factors(q.n_cand, hostf);
      QUIP_HIP(hipMemcpyAsync(fac, hostf, sizeof(float) * q.n_cand, hipMemcpyHostToDevice, s));
      QUIP_TRY(grid_scales(W, m, n, ldw, L, q.n_cand, fac, scales, nullptr, s));
    }
    // With at most one sweep work-group per CU, each sub-block takes the
    // batch's earlier feedback itself (one launch per sub-block instead of
    // two); with more rows a separate product after each sub-block is faster
    // (28672 x 8192 layer: sweeps 3.6 -> 5.9 ms with the in-sweep feedback).
    const bool fold = cdiv(m, 16) <= int64_t(device_cus());
    // Sub-block width: B's, up to 256. Without the fold, B = 128 is swept 256
    // columns at a time (half the sweeps and products: 11008 x 4096 layer
    // LDLQ 3.37 -> 3.05 ms); with it, 256-wide sweeps cost more than the
    // launches they save (4096 x 4096: 1.38 -> 1.45 ms).
    const int bi = (B >= 256 || (!fold && B >= 128)) ? 256 : (B >= 128 ? 128 : (B >= 64 ? 64 : 32));
    uint8_t* cd = static_cast<uint8_t*>(codes);
    for (int64_t j0 = 0; j0 < n; j0 += Bo) {
      const int64_t bo = (n - j0 < Bo) ? n - j0 : Bo;
      for (int64_t s0 = j0; s0 < j0 + bo; s0 += bi) {
        const int bw = int((j0 + bo - s0) < bi ? (j0 + bo - s0) : bi);
        QUIP_TRY(sweep(bi, W, ldw, F, n, fold ? j0 > 0 : s0 > 0, U, n, scales, L, m, s0, bw, cd,
                       n, What, n, Eb + (s0 - j0), Bo, D, rl, Eb, fold ? int(s0 - j0) : 0, s));
        if (!fold)  // rest of this batch
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
  float* ybuf[2];  // pre-rounding vectors, alternating between group steps
  ybuf[0] = c.take<float>(size_t(m) * 8);
  ybuf[1] = c.take<float>(size_t(m) * 8);
  const int64_t rbk = cdiv(m, 32);
  unsigned* done = c.take<unsigned>(size_t(rbk));  // per row block: groups done
  e8_take_book(c, e);
  e.sse = c.take<double>(64);
  e.part = c.take<double>(e8_partial_count(m, n));
  e.cand = fac;
  e.F = F;
  e.Eb = Eb;
  if (!c.fits()) return fail(QUIP_ERR_WORKSPACE, "quip_ldlq: workspace too small");
  const bool compute = q.scale_mode == QUIP_SCALE_COMPUTE;
  QUIP_TRY(timed_launch("rownorm_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL(rownorm_kernel, dim3(unsigned(m)), dim3(256), 0, s, W, n, ldw, e.Wn, scales + 1,
                       compute);
  }));
  QUIP_TRY(e8_prepare_book(codebook, e, s));
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
  QUIP_TRY(fill_f32(reinterpret_cast<float*>(done), rbk, 0.f, s));  // counters <- 0
  uint16_t* cd = static_cast<uint16_t*>(codes);
  const int ysplit = e8_argmin_split(m);
  const dim3 grid{unsigned(rbk), unsigned(ysplit)};
  int par = 0;
  const bool fused_pre = ysplit >= 4;
  for (int64_t j0 = 0; j0 < n; j0 += B) {
    const int64_t bo = (n - j0 < B) ? n - j0 : B;
    for (int64_t c0 = j0; c0 < j0 + bo; c0 += 8) {
      const int nprev = int(c0 - j0);
      float* y8 = ybuf[par];
      // A block's first group needs the outer feedback F just updated. The
      // later groups' vectors come from the previous step's finish when the
      // search splits each row block over several work-groups (only one of
      // them finishes); with few, every group finishes and the separate
      // launch costs less than the finishers' extra latency.
      if (nprev == 0 || !fused_pre)
        QUIP_TRY(timed_launch("e8_prerounding_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
          QUIP_KERNEL(e8_prerounding_kernel, dim3(unsigned(cdiv(m, 16))), dim3(256), 0, s, e.Wn, n,
                      F, j0 > 0, Eb, B, nprev, U, c0, j0, m, y8);
        }, 16.0 * double(m) * double(nprev), 4.0 * double(m) * (double(nprev) + 24.0)));
      const bool more = fused_pre && c0 + 8 < j0 + bo;
      E8Finish fin{e.Wn, n, codebook, scales + 1, c0, cd, n / 8, What, Eb, B, nprev, y8, D, rl,
                   more ? ybuf[par ^ 1] : nullptr, j0 > 0 ? F : nullptr, U, j0};
      // the search, the step's codes, W^, errors and loss term, and the next
      // step's pre-rounding vectors
      QUIP_TRY(timed_launch("e8_argmin_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
        QUIP_KERNEL(e8_argmin_kernel, grid, dim3(256), 0, s, e.book(), sglob, m, e.keys, done, fin);
      }, 16.0 * 65536.0 * double(m), 32.0 * double(m) + 8.0 * double(m) * 8.0));
      par ^= 1;
    }
    QUIP_TRY(feedback_gemm(Eb, B, 0, bo, U, n, j0, j0 + bo, n, F, m, j0 > 0, "gemm:ldlq_outer", s));
  }
  return finish_loss(rl, m, loss, s);
}

}  // namespace quip
