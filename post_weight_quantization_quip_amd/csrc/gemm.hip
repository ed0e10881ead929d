// fp32 GEMM on the CDNA4 matrix cores: C = alpha * op(A) op(B) + beta * C_in.
//
// Used for every dense contraction of the pass: the Hessian X^T X (upper
// tiles only, mirrored), the LDL panel products and trailing updates (upper
// tiles only), the lazy LDLQ trailing update W[:, j+B:] += E U, the two small
// contractions of a Kronecker-factor multiply, and the proxy loss (with a
// fused dot-product epilogue, so E H is never written).
//
// Tiling: one work-group of 4 waves computes a BM x BN tile (BM, BN in
// {64, 128}); each wave owns a (BM/2) x (BN/2) sub-tile made of 32x32 blocks
// computed with v_mfma_f32_32x32x2f32 (wave64: A operand lane = i + 32k,
// B operand lane = j + 32k, D element (i, j) in lane j + 32*((i/4)%2),
// register (i%4) + 4*(i/8)). K advances 32 at a time through double-buffered
// LDS tiles stored K-major, so every operand read is 32 consecutive floats.
// The beta term's C tile is read into registers before the K loop.
// Work-group ids are remapped so that neighbouring tiles share an XCD's L2.
#include "common.h"

namespace quip {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 32;
constexpr int PAD = 4;

__device__ __forceinline__ float4 load4(const float* base, int64_t row, int64_t col, int64_t ld,
                                        int64_t rows, int64_t cols, bool vec) {
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (row >= rows) return v;
  const float* p = base + row * ld + col;
  if (vec && col + 3 < cols) {
    v = *reinterpret_cast<const float4*>(p);
  } else {
    if (col + 0 < cols) v.x = p[0];
    if (col + 1 < cols) v.y = p[1];
    if (col + 2 < cols) v.z = p[2];
    if (col + 3 < cols) v.w = p[3];
  }
  return v;
}

template <int BM, int BN, bool TA, bool TB, int EPI>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmArgs a, int tiles_m, int tiles_n,
                                                      int total, bool vecA, bool vecB) {
  __shared__ __align__(16) float As[2][BK][BM + PAD];
  __shared__ __align__(16) float Bs[2][BK][BN + PAD];

  constexpr int WBM = BM / 64;  // 32x32 blocks per wave along M
  constexpr int WBN = BN / 64;
  constexpr int LA = BM * BK / 4 / 256;  // float4 loads per thread
  constexpr int LB = BN * BK / 4 / 256;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- tile coordinates
  int bid = (EPI == EPI_DOT_SYM) ? int(blockIdx.x) : xcd_remap(blockIdx.x, total);
  int tm, tn;
  if (a.upper_tiles) {
    int rem = bid, r = 0;
    while (rem >= tiles_m - r) {
      rem -= tiles_m - r;
      ++r;
    }
    tm = r;
    tn = r + rem;
  } else if (EPI == EPI_DOT_SYM) {
    // column tile tn has K range [0, (tn+1) BN): longest tiles first, dealt
    // round-robin over the XCDs, so the short ones fill the tail
    tm = bid % tiles_m;
    tn = tiles_n - 1 - bid / tiles_m;
  } else {
    const int G = 8;
    int per_group = G * tiles_n;
    int group = bid / per_group;
    int first = group * G;
    int gsize = min(tiles_m - first, G);
    int in = bid % per_group;
    tm = first + in % gsize;
    tn = in / gsize;
  }
  const int64_t m0 = int64_t(tm) * BM, n0 = int64_t(tn) * BN;
  const int64_t bz = blockIdx.y;
  const float* A = a.A + bz * a.strideA;
  const float* B = a.B + bz * a.strideB;

  float4 ra[LA], rb[LB];

  auto gload = [&](int64_t k0) {
    const bool fullA = vecA && k0 + BK <= a.K && (TA ? (m0 + BM <= a.M) : (m0 + BM <= a.M));
    const bool fullB = vecB && k0 + BK <= a.K && n0 + BN <= a.N;
    if (fullA) {
#pragma unroll
      for (int i = 0; i < LA; ++i) {
        int idx = tid + 256 * i;
        if (TA) {
          int k = idx / (BM / 4), m4 = (idx % (BM / 4)) * 4;
          ra[i] = *reinterpret_cast<const float4*>(A + (k0 + k) * a.lda + m0 + m4);
        } else {
          int m = idx / (BK / 4), k4 = (idx % (BK / 4)) * 4;
          ra[i] = *reinterpret_cast<const float4*>(A + (m0 + m) * a.lda + k0 + k4);
        }
      }
    } else {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      int idx = tid + 256 * i;
      if (TA) {
        int k = idx / (BM / 4), m4 = (idx % (BM / 4)) * 4;
        ra[i] = load4(A, k0 + k, m0 + m4, a.lda, a.K, a.M, vecA);
      } else {
        int m = idx / (BK / 4), k4 = (idx % (BK / 4)) * 4;
        ra[i] = load4(A, m0 + m, k0 + k4, a.lda, a.M, a.K, vecA);
      }
    }
    }
    if (fullB) {
#pragma unroll
      for (int i = 0; i < LB; ++i) {
        int idx = tid + 256 * i;
        if (!TB) {
          int k = idx / (BN / 4), n4 = (idx % (BN / 4)) * 4;
          rb[i] = *reinterpret_cast<const float4*>(B + (k0 + k) * a.ldb + n0 + n4);
        } else {
          int n = idx / (BK / 4), k4 = (idx % (BK / 4)) * 4;
          rb[i] = *reinterpret_cast<const float4*>(B + (n0 + n) * a.ldb + k0 + k4);
        }
      }
    } else {
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      int idx = tid + 256 * i;
      if (!TB) {
        int k = idx / (BN / 4), n4 = (idx % (BN / 4)) * 4;
        rb[i] = load4(B, k0 + k, n0 + n4, a.ldb, a.K, a.N, vecB);
      } else {
        int n = idx / (BK / 4), k4 = (idx % (BK / 4)) * 4;
        rb[i] = load4(B, n0 + n, k0 + k4, a.ldb, a.N, a.K, vecB);
      }
    }
    }
  };
  auto sstore = [&](int buf, int64_t kcur) {
#pragma unroll
    for (int i = 0; i < LA; ++i) {
      int idx = tid + 256 * i;
      if (TA) {
        int k = idx / (BM / 4), m4 = (idx % (BM / 4)) * 4;
        *reinterpret_cast<float4*>(&As[buf][k][m4]) = ra[i];
      } else {
        int m = idx / (BK / 4), k4 = (idx % (BK / 4)) * 4;
        As[buf][k4 + 0][m] = ra[i].x;
        As[buf][k4 + 1][m] = ra[i].y;
        As[buf][k4 + 2][m] = ra[i].z;
        As[buf][k4 + 3][m] = ra[i].w;
      }
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      int idx = tid + 256 * i;
      if (!TB) {
        int k = idx / (BN / 4), n4 = (idx % (BN / 4)) * 4;
        float4 v = rb[i];
        if (EPI == EPI_DOT_SYM) {
          // upper triangle of B, off-diagonal entries doubled
          const int kd = int(kcur - n0) + k - n4;  // row minus column of v.x
          v.x = kd > 0 ? 0.f : (kd == 0 ? v.x : 2.f * v.x);
          v.y = kd > 1 ? 0.f : (kd == 1 ? v.y : 2.f * v.y);
          v.z = kd > 2 ? 0.f : (kd == 2 ? v.z : 2.f * v.z);
          v.w = kd > 3 ? 0.f : (kd == 3 ? v.w : 2.f * v.w);
        }
        *reinterpret_cast<float4*>(&Bs[buf][k][n4]) = v;
      } else {
        int n = idx / (BK / 4), k4 = (idx % (BK / 4)) * 4;
        Bs[buf][k4 + 0][n] = rb[i].x;
        Bs[buf][k4 + 1][n] = rb[i].y;
        Bs[buf][k4 + 2][n] = rb[i].z;
        Bs[buf][k4 + 3][n] = rb[i].w;
      }
    }
  };

  f32x16 acc[WBM][WBN];
#pragma unroll
  for (int i = 0; i < WBM; ++i)
#pragma unroll
    for (int j = 0; j < WBN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  // C_in for the beta term, read before the K loop so its latency overlaps it
  float* C = a.C + bz * a.strideC;
  const float* Cin = a.Cin ? a.Cin + bz * a.strideCin : C;
  const int64_t ldcin = a.Cin ? a.ldcin : a.ldc;
  const int krow = lane >> 5, kcol = lane & 31;
  f32x16 cpre[WBM][WBN];
  const bool useC = (EPI == EPI_STORE || EPI == EPI_SPLIT) && a.beta != 0.f;
  if (useC) {
#pragma unroll
    for (int i = 0; i < WBM; ++i)
#pragma unroll
      for (int j = 0; j < WBN; ++j) {
        const int64_t col = n0 + wn * (BN / 2) + j * 32 + kcol;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + wm * (BM / 2) + i * 32 + 8 * (r / 4) + 4 * krow + (r % 4);
          cpre[i][j][r] = (row < a.M && col < a.N) ? Cin[row * ldcin + col] : 0.f;
        }
      }
  }

  int64_t kend = a.K;
  if (EPI == EPI_DOT_SYM) kend = (n0 + BN < a.K) ? n0 + BN : a.K;  // rows k <= last column
  const int64_t nk = (kend + BK - 1) / BK;
  if (nk > 0) {
    gload(0);
    sstore(0, 0);
    __syncthreads();
  }
  int buf = 0;
  for (int64_t kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < BK / 2; ++kk) {
      float av[WBM], bv[WBN];
#pragma unroll
      for (int i = 0; i < WBM; ++i) av[i] = As[buf][2 * kk + krow][wm * (BM / 2) + i * 32 + kcol];
#pragma unroll
      for (int j = 0; j < WBN; ++j) bv[j] = Bs[buf][2 * kk + krow][wn * (BN / 2) + j * 32 + kcol];
#pragma unroll
      for (int i = 0; i < WBM; ++i)
#pragma unroll
        for (int j = 0; j < WBN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[i], bv[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) sstore(buf ^ 1, (kt + 1) * BK);
    __syncthreads();
    buf ^= 1;
  }

  // ---- epilogue
  double dsum = 0.0;
#pragma unroll
  for (int i = 0; i < WBM; ++i) {
#pragma unroll
    for (int j = 0; j < WBN; ++j) {
      const int64_t col = n0 + wn * (BN / 2) + j * 32 + kcol;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * (BM / 2) + i * 32 + 8 * (r / 4) + 4 * krow + (r % 4);
        if (row >= a.M || col >= a.N) continue;
        float v = a.alpha * acc[i][j][r];
        if (EPI == EPI_DOT || EPI == EPI_DOT_SYM) {
          dsum += double(v) * double(a.E[row * a.lde + col]);
        } else {
          if (useC) v += a.beta * cpre[i][j][r];
          if (EPI == EPI_SPLIT && col >= a.split)
            a.C2[row * a.ldc2 + (col - a.split)] = v;
          else
            C[row * a.ldc + col] = v;
          if (a.mirror && tm != tn) {
            float w = a.alpha * acc[i][j][r];
            if (a.beta != 0.f) w += a.beta * Cin[col * ldcin + row];
            C[col * a.ldc + row] = w;
          }
        }
      }
    }
  }
  if (EPI == EPI_DOT || EPI == EPI_DOT_SYM) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) dsum += __shfl_down(dsum, off, 64);
    if (lane == 0) atomicAdd(a.dot, dsum);
  }
}

template <int BM, int BN, bool TA, bool TB, int EPI>
quip_status launch_t(const GemmArgs& a, hipStream_t s, bool vecA, bool vecB) {
  int tiles_m = int(cdiv(a.M, BM)), tiles_n = int(cdiv(a.N, BN));
  int total = a.upper_tiles ? tiles_m * (tiles_m + 1) / 2 : tiles_m * tiles_n;
  if (total == 0 || a.batch == 0) return QUIP_OK;
  dim3 grid(total, a.batch);
  hipLaunchKernelGGL((gemm_kernel<BM, BN, TA, TB, EPI>), grid, dim3(256), 0, s, a, tiles_m,
                     tiles_n, total, vecA, vecB);
  return launch_check("gemm_kernel");
}

template <bool TA, bool TB, int EPI>
quip_status launch_tiles(const GemmArgs& a, hipStream_t s, bool vecA, bool vecB) {
  // Prefer 128x128 tiles; 64x64 when the 128-tile grid would not give every
  // CU two work-groups (small launches are latency-bound: more, smaller tiles
  // finish sooner); 64 along one dimension when only that one is small.
  int64_t t128 = cdiv(a.M, 128) * cdiv(a.N, 128) * a.batch;
  if (a.upper_tiles) t128 = cdiv(a.M, 128) * (cdiv(a.M, 128) + 1) / 2 * a.batch;
  if (t128 < 512) return launch_t<64, 64, TA, TB, EPI>(a, s, vecA, vecB);
  bool smallM = a.M <= 64;
  bool smallN = a.N <= 64;
  if (a.upper_tiles) smallN = smallM;  // square tiles for the triangular grid
  if (smallM && smallN) return launch_t<64, 64, TA, TB, EPI>(a, s, vecA, vecB);
  if (smallM) return launch_t<64, 128, TA, TB, EPI>(a, s, vecA, vecB);
  if (smallN) return launch_t<128, 64, TA, TB, EPI>(a, s, vecA, vecB);
  return launch_t<128, 128, TA, TB, EPI>(a, s, vecA, vecB);
}

template <int EPI>
quip_status launch_epi(const GemmArgs& a, hipStream_t s, bool vecA, bool vecB) {
  if (a.transA) {
    if (a.transB) return launch_tiles<true, true, EPI>(a, s, vecA, vecB);
    return launch_tiles<true, false, EPI>(a, s, vecA, vecB);
  }
  if (a.transB) return launch_tiles<false, true, EPI>(a, s, vecA, vecB);
  return launch_tiles<false, false, EPI>(a, s, vecA, vecB);
}

}  // namespace

quip_status gemm(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return QUIP_OK;
  if (a.upper_tiles && a.M != a.N) return fail(QUIP_ERR_SHAPE, "gemm: upper_tiles needs M == N");
  bool vecA = aligned16(a.A) && a.lda % 4 == 0 && a.strideA % 4 == 0;
  bool vecB = aligned16(a.B) && a.ldb % 4 == 0 && a.strideB % 4 == 0;
  switch (a.epi) {
    case EPI_STORE: return launch_epi<EPI_STORE>(a, s, vecA, vecB);
    case EPI_DOT: return launch_epi<EPI_DOT>(a, s, vecA, vecB);
    case EPI_SPLIT: return launch_epi<EPI_SPLIT>(a, s, vecA, vecB);
    case EPI_DOT_SYM:
      if (a.transB || a.K != a.N) return fail(QUIP_ERR_ARG, "gemm: symmetric dot needs B square, not transposed");
      return launch_epi<EPI_DOT_SYM>(a, s, vecA, vecB);
  }
  return fail(QUIP_ERR_ARG, "gemm: bad epilogue");
}

}  // namespace quip
