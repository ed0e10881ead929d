// LDL factorization H = (I + U) D (I + U)^T, U strictly (block-)upper, the
// factor through which LDLQ feeds rounding errors back (QuIP, "Adaptive
// Rounding Step"; the 8x8-block form serves BlockLDLQ, named on the QTIP
// page under "Builds on").
//
// Blocked right-looking algorithm working from the last column block to the
// first, with NB = 64 columns per block:
//   1. ldl_diag_kernel (one work-group): factor the NB x NB diagonal block
//      A_KK = (I + U_KK) D_K (I + U_KK)^T in LDS, building on the way the
//      inverse V = (I + U_KK)^{-1} as a product of elementary factors, and
//      emit R = [V^T | V^T D_K^{-1}].
//   2. Panel product on the matrix cores: [X | U_IK] = A_IK R for the rows
//      above the block (X = U_IK D_K).
//   3. Trailing update on the matrix cores, upper tiles only:
//      A_IJ -= X_I U_JK^T for I, J above the block.
// The input is never modified: the first trailing update reads H and writes
// the workspace copy.
#include "common.h"

namespace quip {

quip_status ldl_factor(const float* H, int64_t n, int64_t ldh, int g, float* U, float* D,
                       int32_t* info, void* ws, size_t ws_bytes, hipStream_t s);
size_t ldl_workspace_bytes(int64_t n);

namespace {

constexpr int NB = 64;

// Factor the w x w diagonal block at (k0, k0) of `src` (upper triangle read).
// Writes U[k0.., k0..] (whole w x w block, zeros on/below the diagonal or the
// diagonal blocks), D, R (w x 2w, row-major) and, on the first failure, info.
template <int G>
__global__ __launch_bounds__(256) void ldl_diag_kernel(const float* src, int64_t lds_, int64_t k0,
                                                       int w, float* U, int64_t n, float* D,
                                                       float* R, int32_t* info) {
  __shared__ float S[NB][NB + 1];
  __shared__ float V[NB][NB + 1];
  __shared__ float Us[NB][NB + 1];
  __shared__ float dinv[NB][G];  // G = 1: 1/d_k; G = 8: rows of the inverse diagonal block
  __shared__ float dval[NB][G];
  __shared__ int bad;

  const int tid = threadIdx.x;
  for (int e = tid; e < NB * NB; e += 256) {
    int i = e / NB, j = e % NB;
    float v = 0.f;
    if (i < w && j < w) {
      int a = i < j ? i : j, b = i < j ? j : i;
      v = src[(k0 + a) * lds_ + (k0 + b)];
    }
    S[i][j] = v;
    V[i][j] = i == j ? 1.f : 0.f;
    Us[i][j] = 0.f;
  }
  if (tid == 0) bad = -1;
  __syncthreads();

  if (G == 1) {
    for (int k = w - 1; k >= 0; --k) {
      const float d = S[k][k];
      if (tid == 0) {
        if (!(d > 0.f) && bad < 0) bad = k;
        dval[k][0] = d;
        dinv[k][0] = 1.f / d;
      }
      const float rd = 1.f / d;
      if (tid < k) Us[tid][k] = S[tid][k] * rd;
      __syncthreads();
      // S[i][j] -= S[i][k] * u_j  for i <= j < k ;  V[i][j] -= u_i V[k][j] for i < k <= j
      for (int e = tid; e < k * k; e += 256) {
        int i = e / k, j = e % k;
        if (i <= j) S[i][j] -= S[i][k] * Us[j][k];
      }
      for (int e = tid; e < k * (w - k); e += 256) {
        int i = e / (w - k), j = k + e % (w - k);
        V[i][j] -= Us[i][k] * V[k][j];
      }
      __syncthreads();
    }
  } else {
    __shared__ float Dk[8][8];
    __shared__ float Di[8][8];
    for (int kb = w / 8 - 1; kb >= 0; --kb) {
      const int c0 = kb * 8;
      if (tid == 0) {
        // Cholesky of the 8x8 pivot block, then its inverse.
        float L[8][8];
        bool ok = true;
        for (int a = 0; a < 8; ++a)
          for (int b = 0; b < 8; ++b) {
            int lo = a < b ? a : b, hi = a < b ? b : a;
            Dk[a][b] = S[c0 + lo][c0 + hi];
            L[a][b] = 0.f;
          }
        for (int j = 0; j < 8; ++j) {
          float sdiag = Dk[j][j];
          for (int t = 0; t < j; ++t) sdiag -= L[j][t] * L[j][t];
          if (!(sdiag > 0.f)) ok = false;
          float ljj = sqrtf(sdiag);
          L[j][j] = ljj;
          for (int i = j + 1; i < 8; ++i) {
            float v = Dk[i][j];
            for (int t = 0; t < j; ++t) v -= L[i][t] * L[j][t];
            L[i][j] = v / ljj;
          }
        }
        if (!ok && bad < 0) bad = c0;
        // inverse of L (lower), then Di = L^-T L^-1
        float Li[8][8];
        for (int c = 0; c < 8; ++c)
          for (int i = 0; i < 8; ++i) {
            float v = i == c ? 1.f : 0.f;
            for (int t = c; t < i; ++t) v -= L[i][t] * Li[t][c];
            Li[i][c] = i < c ? 0.f : v / L[i][i];
          }
        for (int a = 0; a < 8; ++a)
          for (int b = 0; b < 8; ++b) {
            float v = 0.f;
            for (int t = 0; t < 8; ++t) v += Li[t][a] * Li[t][b];
            Di[a][b] = v;
          }
        for (int a = 0; a < 8; ++a)
          for (int b = 0; b < 8; ++b) {
            dinv[c0 + a][b] = Di[a][b];
            dval[c0 + a][b] = Dk[a][b];
          }
      }
      __syncthreads();
      // U_{i, c0+b} = sum_a S[i][c0+a] Di[a][b], rows i < c0
      for (int e = tid; e < c0 * 8; e += 256) {
        int i = e / 8, b = e % 8;
        float v = 0.f;
#pragma unroll
        for (int a = 0; a < 8; ++a) v += S[i][c0 + a] * Di[a][b];
        Us[i][c0 + b] = v;
      }
      __syncthreads();
      for (int e = tid; e < c0 * c0; e += 256) {
        int i = e / c0, j = e % c0;
        if (i <= j) {
          float v = 0.f;
#pragma unroll
          for (int a = 0; a < 8; ++a) v += Us[i][c0 + a] * S[j][c0 + a];
          S[i][j] -= v;
        }
      }
      for (int e = tid; e < c0 * (w - c0); e += 256) {
        int i = e / (w - c0), j = c0 + e % (w - c0);
        float v = 0.f;
#pragma unroll
        for (int a = 0; a < 8; ++a) v += Us[i][c0 + a] * V[c0 + a][j];
        V[i][j] -= v;
      }
      __syncthreads();
    }
  }

  // outputs
  for (int e = tid; e < w * w; e += 256) {
    int i = e / w, j = e % w;
    U[(k0 + i) * n + (k0 + j)] = Us[i][j];
    // R[r][c] = V[c][r] ; R[r][w + c] = sum_b V[b][r] Dinv[b][c]
    float rv = V[j][i];
    float rd;
    if (G == 1) {
      rd = V[j][i] * dinv[j][0];
    } else {
      int cb = (j / 8) * 8;
      rd = 0.f;
#pragma unroll
      for (int b = 0; b < 8; ++b) rd += V[cb + b][i] * dinv[cb + b][j - cb];
    }
    R[i * (2 * w) + j] = rv;
    R[i * (2 * w) + w + j] = rd;
  }
  if (G == 1) {
    for (int i = tid; i < w; i += 256) D[k0 + i] = dval[i][0];
  } else {
    for (int e = tid; e < w * 8; e += 256) {
      int i = e / 8, b = e % 8;
      D[(k0 + i) * 8 + b] = dval[i][b];  // block (k0+i)/8, row (k0+i)%8, column b
    }
  }
  if (tid == 0 && bad >= 0) atomicCAS(info, 0, int32_t(k0 + bad + 1));
}

}  // namespace

size_t ldl_workspace_bytes(int64_t n) {
  Carver c(nullptr, 0);
  c.take<float>(size_t(n) * n);       // working copy of the upper triangle
  c.take<float>(size_t(n) * NB);      // X panel
  c.take<float>(size_t(NB) * 2 * NB);  // R
  return c.used;
}

quip_status ldl_factor(const float* H, int64_t n, int64_t ldh, int g, float* U, float* D,
                       int32_t* info, void* ws, size_t ws_bytes, hipStream_t s) {
  Carver c(ws, ws_bytes);
  float* Aw = c.take<float>(size_t(n) * n);
  float* Xp = c.take<float>(size_t(n) * NB);
  float* R = c.take<float>(size_t(NB) * 2 * NB);
  if (!c.fits()) return fail(QUIP_ERR_WORKSPACE, "quip_ldl: workspace too small");

  QUIP_TRY(fill_matrix(U, n, n, n, 0.f, s));
  {
    // info <- 0 (one int32): reuse the float fill on its bit pattern
    QUIP_TRY(fill_f32(reinterpret_cast<float*>(info), 1, 0.f, s));
  }
  const int64_t nblk = cdiv(n, NB);
  bool first = true;
  for (int64_t K = nblk - 1; K >= 0; --K) {
    const int64_t k0 = K * NB;
    const int w = int(n - k0 < NB ? n - k0 : NB);
    const float* src = first ? H : Aw;
    const int64_t lsrc = first ? ldh : n;
    if (g == 1)
      hipLaunchKernelGGL((ldl_diag_kernel<1>), dim3(1), dim3(256), 0, s, src, lsrc, k0, w, U, n, D,
                         R, info);
    else
      hipLaunchKernelGGL((ldl_diag_kernel<8>), dim3(1), dim3(256), 0, s, src, lsrc, k0, w, U, n, D,
                         R, info);
    QUIP_TRY(launch_check("ldl_diag_kernel"));
    if (k0 == 0) break;
    // [X | U_IK] = A_IK R
    GemmArgs p;
    p.M = k0;
    p.N = 2 * w;
    p.K = w;
    p.A = src + k0;
    p.lda = lsrc;
    p.B = R;
    p.ldb = 2 * w;
    p.C = Xp;
    p.ldc = w;
    p.epi = EPI_SPLIT;
    p.split = w;
    p.C2 = U + k0;
    p.ldc2 = n;
    QUIP_TRY(gemm(p, s));
    // A_IJ -= X_I U_J^T  (upper tiles of the leading k0 x k0 block)
    GemmArgs t;
    t.M = k0;
    t.N = k0;
    t.K = w;
    t.A = Xp;
    t.lda = w;
    t.B = U + k0;  // op(B)[k][j] = U[j][k0 + k]
    t.ldb = n;
    t.transB = true;
    t.C = Aw;
    t.ldc = n;
    t.Cin = src;
    t.ldcin = lsrc;
    t.alpha = -1.f;
    t.beta = 1.f;
    t.upper_tiles = true;
    QUIP_TRY(gemm(t, s));
    first = false;
  }
  return QUIP_OK;
}

}  // namespace quip
