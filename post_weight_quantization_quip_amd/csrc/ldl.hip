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

constexpr int LDL_NB = 64;   // columns per diagonal block (one register column per thread)
constexpr int LDL_NO = 256;  // columns per outer block (K of the trailing update)

quip_status ldl_factor(const float* H, int64_t n, int64_t ldh, int g, float* U, float* D,
                       int32_t* info, void* ws, size_t ws_bytes, hipStream_t s);
size_t ldl_workspace_bytes(int64_t n);

namespace {

// Factor the w x w diagonal block at (k0, k0) of `src` (upper triangle read).
//
// Thread (j, q) holds rows [16q, 16q + 16) of column j of the block in
// registers. A column that has not been pivoted yet holds the partially
// reduced block S (full symmetric storage); once column j has been pivoted it
// holds column j of V = (I + U_KK)^{-1}, built as a product of elementary
// factors V <- (I - u_k e_k^T) V. Both updates of pivot k take the same form
//     R[i] -= c_i * h_j   (i < k),   c_i = S[i][k],   h_j = R_j[k] / d,
// except for the pivot column itself, which uses h = 1 + 1/d to turn its S
// column into the V column (-u). Row k of every column is broadcast through
// LDS by the row group that holds it (one barrier per pivot, double-buffered).
// For 8x8 pivots (G = 8) c and h are 8-vectors and 1/d is D_K^{-1}, which one
// thread computes (Cholesky) into LDS.
// Outputs: U[k0.., k0..] (the whole w x w block), D, R = [V^T | V^T D^{-1}]
// (w x 2w, row-major) and, on the first failing pivot, info.
template <int NB, int G>
__global__ __launch_bounds__(NB * NB / 16) void ldl_diag_kernel(const float* src, int64_t lds_,
                                                                int64_t k0, int w, float* U,
                                                                int64_t n, float* D, float* R,
                                                                int32_t* info) {
  constexpr int RG = 16;
  constexpr int NT = NB * NB / RG;
  __shared__ float tile[NB][NB + 1];  // input block, then the U block
  __shared__ __align__(16) float colk[2][G][NB];
  __shared__ float dsh[NB][G];
  __shared__ float dinv[NB][G];
  __shared__ float Dis[8][8];
  __shared__ float Lsh[8][8], Lish[8][8];
  __shared__ int bad_sh;

  const int t = threadIdx.x;
  const int j = t % NB, q = t / NB;
  const int r0 = RG * q;
  {
    constexpr int NL = NB * NB / NT;  // loads per thread, all issued before the stores
    float v[NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int e = t + NT * i;
      const int r = e / NB, c = e % NB;
      v[i] = (r < w && c < w && r <= c) ? src[(k0 + r) * lds_ + (k0 + c)] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int e = t + NT * i;
      tile[e / NB][e % NB] = v[i];
    }
  }
  if (t == 0) bad_sh = -1;
  __syncthreads();
  float Rr[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const int i = r0 + r;
    Rr[r] = (i <= j) ? tile[i][j] : tile[j][i];
  }
  __syncthreads();
  for (int e = t; e < NB * NB; e += NT) tile[e / NB][e % NB] = 0.f;  // becomes the U block
  __syncthreads();

  if constexpr (G == 1) {
    // pivots k = 16 qk + r, last to first; r is a compile-time register index
    for (int qk = (w - 1) / RG; qk >= 0; --qk) {
#pragma unroll
      for (int r = RG - 1; r >= 0; --r) {
        const int k = RG * qk + r;
        if (k < w) {
          float* ck = colk[k & 1][0];
          if (q == qk) ck[j] = Rr[r];
          __syncthreads();
          // every LDS read of this pivot up front, one wait
          const float d = ck[k];
          const float rkj = ck[j];
          float cc[RG];
          {
            const float4* c4 = reinterpret_cast<const float4*>(ck + r0);
#pragma unroll
            for (int v = 0; v < RG / 4; ++v) {
              const float4 c = c4[v];
              cc[4 * v + 0] = c.x;
              cc[4 * v + 1] = c.y;
              cc[4 * v + 2] = c.z;
              cc[4 * v + 3] = c.w;
            }
          }
          const float rd = __builtin_amdgcn_rcpf(d);  // pivot reciprocal (1 ulp)
          const float h = (j == k) ? 1.f + rd : rd * rkj;
          if (t == 0) {
            if (!(d > 0.f) && bad_sh < 0) bad_sh = k;
            dsh[k][0] = d;
            dinv[k][0] = rd;
          }
          if (q == 0 && j < k) tile[j][k] = rkj * rd;
          if (r0 + RG <= k) {  // whole row group above the pivot
#pragma unroll
            for (int rr = 0; rr < RG; ++rr) Rr[rr] = fmaf(-cc[rr], h, Rr[rr]);
          } else if (r0 < k) {  // the row group of the pivot: rows below k are kept
#pragma unroll
            for (int rr = 0; rr < RG; ++rr) Rr[rr] = (rr < r) ? fmaf(-cc[rr], h, Rr[rr]) : Rr[rr];
          }
          if (j == k && q == qk) Rr[r] = 1.f;
        }
      }
    }
  } else {
    for (int qk = (w - 1) / RG; qk >= 0; --qk) {
#pragma unroll
    for (int hb = 1; hb >= 0; --hb) {  // the two 8-row halves of row group qk
      const int kb = 2 * qk + hb;
      const int c0 = kb * 8;
      if (c0 >= w) continue;
      float(*ck)[NB] = colk[kb & 1];
      if (q == qk) {
#pragma unroll
        for (int a = 0; a < 8; ++a) ck[a][j] = Rr[8 * hb + a];
      }
      __syncthreads();
      if (t == 0) {
        float(*Lc)[8] = Lsh;  // thread 0 works in LDS to keep registers free
        bool ok = true;
#pragma unroll
        for (int a = 0; a < 8; ++a) {
          float sd = ck[a][c0 + a];
#pragma unroll
          for (int x = 0; x < a; ++x) sd -= Lc[a][x] * Lc[a][x];
          ok = ok && (sd > 0.f);
          const float la = sqrtf(sd);
          Lc[a][a] = la;
#pragma unroll
          for (int b = a + 1; b < 8; ++b) {
            float v = ck[a][c0 + b];
#pragma unroll
            for (int x = 0; x < a; ++x) v -= Lc[b][x] * Lc[a][x];
            Lc[b][a] = v / la;
          }
        }
        if (!ok && bad_sh < 0) bad_sh = c0;
        float(*Li)[8] = Lish;
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            if (i < c) {
              Li[i][c] = 0.f;
            } else {
              float v = (i == c) ? 1.f : 0.f;
#pragma unroll
              for (int x = c; x < i; ++x) v -= Lc[i][x] * Li[x][c];
              Li[i][c] = v / Lc[i][i];
            }
          }
#pragma unroll
        for (int a = 0; a < 8; ++a)
#pragma unroll
          for (int b = 0; b < 8; ++b) {
            float v = 0.f;
#pragma unroll
            for (int x = 0; x < 8; ++x) v += Li[x][a] * Li[x][b];
            Dis[a][b] = v;
            dinv[c0 + a][b] = v;
            dsh[c0 + a][b] = ck[b][c0 + a];
          }
      }
      __syncthreads();
      const bool piv = (j >= c0) && (j < c0 + 8);
      const int jp = piv ? j - c0 : 0;
      float h[8];
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        float v = 0.f;
#pragma unroll
        for (int a = 0; a < 8; ++a) v = fmaf(Dis[b][a], ck[a][j], v);
        h[b] = piv ? ((b == jp ? 1.f : 0.f) + Dis[b][jp]) : v;
      }
      if (q == 0 && j < c0) {
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          float v = 0.f;
#pragma unroll
          for (int a = 0; a < 8; ++a) v = fmaf(ck[a][j], Dis[a][b], v);
          tile[j][c0 + b] = v;
        }
      }
      if (r0 < c0) {
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const float4* c4 = reinterpret_cast<const float4*>(&ck[b][r0]);
#pragma unroll
          for (int v = 0; v < RG / 4; ++v) {
            const float4 c = c4[v];
            const float cc[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * v + e;
              const float ci = (r0 + r < c0) ? cc[e] : 0.f;
              Rr[r] = fmaf(-ci, h[b], Rr[r]);
            }
          }
        }
      }
      if (piv && q == qk) {
#pragma unroll
        for (int a = 0; a < 8; ++a) Rr[8 * hb + a] = (a == jp) ? 1.f : 0.f;
      }
    }
    }
  }
  __syncthreads();

  // U block
  for (int e = t; e < w * w; e += NT) {
    const int r = e / w, c = e % w;
    U[(k0 + r) * n + (k0 + c)] = tile[r][c];
  }
  if (q == 0 && j < w) {
#pragma unroll
    for (int b = 0; b < G; ++b) D[(k0 + j) * G + b] = dsh[j][b];
  }
  // R[j][c] = V[c][j] for c < j (1 at c = j, 0 above); R[j][w + c] = sum_b V[b][j] Dinv[b][c]
  if (j < w) {
    float* Rrow = R + j * (2 * w);
#pragma unroll
    for (int r = 0; r < RG; ++r) {
      const int c = r0 + r;
      if (c < w) {
        const float v = c < j ? Rr[r] : (c == j ? 1.f : 0.f);
        Rrow[c] = v;
        float vd;
        if constexpr (G == 1) {
          vd = v * dinv[c][0];
        } else {
          const int rb = r & ~7;  // first row of c's 8-block inside this thread
          vd = 0.f;
#pragma unroll
          for (int b = 0; b < 8; ++b) {
            const int cbb = r0 + rb + b;
            const float vb = cbb < j ? Rr[rb + b] : (cbb == j ? 1.f : 0.f);
            vd = fmaf(vb, dinv[cbb][c - (r0 + rb)], vd);
          }
        }
        Rrow[w + c] = vd;
      }
    }
  }
  if (t == 0 && bad_sh >= 0) atomicCAS(info, 0, int32_t(k0 + bad_sh + 1));
}

}  // namespace

size_t ldl_workspace_bytes(int64_t n) {
  Carver c(nullptr, 0);
  c.take<float>(size_t(n) * n);       // working copy of the upper triangle
  c.take<float>(size_t(n) * LDL_NO);          // X panel of an outer block
  c.take<float>(size_t(LDL_NB) * 2 * LDL_NB);  // R
  return c.used;
}

quip_status ldl_factor(const float* H, int64_t n, int64_t ldh, int g, float* U, float* D,
                       int32_t* info, void* ws, size_t ws_bytes, hipStream_t s) {
  Carver c(ws, ws_bytes);
  float* Aw = c.take<float>(size_t(n) * n);
  constexpr int NB = LDL_NB;
  constexpr int NO = LDL_NO;
  float* Xp = c.take<float>(size_t(n) * NO);
  float* R = c.take<float>(size_t(NB) * 2 * NB);
  if (!c.fits()) return fail(QUIP_ERR_WORKSPACE, "quip_ldl: workspace too small");

  QUIP_TRY(fill_matrix(U, n, n, n, 0.f, s));
  QUIP_TRY(fill_f32(reinterpret_cast<float*>(info), 1, 0.f, s));  // info <- 0 (bit pattern)

  // Outer blocks of NO columns from the last to the first; inside each, inner
  // blocks of NB columns (diagonal factor, panel product for every row above,
  // update of the outer block's remaining columns); then one trailing update
  // of the leading block with K = NO.
  const int64_t nouter = cdiv(n, NO);
  // Which copy holds the current values: the leading block [0, o1)^2 is in Aw
  // once an outer trailing update has run (aw_lead); inside an outer block its
  // columns are in Aw once aw_lead held or an inner update has run (aw_outer).
  bool aw_lead = false;
  for (int64_t O = nouter - 1; O >= 0; --O) {
    const int64_t o0 = O * NO;
    const int64_t o1 = (o0 + NO < n) ? o0 + NO : n;
    const int64_t nin = cdiv(o1 - o0, NB);
    bool aw_outer = aw_lead;
    for (int64_t b = nin - 1; b >= 0; --b) {
      const int64_t k0 = o0 + b * NB;
      const int w = int((o1 - k0) < NB ? (o1 - k0) : NB);
      const float* src = aw_outer ? Aw : H;
      const int64_t lsrc = aw_outer ? n : ldh;
      if (g == 1)
        hipLaunchKernelGGL((ldl_diag_kernel<NB, 1>), dim3(1), dim3(NB * NB / 16), 0, s, src, lsrc,
                           k0, w, U, n, D, R, info);
      else
        hipLaunchKernelGGL((ldl_diag_kernel<NB, 8>), dim3(1), dim3(NB * NB / 16), 0, s, src, lsrc,
                           k0, w, U, n, D, R, info);
      QUIP_TRY(launch_check("ldl_diag_kernel"));
      if (k0 == 0) break;
      // [X | U_IK] = A_IK R for all rows above the block
      GemmArgs p;
      p.M = k0;
      p.N = 2 * w;
      p.K = w;
      p.A = src + k0;
      p.lda = lsrc;
      p.B = R;
      p.ldb = 2 * w;
      p.C = Xp + (k0 - o0);
      p.ldc = NO;
      p.epi = EPI_SPLIT;
      p.split = w;
      p.C2 = U + k0;
      p.ldc2 = n;
      QUIP_TRY(gemm(p, s));
      if (b > 0) {
        // the outer block's columns left of this one: A[:k0, o0:k0] -= X U[o0:k0, blk]^T
        GemmArgs t;
        t.M = k0;
        t.N = k0 - o0;
        t.K = w;
        t.A = Xp + (k0 - o0);
        t.lda = NO;
        t.B = U + o0 * n + k0;  // op(B)[k][jj] = U[o0 + jj][k0 + k]
        t.ldb = n;
        t.transB = true;
        t.C = Aw + o0;
        t.ldc = n;
        t.Cin = src + o0;
        t.ldcin = lsrc;
        t.alpha = -1.f;
        t.beta = 1.f;
        QUIP_TRY(gemm(t, s));
        aw_outer = true;
      }
    }
    if (o0 == 0) break;
    // trailing update of the leading o0 x o0 block (upper tiles), K = outer width
    const float* src = aw_lead ? Aw : H;
    const int64_t lsrc = aw_lead ? n : ldh;
    GemmArgs t;
    t.M = o0;
    t.N = o0;
    t.K = o1 - o0;
    t.A = Xp;
    t.lda = NO;
    t.B = U + o0;  // op(B)[k][jj] = U[jj][o0 + k]
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
    aw_lead = true;
  }
  return QUIP_OK;
}

}  // namespace quip
