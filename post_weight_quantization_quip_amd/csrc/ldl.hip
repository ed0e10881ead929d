// LDL factorization H = (I + U) D (I + U)^T, U strictly (block-)upper, the
// factor through which LDLQ feeds rounding errors back (QuIP, "Adaptive
// Rounding Step"; the 8x8-block form serves BlockLDLQ, named on the QTIP
// page under "Builds on").
//
// Blocked right-looking algorithm working from the last column block to the
// first, NB = 64 columns per block:
//   1. ldl_block_kernel: every work-group takes PR rows above the block and
//      the NB x NB diagonal block A_KK, factors A_KK (redundantly: each group
//      computes bit-identical factors, so no group waits for another) and
//      turns its rows into U_IK = A_IK (I + U_KK)^{-T} D_K^{-1} and
//      X_IK = U_IK D_K.
//   2. Trailing update on the matrix cores, upper tiles only:
//      A_IJ -= X_I U_JK^T for I, J above the block (two levels: the columns of
//      the current NO-wide outer block right away, the rest once per outer
//      block with K = NO).
// The input is never modified: the first trailing update reads H and writes
// the workspace copy.
#include <utility>

#include "common.h"

namespace quip {

constexpr int LDL_NB = 64;   // columns per diagonal block
// Columns per outer block (K of the outer trailing update): 256 up to
// n = 4096, 512 above, where each outer update's read-modify-write of the
// leading block costs more than the longer inner updates (28672 columns: LDL
// 94 -> 86 ms; 11008: 8.75 -> 8.35 ms; 4096: unchanged; 1024: slower again).
inline int64_t ldl_outer_width(int64_t n) { return n > 4096 ? 512 : 256; }
constexpr int LDL_PR = 64;   // rows above the diagonal block per work-group

quip_status ldl_factor(const float* H, int64_t n, int64_t ldh, int g, float* U, float* D,
                       int32_t* info, void* ws, size_t ws_bytes, hipStream_t s);
size_t ldl_workspace_bytes(int64_t n);

namespace {

// Compile-time loop: f(std::integral_constant<int, I>) for I = 0 .. N-1.
template <typename F, int... I>
__device__ __forceinline__ void static_for_(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_(f, std::make_integer_sequence<int, N>{});
}

// First float4 slot of column l in the packed strictly-upper 16 x 16 factor.
__host__ __device__ constexpr int ut_off(int l) {
  int o = 0;
  for (int c = 1; c < l; ++c) o += (c + 3) / 4;
  return o;
}
static_assert(ut_off(16) == 36, "packed factor size");

// Value of lane J of this lane's 16-lane row (DPP row_newbcast).
template <int J>
__device__ __forceinline__ float row_bcast(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + J, 0xF, 0xF, false));
}

// Cholesky of the 8x8 block P (upper triangle read) followed by its inverse;
// every lane computes the same values. Returns false on a non-positive pivot.
__device__ bool chol_inv8(const float (*P)[17], int r0, float (&Pinv)[8][8]) {
  float L[8][8];  // lower triangle used
  float rl[8];    // 1 / L[a][a]
  bool ok = true;
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    float sd = P[r0 + a][r0 + a];
#pragma unroll
    for (int x = 0; x < a; ++x) sd = fmaf(-L[a][x], L[a][x], sd);
    ok = ok && (sd > 0.f);
    // 1/sqrt to 1 ulp (the hardware's), and the root from it
    const float r = __builtin_amdgcn_rsqf(sd);
    rl[a] = r;
    L[a][a] = sd * r;
#pragma unroll
    for (int b = a + 1; b < 8; ++b) {
      float v = P[r0 + a][r0 + b];
#pragma unroll
      for (int x = 0; x < a; ++x) v = fmaf(-L[b][x], L[a][x], v);
      L[b][a] = v * rl[a];
    }
  }
  // L^{-1}, lower triangular, column by column (only its nonzero entries:
  // the loops run over the triangle, so no products with known zeros)
  float Li[8][8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    Li[c][c] = rl[c];
#pragma unroll
    for (int i = c + 1; i < 8; ++i) {
      float v = 0.f;
#pragma unroll
      for (int x = c; x < i; ++x) v = fmaf(L[i][x], Li[x][c], v);
      Li[i][c] = -v * rl[i];
    }
  }
  // P^{-1} = L^{-T} L^{-1}, symmetric: entry (a, b), a <= b, sums x >= b
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = a; b < 8; ++b) {
      float v = 0.f;
#pragma unroll
      for (int x = b; x < 8; ++x) v = fmaf(Li[x][a], Li[x][b], v);
      Pinv[a][b] = v;
      Pinv[b][a] = v;
    }
  return ok;
}

// Moves a rows x 64 block between global memory (leading dimension ld, first
// `cols` columns valid, rows below `nrows` absent) and an LDS tile with 65
// floats per row; float4 accesses when `vec`.
template <int NT, int R, bool LOAD>
__device__ __forceinline__ void tile_io(float (*T)[65], const float* gsrc, float* gdst, int64_t ld,
                                        int nrows, int cols, bool vec) {
  const int t = threadIdx.x;
  if (vec) {
    constexpr int NV = (R * 16 + NT - 1) / NT;
    float4 v[NV];
    if (LOAD) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int e = t + NT * i, a = e / 16, c4 = (e % 16) * 4;
        v[i] = (e < R * 16 && a < nrows) ? *reinterpret_cast<const float4*>(gsrc + a * ld + c4)
                                         : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int e = t + NT * i, a = e / 16, c4 = (e % 16) * 4;
        if (e < R * 16) {
          T[a][c4 + 0] = v[i].x;
          T[a][c4 + 1] = v[i].y;
          T[a][c4 + 2] = v[i].z;
          T[a][c4 + 3] = v[i].w;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int e = t + NT * i, a = e / 16, c4 = (e % 16) * 4;
        if (e < R * 16 && a < nrows)
          *reinterpret_cast<float4*>(gdst + a * ld + c4) =
              make_float4(T[a][c4 + 0], T[a][c4 + 1], T[a][c4 + 2], T[a][c4 + 3]);
      }
    }
  } else {
    constexpr int NS = (R * 64 + NT - 1) / NT;
    float v[NS];
    if (LOAD) {
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int e = t + NT * i, a = e / 64, c = e % 64;
        v[i] = (e < R * 64 && a < nrows && c < cols) ? gsrc[a * ld + c] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int e = t + NT * i;
        if (e < R * 64) T[e / 64][e % 64] = v[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int e = t + NT * i, a = e / 64, c = e % 64;
        if (e < R * 64 && a < nrows && c < cols) gdst[a * ld + c] = T[a][c];
      }
    }
  }
}

// One diagonal block and PR rows above it.
//
// Layout: thread t = ROWS * qt + r holds row r of the tall panel (rows
// [0, PR): the rows prow0 + r of the matrix above the block; rows PR + i:
// row i of the diagonal block, stored in full) restricted to the 16 columns
// [16 qt, 16 qt + 16) of the block, in registers s[0..15]. The diagonal block
// is read and its U written through an LDS tile (coalesced, and its lower
// triangle taken from the upper one); the rows above are read and their X
// and U written straight from the registers (64 contiguous bytes per thread).
// Column groups of 16 are processed from the last (gq = 3) to the first:
//   leaf  - the wave holding the group's 16 diagonal rows (one 16-lane DPP
//           row) factors the 16 x 16 sub-block S_gg = (I + U_gg) D_g
//           (I + U_gg)^T; for g = 1 the pivot row is broadcast with DPP, no
//           barrier; for g = 8 the two 8 x 8 pivots are Cholesky-inverted by
//           every lane;
//   solve - every row above the group solves x (I + U_gg)^T = a on its 16
//           columns (x = U D), then u = x D_g^{-1};
//   update- rows above subtract x U_{c,g}^T from their columns c left of the
//           group (U_{c,g} from the diagonal rows of the same pass).
// Outputs: U and X rows above the block from every group; the diagonal block
// of U, D and info from the first group.
template <int PR, int G>
__global__ __launch_bounds__(4 * (PR + 64)) void ldl_block_kernel(const float* src, int64_t lds_,
                                                                  int64_t k0, int w, float* U,
                                                                  int64_t n, float* D, float* Xp,
                                                                  int64_t ldx, int32_t* info) {
  constexpr int NB = 64, ROWS = PR + NB, NT = 4 * ROWS;
  __shared__ float tile[NB][65];   // diagonal block (upper triangle), later U's diagonal block
  __shared__ __align__(16) float Xs[ROWS][20];
  __shared__ __align__(16) float Us[NB][16];
  // column l of U_gg (rows j < l), packed: float4 slots ut_off(l) .. + ceil(l/4)
  __shared__ __align__(16) float4 UtP[36];
  __shared__ float dsh[NB][G];
  __shared__ float dinv[NB][G];
  __shared__ float L16[16][17];
  __shared__ int bad_sh;

  const int t = threadIdx.x;
  const int qt = t / ROWS, r = t % ROWS;
  const int lane = t & 63, wave = t >> 6;
  const bool is_panel = r < PR;
  const int64_t prow0 = int64_t(blockIdx.x) * PR;
  const int64_t grow = prow0 + r;
  const int npan = int(k0 - prow0 < PR ? (k0 - prow0 > 0 ? k0 - prow0 : 0) : PR);
  const bool live = !is_panel || r < npan;
  const int di = r - PR;  // row of the diagonal block (diagonal rows only)

  const bool vin = (w == NB) && (lds_ % 4 == 0) && ((reinterpret_cast<uintptr_t>(src) & 15) == 0);
  const bool vout = (w == NB) && (n % 4 == 0) && ((reinterpret_cast<uintptr_t>(U) & 15) == 0);
  const bool vx = (w == NB) && (ldx % 4 == 0) && ((reinterpret_cast<uintptr_t>(Xp) & 15) == 0);
  tile_io<NT, NB, true>(tile, src + k0 * lds_ + k0, nullptr, lds_, w, w, vin);
  float s[16];
  if (is_panel) {  // (uniform per wave) the row's 16 columns straight into registers
    const float* ar = src + (prow0 + r) * lds_ + k0 + 16 * qt;
    if (live && vin) {
      const float4* a4 = reinterpret_cast<const float4*>(ar);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float4 x = a4[v];
        s[4 * v + 0] = x.x;
        s[4 * v + 1] = x.y;
        s[4 * v + 2] = x.z;
        s[4 * v + 3] = x.w;
      }
    } else {
#pragma unroll
      for (int m = 0; m < 16; ++m) s[m] = (live && 16 * qt + m < w) ? ar[m] : 0.f;
    }
  }
  if (t == 0) bad_sh = -1;
  __syncthreads();
  if (!is_panel) {
    // the diagonal block from its tile (upper triangle stored; identity past w)
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const int c = 16 * qt + m;
      const float va = tile[di][c];
      const float vb = tile[c][di];
      float vd = (di <= c) ? va : vb;
      vd = (di >= w || c >= w) ? (di == c ? 1.f : 0.f) : vd;
      s[m] = vd;
    }
  }

  static_assert((ROWS + 16) % 16 == 0 && PR % 16 == 0, "leaf rows must form one DPP row");
  // a runtime loop: one copy of the group code stays in the instruction cache
#pragma nounroll
  for (int gq = 3; gq >= 0; --gq) {
    const int c0 = 16 * gq;
    const int base = ROWS * gq + PR + c0;  // thread of diagonal row c0 in column group gq
    const int wl = base / 64, lb = base % 64;
    const int il = lane - lb;
    // ---- leaf
    if (wave == wl) {
      if constexpr (G == 1) {
        // on a copy: the other lanes of this wave hold rows that still need s
        float ls[16], uu[16], dd[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) ls[k] = s[k];
        static_for<16>([&](auto KI) {
          constexpr int k = 15 - decltype(KI)::value;
          const float d = row_bcast<k>(ls[k]);
          const float rd = __builtin_amdgcn_rcpf(d);  // pivot reciprocal (1 ulp)
          const float u = ls[k] * rd;
          const float nu = -u;
          uu[k] = u;
          dd[k] = d;
          static_for<k>([&](auto JI) {
            constexpr int j = decltype(JI)::value;
            ls[j] = fmaf(row_bcast<k>(ls[j]), nu, ls[j]);
          });
        });
        if (il >= 0 && il < 16) {
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            const float v = k > il ? uu[k] : 0.f;
            if (k > il) reinterpret_cast<float*>(UtP)[4 * ut_off(k) + il] = v;
            s[k] = v;
          }
        }
        if (lane == lb) {
          int bad = -1;  // first non-positive pivot in processing order (highest index)
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            dsh[c0 + k][0] = dd[k];
            dinv[c0 + k][0] = __builtin_amdgcn_rcpf(dd[k]);
            bad = !(dd[k] > 0.f) ? c0 + k : bad;
          }
          if (bad >= 0 && bad_sh < 0) bad_sh = bad;
        }
      } else {
        if (il >= 0 && il < 16) {
#pragma unroll
          for (int k = 0; k < 16; ++k) L16[il][k] = s[k];
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        float Pinv[8][8];
        // second 8-block first
        const bool ok1 = chol_inv8(L16, 8, Pinv);
        float u8[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          float v = 0.f;
#pragma unroll
          for (int a = 0; a < 8; ++a) v = fmaf(s[8 + a], Pinv[a][b], v);
          u8[b] = v;  // rows il < 8: U[c0 + il][c0 + 8 + b]
        }
        if (lane == lb) {
#pragma unroll
          for (int a = 0; a < 8; ++a)
#pragma unroll
            for (int b = 0; b < 8; ++b) {
              dsh[c0 + 8 + a][b] = a <= b ? L16[8 + a][8 + b] : L16[8 + b][8 + a];
              dinv[c0 + 8 + a][b] = Pinv[a][b];
            }
          if (!ok1 && bad_sh < 0) bad_sh = c0 + 8;
        }
        // Schur complement of the first 8 rows: S00 -= u S10
        float s00[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float v = s[j];
#pragma unroll
          for (int b = 0; b < 8; ++b) v = fmaf(-u8[b], L16[j][8 + b], v);
          s00[j] = v;
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        if (il >= 0 && il < 8) {
#pragma unroll
          for (int j = 0; j < 8; ++j) L16[il][j] = s00[j];
        }
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        __builtin_amdgcn_wave_barrier();
        const bool ok0 = chol_inv8(L16, 0, Pinv);
        if (lane == lb) {
#pragma unroll
          for (int a = 0; a < 8; ++a)
#pragma unroll
            for (int b = 0; b < 8; ++b) {
              dsh[c0 + a][b] = a <= b ? L16[a][b] : L16[b][a];
              dinv[c0 + a][b] = Pinv[a][b];
            }
          if (!ok0 && ok1 && bad_sh < 0) bad_sh = c0;
        }
        if (il >= 0 && il < 16) {
#pragma unroll
          for (int k = 0; k < 16; ++k) {
            const float v = (il < 8 && k >= 8) ? u8[k - 8] : 0.f;
            if (k > il) reinterpret_cast<float*>(UtP)[4 * ut_off(k) + il] = v;
            s[k] = v;
          }
        }
      }
    }
    __syncthreads();
    const bool above = live && (is_panel || di < c0);
    // ---- solve x (I + U_gg)^T = a, then u = x D_g^{-1}
    {
      if (qt == gq && above) {
        // every column of U_gg up front (144 floats), then the back substitution
        float4 up[36];
#pragma unroll
        for (int v = 0; v < 36; ++v) up[v] = UtP[v];
        const float* uf = reinterpret_cast<const float*>(up);
#pragma unroll
        for (int l = 15; l > 0; --l) {
          const float xl = s[l];
#pragma unroll
          for (int j = 0; j < l; ++j) s[j] = fmaf(-xl, uf[4 * ut_off(l) + j], s[j]);
        }
        float4* x4 = reinterpret_cast<float4*>(Xs[r]);
#pragma unroll
        for (int v = 0; v < 4; ++v)
          x4[v] = make_float4(s[4 * v], s[4 * v + 1], s[4 * v + 2], s[4 * v + 3]);
        if (is_panel) {  // X of this row straight from the registers (64 bytes)
          float* xr = Xp + (prow0 + r) * ldx + c0;
          if (vx) {
            float4* x4g = reinterpret_cast<float4*>(xr);
#pragma unroll
            for (int v = 0; v < 4; ++v)
              x4g[v] = make_float4(s[4 * v], s[4 * v + 1], s[4 * v + 2], s[4 * v + 3]);
          } else {
#pragma unroll
            for (int l = 0; l < 16; ++l)
              if (c0 + l < w) xr[l] = s[l];
          }
        }
        if constexpr (G == 1) {
#pragma unroll
          for (int l = 0; l < 16; ++l) s[l] *= dinv[c0 + l][0];
        } else {
          float x[16];
#pragma unroll
          for (int l = 0; l < 16; ++l) x[l] = s[l];
#pragma unroll
          for (int hb = 0; hb < 2; ++hb)
#pragma unroll
            for (int a = 0; a < 8; ++a) {
              float v = 0.f;
#pragma unroll
              for (int b = 0; b < 8; ++b) v = fmaf(x[8 * hb + b], dinv[c0 + 8 * hb + b][a], v);
              s[8 * hb + a] = v;
            }
        }
        if (!is_panel) {
          float4* o4 = reinterpret_cast<float4*>(Us[di]);
#pragma unroll
          for (int v = 0; v < 4; ++v)
            o4[v] = make_float4(s[4 * v], s[4 * v + 1], s[4 * v + 2], s[4 * v + 3]);
        }
      }
    }
    if (gq > 0) {
      __syncthreads();
      // ---- update the columns left of the group
      if (qt < gq && above) {
        float x[16];
        const float4* x4 = reinterpret_cast<const float4*>(Xs[r]);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float4 c = x4[v];
          x[4 * v + 0] = c.x;
          x[4 * v + 1] = c.y;
          x[4 * v + 2] = c.z;
          x[4 * v + 3] = c.w;
        }
        const float4* us = reinterpret_cast<const float4*>(Us[16 * qt]);
        float4 cur[16], nxt[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) cur[v] = us[v];
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {  // columns 4 ch .. 4 ch + 3
          if (ch < 3) {
#pragma unroll
            for (int v = 0; v < 16; ++v) nxt[v] = us[16 * (ch + 1) + v];
          }
#pragma unroll
          for (int mm = 0; mm < 4; ++mm) {
            float acc = s[4 * ch + mm];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const float4 c = cur[4 * mm + v];
              acc = fmaf(-x[4 * v + 0], c.x, acc);
              acc = fmaf(-x[4 * v + 1], c.y, acc);
              acc = fmaf(-x[4 * v + 2], c.z, acc);
              acc = fmaf(-x[4 * v + 3], c.w, acc);
            }
            s[4 * ch + mm] = acc;
          }
          if (ch < 3) {
#pragma unroll
            for (int v = 0; v < 16; ++v) cur[v] = nxt[v];
          }
        }
      }
    }
  }

  // ---- outputs: the rows above straight from the registers (16 columns,
  // 64 bytes, per thread); the diagonal block through its LDS tile
  if (is_panel) {
    if (live) {
      float* ur = U + (prow0 + r) * n + k0 + 16 * qt;
      if (vout) {
        float4* u4 = reinterpret_cast<float4*>(ur);
#pragma unroll
        for (int v = 0; v < 4; ++v)
          u4[v] = make_float4(s[4 * v], s[4 * v + 1], s[4 * v + 2], s[4 * v + 3]);
      } else {
#pragma unroll
        for (int m = 0; m < 16; ++m)
          if (16 * qt + m < w) ur[m] = s[m];
      }
    }
  } else if (blockIdx.x == 0) {
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const int c = 16 * qt + m;
      const bool up = (G == 1) ? (c > di) : (c / 8 > di / 8);
      tile[di][c] = up ? s[m] : 0.f;
    }
  }
  if (blockIdx.x == 0) {
    __syncthreads();
    tile_io<NT, NB, false>(tile, nullptr, U + k0 * n + k0, n, w, w, vout);
    if (t < w) {
#pragma unroll
      for (int b = 0; b < G; ++b) D[(k0 + t) * G + b] = dsh[t][b];
    }
    if (t == 0 && bad_sh >= 0) atomicCAS(info, 0, int32_t(k0 + bad_sh + 1));
  }
}

typedef float ldl_f32x4 __attribute__((ext_vector_type(4)));

// Small trailing updates straight on the matrix cores: C[m][c] = Cin[m][c] -
// sum_k X[m][k] U[c][k], with K = 64 (an outer block's inner update) or
// K = 256 (the update of a small leading block, upper tiles only: tile row <=
// tile column, row-major). One work-group of four waves per 32 x 32 tile,
// each wave a 16 x 16 block on v_mfma_f32_16x16x4f32 with its operands
// straight from memory: lane (i, h) = (lane % 16, lane / 16) loads the K / 4
// consecutive k of quarter h of row i of X and of U (step t takes
// k = h K / 4 + t), and holds C's rows 4 h + r of column i. Two accumulators
// (even and odd steps) halve the dependent chain. No LDS and no barrier:
// these products are too small for operand reuse to pay, and the latency of
// their few steps is what they cost.
template <int K, bool UPPER>
__global__ __launch_bounds__(256) void ldl_update_kernel(const float* __restrict__ X, int64_t ldx,
                                                         const float* __restrict__ Ub, int64_t ldu,
                                                         const float* Cin, int64_t ldcin, float* C,
                                                         int64_t ldc, int tiles_n) {
  constexpr int KQ = K / 4;  // steps, and k per lane and quarter
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int i = lane & 15, h = lane >> 4;
  int tm, tn;
  if (UPPER) {  // row-major over the upper tiles of a tiles_n x tiles_n grid
    int rem = int(blockIdx.x), r = 0;
    while (rem >= tiles_n - r) {
      rem -= tiles_n - r;
      ++r;
    }
    tm = r;
    tn = r + rem;
  } else {
    tm = int(blockIdx.x) / tiles_n;
    tn = int(blockIdx.x) % tiles_n;
  }
  const int64_t m0 = int64_t(tm) * 32 + (wave >> 1) * 16;
  const int64_t n0 = int64_t(tn) * 32 + (wave & 1) * 16;
  const float4* xa = reinterpret_cast<const float4*>(X + (m0 + i) * ldx + KQ * h);
  const float4* ub = reinterpret_cast<const float4*>(Ub + (n0 + i) * ldu + KQ * h);
  float a[KQ], b[KQ];
#pragma unroll
  for (int v = 0; v < KQ / 4; ++v) {
    const float4 p = xa[v], q = ub[v];
    a[4 * v] = p.x;
    a[4 * v + 1] = p.y;
    a[4 * v + 2] = p.z;
    a[4 * v + 3] = p.w;
    b[4 * v] = q.x;
    b[4 * v + 1] = q.y;
    b[4 * v + 2] = q.z;
    b[4 * v + 3] = q.w;
  }
  float cin[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) cin[r] = Cin[(m0 + 4 * h + r) * ldcin + n0 + i];
  ldl_f32x4 e = {0.f, 0.f, 0.f, 0.f}, o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < KQ; t += 2) {
    e = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t], b[t], e, 0, 0, 0);
    o = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t + 1], b[t + 1], o, 0, 0, 0);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) C[(m0 + 4 * h + r) * ldc + n0 + i] = cin[r] - (e[r] + o[r]);
}

}  // namespace

size_t ldl_workspace_bytes(int64_t n) {
  Carver c(nullptr, 0);
  c.take<float>(size_t(n) * n);       // working copy of the upper triangle
  c.take<float>(size_t(n) * ldl_outer_width(n));  // X panel of an outer block
  return c.used;
}

quip_status ldl_factor(const float* H, int64_t n, int64_t ldh, int g, float* U, float* D,
                       int32_t* info, void* ws, size_t ws_bytes, hipStream_t s) {
  Carver c(ws, ws_bytes);
  float* Aw = c.take<float>(size_t(n) * n);
  constexpr int NB = LDL_NB;
  const int64_t NO = ldl_outer_width(n);
  constexpr int PR = LDL_PR;
  static_assert(NB % PR == 0, "block sizes");
  float* Xp = c.take<float>(size_t(n) * NO);
  if (!c.fits()) return fail(QUIP_ERR_WORKSPACE, "quip_ldl: workspace too small");

  // the kernels write every entry of U from each diagonal block's rows up
  // (zeros below the diagonal inside the block); the rest is zero, and so is
  // info, in the same launch
  QUIP_TRY(fill_lower_blocks(U, n, n, NB, info, s));

  // Outer blocks of NO columns from the last to the first; inside each, blocks
  // of NB columns (factor + rows above in one kernel, then the update of the
  // outer block's remaining columns); then one trailing update of the leading
  // block with K = NO.
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
      const dim3 grid(unsigned(k0 > 0 ? k0 / PR : 1));
      // work: the w x w factorization, then per row above a triangular solve
      // and the D^{-1} scaling; reads the block column, writes U, X and D
      const double wd = double(w), kd = double(k0);
      QUIP_TRY(timed_launch("ldl_block_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
        if (g == 1)
          QUIP_KERNEL((ldl_block_kernel<PR, 1>), grid, dim3(4 * (PR + NB)), 0, s, src, lsrc,
                             k0, w, U, n, D, Xp + (k0 - o0), int64_t(NO), info);
        else
          QUIP_KERNEL((ldl_block_kernel<PR, 8>), grid, dim3(4 * (PR + NB)), 0, s, src, lsrc,
                             k0, w, U, n, D, Xp + (k0 - o0), int64_t(NO), info);
      }, 2.0 / 3.0 * wd * wd * wd + kd * (wd * wd + wd),
         4.0 * ((kd + wd) * wd + 2.0 * kd * wd + wd * wd + wd * g)));
      if (k0 == 0) break;
      // the direct kernel while its 32 x 32 grid fits one round of four
      // work-groups per CU; larger products reuse operands through LDS tiles
      // (n = 28672: 283 against 281 ms per pass with the direct kernel throughout)
      if (b > 0 && w == NB && k0 % 32 == 0 && (k0 - o0) % 32 == 0 && NO % 4 == 0 &&
          n % 4 == 0 && aligned16(Xp) && aligned16(U) &&
          (k0 / 32) * ((k0 - o0) / 32) <= 4 * int64_t(device_cus())) {
        // the outer block's columns left of this one: A[:k0, o0:k0] -= X U[o0:k0, blk]^T
        const int tiles_n = int((k0 - o0) / 32);
        const double md = double(k0), nd = double(k0 - o0);
        QUIP_TRY(timed_launch("gemm:ldl_inner", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
          QUIP_KERNEL((ldl_update_kernel<64, false>), dim3(unsigned((k0 / 32) * tiles_n)), dim3(256), 0, s,
                      Xp + (k0 - o0), int64_t(NO), U + o0 * n + k0, n, src + o0, lsrc, Aw + o0,
                      n, tiles_n);
        }, 2.0 * md * nd * NB, 4.0 * (md * NB + nd * NB + 2.0 * md * nd)));
        aw_outer = true;
      } else if (b > 0) {
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
        t.tag = "gemm:ldl_inner";
        QUIP_TRY(gemm(t, s));
        aw_outer = true;
      }
    }
    if (o0 == 0) break;
    // trailing update of the leading o0 x o0 block (upper tiles), K = outer width
    const float* src = aw_lead ? Aw : H;
    const int64_t lsrc = aw_lead ? n : ldh;
    const int64_t tu = o0 / 32;  // 32 x 32 tiles per side
    if (o1 - o0 == 256 && o0 % 32 == 0 && NO % 4 == 0 && n % 4 == 0 && aligned16(Xp) &&
        aligned16(U) && tu * (tu + 1) / 2 <= 2 * int64_t(device_cus())) {
      // a small leading block (o0 <= 992 here): the direct kernel, 6-7 us
      // against 13 us for the LDS-tiled product, whose eight K steps each wait
      // on their loads; larger grids read too much from L2 without LDS reuse
      const double od = double(o0);
      QUIP_TRY(timed_launch("gemm:ldl_outer", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
        QUIP_KERNEL((ldl_update_kernel<256, true>), dim3(unsigned(tu * (tu + 1) / 2)), dim3(256),
                    0, s, Xp, int64_t(NO), U + o0, n, src, lsrc, Aw, n, int(tu));
      }, od * (od + 32.0) * 256.0, 4.0 * (2.0 * od * 256.0 + od * (od + 32.0))));
      aw_lead = true;
      continue;
    }
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
    t.tag = "gemm:ldl_outer";
    QUIP_TRY(gemm(t, s));
    aw_lead = true;
  }
  return QUIP_OK;
}

}  // namespace quip
