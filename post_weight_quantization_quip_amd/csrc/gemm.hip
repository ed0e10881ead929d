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
// LDS tiles kept in the operand's own memory order, so every store is one
// float4: a k-contiguous operand (A not transposed, B transposed) as rows of
// 32 k values padded to 36 floats, an m/n-contiguous one as 32 rows of BM
// (BN) floats padded by 8. Inside a 32-wide K step, sub-step kk (0..15) of
// lane half h sums k = 8 (kk / 4) + 4 h + kk % 4, so a k-contiguous operand
// gives four sub-steps per 128-bit LDS read, and the two lane halves of an
// m/n-contiguous read are 4 rows apart (a shift of 32 banks with these pads).
// The reads of the next four sub-steps are issued before the current four
// sub-steps' MFMAs.
// The beta term's C tile is read into registers before the K loop.
// Work-group ids are remapped so that neighbouring tiles share an XCD's L2.
#include "common.h"

namespace quip {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BK = 32;
constexpr int KC_LD = BK + 4;  // row length of a k-contiguous LDS tile
constexpr int MC_PAD = 8;      // row padding of an m/n-contiguous LDS tile

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

// Tile (tm, tn), tm <= tn, of an upper-triangular tile grid with tiles_m
// tile rows. `blocked` (products with a long K, where the operand panels are
// the traffic): numbered super-block by super-block, blocks of 8 x 8 tiles,
// the off-diagonal blocks first (row-major), then the diagonal blocks (their
// upper tiles, row-major inside). With the XCD remap giving each XCD a
// contiguous range of numbers, the 64 work-groups an XCD holds at once cover
// one block: 16 operand panels (8 on the diagonal) instead of up to 35 for a
// run of row-major tiles, so each L2 re-reads fewer panels. Otherwise
// (short K: the C tiles are the traffic) row-major, so that consecutive tiles
// read and write neighbouring stretches of C's rows.
__device__ __forceinline__ void upper_tile(int bid, int tiles_m, bool blocked, int& tm, int& tn) {
  if (!blocked) {  // row-major: consecutive tiles along a tile row
    int rem = bid, r = 0;
    while (rem >= tiles_m - r) {
      rem -= tiles_m - r;
      ++r;
    }
    tm = r;
    tn = r + rem;
    return;
  }
  constexpr int S = 8;
  const int sg = (tiles_m + S - 1) / S;
  auto ext = [&](int I) { return tiles_m - S * I < S ? tiles_m - S * I : S; };
  int rem = bid;
  for (int I = 0; I < sg; ++I)
    for (int J = I + 1; J < sg; ++J) {
      const int cnt = ext(I) * ext(J);
      if (rem < cnt) {
        const int cj = ext(J);
        tm = S * I + rem / cj;
        tn = S * J + rem % cj;
        return;
      }
      rem -= cnt;
    }
  for (int I = 0; I < sg; ++I) {
    const int e = ext(I);
    const int cnt = e * (e + 1) / 2;
    if (rem < cnt) {
      int r = 0;
      while (rem >= e - r) {
        rem -= e - r;
        ++r;
      }
      tm = S * I + r;
      tn = S * I + r + rem;
      return;
    }
    rem -= cnt;
  }
  tm = tn = 0;  // not reached: bid < tiles_m (tiles_m + 1) / 2
}

template <int BM, int BN, bool TA, bool TB, int EPI>
__global__ __launch_bounds__(256, 2) void gemm_kernel(GemmArgs a, int tiles_m, int tiles_n,
                                                      int total, bool vecA, bool vecB) {
  constexpr bool KCA = !TA, KCB = TB;  // operand tiles stored k-contiguous
  constexpr int LDA_S = KCA ? KC_LD : BM + MC_PAD;
  constexpr int LDB_S = KCB ? KC_LD : BN + MC_PAD;
  __shared__ __align__(16) float As[2][KCA ? BM * KC_LD : BK * (BM + MC_PAD)];
  __shared__ __align__(16) float Bs[2][KCB ? BN * KC_LD : BK * (BN + MC_PAD)];

  constexpr int WBM = BM / 64;  // 32x32 blocks per wave along M
  constexpr int WBN = BN / 64;
  constexpr int LA = BM * BK / 4 / 256;  // float4 loads per thread
  constexpr int LB = BN * BK / 4 / 256;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // ---- tile coordinates
  int bid = (EPI == EPI_DOT_SYM) ? int(blockIdx.x) : xcd_remap(blockIdx.x, total);
  int piece = 0;
  if (a.kpieces > 1) {
    piece = bid % a.kpieces;
    bid /= a.kpieces;
  }
  bid += a.tile0;
  int tm, tn;
  if (a.upper_tiles) {
    upper_tile(bid, tiles_m, a.K >= 1024, tm, tn);
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

  // K range of this work-group: [kbeg, kend)
  int64_t kbeg = 0, kend = a.K;
  if (a.kpieces > 1) {
    kbeg = piece * a.kchunk;
    kend = (kbeg + a.kchunk < a.K) ? kbeg + a.kchunk : a.K;
  }
  if (EPI == EPI_DOT_SYM) kend = (n0 + BN < a.K) ? n0 + BN : a.K;  // rows k <= last column
  const int64_t klim = kend;

  auto gload = [&](int64_t k0) {
    const bool fullA = vecA && k0 + BK <= klim && m0 + BM <= a.M;
    const bool fullB = vecB && k0 + BK <= klim && n0 + BN <= a.N;
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
        ra[i] = load4(A, k0 + k, m0 + m4, a.lda, klim, a.M, vecA);
      } else {
        int m = idx / (BK / 4), k4 = (idx % (BK / 4)) * 4;
        ra[i] = load4(A, m0 + m, k0 + k4, a.lda, a.M, klim, vecA);
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
        rb[i] = load4(B, k0 + k, n0 + n4, a.ldb, klim, a.N, vecB);
      } else {
        int n = idx / (BK / 4), k4 = (idx % (BK / 4)) * 4;
        rb[i] = load4(B, n0 + n, k0 + k4, a.ldb, a.N, klim, vecB);
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
        *reinterpret_cast<float4*>(&As[buf][k * LDA_S + m4]) = ra[i];
      } else {
        int m = idx / (BK / 4), k4 = (idx % (BK / 4)) * 4;
        *reinterpret_cast<float4*>(&As[buf][m * LDA_S + k4]) = ra[i];
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
        *reinterpret_cast<float4*>(&Bs[buf][k * LDB_S + n4]) = v;
      } else {
        int n = idx / (BK / 4), k4 = (idx % (BK / 4)) * 4;
        *reinterpret_cast<float4*>(&Bs[buf][n * LDB_S + k4]) = rb[i];
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

  const int64_t nk = (kend - kbeg + BK - 1) / BK;
  if (nk > 0) gload(kbeg);
  // C_in for the beta term: read at the start of the last K step, when no
  // tile loads are in flight (their registers are free) and the step's MFMAs
  // cover the latency
  float* C = a.C + bz * a.strideC;
  const float* Cin = a.Cin ? a.Cin + bz * a.strideCin : C;
  const int64_t ldcin = a.Cin ? a.ldcin : a.ldc;
  const int krow = lane >> 5, kcol = lane & 31;
  f32x16 cpre[WBM][WBN];
  const bool useC = (EPI == EPI_STORE || EPI == EPI_SPLIT) && a.beta != 0.f;
  auto load_c = [&]() {
    if (!useC) return;
    if (m0 + BM <= a.M && n0 + BN <= a.N) {  // interior tile: no per-element checks
#pragma unroll
      for (int i = 0; i < WBM; ++i)
#pragma unroll
        for (int j = 0; j < WBN; ++j) {
          const float* cp = Cin + (m0 + wm * (BM / 2) + i * 32 + 4 * krow) * ldcin + n0 +
                            wn * (BN / 2) + j * 32 + kcol;
#pragma unroll
          for (int r = 0; r < 16; ++r) cpre[i][j][r] = cp[(8 * (r / 4) + (r % 4)) * ldcin];
        }
      return;
    }
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
  };

  // sub-steps 4q .. 4q+3 of LDS buffer bf: aq[s][i] / bq[s][j] are the
  // operands of sub-step 4q + s
  auto read_quad = [&](int bf, int q, float (&aq)[4][WBM], float (&bq)[4][WBN]) {
    const int kq = 8 * q + 4 * krow;
#pragma unroll
    for (int i = 0; i < WBM; ++i) {
      const int m = wm * (BM / 2) + i * 32 + kcol;
      if (KCA) {
        const float4 v = *reinterpret_cast<const float4*>(&As[bf][m * LDA_S + kq]);
        aq[0][i] = v.x;
        aq[1][i] = v.y;
        aq[2][i] = v.z;
        aq[3][i] = v.w;
      } else {
#pragma unroll
        for (int st = 0; st < 4; ++st) aq[st][i] = As[bf][(kq + st) * LDA_S + m];
      }
    }
#pragma unroll
    for (int j = 0; j < WBN; ++j) {
      const int n = wn * (BN / 2) + j * 32 + kcol;
      if (KCB) {
        const float4 v = *reinterpret_cast<const float4*>(&Bs[bf][n * LDB_S + kq]);
        bq[0][j] = v.x;
        bq[1][j] = v.y;
        bq[2][j] = v.z;
        bq[3][j] = v.w;
      } else {
#pragma unroll
        for (int st = 0; st < 4; ++st) bq[st][j] = Bs[bf][(kq + st) * LDB_S + n];
      }
    }
  };
  // MFMAs of sub-steps s0 .. s1-1 of a quad
  auto mfma_quad = [&](const float (&aq)[4][WBM], const float (&bq)[4][WBN], int s0, int s1) {
#pragma unroll
    for (int st = s0; st < s1; ++st)
#pragma unroll
      for (int i = 0; i < WBM; ++i)
#pragma unroll
        for (int j = 0; j < WBN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(aq[st][i], bq[st][j], acc[i][j], 0, 0, 0);
  };
  // LDS read instructions per quad (pairs 32 floats apart share a ds_read2)
  constexpr int kReads = (KCA ? WBM : 4 * ((WBM + 1) / 2)) + (KCB ? WBN : 4 * ((WBN + 1) / 2));
  constexpr int kQuads = BK / 8;
  static_assert(kQuads % 2 == 0, "quads alternate between the two operand register sets");

  // Software pipeline: the reads of quad q + 1 are issued before the MFMAs of
  // quad q; at a step boundary half of the last quad's MFMAs go before the
  // LDS stores and the barrier, the other half after the next step's first
  // reads, so that they cover the read latency.
  float aq[2][4][WBM], bq[2][4][WBN];
  int buf = 0;
  if (nk > 0) {
    sstore(0, kbeg);
    __syncthreads();
    read_quad(0, 0, aq[0], bq[0]);
  }
  // quads 0 .. kQuads-2 of the current step, each after the next one's reads
  auto step_quads = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);
#pragma unroll
    for (int q = 0; q + 1 < kQuads; ++q) {
      const int cur = q & 1;
      read_quad(buf, q + 1, aq[cur ^ 1], bq[cur ^ 1]);
      mfma_quad(aq[cur], bq[cur], 0, 4);
      __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 4 * WBM * WBN, 0);
    }
  };
  constexpr int last = (kQuads - 1) & 1;
  // every step but the last (no branch inside, so the accumulators stay in place)
  for (int64_t kt = 0; kt + 1 < nk; ++kt) {
    gload(kbeg + (kt + 1) * BK);
    step_quads();
    mfma_quad(aq[last], bq[last], 0, 2);
    sstore(buf ^ 1, kbeg + (kt + 1) * BK);
    __syncthreads();
    read_quad(buf ^ 1, 0, aq[last ^ 1], bq[last ^ 1]);
    mfma_quad(aq[last], bq[last], 2, 4);
    buf ^= 1;
  }
  load_c();
  if (nk > 0) {
    step_quads();
    mfma_quad(aq[last], bq[last], 0, 4);
  }

  // ---- epilogue
  if (a.kpieces > 1) {  // raw partial tile, summed later by tail_reduce_kernel
    float* Pt = a.P + (size_t((bid - a.tile0) * a.kpieces + piece) * BM * BN);
#pragma unroll
    for (int i = 0; i < WBM; ++i)
#pragma unroll
      for (int j = 0; j < WBN; ++j) {
        const int c = wn * (BN / 2) + j * 32 + kcol;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rr = wm * (BM / 2) + i * 32 + 8 * (r / 4) + 4 * krow + (r % 4);
          Pt[rr * BN + c] = acc[i][j][r];
        }
      }
    return;
  }
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

// Sums the K pieces of the leftover tiles (fixed order) and applies alpha,
// beta and the mirror like the regular epilogue.
template <int BM, int BN>
__global__ __launch_bounds__(256) void tail_reduce_kernel(GemmArgs a, int tiles_m) {
  const int r = blockIdx.x;  // leftover tile
  int tm, tn;
  upper_tile(a.tile0 + r, tiles_m, a.K >= 1024, tm, tn);
  const int e4 = (int(blockIdx.y) * 256 + int(threadIdx.x)) * 4;  // 4 consecutive elements
  if (e4 >= BM * BN) return;
  const int i = e4 / BN, j0 = e4 % BN;
  const float* Pr = a.P + size_t(r) * a.kpieces * BM * BN + e4;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int p = 0; p < a.kpieces; ++p) {
    const float4 x = *reinterpret_cast<const float4*>(Pr + size_t(p) * BM * BN);
    v.x += x.x;
    v.y += x.y;
    v.z += x.z;
    v.w += x.w;
  }
  const float vv[4] = {v.x, v.y, v.z, v.w};
  const int64_t row = int64_t(tm) * BM + i;
  const float* Cin = a.Cin ? a.Cin : a.C;
  const int64_t ldcin = a.Cin ? a.ldcin : a.ldc;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t col = int64_t(tn) * BN + j0 + e;
    if (row >= a.M || col >= a.N) continue;
    float o = a.alpha * vv[e];
    if (a.beta != 0.f) o += a.beta * Cin[row * ldcin + col];
    a.C[row * a.ldc + col] = o;
    if (a.mirror && tm != tn) {
      float w = a.alpha * vv[e];
      if (a.beta != 0.f) w += a.beta * Cin[col * ldcin + row];
      a.C[col * a.ldc + row] = w;
    }
  }
}


struct TailPlan {
  int T = 0, R = 0, kp = 1;
  int64_t kchunk = 0;
  size_t floats = 0;
};

// Leftover-tile split of an upper-tile grid: T tiles, `slots` resident
// work-groups; the T mod slots tiles of the last round are cut into K pieces
// so that they fill (at most) one round.
template <int BM, int BN, bool TA, bool TB, int EPI>
TailPlan plan_tail(int64_t M, int64_t K) {
  TailPlan pl;
  const int tiles_m = int(cdiv(M, BM));
  pl.T = tiles_m * (tiles_m + 1) / 2;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(&gemm_kernel<BM, BN, TA, TB, EPI>), 256, 0) !=
          hipSuccess ||
      per_cu <= 0)
    return pl;
  const int slots = per_cu * device_cus();
  pl.R = pl.T % slots;
  if (pl.R == 0) return pl;
  int kp = slots / pl.R;
  const int64_t kchunk = cdiv(cdiv(K, kp), BK) * BK;
  kp = int(cdiv(K, kchunk));
  if (kp < 2) return pl;
  pl.kp = kp;
  pl.kchunk = kchunk;
  pl.floats = size_t(pl.R) * kp * BM * BN;
  return pl;
}

// Algorithmic work of one gemm() call: useful flops (the upper triangle only
// for upper tiles, k <= j only for the symmetric dot) and compulsory bytes.
void gemm_work(const GemmArgs& a, double& flops, double& bytes) {
  const double M = double(a.M), N = double(a.N), K = double(a.K), b = double(a.batch);
  if (a.upper_tiles) {
    flops = M * (M + 1.0) * K * b;
    bytes = 4.0 * b * (K * M * (a.A == a.B ? 1.0 : 2.0) + M * M * (a.beta != 0.f ? 2.0 : 1.0));
  } else if (a.epi == EPI_DOT_SYM) {
    flops = M * N * (N + 1.0) * b + 2.0 * M * N * b;
    bytes = 4.0 * b * (M * K + N * (N + 1.0) / 2.0 + M * N);
  } else {
    flops = 2.0 * M * N * K * b + (a.epi == EPI_DOT ? 2.0 * M * N * b : 0.0);
    bytes = 4.0 * b * (M * K + K * N +
                       (a.epi == EPI_DOT ? M * N : M * N * (a.beta != 0.f ? 2.0 : 1.0)));
  }
}

template <int BM, int BN, bool TA, bool TB, int EPI>
quip_status launch_t(const GemmArgs& a, hipStream_t s, bool vecA, bool vecB) {
  double wf = 0.0, wb = 0.0;  // attributed to the call's first launch
  if (timing_on()) gemm_work(a, wf, wb);
  int tiles_m = int(cdiv(a.M, BM)), tiles_n = int(cdiv(a.N, BN));
  int total = a.upper_tiles ? tiles_m * (tiles_m + 1) / 2 : tiles_m * tiles_n;
  if (total == 0 || a.batch == 0) return QUIP_OK;
  if (EPI == EPI_STORE && a.upper_tiles && a.P && a.batch == 1) {
    const TailPlan pl = plan_tail<BM, BN, TA, TB, EPI>(a.M, a.K);
    if (pl.kp > 1 && pl.floats <= a.P_floats) {
      const int full = pl.T - pl.R;
      if (full > 0) {
        GemmArgs f = a;
        f.tile0 = 0;
        f.kpieces = 1;
        QUIP_TRY(timed_launch(a.tag, s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
          QUIP_KERNEL((gemm_kernel<BM, BN, TA, TB, EPI>), dim3(full, 1), dim3(256), 0, s, f,
                             tiles_m, tiles_n, full, vecA, vecB);
        }, wf, wb));
        wf = wb = 0.0;
      }
      GemmArgs t = a;
      t.tile0 = full;
      t.kpieces = pl.kp;
      t.kchunk = pl.kchunk;
      const int np = pl.R * pl.kp;
      QUIP_TRY(timed_launch(a.tag, s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
        QUIP_KERNEL((gemm_kernel<BM, BN, TA, TB, EPI>), dim3(np, 1), dim3(256), 0, s, t,
                           tiles_m, tiles_n, np, vecA, vecB);
      }, wf, wb));
      return timed_launch("gemm_tail_reduce", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
        QUIP_KERNEL((tail_reduce_kernel<BM, BN>), dim3(pl.R, BM * BN / 1024), dim3(256), 0, s,
                           t, tiles_m);
      });
    }
  }
  dim3 grid(total, a.batch);
  return timed_launch(a.tag, s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL((gemm_kernel<BM, BN, TA, TB, EPI>), grid, dim3(256), 0, s, a, tiles_m,
                       tiles_n, total, vecA, vecB);
  }, wf, wb);
}

template <bool TA, bool TB, int EPI>
quip_status launch_tiles(const GemmArgs& a, hipStream_t s, bool vecA, bool vecB) {
  // Prefer 128x128 tiles; 64x64 when the 128-tile grid would not give every
  // CU two work-groups (small launches are latency-bound: more, smaller tiles
  // finish sooner); 64 along one dimension when only that one is small.
  int64_t t128 = cdiv(a.M, 128) * cdiv(a.N, 128) * a.batch;
  if (a.upper_tiles) t128 = cdiv(a.M, 128) * (cdiv(a.M, 128) + 1) / 2 * a.batch;
  if (t128 < 512) return launch_t<64, 64, TA, TB, EPI>(a, s, vecA, vecB);
  // a plain product of a few rounds whose 64x64 grid fills whole rounds of
  // resident work-groups (two per CU) where the 128x128 grid would leave the
  // last round part empty (the LDLQ feedback with N = 3072 or 2560 at
  // M = 4096: 1.5 and 1.25 rounds): all products 0.669 -> 0.635 ms per
  // 4096 x 4096 pass. With many rounds the part-empty last one costs less
  // than the smaller tiles (8192 x 28672 layer: 59.3 against 61.4 ms).
  if (!a.upper_tiles && EPI == EPI_STORE) {
    const int64_t slots = 2 * int64_t(device_cus());
    const int64_t t64 = cdiv(a.M, 64) * cdiv(a.N, 64) * a.batch;
    if (t128 < 4 * slots && t128 % slots != 0 && t64 % slots == 0)
      return launch_t<64, 64, TA, TB, EPI>(a, s, vecA, vecB);
  }
  // 64 along a dimension that 128-wide tiles would pad by more than half a
  // 64-tile beyond what 64-wide tiles need (172: 256 against 192). The tile
  // shape does not change any element's summation order.
  auto pads = [](int64_t d) { return cdiv(d, 128) * 128 > cdiv(d, 64) * 64 + 32; };
  bool smallM = a.M <= 64 || pads(a.M);
  bool smallN = a.N <= 64 || pads(a.N);
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

// Compute units of the current device (256 if the query fails), cached per device.
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    cached[dev] = cus;
  }
  return cached[dev];
}

size_t gemm_upper_tail_floats(int64_t n, int64_t K) {
  // the Hessian product: upper tiles, op(A) = X^T, op(B) = X, tile size as launch_tiles picks it
  const int64_t t = cdiv(n, 128) * (cdiv(n, 128) + 1) / 2;
  if (t < 512) return plan_tail<64, 64, true, false, EPI_STORE>(n, K).floats;
  return plan_tail<128, 128, true, false, EPI_STORE>(n, K).floats;
}

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
