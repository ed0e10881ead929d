// Randomized Hadamard transform (random signs, then the natural-order
// Sylvester Hadamard matrix, then 1/sqrt(d)) -- the incoherence transform of
// QuIP# (abstract) applied to one side of a matrix.
//
// RIGHT side (along a row, contiguous): rht_rows_kernel. A row of N = 2^LOGN
// floats is held by N/E threads with E floats each. The first E-point
// butterfly round runs on what each thread loaded (index bits {0,1} and the
// top bits, so that every load is a lane-contiguous float4); the remaining
// index bits are covered by rounds of E-point butterflies in registers, with an
// LDS transpose between rounds (one buffer per row, so that more work-groups
// fit on a CU; XOR swizzle on bits 2..4 so the strided round patterns hit
// distinct banks). A last transpose brings the data back to the float4 layout
// for the store. As many work-groups as fit at once, each looping over rows
// with the next row's loads issued before the current row's transform. Rows
// are read with non-temporal loads (whole 16-byte chunks of contiguous rows,
// which no other work-group touches), and written with non-temporal stores
// when no other pass of the same transform follows (a following column pass
// reads the result back while it is still in the last-level cache).
//
// LEFT side (along a column, strided by the row pitch). For d = 4096 and
// float4-aligned rows, one pass over memory, a work-group per column block:
// rht_cols_panel16 (16 columns, 64-byte row segments, the panel in registers,
// one LDS exchange in halves) when the column count is a multiple of 16, else
// rht_cols_panel (8 columns in LDS, 128 KB + padding: the top four index bits
// in registers right after the load, the middle four through one LDS round
// trip, the low four in registers right before the store). Row segments
// narrower than a 128-byte line cost per-CU throughput, so column blocks are
// dealt out such that the work-groups sharing a line run on one XCD. Otherwise rht_cols_pass: the d-point transform is split
// H_d = H_{2^k1} (x) H_{2^k2} (x) ... into passes that each transform 2^KR
// rows spaced 2^lo apart, for 64 consecutive columns per work-group (lanes run
// along the columns, so every access is a 256-byte row segment). Inside a
// pass: butterflies on the rows a thread holds, one LDS transpose, butterflies
// on the rest.
#include "common.h"

namespace quip {
namespace {

__device__ __forceinline__ int swz(int i) {
  int f = ((i >> 5) ^ (i >> 8) ^ (i >> 11)) & 7;
  return i ^ (f << 2);
}

typedef float rht_f4 __attribute__((ext_vector_type(4)));

template <int LOGN, int LE>
__global__ __launch_bounds__(512) void rht_rows_kernel(const float* A, float* out, int64_t rows,
                                                       int64_t ld, const float* __restrict__ signs,
                                                       float scale, bool inverse, bool vec,
                                                       bool nt_out) {
  constexpr int N = 1 << LOGN;
  constexpr int E = 1 << LE;
  constexpr int T = N / E;                    // threads per row
  constexpr int RW = T >= 256 ? 1 : 256 / T;  // rows per work-group
  constexpr int TOP = LE - 2;                 // register bits placed at the top of the index
  constexpr int MID_LO = 2, MID_HI = LOGN - TOP;
  constexpr int MID = MID_HI - MID_LO;
  constexpr int NFULL = MID / LE;
  constexpr int REM = MID % LE;
  constexpr int NR = NFULL + (REM ? 1 : 0);

  extern __shared__ __align__(16) float lds[];  // RW * N floats

  const int tid = threadIdx.x;
  const int rw = tid / T, p = tid % T;
  // rows of this work-group: (blockIdx.x + k gridDim.x) RW + rw, k = 0, 1, ...;
  // the next row's loads are issued before the current row's transform
  int64_t row = int64_t(blockIdx.x) * RW + rw;
  int64_t wbase = int64_t(blockIdx.x) * RW;  // uniform over the work-group
  const int64_t wstep = int64_t(gridDim.x) * RW;

  float x[E], xn[E];

  // round-0 layout: i = (r & 3) | (p << 2) | ((r >> 2) << MID_HI)
  auto idx0 = [&](int r) { return (r & 3) | (p << 2) | ((r >> 2) << MID_HI); };
  auto idxa = [&](int a, int r) {
    return (p & ((1 << a) - 1)) | (r << a) | ((p >> a) << (a + LE));
  };

  auto load_row = [&](int64_t r, float (&y)[E]) {
    const float* src = A + r * ld;
#pragma unroll
    for (int c = 0; c < E / 4; ++c) {
      int i = idx0(4 * c);
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (r < rows) {
        if (vec) {
          const rht_f4 t = __builtin_nontemporal_load(reinterpret_cast<const rht_f4*>(src + i));
          v = make_float4(t.x, t.y, t.z, t.w);
        } else {
          v.x = src[i];
          v.y = src[i + 1];
          v.z = src[i + 2];
          v.w = src[i + 3];
        }
      }
      y[4 * c + 0] = v.x;
      y[4 * c + 1] = v.y;
      y[4 * c + 2] = v.z;
      y[4 * c + 3] = v.w;
    }
  };
  load_row(row, xn);
  for (;;) {
    const bool live = row < rows;
#pragma unroll
    for (int e = 0; e < E; ++e) x[e] = xn[e];
    const bool more = wbase + wstep < rows;
    if (more) load_row(row + wstep, xn);
    if (!inverse) {
#pragma unroll
      for (int c = 0; c < E / 4; ++c) {
        float4 s = *reinterpret_cast<const float4*>(signs + idx0(4 * c));
        x[4 * c + 0] *= s.x;
        x[4 * c + 1] *= s.y;
        x[4 * c + 2] *= s.z;
        x[4 * c + 3] *= s.w;
      }
    }
    // round 0: every register bit is a new index bit
#pragma unroll
    for (int t = 0; t < LE; ++t) {
#pragma unroll
      for (int r = 0; r < E; ++r) {
        if (r & (1 << t)) continue;
        float u = x[r], w = x[r | (1 << t)];
        x[r] = u + w;
        x[r | (1 << t)] = u - w;
      }
    }

    float* const L = lds + rw * N;  // one transpose buffer per row
    int prev = -1;  // -1: round-0 layout, else base bit of the previous round
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const int a = j < NFULL ? MID_LO + j * LE : (MID_HI - LE > 0 ? MID_HI - LE : 0);
      const int new_lo = j < NFULL ? a : MID_LO + NFULL * LE;
      const int new_hi = j < NFULL ? a + LE : MID_HI;
      if (j > 0) __syncthreads();  // the previous round's reads are done
      if (prev < 0) {
#pragma unroll
        for (int c = 0; c < E / 4; ++c)
          *reinterpret_cast<float4*>(L + swz(idx0(4 * c))) =
              make_float4(x[4 * c], x[4 * c + 1], x[4 * c + 2], x[4 * c + 3]);
      } else {
#pragma unroll
        for (int r = 0; r < E; ++r) L[swz(idxa(prev, r))] = x[r];
      }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < E; ++r) x[r] = L[swz(idxa(a, r))];
#pragma unroll
      for (int t = 0; t < LE; ++t) {
        if (a + t < new_lo || a + t >= new_hi) continue;
#pragma unroll
        for (int r = 0; r < E; ++r) {
          if (r & (1 << t)) continue;
          float u = x[r], w = x[r | (1 << t)];
          x[r] = u + w;
          x[r | (1 << t)] = u - w;
        }
      }
      prev = a;
    }
    if (NR > 0) {
      __syncthreads();
#pragma unroll
      for (int r = 0; r < E; ++r) L[swz(idxa(prev, r))] = x[r];
      __syncthreads();
#pragma unroll
      for (int c = 0; c < E / 4; ++c) {
        float4 v = *reinterpret_cast<const float4*>(L + swz(idx0(4 * c)));
        x[4 * c + 0] = v.x;
        x[4 * c + 1] = v.y;
        x[4 * c + 2] = v.z;
        x[4 * c + 3] = v.w;
      }
    }
#pragma unroll
    for (int c = 0; c < E / 4; ++c) {
      float4 s = make_float4(1.f, 1.f, 1.f, 1.f);
      if (inverse) s = *reinterpret_cast<const float4*>(signs + idx0(4 * c));
      x[4 * c + 0] *= s.x * scale;
      x[4 * c + 1] *= s.y * scale;
      x[4 * c + 2] *= s.z * scale;
      x[4 * c + 3] *= s.w * scale;
    }
    if (live) {
      float* dst = out + row * ld;
#pragma unroll
      for (int c = 0; c < E / 4; ++c) {
        int i = idx0(4 * c);
        if (vec && nt_out) {
          __builtin_nontemporal_store(rht_f4{x[4 * c], x[4 * c + 1], x[4 * c + 2], x[4 * c + 3]},
                                      reinterpret_cast<rht_f4*>(dst + i));
        } else if (vec) {
          *reinterpret_cast<float4*>(dst + i) =
              make_float4(x[4 * c], x[4 * c + 1], x[4 * c + 2], x[4 * c + 3]);
        } else {
          dst[i] = x[4 * c];
          dst[i + 1] = x[4 * c + 1];
          dst[i + 2] = x[4 * c + 2];
          dst[i + 3] = x[4 * c + 3];
        }
      }
    }
    if (!more) break;
    __syncthreads();  // the LDS buffer is reused by the next row
    row += wstep;
    wbase += wstep;
  }
}

// Rows of length 2, 4 or 8: one thread per row.
template <int N>
__global__ void rht_rows_small_kernel(const float* A, float* out, int64_t rows, int64_t ld,
                                      const float* signs, float scale, bool inverse) {
  int64_t row = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (row >= rows) return;
  float x[N];
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] = A[row * ld + i] * (inverse ? 1.f : signs[i]);
#pragma unroll
  for (int h = 1; h < N; h <<= 1)
#pragma unroll
    for (int i = 0; i < N; ++i)
      if (!(i & h)) {
        float u = x[i], w = x[i | h];
        x[i] = u + w;
        x[i | h] = u - w;
      }
#pragma unroll
  for (int i = 0; i < N; ++i) out[row * ld + i] = x[i] * scale * (inverse ? signs[i] : 1.f);
}

// One pass of the column transform: rows {base + (t << lo) : t < 2^KR} for the
// 64 columns [c0, c0 + 64). 256 threads = 64 columns x 4 groups.
template <int KR>
__global__ __launch_bounds__(256) void rht_cols_pass(const float* A, float* out, int64_t cols,
                                                     int64_t ld, int lo,
                                                     const float* __restrict__ signs,
                                                     float scale, int mode) {
  // mode bit 0: multiply by the sign of the row before the butterflies
  //          1: multiply by the sign of the row after (and apply `scale`)
  constexpr int R = 1 << KR;
  constexpr int NREG = R / 4;
  __shared__ float lds[R][65];

  const int tid = threadIdx.x;
  const int c = tid & 63, g = tid >> 6;
  const int64_t b = blockIdx.x;
  const int64_t base = (b & ((int64_t(1) << lo) - 1)) | ((b >> lo) << (lo + KR));
  const int64_t col = int64_t(blockIdx.y) * 64 + c;
  const bool live = col < cols;

  float x[NREG];
  // layout A: t = g + 4 r
#pragma unroll
  for (int r = 0; r < NREG; ++r) {
    int64_t rowi = base + (int64_t(g + 4 * r) << lo);
    float v = live ? A[rowi * ld + col] : 0.f;
    if (mode & 1) v *= signs[rowi];
    x[r] = v;
  }
#pragma unroll
  for (int t = 0; t < KR - 2; ++t)
#pragma unroll
    for (int r = 0; r < NREG; ++r) {
      if (r & (1 << t)) continue;
      float u = x[r], w = x[r | (1 << t)];
      x[r] = u + w;
      x[r | (1 << t)] = u - w;
    }
#pragma unroll
  for (int r = 0; r < NREG; ++r) lds[g + 4 * r][c] = x[r];
  __syncthreads();
  // layout B: t = (r & 3) | (g << 2) | ((r >> 2) << 4)
#pragma unroll
  for (int r = 0; r < NREG; ++r) x[r] = lds[(r & 3) | (g << 2) | ((r >> 2) << 4)][c];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < NREG; ++r) {
      if (r & (1 << t)) continue;
      float u = x[r], w = x[r | (1 << t)];
      x[r] = u + w;
      x[r | (1 << t)] = u - w;
    }
  if (!live) return;
#pragma unroll
  for (int r = 0; r < NREG; ++r) {
    int t = (r & 3) | (g << 2) | ((r >> 2) << 4);
    int64_t rowi = base + (int64_t(t) << lo);
    float v = x[r] * scale;
    if (mode & 2) v *= signs[rowi];
    out[rowi * ld + col] = v;
  }
}

// In-register butterflies over the index bits of v[0..15] (one float4 of
// four columns per index).
__device__ __forceinline__ void fwht16_f4(float4 (&v)[16]) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i & h) continue;
      const float4 u = v[i], w = v[i | h];
      v[i] = make_float4(u.x + w.x, u.y + w.y, u.z + w.z, u.w + w.w);
      v[i | h] = make_float4(u.x - w.x, u.y - w.y, u.z - w.z, u.w - w.w);
    }
}

// Column transform of length 4096 for 8 consecutive columns per work-group,
// in one pass over memory (see the file header). 512 threads; the panel sits
// in LDS as float4 slots: row r, column group cg (4 columns) at
// 2 r + cg + r / 16 (one slot of padding per 16 rows keeps every phase's
// 16-lane groups on distinct banks). Needs ld % 4 == 0 and 16-byte aligned
// A and out; A == out is allowed (each column block is read and written by
// one work-group only, and read in full before it is written).
constexpr int PANEL_SLOTS = 2 * 4096 + 4096 / 16;

__global__ __launch_bounds__(512) void rht_cols_panel(const float* A, float* out, int64_t cols,
                                                      int64_t ld,
                                                      const float* __restrict__ signs,
                                                      float scale, bool inverse) {
  extern __shared__ __align__(16) float4 P[];
  auto slot = [](int r, int cg) { return 2 * r + cg + (r >> 4); };
  const int t = threadIdx.x;
  const int cg = t & 1;
  const int nblk = int((cols + 7) / 8);
  const int64_t c = int64_t(xcd_remap(int(blockIdx.x), nblk)) * 8 + 4 * cg;  // first of 4 columns
  const int ncol = cols - c >= 4 ? 4 : (cols - c > 0 ? int(cols - c) : 0);
  float4 v[16];

  // ---- load rows rb + 256 i, i = 0..15; bits 8..11 in registers
  {
    const int rb = t >> 1;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float* p = A + int64_t(rb + 256 * i) * ld + c;
      if (ncol == 4) {
        v[i] = *reinterpret_cast<const float4*>(p);
      } else {
        v[i] = make_float4(ncol > 0 ? p[0] : 0.f, ncol > 1 ? p[1] : 0.f, ncol > 2 ? p[2] : 0.f, 0.f);
      }
    }
    if (!inverse) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float sg = signs[rb + 256 * i];
        v[i] = make_float4(v[i].x * sg, v[i].y * sg, v[i].z * sg, v[i].w * sg);
      }
    }
    fwht16_f4(v);
#pragma unroll
    for (int i = 0; i < 16; ++i) P[slot(rb + 256 * i, cg)] = v[i];
  }
  __syncthreads();
  // ---- rows lo + 16 i + 256 hi: bits 4..7
  {
    const int lo = (t >> 1) & 15, hi = t >> 5;
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = P[slot(lo + 16 * i + 256 * hi, cg)];
    fwht16_f4(v);
#pragma unroll
    for (int i = 0; i < 16; ++i) P[slot(lo + 16 * i + 256 * hi, cg)] = v[i];
  }
  __syncthreads();
  // ---- rows i + 16 mid + 256 hi: bits 0..3, then the store
  {
    const int mid = (t >> 1) & 15, hi = t >> 5;
    const int r0 = 16 * mid + 256 * hi;
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = P[slot(r0 + i, cg)];
    fwht16_f4(v);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float sg = scale * (inverse ? signs[r0 + i] : 1.f);
      v[i] = make_float4(v[i].x * sg, v[i].y * sg, v[i].z * sg, v[i].w * sg);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float* p = out + int64_t(r0 + i) * ld + c;
      if (ncol == 4) {
        *reinterpret_cast<float4*>(p) = v[i];
      } else {
        if (ncol > 0) p[0] = v[i].x;
        if (ncol > 1) p[1] = v[i].y;
        if (ncol > 2) p[2] = v[i].z;
      }
    }
  }
}

// In-register butterflies over the index bits of v[0..31] (float4 of four
// columns per index).
__device__ __forceinline__ void fwht32_f4(float4 (&v)[32]) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1)
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (i & h) continue;
      const float4 u = v[i], w = v[i | h];
      v[i] = make_float4(u.x + w.x, u.y + w.y, u.z + w.z, u.w + w.w);
      v[i | h] = make_float4(u.x - w.x, u.y - w.y, u.z - w.z, u.w - w.w);
    }
}

// In-register butterflies over the index bits of v[0..63] (float2 of two
// columns per index).
__device__ __forceinline__ void fwht64_f2(float2 (&v)[64]) {
#pragma unroll
  for (int h = 1; h < 64; h <<= 1)
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      if (i & h) continue;
      const float2 u = v[i], w = v[i | h];
      v[i] = make_float2(u.x + w.x, u.y + w.y);
      v[i | h] = make_float2(u.x - w.x, u.y - w.y);
    }
}

// Column transform of length 4096 for 16 consecutive columns per work-group
// (64-byte row segments: eight lanes per row), in one pass over memory. 512
// threads; thread t holds the column pair g = t % 8 of 64 rows in registers
// (the 256 KB panel lives in registers). Index bits 6..11 are done right after
// the load (rows k + 64 i), bits 0..5 after one exchange (rows 64 k + i), then
// the store. The exchange goes through LDS in two halves of 8 columns (128 KB
// + padding: float2 slot 4 r + g' + r / 16 of a half, so that both the
// row-contiguous writes and the 64-row-strided reads of a wave's active lanes
// fall on distinct banks). Both directions stage the signs, times the scale,
// in LDS (each thread's 64 signs are 16 float4 reads). Needs
// cols % 16 == 0, ld % 2 == 0, 8-byte aligned A and out and 16-byte aligned
// signs; A == out is allowed.
template <bool INV>
__global__ __launch_bounds__(512) void rht_cols_panel16(const float* A, float* out, int64_t ld,
                                                        int nblk,
                                                        const float* __restrict__ signs,
                                                        float scale) {
  constexpr bool inverse = INV;
  extern __shared__ __align__(16) float2 P2[];
  // the signs times the scale, rows of 68 floats after the exchange buffer:
  // forward Sg[k][i] = s[k + 64 i] / 64, inverse Sg[k][i] = s[64 k + i] / 64
  // (a power-of-two scale commutes exactly with the butterflies, so it is
  // applied once, with the signs)
  float* Sg = reinterpret_cast<float*>(P2 + (4 * 4096 + 4096 / 16));
  auto slot = [](int r, int g4) { return 4 * r + g4 + (r >> 4); };
  const int t = threadIdx.x;
  const int g = t & 7, k = t >> 3;  // column pair, row index of the thread (0..63)
  // the block's first column (uniform) and the lane's offset from it, so that
  // every access is a uniform base plus one 32-bit lane offset
  const int64_t cb = int64_t(xcd_remap(int(blockIdx.x), nblk)) * 16;
  const uint32_t lin = uint32_t(k * ld + 2 * g);        // rows k + 64 i
  const uint32_t lout = uint32_t(64 * k * ld + 2 * g);  // rows 64 k + i
  float2 v[64];

  // ---- rows k + 64 i: bits 6..11
#pragma unroll
  for (int i = 0; i < 64; ++i)
    v[i] = *reinterpret_cast<const float2*>(A + cb + int64_t(64 * i) * ld + lin);
  {
    // thread t stages s[8 t .. 8 t + 7]: element e sits at Sg[e % 64][e / 64]
    // (forward: thread k applies s[k + 64 i] after the load) or at
    // Sg[e / 64][e % 64] (inverse: s[64 k + i] before the store)
    const float4 s0 = *reinterpret_cast<const float4*>(signs + 8 * t);
    const float4 s1 = *reinterpret_cast<const float4*>(signs + 8 * t + 4);
    const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int e = 8 * t + q;
      if (inverse)
        Sg[(e >> 6) * 68 + (e & 63)] = sv[q] * scale;
      else
        Sg[(e & 63) * 68 + (e >> 6)] = sv[q] * scale;
    }
  }
  if (!inverse) {
    __syncthreads();
    const float4* sk = reinterpret_cast<const float4*>(Sg + k * 68);
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const float4 sq = sk[c];
      const float sw[4] = {sq.x, sq.y, sq.z, sq.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = 4 * c + q;
        v[i] = make_float2(v[i].x * sw[q], v[i].y * sw[q]);
      }
    }
  }
  fwht64_f2(v);
  // ---- exchange to rows 64 k + i: bits 0..5 (and the store layout)
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const bool mine = (g >> 2) == half;
    if (half) __syncthreads();  // the first half's reads are done
    if (mine) {
#pragma unroll
      for (int i = 0; i < 64; ++i) P2[slot(k + 64 * i, g & 3)] = v[i];
    }
    __syncthreads();
    if (mine) {
#pragma unroll
      for (int i = 0; i < 64; ++i) v[i] = P2[slot(64 * k + i, g & 3)];
    }
  }
  fwht64_f2(v);
  if (inverse) {  // staged before the exchange's barriers
    const float4* sk = reinterpret_cast<const float4*>(Sg + k * 68);
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const float4 sq = sk[c];
      const float sw[4] = {sq.x, sq.y, sq.z, sq.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = 4 * c + q;
        v[i] = make_float2(v[i].x * sw[q], v[i].y * sw[q]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 64; ++i)
    *reinterpret_cast<float2*>(out + cb + int64_t(i) * ld + lout) = v[i];
}

// Column transform of length 2, 4 or 8: one thread per column.
template <int D>
__global__ void rht_cols_small_kernel(const float* A, float* out, int64_t cols, int64_t ld,
                                      const float* signs, float scale, bool inverse) {
  int64_t col = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (col >= cols) return;
  float x[D];
#pragma unroll
  for (int i = 0; i < D; ++i) x[i] = A[i * ld + col] * (inverse ? 1.f : signs[i]);
#pragma unroll
  for (int h = 1; h < D; h <<= 1)
#pragma unroll
    for (int i = 0; i < D; ++i)
      if (!(i & h)) {
        float u = x[i], w = x[i | h];
        x[i] = u + w;
        x[i | h] = u - w;
      }
#pragma unroll
  for (int i = 0; i < D; ++i) out[i * ld + col] = x[i] * scale * (inverse ? signs[i] : 1.f);
}

template <int LOGN>
quip_status rows_t(const float* A, float* out, int64_t rows, int64_t ld, const float* s,
                   bool inverse, bool nt_out, hipStream_t st) {
  constexpr int LE = LOGN >= 14 ? 5 : 4;
  constexpr int N = 1 << LOGN;
  constexpr int T = N >> LE;
  constexpr int RW = T >= 256 ? 1 : 256 / T;
  const float scale = 1.0f / sqrtf(float(N));
  bool vec = aligned16(A) && aligned16(out) && ld % 4 == 0;
  size_t shmem = size_t(RW) * N * sizeof(float);
  if (shmem > 65536)
    QUIP_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(&rht_rows_kernel<LOGN, LE>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, int(shmem)));
  // as many work-groups as fit at once (each loops over rows), at most one per row group
  int64_t nwg = cdiv(rows, RW);
  int per_cu = 0, dev = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
          &per_cu, reinterpret_cast<const void*>(&rht_rows_kernel<LOGN, LE>), T * RW, shmem) ==
          hipSuccess &&
      hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      per_cu > 0 && cus > 0 && int64_t(per_cu) * cus < nwg)
    nwg = int64_t(per_cu) * cus;
  const dim3 grid{unsigned(nwg)};
  return timed_launch("rht_rows_kernel", st, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL((rht_rows_kernel<LOGN, LE>), grid, dim3(T * RW), shmem, st, A, out, rows, ld,
                       s, scale, inverse, vec, nt_out);
  }, double(rows) * N * (LOGN + 2), 8.0 * double(rows) * N);
}

template <int N>
quip_status rows_small_t(const float* A, float* out, int64_t rows, int64_t ld, const float* s,
                         bool inverse, hipStream_t st) {
  const float scale = 1.0f / sqrtf(float(N));
  return timed_launch("rht_rows_small_kernel", st, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL((rht_rows_small_kernel<N>), dim3(unsigned(cdiv(rows, 256))), dim3(256), 0, st,
                       A, out, rows, ld, s, scale, inverse);
  });
}

template <int D>
quip_status cols_small_t(const float* A, float* out, int64_t cols, int64_t ld, const float* s,
                         bool inverse, hipStream_t st) {
  const float scale = 1.0f / sqrtf(float(D));
  return timed_launch("rht_cols_small_kernel", st, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL((rht_cols_small_kernel<D>), dim3(unsigned(cdiv(cols, 256))), dim3(256), 0, st,
                       A, out, cols, ld, s, scale, inverse);
  });
}

quip_status cols_pass(int kr, const float* A, float* out, int64_t d, int64_t cols, int64_t ld,
                      int lo, const float* s, float scale, int mode, hipStream_t st) {
  dim3 grid(unsigned(d >> kr), unsigned(cdiv(cols, 64)));
  if (kr < 4 || kr > 7) return fail(QUIP_ERR_UNSUPPORTED, "rht_cols: pass size");
  // one pass reads and writes the whole matrix once (kr butterfly levels)
  return timed_launch("rht_cols_pass", st, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    switch (kr) {
#define CASE(K)                                                                                \
  case K:                                                                                      \
    QUIP_KERNEL((rht_cols_pass<K>), grid, dim3(256), 0, st, A, out, cols, ld, lo, s,   \
                       scale, mode);                                                           \
    break;
      CASE(4) CASE(5) CASE(6) CASE(7)
#undef CASE
    }
  }, double(d) * double(cols) * (kr + 1), 8.0 * double(d) * double(cols));
}

}  // namespace

quip_status rht_rows(const float* A, float* out, int64_t rows, int64_t cols, int64_t ld,
                     const float* signs, bool inverse, hipStream_t st, bool last_pass) {
  if (rows == 0) return QUIP_OK;
  switch (ilog2(cols)) {
    case 1: return rows_small_t<2>(A, out, rows, ld, signs, inverse, st);
    case 2: return rows_small_t<4>(A, out, rows, ld, signs, inverse, st);
    case 3: return rows_small_t<8>(A, out, rows, ld, signs, inverse, st);
#define CASE(L) \
  case L: return rows_t<L>(A, out, rows, ld, signs, inverse, last_pass, st);
    CASE(4) CASE(5) CASE(6) CASE(7) CASE(8) CASE(9) CASE(10) CASE(11) CASE(12) CASE(13) CASE(14)
#undef CASE
  }
  return fail(QUIP_ERR_SHAPE, "rht: the transform length must be a power of two in [2, 16384]");
}

quip_status rht_cols(const float* A, float* out, int64_t rows, int64_t cols, int64_t ld,
                     const float* signs, bool inverse, hipStream_t st) {
  if (cols == 0) return QUIP_OK;
  const int k = ilog2(rows);
  switch (k) {
    case 1: return cols_small_t<2>(A, out, cols, ld, signs, inverse, st);
    case 2: return cols_small_t<4>(A, out, cols, ld, signs, inverse, st);
    case 3: return cols_small_t<8>(A, out, cols, ld, signs, inverse, st);
  }
  if (k < 4 || k > 14) return fail(QUIP_ERR_SHAPE, "rht: the transform length must be a power of two in [2, 16384]");
  if (k == 12 && aligned16(A) && aligned16(out) && ld % 4 == 0) {
    const size_t shmem = size_t(PANEL_SLOTS) * sizeof(float4);
    QUIP_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(&rht_cols_panel),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, int(shmem)));
    const float scale = 1.0f / 64.0f;  // 1 / sqrt(4096)
    if (cols % 16 == 0 && aligned16(signs)) {  // 64-byte row segments
      // half a panel (8 columns x 4096 rows) plus one float2 of padding per 16
      // rows, then the scaled signs (64 rows of 68 floats)
      const size_t shmem16 = size_t(4 * 4096 + 4096 / 16) * sizeof(float2) + 64 * 68 * sizeof(float);
      QUIP_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(&rht_cols_panel16<false>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, int(shmem16)));
      QUIP_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(&rht_cols_panel16<true>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, int(shmem16)));
      const int nblk = int(cols / 16);
      return timed_launch("rht_cols_panel16", st, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
        if (inverse)
          QUIP_KERNEL(rht_cols_panel16<true>, dim3(unsigned(nblk)), dim3(512), shmem16, st, A,
                      out, ld, nblk, signs, scale);
        else
          QUIP_KERNEL(rht_cols_panel16<false>, dim3(unsigned(nblk)), dim3(512), shmem16, st, A,
                      out, ld, nblk, signs, scale);
      }, double(rows) * double(cols) * 14.0, 8.0 * double(rows) * double(cols));
    }
    const dim3 grid{unsigned(cdiv(cols, 8))};
    return timed_launch("rht_cols_panel", st, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
      QUIP_KERNEL(rht_cols_panel, grid, dim3(512), shmem, st, A, out, cols, ld, signs, scale,
                  inverse);
    }, double(rows) * double(cols) * 14.0, 8.0 * double(rows) * double(cols));
  }
  const int npass = (k + 6) / 7;
  int lo = 0;
  const float* src = A;
  for (int pidx = 0; pidx < npass; ++pidx) {
    int kr = (k - lo) / (npass - pidx);
    bool first = pidx == 0, last = pidx == npass - 1;
    int mode = (first && !inverse ? 1 : 0) | (last && inverse ? 2 : 0);
    float scale = last ? 1.0f / sqrtf(float(int64_t(1) << k)) : 1.0f;
    QUIP_TRY(cols_pass(kr, src, out, rows, cols, ld, lo, signs, scale, mode, st));
    src = out;
    lo += kr;
  }
  return QUIP_OK;
}

}  // namespace quip
