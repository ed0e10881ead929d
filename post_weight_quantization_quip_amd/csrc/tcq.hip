// Trellis-coded quantization with a bitshift trellis ([QTIP] summary page,
// Approach): a sequence x_0..x_{T-1} is quantized to the state sequence of an
// L-bit shift register that takes k = 2 new bits per step, each state s
// standing for the value c(s) of a computed pseudorandom Gaussian code, so
// that decoding needs only a window of L bits of the stream. The search is the
// exact Viterbi recursion: the best cost of reaching state s' = 4m + b at step
// t is min over a of the cost of state m + a 2^(L-2) at step t-1, plus
// (x_t - c(s'))^2. Ties go to the lowest a and, at the end, to the lowest
// state; the first state is free (no tail-biting).
//
// The code: h = 1664525 s + 1013904223 (mod 2^32, one 24-bit multiply-add
// since s < 2^16), c(s) = fma(sum of the four bytes of h, alpha, beta) with
// alpha = scale / sqrt(21845), beta = -510 alpha (the byte sum of a uniform
// word has mean 510 and variance 21845).
//
// tcq_forward_kernel: one work-group per sequence; the 2^L costs live in one
// LDS buffer (L <= 15: at most 128 KB) that every step updates in place: each
// thread reads the four predecessor costs of its groups (float4 reads of four
// consecutive groups), a barrier, then it writes the costs of the groups'
// successors (16 consecutive states per quad of groups) and one back-pointer
// byte per quad (2 bits per group), a barrier. The code of a state is
// recomputed each step (4 VALU ops). After the last step the work-group
// reduces the best final state.
//
// tcq_traceback_kernel: one thread per sequence walks the back-pointers from
// the best final state (all sequences of a chunk in parallel, so the chains of
// dependent loads overlap) and writes the states and their values.
#include "common.h"

namespace quip {
namespace {

constexpr uint32_t TCQ_MUL = 1664525u;
constexpr uint32_t TCQ_ADD = 1013904223u;
constexpr int64_t TCQ_CHUNK_ROWS = 2048;  // sequences per forward/traceback round

__device__ __forceinline__ float tcq_from_hash(uint32_t h, float alpha, float beta) {
  return fmaf(float(__builtin_amdgcn_sad_u8(h, 0u, 0u)), alpha, beta);
}

template <int L>
constexpr int tcq_threads() {
  return (1 << (L - 4)) < 64 ? 64 : ((1 << (L - 4)) > 1024 ? 1024 : (1 << (L - 4)));
}

template <int L>
__global__ __launch_bounds__(tcq_threads<L>()) void tcq_forward_kernel(
    const float* __restrict__ X, int64_t T, int64_t ldx, float alpha, float beta,
    uint8_t* __restrict__ bp, int32_t* __restrict__ best_state, float* __restrict__ best_cost) {
  constexpr int THREADS = tcq_threads<L>();
  constexpr int S = 1 << L;       // states
  constexpr int G = S >> 2;       // groups of states sharing their 4 predecessors
  constexpr int NQ = G >> 2;      // quads of groups
  constexpr int QPT = (NQ + THREADS - 1) / THREADS;
  extern __shared__ float4 cost4[];  // S floats
  float* const cost = reinterpret_cast<float*>(cost4);
  constexpr bool FULL = NQ % THREADS == 0;  // every thread owns QPT quads
  __shared__ float red_c[THREADS];
  __shared__ int32_t red_s[THREADS];

  const int tid = threadIdx.x;
  const float* x = X + int64_t(blockIdx.x) * ldx;
  uint8_t* bpr = bp + int64_t(blockIdx.x) * T * NQ;

  // step 0: every state may start the sequence
  {
    const float x0 = x[0];
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int q = tid + i * THREADS;
      if (FULL || q < NQ) {
        const uint32_t hb = __umul24(uint32_t(16 * q), TCQ_MUL) + TCQ_ADD;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          float4 v;
          float* vp = reinterpret_cast<float*>(&v);
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const float d = x0 - tcq_from_hash(hb + TCQ_MUL * uint32_t(4 * u + b), alpha, beta);
            vp[b] = d * d;
          }
          cost4[4 * q + u] = v;
        }
      }
    }
  }
  __syncthreads();

  for (int64_t t = 1; t < T; ++t) {
    const float xt = x[t];
    float4 P[QPT][4];
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int q = tid + i * THREADS;
      if (FULL || q < NQ) {
#pragma unroll
        for (int a = 0; a < 4; ++a) P[i][a] = cost4[q + a * (G / 4)];
      }
    }
    __syncthreads();  // every predecessor read before the in-place update
#pragma unroll
    for (int i = 0; i < QPT; ++i) {
      const int q = tid + i * THREADS;
      if (FULL || q < NQ) {
        const uint32_t hb = __umul24(uint32_t(16 * q), TCQ_MUL) + TCQ_ADD;
        uint32_t byte = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          float M = reinterpret_cast<const float*>(&P[i][0])[u];
          uint32_t am = 0;
#pragma unroll
          for (int a = 1; a < 4; ++a) {
            const float v = reinterpret_cast<const float*>(&P[i][a])[u];
            const bool lt = v < M;
            am = lt ? uint32_t(a) : am;
            M = lt ? v : M;
          }
          byte |= am << (2 * u);
          float4 nv;
          float* np = reinterpret_cast<float*>(&nv);
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const float d = xt - tcq_from_hash(hb + TCQ_MUL * uint32_t(4 * u + b), alpha, beta);
            np[b] = fmaf(d, d, M);
          }
          cost4[4 * q + u] = nv;
        }
        bpr[t * NQ + q] = uint8_t(byte);
      }
    }
    __syncthreads();
  }

  // best final state: lowest cost, then lowest index
  float bc = INFINITY;
  int32_t bs = S;
#pragma unroll
  for (int i = 0; i < QPT; ++i) {
    const int q = tid + i * THREADS;
    if (FULL || q < NQ) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float v = cost[16 * q + j];
        if (v < bc || (bs == S && !(v >= bc))) {  // the first state also takes NaN
          bc = v;
          bs = 16 * q + j;
        }
      }
    }
  }
  red_c[tid] = bc;
  red_s[tid] = bs;
  __syncthreads();
  for (int w = THREADS / 2; w > 0; w >>= 1) {
    if (tid < w) {
      const float oc = red_c[tid + w];
      const int32_t os = red_s[tid + w];
      const float mc = red_c[tid];
      const int32_t ms = red_s[tid];
      if (os < S && (ms == S || oc < mc || (oc == mc && os < ms) || (mc != mc && oc == oc))) {
        red_c[tid] = oc;
        red_s[tid] = os;
      }
    }
    __syncthreads();
  }
  if (tid == 0) {
    best_state[blockIdx.x] = red_s[0];
    best_cost[blockIdx.x] = red_c[0];
  }
}

__global__ __launch_bounds__(256) void tcq_traceback_kernel(
    const uint8_t* __restrict__ bp, int64_t rows, int64_t T, int L, const int32_t* __restrict__ best,
    uint16_t* __restrict__ states, int64_t lds, float* __restrict__ xhat, int64_t ldq, float alpha,
    float beta) {
  const int64_t r = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (r >= rows) return;
  const int64_t NQ = int64_t(1) << (L - 4);
  const uint32_t G = 1u << (L - 2);
  const uint8_t* bpr = bp + r * T * NQ;
  uint16_t* st = states + r * lds;
  float* xq = xhat ? xhat + r * ldq : nullptr;
  uint32_t s = uint32_t(best[r]) & ((1u << L) - 1);
  for (int64_t t = T - 1; t >= 1; --t) {
    st[t] = uint16_t(s);
    if (xq) xq[t] = tcq_from_hash(__umul24(s, TCQ_MUL) + TCQ_ADD, alpha, beta);
    const uint32_t m = s >> 2;
    const uint32_t a = (uint32_t(bpr[t * NQ + (m >> 2)]) >> (2 * (m & 3))) & 3u;
    s = m + a * G;
  }
  st[0] = uint16_t(s);
  if (xq) xq[0] = tcq_from_hash(__umul24(s, TCQ_MUL) + TCQ_ADD, alpha, beta);
}

template <int L>
quip_status tcq_forward_t(const float* X, int64_t n, int64_t T, int64_t ldx, float alpha,
                          float beta, uint8_t* bp, int32_t* best, float* cost, hipStream_t s) {
  constexpr int THREADS = tcq_threads<L>();
  const size_t shmem = sizeof(float) << L;
  QUIP_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(&tcq_forward_kernel<L>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, int(shmem)));
  // trellis edges relaxed: 4 per state and step
  const double edges = double(n) * double(T - 1) * 4.0 * double(1 << L);
  const double bytes = 4.0 * double(n) * double(T) + double(n) * double(T) * double(1 << (L - 4));
  return timed_launch("tcq_forward_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL(tcq_forward_kernel<L>, dim3(unsigned(n)), dim3(THREADS), shmem, s, X, T, ldx, alpha,
                beta, bp, best, cost);
  }, edges, bytes);
}

}  // namespace

int64_t tcq_chunk_rows(int64_t rows) { return rows < TCQ_CHUNK_ROWS ? rows : TCQ_CHUNK_ROWS; }

size_t tcq_workspace_bytes(int64_t rows, int64_t T, int L) {
  const int64_t c = tcq_chunk_rows(rows);
  Carver w(nullptr, 0);
  w.take<uint8_t>(size_t(c) * size_t(T) * (size_t(1) << (L - 4)));  // back-pointers
  w.take<int32_t>(size_t(c));                                         // best final states
  return w.used;
}

quip_status tcq_quantize(const float* X, int64_t rows, int64_t T, int64_t ldx, int L, float scale,
                         uint16_t* states, int64_t lds, float* xhat, int64_t ldq, float* cost,
                         void* ws, size_t ws_bytes, hipStream_t s) {
  const int64_t chunk = tcq_chunk_rows(rows);
  Carver w(ws, ws_bytes);
  uint8_t* bp = w.take<uint8_t>(size_t(chunk) * size_t(T) * (size_t(1) << (L - 4)));
  int32_t* best = w.take<int32_t>(size_t(chunk));
  if (!w.fits()) return fail(QUIP_ERR_WORKSPACE, "quip_tcq_quantize: workspace too small");
  const double sd = 147.80054127099805;  // sqrt(4 (256^2 - 1) / 12)
  const float alpha = float(double(scale) / sd);
  const float beta = float(-510.0 * double(scale) / sd);
  for (int64_t r0 = 0; r0 < rows; r0 += chunk) {
    const int64_t n = rows - r0 < chunk ? rows - r0 : chunk;
    const float* Xc = X + r0 * ldx;
    switch (L) {
#define CASE(LL) \
  case LL: QUIP_TRY(tcq_forward_t<LL>(Xc, n, T, ldx, alpha, beta, bp, best, cost + r0, s)); break;
      CASE(4) CASE(5) CASE(6) CASE(7) CASE(8) CASE(9) CASE(10) CASE(11) CASE(12) CASE(13) CASE(14)
      CASE(15)
#undef CASE
      default: return fail(QUIP_ERR_UNSUPPORTED, "quip_tcq_quantize: L must be in [4, 15]");
    }
    const double tb_bytes = double(n) * double(T) * (1.0 + 2.0 + (xhat ? 4.0 : 0.0));
    QUIP_TRY(timed_launch("tcq_traceback_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
      QUIP_KERNEL(tcq_traceback_kernel, dim3(unsigned(cdiv(n, 256))), dim3(256), 0, s, bp, n, T, L,
                  best, states + r0 * lds, lds, xhat ? xhat + r0 * ldq : nullptr, ldq, alpha, beta);
    }, 0.0, tb_bytes));
  }
  return QUIP_OK;
}

}  // namespace quip
