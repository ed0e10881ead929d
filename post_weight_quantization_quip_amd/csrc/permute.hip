// Permutations for the QuIP variants: the random permutation inside the fast
// orthogonal multiplication ([QuIP] "Further Ablation", Table 5) and LDLQ-RG's
// quantization order by diag(H) ([QuIP] "Experiments / Methods").
//
// permute_gather_kernel / permute_scatter_kernel move whole rows: one
// work-group per row (looping), the row staged in LDS when the columns are
// permuted, so that both the global read and the global write are contiguous
// (float4 when the shapes allow) and only LDS sees the scattered indices.
//
// The diag(H) order is a rank count: column i lands at position
//   #{j : key_j > key_i} + #{j < i : key_j == key_i},
// a strict total order, so the positions form a permutation. The count is
// split over slices of j (one partial count per slice and column, no atomics)
// and a second launch sums the partials and writes order[position] = i.
#include "common.h"

namespace quip {
namespace {

constexpr int PERM_THREADS = 256;
constexpr int RANK_SLICE = 512;

__device__ __forceinline__ bool in_range(int32_t v, int64_t n) { return v >= 0 && int64_t(v) < n; }

template <bool VEC>
__device__ __forceinline__ void copy_row(const float* __restrict__ a, float* __restrict__ o,
                                         int64_t cols) {
  if (VEC) {
    const float4* a4 = reinterpret_cast<const float4*>(a);
    float4* o4 = reinterpret_cast<float4*>(o);
    for (int64_t j = threadIdx.x; j < cols / 4; j += PERM_THREADS) o4[j] = a4[j];
  } else {
    for (int64_t j = threadIdx.x; j < cols; j += PERM_THREADS) o[j] = a[j];
  }
}

// out[i][j] = A[r(i)][c(j)]; an index outside the matrix gives NaN.
template <bool VEC>
__global__ __launch_bounds__(PERM_THREADS) void permute_gather_kernel(
    const float* __restrict__ A, int64_t lda, float* __restrict__ out, int64_t ldo, int64_t rows,
    int64_t cols, const int32_t* __restrict__ ridx, const int32_t* __restrict__ cidx) {
  extern __shared__ float row[];
  const float qnan = __builtin_nanf("");
  for (int64_t i = blockIdx.x; i < rows; i += gridDim.x) {
    const int64_t src = ridx ? int64_t(ridx[i]) : i;  // the same for the whole work-group
    float* o = out + i * ldo;
    if (src < 0 || src >= rows) {
      for (int64_t j = threadIdx.x; j < cols; j += PERM_THREADS) o[j] = qnan;
      continue;
    }
    const float* a = A + src * lda;
    if (!cidx) {
      copy_row<VEC>(a, o, cols);
      continue;
    }
    __syncthreads();  // the previous row's LDS reads are done
    if (VEC) {
      const float4* a4 = reinterpret_cast<const float4*>(a);
      float4* r4 = reinterpret_cast<float4*>(row);
      for (int64_t j = threadIdx.x; j < cols / 4; j += PERM_THREADS) r4[j] = a4[j];
    } else {
      for (int64_t j = threadIdx.x; j < cols; j += PERM_THREADS) row[j] = a[j];
    }
    __syncthreads();
    if (VEC) {
      float4* o4 = reinterpret_cast<float4*>(o);
      const int4* c4 = reinterpret_cast<const int4*>(cidx);
      for (int64_t j = threadIdx.x; j < cols / 4; j += PERM_THREADS) {
        const int4 c = c4[j];
        float4 v;
        v.x = in_range(c.x, cols) ? row[c.x] : qnan;
        v.y = in_range(c.y, cols) ? row[c.y] : qnan;
        v.z = in_range(c.z, cols) ? row[c.z] : qnan;
        v.w = in_range(c.w, cols) ? row[c.w] : qnan;
        o4[j] = v;
      }
    } else {
      for (int64_t j = threadIdx.x; j < cols; j += PERM_THREADS) {
        const int32_t c = cidx[j];
        o[j] = in_range(c, cols) ? row[c] : qnan;
      }
    }
  }
}

// out[r(i)][c(j)] = A[i][j]; entries with an index outside the matrix are
// dropped (with index vectors that are not permutations, the entries of out
// that nothing lands on are unspecified).
template <bool VEC>
__global__ __launch_bounds__(PERM_THREADS) void permute_scatter_kernel(
    const float* __restrict__ A, int64_t lda, float* __restrict__ out, int64_t ldo, int64_t rows,
    int64_t cols, const int32_t* __restrict__ ridx, const int32_t* __restrict__ cidx) {
  extern __shared__ float row[];
  for (int64_t i = blockIdx.x; i < rows; i += gridDim.x) {
    const int64_t dst = ridx ? int64_t(ridx[i]) : i;
    if (dst < 0 || dst >= rows) continue;
    const float* a = A + i * lda;
    float* o = out + dst * ldo;
    if (!cidx) {
      copy_row<VEC>(a, o, cols);
      continue;
    }
    __syncthreads();
    if (VEC) {
      const float4* a4 = reinterpret_cast<const float4*>(a);
      const int4* c4 = reinterpret_cast<const int4*>(cidx);
      for (int64_t j = threadIdx.x; j < cols / 4; j += PERM_THREADS) {
        const float4 v = a4[j];
        const int4 c = c4[j];
        if (in_range(c.x, cols)) row[c.x] = v.x;
        if (in_range(c.y, cols)) row[c.y] = v.y;
        if (in_range(c.z, cols)) row[c.z] = v.z;
        if (in_range(c.w, cols)) row[c.w] = v.w;
      }
    } else {
      for (int64_t j = threadIdx.x; j < cols; j += PERM_THREADS) {
        const int32_t c = cidx[j];
        if (in_range(c, cols)) row[c] = a[j];
      }
    }
    __syncthreads();
    if (VEC) {
      const float4* r4 = reinterpret_cast<const float4*>(row);
      float4* o4 = reinterpret_cast<float4*>(o);
      for (int64_t j = threadIdx.x; j < cols / 4; j += PERM_THREADS) o4[j] = r4[j];
    } else {
      for (int64_t j = threadIdx.x; j < cols; j += PERM_THREADS) o[j] = row[j];
    }
  }
}

// NaN orders after every number (as -inf); +0 and -0 are equal.
__device__ __forceinline__ float order_key(float x) { return x != x ? -INFINITY : x; }

// part[s][i] = #{j in slice s : key_j > key_i or (key_j == key_i and j < i)}
__global__ __launch_bounds__(256) void diag_rank_kernel(const float* __restrict__ H, int64_t n,
                                                        int64_t ldh, int32_t* __restrict__ part) {
  __shared__ float key[RANK_SLICE];
  const int64_t j0 = int64_t(blockIdx.y) * RANK_SLICE;
  const int jn = int(n - j0 < RANK_SLICE ? n - j0 : RANK_SLICE);
  for (int t = threadIdx.x; t < jn; t += 256) key[t] = order_key(H[(j0 + t) * (ldh + 1)]);
  __syncthreads();
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  const float ki = order_key(H[i * (ldh + 1)]);
  // j < i holds for the whole slice, for none of it, or up to i - j0
  const int64_t below = i - j0 < 0 ? 0 : (i - j0 > jn ? jn : i - j0);
  int c = 0;
  for (int t = 0; t < below; ++t) c += key[t] >= ki;
  for (int t = int(below); t < jn; ++t) c += key[t] > ki;
  part[int64_t(blockIdx.y) * n + i] = c;
}

__global__ __launch_bounds__(256) void diag_order_finish_kernel(const int32_t* __restrict__ part,
                                                                int slices, int64_t n,
                                                                int32_t* __restrict__ order) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n) return;
  int64_t c = 0;
  for (int s = 0; s < slices; ++s) c += part[int64_t(s) * n + i];
  order[c] = int32_t(i);  // 0 <= c < n: at most n - 1 columns precede column i
}

}  // namespace

int64_t permute_max_cols() { return 32768; }

quip_status permute(const float* A, int64_t lda, float* out, int64_t ldo, int64_t rows,
                    int64_t cols, const int32_t* ridx, const int32_t* cidx, bool scatter,
                    hipStream_t s) {
  if (rows == 0 || cols == 0) return QUIP_OK;
  const bool vec = cols % 4 == 0 && lda % 4 == 0 && ldo % 4 == 0 && aligned16(A) &&
                   aligned16(out) && (!cidx || aligned16(cidx));
  const size_t shmem = cidx ? size_t(cols) * sizeof(float) : 0;
  const dim3 grid{unsigned(rows < 65535 ? rows : 65535)};
  const double bytes = 8.0 * double(rows) * double(cols) + 4.0 * (ridx ? double(rows) : 0.0) +
                       4.0 * (cidx ? double(cols) : 0.0);
  const char* name = scatter ? "permute_scatter_kernel" : "permute_gather_kernel";
  if (cidx) {
#define SET_LDS(K) \
  QUIP_HIP(hipFuncSetAttribute(reinterpret_cast<const void*>(&K), \
                               hipFuncAttributeMaxDynamicSharedMemorySize, int(shmem)))
    if (scatter) {
      if (vec) SET_LDS(permute_scatter_kernel<true>); else SET_LDS(permute_scatter_kernel<false>);
    } else {
      if (vec) SET_LDS(permute_gather_kernel<true>); else SET_LDS(permute_gather_kernel<false>);
    }
#undef SET_LDS
  }
  return timed_launch(name, s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    if (scatter) {
      if (vec)
        QUIP_KERNEL(permute_scatter_kernel<true>, grid, dim3(PERM_THREADS), shmem, s, A, lda, out,
                    ldo, rows, cols, ridx, cidx);
      else
        QUIP_KERNEL(permute_scatter_kernel<false>, grid, dim3(PERM_THREADS), shmem, s, A, lda, out,
                    ldo, rows, cols, ridx, cidx);
    } else {
      if (vec)
        QUIP_KERNEL(permute_gather_kernel<true>, grid, dim3(PERM_THREADS), shmem, s, A, lda, out,
                    ldo, rows, cols, ridx, cidx);
      else
        QUIP_KERNEL(permute_gather_kernel<false>, grid, dim3(PERM_THREADS), shmem, s, A, lda, out,
                    ldo, rows, cols, ridx, cidx);
    }
  }, 0.0, bytes);
}

size_t diag_order_workspace_bytes(int64_t n) {
  Carver c(nullptr, 0);
  c.take<int32_t>(size_t(cdiv(n, RANK_SLICE) * n));
  return c.used;
}

quip_status diag_order(const float* H, int64_t n, int64_t ldh, int32_t* order, void* ws,
                       size_t ws_bytes, hipStream_t s) {
  const int slices = int(cdiv(n, RANK_SLICE));
  Carver c(ws, ws_bytes);
  int32_t* part = c.take<int32_t>(size_t(slices) * size_t(n));
  if (!c.fits()) return fail(QUIP_ERR_WORKSPACE, "quip_diag_order: workspace too small");
  const dim3 grid{unsigned(cdiv(n, 256)), unsigned(slices)};
  QUIP_TRY(timed_launch("diag_rank_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL(diag_rank_kernel, grid, dim3(256), 0, s, H, n, ldh, part);
  }, double(n) * double(n), 4.0 * double(n) * (1.0 + double(slices))));
  return timed_launch("diag_order_finish_kernel", s, [&](hipEvent_t ev_start_, hipEvent_t ev_stop_) {
    QUIP_KERNEL(diag_order_finish_kernel, dim3(unsigned(cdiv(n, 256))), dim3(256), 0, s, part,
                slices, n, order);
  }, 0.0, 4.0 * double(n) * double(slices) + 4.0 * double(n));
}

}  // namespace quip
