// Multiplication by Q = F1 (x) F2, a Kronecker product of two orthogonal
// factors (QuIP, "Introduction" / "Conclusion": incoherence processing by a
// Kronecker product of random orthogonal matrices). Index i = a*q + b.
//
// RIGHT (out = A Q^T): every row x, seen as a p x q matrix X, becomes
// F1 X F2^T. Two contractions on the matrix cores:
//   T = X F2^T  : one GEMM over all rows*p sub-rows (M = rows*p, K = N = q)
//   out_r = F1 T_r : batched over rows (M = p, K = p, N = q)
// LEFT (out = Q A): A seen as p blocks of q rows.
//   T_a = F2 A_a : batched over a (M = q, K = q, N = cols)
//   out = F1 T   : one GEMM with T viewed as p x (q*cols)
// The inverse uses F1^T (x) F2^T (the GEMMs read the factors transposed).
#include "common.h"

namespace quip {

quip_status kron_apply(const float* A, float* out, int64_t rows, int64_t cols, int64_t ld,
                       const float* F1, int64_t p, const float* F2, int64_t q, bool left,
                       bool inverse, void* ws, size_t ws_bytes, hipStream_t s) {
  Carver c(ws, ws_bytes);
  float* T = c.take<float>(size_t(rows) * cols);
  if (!c.fits()) return fail(QUIP_ERR_WORKSPACE, "quip_kron_orth: workspace too small");
  if (!left) {
    // T[(r, a), b] = sum_b' A[r, a*q + b'] F2[b][b']   (F2^T for the forward map)
    GemmArgs g1;
    if (ld == cols) {
      g1.M = rows * p;
      g1.N = q;
      g1.K = q;
      g1.A = A;
      g1.lda = q;
    } else {
      g1.M = p;
      g1.N = q;
      g1.K = q;
      g1.A = A;
      g1.lda = q;
      g1.strideA = ld;
      g1.batch = int(rows);
    }
    g1.B = F2;
    g1.ldb = q;
    g1.transB = !inverse;  // forward: op(B)[k][j] = F2[j][k]; inverse: F2[k][j]
    g1.C = T;
    g1.ldc = q;
    g1.strideC = p * q;
    g1.tag = "gemm:kron";
    QUIP_TRY(gemm(g1, s));
    // out_r[a, b] = sum_a' F1[a][a'] T_r[a', b]  (inverse: F1^T)
    GemmArgs g2;
    g2.M = p;
    g2.N = q;
    g2.K = p;
    g2.A = F1;
    g2.lda = p;
    g2.transA = inverse;  // inverse: op(A)[a][a'] = F1[a'][a]
    g2.B = T;
    g2.ldb = q;
    g2.strideB = p * q;
    g2.C = out;
    g2.ldc = q;
    g2.strideC = ld;
    g2.batch = int(rows);
    g2.tag = "gemm:kron";
    return gemm(g2, s);
  }
  // LEFT: T_a = F2 A_a (q x cols), a = 0..p-1
  GemmArgs g1;
  g1.M = q;
  g1.N = cols;
  g1.K = q;
  g1.A = F2;
  g1.lda = q;
  g1.transA = inverse;
  g1.B = A;
  g1.ldb = ld;
  g1.strideB = q * ld;
  g1.C = T;
  g1.ldc = cols;
  g1.strideC = q * cols;
  g1.batch = int(p);
  g1.tag = "gemm:kron";
  QUIP_TRY(gemm(g1, s));
  // out[(a, b), :] = sum_a' F1[a][a'] T[(a', b), :] : batched over b (row stride q*ld)
  GemmArgs g2;
  g2.A = F1;
  g2.lda = p;
  g2.transA = inverse;
  g2.M = p;
  g2.K = p;
  if (ld == cols) {
    g2.N = q * cols;
    g2.B = T;
    g2.ldb = q * cols;
    g2.C = out;
    g2.ldc = q * cols;
  } else {
    g2.N = cols;
    g2.B = T;
    g2.ldb = q * cols;
    g2.strideB = cols;
    g2.C = out;
    g2.ldc = q * ld;
    g2.strideC = ld;
    g2.batch = int(q);
  }
  g2.tag = "gemm:kron";
  return gemm(g2, s);
}

size_t kron_workspace_bytes(int64_t rows, int64_t cols) {
  Carver c(nullptr, 0);
  c.take<float>(size_t(rows) * cols);
  return c.used;
}

}  // namespace quip
