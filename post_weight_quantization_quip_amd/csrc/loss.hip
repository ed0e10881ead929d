// Proxy loss tr((W^ - W) H (W^ - W)^T) (QuIP, "Introduction": the quadratic
// proxy objective): E = W^ - W, then the contraction E H on the matrix cores
// with a fused epilogue that multiplies by E and sums in float64, so the
// m x n product E H is never written to memory. H is symmetric, so only its
// upper triangle is used (sum_{i<=j} E_ri H'_ij E_rj with H'_ij = 2 H_ij off the
// diagonal): half the flops of the full product.
#include "common.h"

namespace quip {

size_t loss_workspace_bytes(int64_t m, int64_t n) {
  Carver c(nullptr, 0);
  c.take<float>(size_t(m) * n);
  return c.used;
}

quip_status proxy_loss(const float* W, const float* What, int64_t m, int64_t n, int64_t ld,
                       const float* H, int64_t ldh, double* loss, void* ws, size_t ws_bytes,
                       hipStream_t s) {
  Carver c(ws, ws_bytes);
  float* E = c.take<float>(size_t(m) * n);
  if (!c.fits()) return fail(QUIP_ERR_WORKSPACE, "quip_proxy_loss: workspace too small");
  QUIP_TRY(fill_f64(loss, 1, 0.0, s));
  QUIP_TRY(sub_matrix(What, W, E, m, n, ld, ld, n, s));
  GemmArgs g;
  g.M = m;
  g.N = n;
  g.K = n;
  g.A = E;
  g.lda = n;
  g.B = H;
  g.ldb = ldh;
  g.epi = EPI_DOT_SYM;  // H symmetric: its upper triangle, off-diagonal counted twice
  g.E = E;
  g.lde = n;
  g.dot = loss;
  g.C = nullptr;
  g.tag = "gemm:proxy_loss";
  return gemm(g, s);
}

}  // namespace quip
