"""GPU parity of every entry point of the C ABI against the CPU oracle, at sizes
the oracle finishes in seconds that still span several tiles and ragged tails.

Tolerances:
  * transforms (RHT, Kronecker): per-row normwise relative error <= 1e-5;
  * Hessian: |dH_ij| <= 2e-5 sqrt(H_ii H_jj)  (float32 sums of N products);
  * LDL: backward error ||(I+U)D(I+U)^T - H|| / ||H|| <= 2e-6 * sqrt(n);
  * codes: conditional replay, every mismatch inside the 1e-5 boundary band
    and at most 1e-4 of all codes;
  * proxy loss: 1e-4 relative (float64 accumulation of float32 products).
"""
import numpy as np
import pytest
import torch

import oracle as O
import post_weight_quantization_quip_amd as Q
import workloads as wl
from tests import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda"


def dev(x, dtype=torch.float32):
    return torch.as_tensor(np.ascontiguousarray(x)).to(device=DEV, dtype=dtype)


def host(t):
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def rng(seed):
    return np.random.default_rng(seed)


def signs(seed, d):
    return np.where(rng(seed).random(d) < 0.5, -1.0, 1.0).astype(np.float32)


def spd32(seed, n, N=None, sigma=1.0):
    r = rng(seed)
    N = 2 * n if N is None else N
    X = (r.standard_normal((N, n)) * np.exp(sigma * r.standard_normal(n))[None, :]).astype(np.float32)
    return O.damp(O.proxy_hessian(X), 0.01).astype(np.float32)


# ------------------------------------------------------------------ Hessian

# N >= 1024 numbers the output tiles by 8 x 8 super-blocks: 1500 x 1100 has 18
# tile rows of 64, so the last super-blocks are partial
@pytest.mark.parametrize("N,n", [(2048, 256), (1000, 200), (64, 1000), (5, 3), (1, 1), (300, 129),
                                 (1500, 1100)])
def test_hessian_parity(N, n):
    X = (rng(N * 7 + n).standard_normal((N, n)) * np.exp(rng(n).standard_normal(n))).astype(np.float32)
    H = torch.empty((n, n), device=DEV)
    Xd = dev(X)
    Q.quip_hessian(Xd, H)
    Q.quip_hessian_finalize(H, N, 0.01)
    got = host(H).astype(np.float64)
    ref = O.damp(O.proxy_hessian(X), 0.01)
    d = np.sqrt(np.diag(ref))
    assert (np.abs(got - ref) <= 2e-5 * d[:, None] * d[None, :]).all()
    assert np.array_equal(got, got.T)


def hessian_raw(Xd, n, ws):
    """X^T X through the C ABI, with or without the leftover-tile workspace."""
    N = Xd.shape[0]
    H = torch.empty((n, n), device=DEV)
    Q.native._check(Q.native.lib.quip_hessian(
        Xd.data_ptr(), N, n, n, H.data_ptr(), n, 0, None if ws is None else ws.data_ptr(),
        0 if ws is None else ws.numel(), torch.cuda.current_stream().cuda_stream), "quip_hessian")
    return host(H)


@pytest.mark.parametrize("N,n", [(4096, 4096), (2048, 256), (333, 1100)])
def test_hessian_leftover_split(N, n):
    # the leftover tiles split along N (with the workspace) and the plain grid
    # both match float64 sums; each path is bitwise reproducible
    X = (rng(N + n).standard_normal((N, n)) * np.exp(0.5 * rng(n + 1).standard_normal(n))).astype(np.float32)
    Xd = dev(X)
    need = Q.native._ws_query(Q.native.lib.quip_hessian_workspace, N, n)
    ws = Q.native._workspace(need, DEV) if need else None
    a = hessian_raw(Xd, n, ws)
    a2 = hessian_raw(Xd, n, ws)
    b = hessian_raw(Xd, n, None)
    assert np.array_equal(a, a2)
    assert np.array_equal(a, a.T) and np.array_equal(b, b.T)
    cols = rng(5).choice(n, min(n, 64), replace=False)
    ref = X[:, cols].astype(np.float64).T @ X.astype(np.float64)  # rows `cols` of X^T X
    d = np.sqrt(np.einsum("ij,ij->j", X.astype(np.float64), X.astype(np.float64)))
    tol = 2e-5 * d[cols][:, None] * d[None, :]
    assert (np.abs(a[cols] - ref) <= tol).all()
    assert (np.abs(b[cols] - ref) <= tol).all()


def test_hessian_accumulates_in_chunks():
    X = rng(3).standard_normal((700, 130)).astype(np.float32)
    H = torch.empty((130, 130), device=DEV)
    Q.quip_hessian(dev(X[:300]), H)
    Q.quip_hessian(dev(X[300:]), H, accumulate=True)
    Q.quip_hessian_finalize(H, 700, 0.0)
    ref = O.proxy_hessian(X)
    d = np.sqrt(np.diag(ref))
    assert (np.abs(host(H) - ref) <= 2e-5 * d[:, None] * d[None, :]).all()


def test_hessian_of_no_rows():
    # an empty chunk of calibration rows: H = 0, or H unchanged when accumulating
    X = torch.empty((0, 70), device=DEV)
    H = torch.full((70, 70), 3.0, device=DEV)
    Q.quip_hessian(X, H, accumulate=True)
    torch.cuda.synchronize()
    assert bool((H == 3.0).all())
    Q.quip_hessian(X, H)
    torch.cuda.synchronize()
    assert bool((H == 0.0).all())


def test_permute_of_empty_matrix_is_a_no_op():
    out = torch.full((4, 3), 7.0, device=DEV)
    A = torch.zeros((4, 3), device=DEV)
    lib = Q.native.lib
    assert lib.quip_permute(A.data_ptr(), 3, out.data_ptr(), 3, 0, 3, None, None, 0, None) == 0
    assert lib.quip_permute(A.data_ptr(), 3, out.data_ptr(), 3, 4, 0, None, None, 1, None) == 0
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())


# ------------------------------------------------------------------ RHT

@pytest.mark.parametrize("rows,d", [(37, 2), (5, 4), (9, 8), (33, 16), (17, 32), (17, 64), (300, 256),
                                    (3, 1024), (70, 4096), (5, 8192), (3, 16384)])
def test_rht_right(rows, d):
    A = rng(d + rows).standard_normal((rows, d)).astype(np.float32)
    s = signs(d, d)
    Ad, sd = dev(A), dev(s)
    out = torch.empty_like(Ad)
    Q.quip_rht(Ad, out, sd, Q.RIGHT)
    assert P.rel_rows(host(out), O.rht(A, s, "right")) <= 1e-5
    back = torch.empty_like(Ad)
    Q.quip_rht_inv(out, back, sd, Q.RIGHT)
    assert P.rel_rows(host(back), O.rht_inv(host(out), s, "right")) <= 1e-5
    assert P.rel_rows(host(back), A) <= 1e-5
    Q.quip_rht(Ad, Ad, sd, Q.RIGHT)  # in place
    assert np.array_equal(host(Ad), host(out))


# d = 4096 with aligned rows takes a one-pass panel kernel: 16 columns per
# work-group when the count is a multiple of 16 (128, 16, 4096), else 8 (13
# and 1030 leave ragged last blocks)
@pytest.mark.parametrize("d,cols", [(2, 5), (4, 65), (8, 1), (16, 64), (64, 130), (128, 64), (256, 300),
                                    (512, 64), (2048, 65), (4096, 128), (4096, 16), (4096, 13),
                                    (4096, 1030), (8192, 64)])
def test_rht_left(d, cols):
    A = rng(d * 3 + cols).standard_normal((d, cols)).astype(np.float32)
    s = signs(d + 1, d)
    Ad, sd = dev(A), dev(s)
    out = torch.empty_like(Ad)
    Q.quip_rht(Ad, out, sd, Q.LEFT)
    ref = O.rht(A, s, "left")
    assert P.rel_rows(host(out).T, ref.T) <= 1e-5
    back = torch.empty_like(Ad)
    Q.quip_rht_inv(out, back, sd, Q.LEFT)
    assert P.rel_rows(host(back).T, O.rht_inv(host(out), s, "left").T) <= 1e-5
    assert P.rel_rows(host(back).T, A.T) <= 1e-5
    Q.quip_rht(Ad, Ad, sd, Q.LEFT)  # in place
    assert np.array_equal(host(Ad), host(out))


@pytest.mark.parametrize("cols,ld", [(48, 64), (4112, 4112)])
def test_rht_left_panel16_strided_and_many_panels(cols, ld):
    """The 16-column panel kernel (d = 4096) with rows wider than the block
    (ld > cols) and with more panels than one work-group per CU (4112 columns:
    257 panels), both directions against the oracle."""
    d = 4096
    base = rng(cols + 7).standard_normal((d, ld)).astype(np.float32)
    s = signs(cols + 11, d)
    A = dev(base)[:, :cols]
    out_full = torch.zeros((d, ld), device=DEV)
    out = out_full[:, :cols]
    Q.quip_rht(A, out, dev(s), Q.LEFT)
    ref = O.rht(base[:, :cols], s, "left")
    assert P.rel_rows(host(out).T, ref.T) <= 1e-5
    back = torch.zeros((d, ld), device=DEV)[:, :cols]
    Q.quip_rht_inv(out, back, dev(s), Q.LEFT)
    assert P.rel_rows(host(back).T, base[:, :cols].T) <= 1e-5
    assert np.all(host(out_full[:, cols:]) == 0)  # the columns past the block are untouched


def test_rht_left_unaligned_rows():
    # row pitch 131 floats: not float4-aligned, so d = 4096 goes through the
    # multi-pass column kernels; it must agree with the oracle all the same
    base = rng(11).standard_normal((4096, 131)).astype(np.float32)
    A = dev(base)[:, :130]
    s = signs(12, 4096)
    out = torch.zeros((4096, 131), device=DEV)[:, :130]
    Q.quip_rht(A, out, dev(s), Q.LEFT)
    ref = O.rht(base[:, :130], s, "left")
    assert P.rel_rows(host(out).T, ref.T) <= 1e-5


def test_rht_leading_dimension():
    base = rng(5).standard_normal((64, 300)).astype(np.float32)
    A = dev(base)[:, :256]  # ld = 300 > cols
    s = signs(9, 256)
    out_full = torch.zeros((64, 300), device=DEV)
    out = out_full[:, :256]
    Q.quip_rht(A, out, dev(s), Q.RIGHT)
    assert P.rel_rows(host(out), O.rht(base[:, :256], s, "right")) <= 1e-5
    assert np.all(host(out_full[:, 256:]) == 0)  # the columns past the rows are untouched


@pytest.mark.parametrize("m,n", [(256, 256), (64, 4096), (4096, 64), (2, 2)])
def test_rht_two_sided(m, n):
    A = rng(m + n).standard_normal((m, n)).astype(np.float32)
    sl, sr = signs(1, m), signs(2, n)
    Ad = dev(A)
    out = torch.empty_like(Ad)
    Q.quip_rht2(Ad, out, dev(sl), dev(sr))
    ref = O.incoherence_W(A, {"signs": sl}, {"signs": sr})
    assert P.rel_rows(host(out), ref) <= 1e-5
    back = torch.empty_like(Ad)
    Q.quip_rht2_inv(out, back, dev(sl), dev(sr))
    assert P.rel_rows(host(back), A) <= 1e-5


# ------------------------------------------------------------------ Kronecker

@pytest.mark.parametrize("side,rows,cols,p,q", [
    ("right", 10, 24, 4, 6), ("left", 24, 10, 4, 6), ("right", 40, 11008, 64, 172),
    ("left", 11008, 48, 64, 172), ("right", 7, 28672, 128, 224), ("left", 3, 5, 3, 1)])
def test_kron(side, rows, cols, p, q):
    r = rng(rows + cols)
    A = r.standard_normal((rows, cols)).astype(np.float32)
    F1 = wl.haar_orthogonal(r, p)
    F2 = wl.haar_orthogonal(r, q)
    Ad = dev(A)
    out = torch.empty_like(Ad)
    sd = Q.LEFT if side == "left" else Q.RIGHT
    Q.quip_kron_orth(Ad, out, dev(F1), dev(F2), sd)
    ref = O.kron_apply(A, F1, F2, side)
    got = host(out)
    if side == "left":
        assert P.rel_rows(got.T, ref.T) <= 1e-5
    else:
        assert P.rel_rows(got, ref) <= 1e-5
    back = torch.empty_like(Ad)
    Q.quip_kron_orth_inv(out, back, dev(F1), dev(F2), sd)
    refb = O.kron_apply(got, F1, F2, side, inverse=True)
    if side == "left":
        assert P.rel_rows(host(back).T, refb.T) <= 1e-5
    else:
        assert P.rel_rows(host(back), refb) <= 1e-5


def test_kron_leading_dimension_in_place():
    r = rng(77)
    base = r.standard_normal((12, 40)).astype(np.float32)
    F1, F2 = wl.haar_orthogonal(r, 4), wl.haar_orthogonal(r, 8)
    full = dev(base)
    view = full[:, :32]
    Q.quip_kron_orth(view, view, dev(F1), dev(F2), Q.RIGHT)
    got = host(full)
    assert P.rel_rows(got[:, :32], O.kron_apply(base[:, :32], F1, F2, "right")) <= 1e-5
    assert np.array_equal(got[:, 32:], base[:, 32:])


# ------------------------------------------------------------------ LDL

def ldl_gpu(H32, g):
    n = H32.shape[0]
    U = torch.empty((n, n), device=DEV)
    D = torch.empty(n * 8 if g == 8 else n, device=DEV)
    info = torch.full((1,), 7, dtype=torch.int32, device=DEV)
    Q.quip_ldl(dev(H32), g, U, D, info)
    return host(U), host(D), int(host(info)[0])


# above n = 4096 the outer blocks are 512 columns wide (4500 and 4616 end in a
# partial one)
@pytest.mark.parametrize("n,g", [(256, 1), (256, 8), (200, 1), (200, 8), (8, 8), (1, 1), (130, 1),
                                 (600, 1), (600, 8), (520, 1), (1000, 1), (2000, 1), (1536, 8),
                                 (3000, 1), (4500, 1), (4616, 8)])
def test_ldl_parity(n, g):
    H = spd32(n * 11 + g, n)
    U, D, info = ldl_gpu(H, g)
    assert info == 0
    assert P.recon_residual(H, U, D, g) <= 2e-6 * np.sqrt(n)
    mask = np.triu(np.ones((n, n), bool), 1)
    if g > 1:
        blk = np.arange(n) // g
        mask = blk[:, None] < blk[None, :]
    assert np.all(U[~mask] == 0)
    Uo, Do = O.udu_cholesky(H.astype(np.float64), g)
    # forward error of the factors, relative to the oracle's on the same float32 H
    assert np.linalg.norm(U - Uo) / max(np.linalg.norm(Uo), 1e-30) <= 1e-3
    assert np.linalg.norm(D.reshape(-1) - Do.reshape(-1)) / np.linalg.norm(Do) <= 1e-3


def test_ldl_diagonal():
    d = rng(4).uniform(0.5, 3.0, 100).astype(np.float32)
    U, D, info = ldl_gpu(np.diag(d), 1)
    assert info == 0 and np.all(U == 0) and np.array_equal(D, d)


@pytest.mark.parametrize("n,g,bad,want", [(16, 1, 9, 10), (16, 8, 9, 9), (200, 1, 9, 10), (200, 8, 9, 9)])
def test_ldl_not_positive_definite(n, g, bad, want):
    H = spd32(5, n)
    H[bad, :] = 0
    H[:, bad] = 0
    _, _, info = ldl_gpu(H, g)
    assert info == want
    with pytest.raises(O.NotPositiveDefinite):
        O.udu(H.astype(np.float64), g)


# ------------------------------------------------------------------ scales

@pytest.mark.parametrize("bits", [2, 3, 4])
def test_grid_scale_parity(bits):
    L = 1 << bits
    W = (rng(bits).standard_normal((37, 300)) * np.exp(rng(9).standard_normal(37))[:, None]).astype(np.float32)
    W[5] = 0
    s = torch.empty(37, device=DEV)
    mse = torch.empty((37, 32), device=DEV)
    Q.quip_scales(dev(W), Q.quantizer(Q.Q_UNIFORM, bits), s, mse_out=mse)
    s_ref, c_ref, mse_ref = O.uniform_scale_search(W, L)
    sg, mg = host(s).astype(np.float64), host(mse).astype(np.float64)
    assert sg[5] == 1.0
    assert np.allclose(mg, mse_ref, rtol=2e-5, atol=1e-30)
    live = np.arange(37) != 5
    cand = O.uniform_scale_candidates(np.abs(W).max(axis=1), L)  # (37, 32)
    cg = np.argmin(np.abs(cand - sg[:, None]), axis=1)
    rows = np.nonzero(live)[0]
    assert np.allclose(sg[rows], cand[rows, cg[rows]], rtol=1e-6)
    best = mse_ref[rows, c_ref[rows]]
    # the GPU's pick is the oracle's argmin, or ties with it to 1e-5
    assert np.all(mse_ref[rows, cg[rows]] <= best * (1 + 1e-5))


# ------------------------------------------------------------------ LDLQ

def ldlq_gpu(Wt32, U32, D32, g, B, bits, scales=None, codebook=None, kind=None):
    m, n = Wt32.shape
    kind = (Q.Q_UNIFORM if g == 1 else Q.Q_E8) if kind is None else kind
    mode = Q.SCALE_GIVEN if scales is not None else Q.SCALE_COMPUTE
    q = Q.quantizer(kind, bits if kind == Q.Q_UNIFORM else 2, 32, mode)
    sd = dev(scales) if scales is not None else torch.empty(m + (1 if kind == Q.Q_E8 else 0), device=DEV)
    if kind == Q.Q_UNIFORM:
        codes = torch.empty((m, n), dtype=torch.uint8, device=DEV)
    else:
        codes = torch.empty((m, n // 8), dtype=torch.int16, device=DEV)
    What = torch.empty((m, n), device=DEV)
    Q.quip_ldlq(dev(Wt32), dev(U32), dev(D32), g, B, q, sd, codes, What,
                None if codebook is None else dev(codebook))
    return host(sd), host(codes), host(What)


def ldlq_gpu_loss(Wt32, U32, D32, g, B, bits, codebook=None):
    """LDLQ with the fused proxy-loss outputs: (What, row_loss, loss)."""
    m, n = Wt32.shape
    kind = Q.Q_UNIFORM if g == 1 else Q.Q_E8
    q = Q.quantizer(kind, bits if kind == Q.Q_UNIFORM else 2, 32, Q.SCALE_COMPUTE)
    sd = torch.empty(m + (1 if kind == Q.Q_E8 else 0), device=DEV)
    codes = torch.empty((m, n) if g == 1 else (m, n // 8), dtype=torch.uint8 if g == 1 else torch.int16,
                        device=DEV)
    What = torch.empty((m, n), device=DEV)
    rl = torch.full((m,), -1.0, dtype=torch.float64, device=DEV)
    tot = torch.full((1,), -1.0, dtype=torch.float64, device=DEV)
    Q.quip_ldlq(dev(Wt32), dev(U32), dev(D32), g, B, q, sd, codes, What,
                None if codebook is None else dev(codebook), row_loss=rl, loss=tot)
    return host(What), host(rl), float(host(tot)[0])


# The fused loss sums D_K |P_K - W^_K|^2 with the GPU's float32 factors and
# targets; the oracle evaluates tr(E H E^T) in float64 on the same W^ and the
# float32 H. They differ by the LDL's backward error (a few 1e-7 relative to
# H's entries) and the float32 feedback sums, i.e. ~1e-6 of the loss; 2e-5
# per row and 1e-5 in total leave an order of magnitude.
FUSED_LOSS_RTOL_ROW = 2e-5
FUSED_LOSS_RTOL = 1e-5


def check_fused_loss(Wt, What, H, row_loss, loss):
    E = What.astype(np.float64) - Wt.astype(np.float64)
    want = np.einsum("ij,ij->i", E @ H.astype(np.float64), E)
    assert np.all(row_loss >= 0)
    assert np.allclose(row_loss, want, rtol=FUSED_LOSS_RTOL_ROW, atol=1e-12 * want.max())
    assert abs(loss - want.sum()) <= FUSED_LOSS_RTOL * want.sum()
    assert abs(loss - row_loss.sum()) <= 1e-12 * loss


@pytest.mark.parametrize("m,n,B,bits", [(256, 256, 32, 2), (37, 200, 64, 3), (300, 384, 128, 4),
                                        (1, 8, 8, 2), (70, 1100, 256, 2), (4112, 520, 128, 2)])
def test_ldlq_fused_loss(m, n, B, bits):
    H = spd32(m + 3 * n, n)
    Wt = (rng(m + n).standard_normal((m, n)) * 0.7).astype(np.float32)
    U, D, info = ldl_gpu(H, 1)
    assert info == 0
    What, rl, loss = ldlq_gpu_loss(Wt, U, D, 1, B, bits)
    check_fused_loss(Wt, What, H, rl, loss)


def test_ldlq_fused_loss_diagonal_H():
    # H diagonal: U = 0, P = W, the loss is sum_j d_j (w_j - q_j)^2; the kernel
    # forms w_j - q_j in float32 (one rounding, relative 2^-24), squares and
    # weights it in float64, so each term is within 2^-23 relative
    m, n = 40, 96
    Wt = rng(31).standard_normal((m, n)).astype(np.float32)
    d = rng(32).uniform(0.5, 2.0, n).astype(np.float32)
    U, D, _ = ldl_gpu(np.diag(d), 1)
    What, rl, loss = ldlq_gpu_loss(Wt, U, D, 1, 32, 2)
    E = What.astype(np.float64) - Wt.astype(np.float64)
    want = (E * E * d.astype(np.float64)[None, :]).sum(axis=1)
    assert np.allclose(rl, want, rtol=2.0 ** -23)


def check_uniform_replay(Wt, U, What, s, codes, L):
    mism, bad, tot = P.replay_uniform(Wt, U, What, s, codes, L)
    assert bad == 0, f"{bad} codes differ outside the boundary band"
    assert mism <= P.MAX_MISMATCH * tot
    lv = ((codes.astype(np.float32) - np.float32((L - 1) / 2)) * s.astype(np.float32)[:, None])
    assert np.array_equal(What, lv)


# more rows than one sweep work-group per CU (16 x 256) take the path with a
# product after each sub-block, and B = 128 is then swept 256 columns at a
# time; fewer take the batch's earlier feedback inside the sweep. Above
# n = 4096 the batches are 1024 columns wide.
@pytest.mark.parametrize("m,n,B,bits", [(256, 256, 32, 2), (37, 200, 64, 3), (100, 512, 256, 4),
                                        (16, 48, 32, 2), (1, 8, 8, 2), (300, 384, 128, 2),
                                        (4112, 520, 128, 3), (4200, 300, 32, 2),
                                        (4097, 1100, 256, 4), (64, 4500, 128, 2),
                                        (4112, 4200, 64, 3)])
def test_ldlq_replay(m, n, B, bits):
    L = 1 << bits
    H = spd32(m + n, n)
    Wt = (rng(m * n).standard_normal((m, n)) * 1.3).astype(np.float32)
    U, D, info = ldl_gpu(H, 1)
    assert info == 0
    s, codes, What = ldlq_gpu(Wt, U, D, 1, B, bits)
    s_ref, _, _ = O.uniform_scale_search(Wt, L)
    assert np.allclose(s, s_ref, rtol=1e-5)
    check_uniform_replay(Wt, U, What, s, codes, L)


def test_ldlq_diagonal_H_is_nearest_rounding():
    m, n = 64, 256
    Wt = rng(21).standard_normal((m, n)).astype(np.float32)
    d = rng(22).uniform(0.5, 2.0, n).astype(np.float32)
    U, D, _ = ldl_gpu(np.diag(d), 1)
    assert np.all(U == 0)
    s, codes, What = ldlq_gpu(Wt, U, D, 1, 64, 2)
    assert np.array_equal(codes.astype(np.int64), O.uniform_code(Wt, s[:, None], 4))


def test_ldlq_given_scales_are_used():
    m, n = 32, 128
    Wt = rng(23).standard_normal((m, n)).astype(np.float32)
    H = spd32(24, n)
    U, D, _ = ldl_gpu(H, 1)
    given = np.full(m, 0.7, np.float32)
    s, codes, What = ldlq_gpu(Wt, U, D, 1, 64, 2, scales=given)
    assert np.array_equal(s, given)
    check_uniform_replay(Wt, U, What, s, codes, 4)


# ------------------------------------------------------------------ loss

@pytest.mark.parametrize("m,n", [(256, 256), (37, 200), (5, 1000)])
def test_proxy_loss_parity(m, n):
    r = rng(m + 3 * n)
    W = r.standard_normal((m, n)).astype(np.float32)
    Wh = (W + 0.1 * r.standard_normal((m, n))).astype(np.float32)
    H = spd32(m, n)
    loss = torch.empty(1, dtype=torch.float64, device=DEV)
    Q.quip_proxy_loss(dev(W), dev(Wh), dev(H), loss)
    ref = O.proxy_loss(W, Wh, H)
    assert abs(float(host(loss)[0]) - ref) <= 1e-4 * abs(ref)


# ------------------------------------------------------------------ E8 / BlockLDLQ

@pytest.fixture(scope="module")
def codebook():
    return O.e8_codebook().astype(np.float32)


def test_e8_scale_search_parity(codebook):
    m, n = 64, 128
    W = rng(31).standard_normal((m, n)).astype(np.float32)
    scales = torch.empty(m + 1, device=DEV)
    sse = torch.empty(32, dtype=torch.float64, device=DEV)
    Q.quip_scales(dev(W), Q.quantizer(Q.Q_E8, 2), scales, mse_out=sse, codebook=dev(codebook))
    sg, eg = host(scales), host(sse)
    rms = O.row_rms(W)
    assert np.allclose(sg[1:], rms, rtol=1e-6)
    Wn = (W / sg[1:, None].astype(np.float64))
    s_ref, c_ref, sse_ref = O.e8_scale_search(Wn, codebook)
    assert np.allclose(eg, sse_ref, rtol=1e-4)
    cg = int(np.argmin(np.abs(O.e8_scale_candidates() - sg[0])))
    assert sse_ref[cg] <= sse_ref[c_ref] * (1 + 1e-5)


# 16448 rows: two work-groups per 32-row block, so every step launches its own
# pre-rounding kernel (the smaller sizes form the next step's vectors in the
# finishing work-group)
@pytest.mark.parametrize("m,n,B", [(64, 128, 64), (40, 64, 32), (33, 256, 128), (16448, 64, 32)])
def test_block_ldlq_e8_replay(m, n, B, codebook):
    H = spd32(m + n + 1, n)
    Wt = (rng(n).standard_normal((m, n)) * np.exp(0.3 * rng(m).standard_normal(m))[:, None]).astype(np.float32)
    U, D, info = ldl_gpu(H, 8)
    assert info == 0
    s, codes, What = ldlq_gpu(Wt, U, D, 8, B, 2, codebook=codebook)
    rms = s[1:].astype(np.float64)
    assert np.allclose(rms, O.row_rms(Wt), rtol=1e-6)
    Wn = Wt / rms[:, None]
    Whn = What / rms[:, None]
    mism, bad, tot = P.replay_e8(Wn, U, Whn, float(s[0]), codes, codebook)
    assert bad == 0
    assert mism <= max(1, P.MAX_MISMATCH * tot)
    # W^ is the scaled codeword times the row RMS
    cw = codebook[codes.astype(np.int64).reshape(m, -1) & 0xFFFF].reshape(m, n)
    assert np.allclose(What, rms[:, None] * float(s[0]) * cw, rtol=1e-6, atol=1e-7)


def test_e8_search_any_codebook_order(codebook):
    """A codebook without the shells' negation pairing (a random row order)
    takes the plain search over all 65536 codewords: the scale table and the
    replayed codes against the oracle on that same codebook."""
    perm = rng(77).permutation(65536)
    cb = np.ascontiguousarray(codebook[perm])
    m, n = 64, 128
    W = rng(31).standard_normal((m, n)).astype(np.float32)
    scales = torch.empty(m + 1, device=DEV)
    sse = torch.empty(32, dtype=torch.float64, device=DEV)
    Q.quip_scales(dev(W), Q.quantizer(Q.Q_E8, 2), scales, mse_out=sse, codebook=dev(cb))
    sg, eg = host(scales), host(sse)
    Wn = (W / sg[1:, None].astype(np.float64))
    _, _, sse_ref = O.e8_scale_search(Wn, cb)
    assert np.allclose(eg, sse_ref, rtol=1e-4)
    H = spd32(m + n + 1, n)
    U, D, info = ldl_gpu(H, 8)
    assert info == 0
    s, codes, What = ldlq_gpu(W, U, D, 8, 64, 2, codebook=cb)
    rms = s[1:].astype(np.float64)
    mism, bad, tot = P.replay_e8(W / rms[:, None], U, What / rms[:, None], float(s[0]), codes, cb)
    assert bad == 0
    assert mism <= max(1, P.MAX_MISMATCH * tot)


@pytest.mark.parametrize("m,n,B", [(64, 128, 64), (33, 256, 128)])
def test_block_ldlq_e8_fused_loss(m, n, B, codebook):
    H = spd32(m + n + 5, n)
    Wt = (rng(n + 1).standard_normal((m, n)) * np.exp(0.3 * rng(m + 1).standard_normal(m))[:, None]).astype(np.float32)
    U, D, info = ldl_gpu(H, 8)
    assert info == 0
    What, rl, loss = ldlq_gpu_loss(Wt, U, D, 8, B, 2, codebook=codebook)
    check_fused_loss(Wt, What, H, rl, loss)


# ------------------------------------------------------------------ end to end

PASS_KEYS = ("Wt", "H", "U", "D", "scales", "codes", "What_t")


def gpu_pass(b):
    """The LayerPass outputs the independent-run comparison reads, on the host."""
    return {k: host(b[k]) for k in PASS_KEYS}


def check_independent_run(b, ref, g=1, L=None, C=None):
    """The GPU pass against the oracle's own pass (tests/parity.py gives the
    rule: 1e-4 on agreeing rows and on the total when no row diverges; a
    diverged row must start at an explained near-tie and is bounded by its
    larger tail)."""
    st = P.compare_independent_run(gpu_pass(b), ref, g=g, L=L, C=C)
    print(f"independent run: {st['diverged']} of {st['rows']} rows diverged; loss "
          f"{st['loss_gpu']:.8g} vs {st['loss_oracle']:.8g} (extra bound {st['extra_bound']:.3g})")
    return st

def test_layer_pass_end_to_end_c1():
    L = wl.make_layer("c1")
    W, X = dev(L.W), dev(L.X)
    lp = Q.LayerPass(256, 256, Q.SideSpec.from_numpy(L.left, DEV), Q.SideSpec.from_numpy(L.right, DEV),
                     bits=2, B=32)
    b = lp.run(W, X)
    ref = O.quantize_layer(L.W, L.X, L.left, L.right, quant="uniform", bits=2)
    H = host(b["H"])
    d = np.sqrt(np.diag(ref["Ht"]))
    assert np.abs(H - ref["Ht"]).max() <= 1e-5 * d.max() ** 2
    assert P.rel_rows(host(b["Wt"]), ref["Wt"]) <= 1e-5
    assert int(host(b["info"])[0]) == 0
    # conditional replay on the GPU's own factors and decisions
    check_uniform_replay(host(b["Wt"]), host(b["U"]), host(b["What_t"]), host(b["scales"]),
                         host(b["codes"]), 4)
    # independent end-to-end run (float64 factors of its own): rows whose codes
    # agree everywhere must have the same loss; a row may diverge only after a
    # near-tie, after which LDLQ follows another (equally valid) path, so the
    # total is compared with a bound for a few diverged rows.
    loss = float(host(b["loss"])[0])
    check_fused_loss(host(b["Wt"]), host(b["What_t"]), host(b["H"]), host(b["row_loss"]), loss)
    check_independent_run(b, ref, g=1, L=4)
    # post-processing inverts the incoherence transforms
    back = O.incoherence_W_inv(host(b["What_t"]), L.left, L.right)
    assert P.rel_rows(host(b["What"]), back) <= 1e-5


def e8_small_layer():
    """The 256 x 256 layer (random-sign Hadamard sides, N = 2048) quantized with
    the E8 codebook: BlockLDLQ, g = 8, B = 32."""
    L = wl.make_layer("c1")
    lp = Q.LayerPass(256, 256, Q.SideSpec.from_numpy(L.left, DEV), Q.SideSpec.from_numpy(L.right, DEV),
                     quant="e8", bits=2, g=8, B=32)
    return L, lp


def test_layer_pass_e8_end_to_end_small(codebook):
    L, lp = e8_small_layer()
    b = lp.run(dev(L.W), dev(L.X))
    assert int(host(b["info"])[0]) == 0
    C = codebook.astype(np.float64)
    ref = O.quantize_layer(L.W, L.X, L.left, L.right, quant="e8", g=8, codebook=C)
    H = host(b["H"])
    d = np.sqrt(np.diag(ref["Ht"]))
    assert np.abs(H - ref["Ht"]).max() <= 1e-5 * d.max() ** 2
    Wt = host(b["Wt"])
    assert P.rel_rows(Wt, ref["Wt"]) <= 1e-5
    sc = host(b["scales"])
    rms = sc[1:].astype(np.float64)
    assert np.allclose(rms, O.row_rms(Wt), rtol=1e-6)
    # the global scale is the oracle's argmin on the GPU's own normalized W~
    cands = O.e8_scale_candidates()
    choice = int(np.argmin(np.abs(cands - sc[0])))
    assert abs(cands[choice] - sc[0]) <= 1e-6 * sc[0]
    Wn = Wt / rms[:, None]
    ok, info = P.e8_scale_is_argmin(Wn, C, choice)
    assert ok, info
    # conditional replay of BlockLDLQ on the GPU's own factors and decisions
    Whn = host(b["What_t"]) / rms[:, None]
    mism, bad, tot = P.replay_e8(Wn, host(b["U"]), Whn, float(sc[0]), host(b["codes"]), C)
    assert bad == 0 and mism <= max(1, P.MAX_MISMATCH * tot)
    loss = float(host(b["loss"])[0])
    check_fused_loss(Wt, host(b["What_t"]), H, host(b["row_loss"]), loss)
    # the oracle's own E8 pass
    check_independent_run(b, ref, g=8, C=C)
    back = O.incoherence_W_inv(host(b["What_t"]), L.left, L.right)
    assert P.rel_rows(host(b["What"]), back) <= 1e-5


def test_e8_layer_pass_is_deterministic():
    # the E8 scale search adds per-work-group partial sums in a fixed order
    # (no floating-point atomics): two passes agree bit for bit
    L, _ = e8_small_layer()
    W, X = dev(L.W), dev(L.X)
    outs = []
    for _ in range(2):
        _, lp = e8_small_layer()
        b = lp.run(W, X)
        sse = torch.empty(32, dtype=torch.float64, device=DEV)
        sc = torch.empty(257, device=DEV)
        Q.quip_scales(b["Wt"], lp.q, sc, mse_out=sse, codebook=lp.codebook)
        outs.append({k: host(b[k]).copy() for k in ("H", "Wt", "U", "D", "scales", "codes", "What_t",
                                                     "What", "row_loss", "loss")})
        outs[-1]["sse"] = host(sse).copy()
    for k in outs[0]:
        assert np.array_equal(outs[0][k], outs[1][k]), k


def _golden(name):
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", name)) as f:
        return json.load(f)


def test_e8_gaussian_source_mse(codebook):
    # The E8 codebook at 2 bits per weight on an i.i.d. N(0,1) source, through
    # the GPU search (the scale search of the E8 configuration). Per-candidate
    # squared errors match the oracle on a small sample; on a large sample the
    # best mean squared error lies between the Gaussian distortion-rate bound
    # 2^-4 (the QTIP page prints 0.063) and the best 2-bit scalar grid (Max
    # 1960), and agrees with the oracle's estimate within sampling error.
    gd = _golden("qtip_gaussian_2bit_mse.json")
    scalar = _golden("max1960_uniform_gaussian.json")["levels"]["4"]["mse"]
    q = Q.quantizer(Q.Q_E8, 2)

    def gpu_sse(W):
        m = W.shape[0]
        scales = torch.empty(m + 1, device=DEV)
        sse = torch.empty(32, dtype=torch.float64, device=DEV)
        Q.quip_scales(dev(W), q, scales, mse_out=sse, codebook=dev(codebook))
        return host(scales), host(sse)

    small = wl.gaussian_rows(11, 64, 256)  # 2048 8-vectors
    sg, eg = gpu_sse(small)
    Wn = small / sg[1:, None].astype(np.float64)
    _, c_ref, sse_ref = O.e8_scale_search(Wn, codebook)
    assert np.allclose(eg, sse_ref, rtol=1e-4)
    mse_oracle = sse_ref[c_ref] / small.size

    large = wl.gaussian_rows(12, 1024, 1024)  # 131072 8-vectors
    _, el = gpu_sse(large)
    mse = el.min() / large.size
    assert 2.0 ** -4 <= mse < scalar
    assert abs(mse - mse_oracle) <= 0.005
    assert 0 < int(np.argmin(el)) < 31


# ------------------------------------------------------------------ inference product

@pytest.mark.parametrize("m,n,bits", [(3, 5, 2), (7, 37, 3), (16, 1024, 2), (5, 33, 1), (9, 19, 4),
                                      (4, 7, 8)])
def test_pack_codes_bit_exact(m, n, bits):
    codes = rng(m * n + bits).integers(0, 1 << bits, size=(m, n)).astype(np.uint8)
    rb = Q.quip_packed_row_bytes(n, bits)
    packed = torch.zeros((m, rb), dtype=torch.uint8, device=DEV)
    Q.quip_pack_codes(torch.from_numpy(codes).to(DEV), bits, packed)
    assert np.array_equal(host(packed), O.pack_codes(codes, bits))


def qmatvec_gpu(codes, scales, bits, sl, sr, x):
    m, n = codes.shape
    packed = torch.empty((m, Q.quip_packed_row_bytes(n, bits)), dtype=torch.uint8, device=DEV)
    Q.quip_pack_codes(torch.from_numpy(codes).to(DEV), bits, packed)
    y = torch.empty(m, device=DEV)
    Q.quip_qmatvec_rht(packed, n, bits, dev(scales), dev(sl), dev(sr), dev(x), y)
    return host(y).astype(np.float64)


@pytest.mark.parametrize("m,n,bits", [(256, 1024, 2), (1024, 4096, 2), (64, 2048, 3), (128, 8192, 4),
                                      (32, 16384, 2), (2, 1024, 8), (4096, 1024, 3), (16, 2048, 1),
                                      (64, 4096, 5), (8, 1024, 6), (512, 2048, 7), (16384, 1024, 4)])
def test_qmatvec_rht_parity(m, n, bits):
    r = rng(m + 3 * n + bits)
    L = 1 << bits
    codes = r.integers(0, L, size=(m, n)).astype(np.uint8)
    scales = np.exp(0.5 * r.standard_normal(m)).astype(np.float32)
    sl = r.choice([-1.0, 1.0], m).astype(np.float32)
    sr = r.choice([-1.0, 1.0], n).astype(np.float32)
    x = r.standard_normal(n).astype(np.float32)
    y = qmatvec_gpu(codes, scales, bits, sl, sr, x)
    ref = O.qmatvec_rht(codes, scales, L, sl, sr, x)
    # float32 sums of n terms: bounded by the product of absolute values
    xp = O.rht(x.astype(np.float64)[None, :], sr, "right")[0]
    absprod = np.abs(O.uniform_level(codes, scales[:, None], L)) @ np.abs(xp)
    assert np.linalg.norm(y - ref) <= 1e-5 * np.linalg.norm(ref)
    assert np.linalg.norm(y - ref) <= 2e-6 * np.sqrt(n) * np.linalg.norm(absprod)


def test_qmatvec_rht_rejects_unsupported_shapes():
    z = torch.zeros(1024, device=DEV)
    packed = torch.zeros((6, 256), dtype=torch.uint8, device=DEV)
    with pytest.raises(Q.QuipError, match="QUIP_ERR_SHAPE"):  # m = 6 is not a power of two
        Q.quip_qmatvec_rht(packed, 1024, 2, torch.ones(6, device=DEV), torch.ones(8, device=DEV),
                           z, z, torch.empty(6, device=DEV))


# ------------------------------------------------------------------ QuIP variants: permutations

@pytest.mark.parametrize("rows,cols,lda,ldo,use_r,use_c", [
    (7, 13, 13, 13, True, True),        # scalar path, ragged
    (64, 256, 256, 256, True, True),    # float4 path
    (33, 4100, 4104, 4100, True, True),  # padded leading dimension
    (5, 11, 16, 12, False, True),       # columns only, scalar path
    (100, 64, 64, 64, True, False),     # rows only
    (2, 32768, 32768, 32768, True, True),  # longest staged row
    (1, 1, 1, 1, True, True),
])
def test_permute_bit_exact(rows, cols, lda, ldo, use_r, use_c):
    r = rng(rows * 7 + cols)
    A = r.standard_normal((rows, lda)).astype(np.float32)
    pr = r.permutation(rows).astype(np.int32) if use_r else None
    pc = r.permutation(cols).astype(np.int32) if use_c else None
    Ad = dev(A)[:, :cols] if lda > cols else dev(A)
    for scatter in (False, True):
        out = torch.full((rows, ldo), -7.0, device=DEV)
        o = out[:, :cols] if ldo > cols else out
        Q.quip_permute(Ad, o, None if pr is None else dev(pr, torch.int32),
                       None if pc is None else dev(pc, torch.int32), scatter=scatter)
        f = O.permute_scatter if scatter else O.permute_gather
        want = f(A[:, :cols], pr, pc)
        got = host(out)
        assert np.array_equal(got[:, :cols], want)
        assert np.all(got[:, cols:] == -7.0)  # nothing written past the row


def test_permute_gather_out_of_range_index_gives_nan():
    A = np.arange(12, dtype=np.float32).reshape(3, 4)
    pc = np.array([3, 9, 0, -1], dtype=np.int32)
    pr = np.array([2, 0, 5], dtype=np.int32)
    out = torch.empty((3, 4), device=DEV)
    Q.quip_permute(dev(A), out, dev(pr, torch.int32), dev(pc, torch.int32))
    got = host(out)
    assert np.array_equal(got[0], [11.0, np.nan, 8.0, np.nan], equal_nan=True)
    assert np.array_equal(got[1], [3.0, np.nan, 0.0, np.nan], equal_nan=True)
    assert np.all(np.isnan(got[2]))


def test_permute_rejects_overlap_and_long_staged_rows():
    A = torch.zeros((4, 8), device=DEV)
    with pytest.raises(Q.QuipError):
        Q.quip_permute(A, A, None, dev(np.arange(8, dtype=np.int32), torch.int32))
    big = torch.zeros((1, 32769), device=DEV)
    with pytest.raises(Q.QuipError):
        Q.quip_permute(big, torch.zeros_like(big), None,
                       dev(np.arange(32769, dtype=np.int32), torch.int32))


@pytest.mark.parametrize("n", [1, 5, 511, 512, 513, 4099, 11008])
def test_diag_order_bit_exact(n):
    r = rng(n)
    # integer-valued diagonal: many exact ties; plus a few signed zeros
    d = r.integers(0, max(2, n // 8), n).astype(np.float32)
    if n > 4:
        d[1], d[3] = 0.0, -0.0
    H = np.zeros((n, n + 3), dtype=np.float32)
    H[np.arange(n), np.arange(n)] = d
    Hd = dev(H)[:, :n]
    order = torch.empty(n, dtype=torch.int32, device=DEV)
    Q.quip_diag_order(Hd, order)
    assert np.array_equal(host(order), O.diag_order(H[:, :n]))
    # distinct random values
    H2 = np.diag(r.standard_normal(n).astype(np.float32)) + 1.0
    Q.quip_diag_order(dev(H2), order)
    assert np.array_equal(host(order), O.diag_order(H2))


def test_layer_pass_with_permutations_and_rg_order():
    cfg = wl.custom_config("perm-rg", 902, 64, 96, 512, left=wl.Side("rht", perm=True),
                           right=wl.KRON(8, 12, perm=True), bits=2, B=32, rg_order=True)
    L = wl.make_layer(cfg)
    W, X = dev(L.W), dev(L.X)
    lp = Q.LayerPass(cfg.m, cfg.n, Q.SideSpec.from_numpy(L.left, DEV),
                     Q.SideSpec.from_numpy(L.right, DEV), bits=2, B=32, rg_order=True)
    b = lp.run(W, X)
    assert int(host(b["info"])[0]) == 0
    order = host(b["order"]).astype(np.int64)
    H = host(b["H"])
    # the GPU's order is the diag order of its own transformed H (bit-exact)
    H0 = O.permute_scatter(H, order, order)
    assert np.array_equal(order, O.diag_order(H0))
    # H~ and W~ against the oracle's transforms (permutation inside), in the GPU's order
    ref = O.quantize_layer(L.W, L.X, L.left, L.right, quant="uniform", bits=2, rg_order=True)
    Ht_ref = O.permute_gather(O.incoherence_H(ref["H"], L.right), order, order)
    d = np.sqrt(np.diag(Ht_ref))
    assert np.abs(H - Ht_ref).max() <= 1e-5 * d.max() ** 2
    Wt_ref = O.permute_gather(O.incoherence_W(L.W, L.left, L.right), cols=order)
    assert P.rel_rows(host(b["Wt"]), Wt_ref) <= 1e-5
    # the oracle's own order agrees except between near-equal diagonal entries
    dref = np.diag(O.incoherence_H(ref["H"], L.right))
    diff = ref["order"] != order
    assert np.all(np.abs(dref[ref["order"][diff]] - dref[order[diff]]) <= 1e-5 * dref.max())
    check_uniform_replay(host(b["Wt"]), host(b["U"]), host(b["What_t"]), host(b["scales"]),
                         host(b["codes"]), 4)
    loss = float(host(b["loss"])[0])
    check_fused_loss(host(b["Wt"]), host(b["What_t"]), H, host(b["row_loss"]), loss)
    if not diff.any():  # the same order: the same problem, so compare the runs
        check_independent_run(b, ref, g=1, L=4)
    # post-processing: columns back to the transform's order, inverse transforms
    # (permutations inside)
    back = O.incoherence_W_inv(O.permute_scatter(host(b["What_t"]), cols=order), L.left, L.right)
    assert P.rel_rows(host(b["What"]), back) <= 1e-5


# ------------------------------------------------------------------ trellis-coded quantization

def tcq_gpu(X, L, scale=1.0, ldx=None, with_xhat=True):
    rows, T = X.shape
    ldx = T if ldx is None else ldx
    Xp = np.zeros((rows, ldx), np.float32)
    Xp[:, :T] = X
    Xd = dev(Xp)[:, :T] if ldx > T else dev(Xp)
    st = torch.empty((rows, T), dtype=torch.int16, device=DEV)
    xh = torch.empty((rows, T), device=DEV) if with_xhat else None
    cost = torch.empty(rows, device=DEV)
    Q.quip_tcq_quantize(Xd, L, st, cost, Xhat=xh, scale=scale)
    s = host(st).astype(np.int64) & 0xFFFF
    return s, (host(xh) if with_xhat else None), host(cost)


def check_tcq_rows(X, L, s, xh, cost, scale=1.0, oracle_rows=None):
    """Every row: a valid path, values c(states) bit-exact, the reported float32
    minimum equal to the path's cost up to float32 summation, and the path
    optimal up to that rounding (the oracle's float64 Viterbi)."""
    rows, T = X.shape
    for r in range(rows):
        assert O.tcq_path_is_valid(s[r], L, 2), r
        if xh is not None:
            assert np.array_equal(xh[r], O.tcq_code(s[r], scale)), r
        pc = O.tcq_path_cost(X[r], s[r], scale)
        tol = 4e-7 * T * max(pc, 1e-3)  # float32 sums of T terms
        assert abs(float(cost[r]) - pc) <= tol, (r, float(cost[r]), pc)
        if oracle_rows is None or r in oracle_rows:
            _, best = O.tcq_viterbi(X[r], L, 2, scale)
            assert best - 1e-12 <= pc <= best + tol, (r, pc, best)


@pytest.mark.parametrize("L,T,rows,ldx", [(4, 5, 3, 5), (8, 64, 17, 70), (12, 256, 24, 256),
                                          (15, 256, 6, 260), (10, 1000, 5, 1000), (13, 1, 9, 4)])
def test_tcq_parity(L, T, rows, ldx):
    X = wl.gaussian_rows(100 + L, rows, T)
    s, xh, cost = tcq_gpu(X, L, ldx=ldx)
    check_tcq_rows(X, L, s, xh, cost)


def test_tcq_scale_and_chunks():
    # more rows than one round of back-pointers (2048), and a scale
    X = wl.gaussian_rows(111, 4100, 6) * np.float32(0.4)
    s, xh, cost = tcq_gpu(X, 6, scale=0.37)
    check_tcq_rows(X, 6, s, xh, cost, scale=0.37, oracle_rows=set(range(0, 4100, 97)))


def test_tcq_without_values_and_rejections():
    X = wl.gaussian_rows(112, 4, 32)
    s, _, cost = tcq_gpu(X, 9, with_xhat=False)
    check_tcq_rows(X, 9, s, None, cost)
    st = torch.empty((4, 32), dtype=torch.int16, device=DEV)
    c = torch.empty(4, device=DEV)
    for kw in ({"k": 3}, {"scale": 0.0}, {"scale": float("nan")}):
        with pytest.raises(Q.QuipError):
            Q.quip_tcq_quantize(dev(X), 9, st, c, **kw)
    with pytest.raises(Q.QuipError):
        Q.quip_tcq_quantize(dev(X), 16, st, c)


def test_layer_pass_is_deterministic():
    # the scalar-grid pass sums in fixed orders (no floating-point atomics):
    # two passes over the same inputs agree bit for bit, permutations included
    cfg = wl.custom_config("det", 903, 128, 96, 512, left=wl.RHT, right=wl.KRON(8, 12, perm=True),
                           bits=3, B=32, rg_order=True)
    L = wl.make_layer(cfg)
    W, X = dev(L.W), dev(L.X)
    outs = []
    for _ in range(2):
        lp = Q.LayerPass(cfg.m, cfg.n, Q.SideSpec.from_numpy(L.left, DEV),
                         Q.SideSpec.from_numpy(L.right, DEV), bits=3, B=32, rg_order=True)
        b = lp.run(W, X)
        outs.append({k: host(b[k]).copy() for k in ("H", "Wt", "U", "D", "scales", "codes", "What_t",
                                                     "What", "row_loss", "loss", "order")})
    for k in outs[0]:
        assert np.array_equal(outs[0][k], outs[1][k]), k


def test_peak_probes():
    # measurement aids: the copy probe copies (float4 body and scalar tail),
    # the compute probes run and count their flops as documented
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    rnd = 16 * cus * 256 * 4  # 16-byte chunks per round of the whole grid
    for count in (1, 7, 4096 + 3, 4 * (2 * rnd + 700) + 2):
        src = torch.arange(count, dtype=torch.float32, device=DEV) * 0.5 - 3.0
        dst = torch.full_like(src, float("nan"))
        Q.quip_peak_copy(src, dst)
        torch.cuda.synchronize()
        assert torch.equal(src, dst), count
    out = torch.zeros(1, device=DEV)
    waves = 4 * cus * 4
    assert Q.quip_peak_compute(0, 3, out) == waves * 3 * 4 * (32 * 32 * 2 * 2)
    assert Q.quip_peak_compute(1, 3, out) == waves * 3 * 4 * (32 * 32 * 16 * 2)
    assert Q.quip_peak_compute(2, 3, out) == waves * 64 * 3 * 8 * 2
    torch.cuda.synchronize()
