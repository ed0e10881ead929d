"""Comparison helpers for the GPU parity tests (test infrastructure: uses the
oracle; never imported by the library)."""
from __future__ import annotations

import numpy as np

import oracle as O

BAND = 1e-5  # pre-rounding value within 1e-5 relative of a decision boundary
MAX_MISMATCH = 1e-4  # fraction of codes allowed to differ, all inside the band


def rel_rows(got, ref):
    """Per-row normwise relative error max_r ||got_r - ref_r|| / ||ref_r||."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.linalg.norm(got - ref, axis=1)
    den = np.maximum(np.linalg.norm(ref, axis=1), 1e-300)
    return float((num / den).max())


def replay_uniform(Wt, U, What, scales, codes, L):
    """Conditional replay of scalar LDLQ: recompute every pre-rounding value in
    float64 from the GPU's own earlier decisions, decide in float32 like the
    kernel, and compare. Returns (n_mismatch, n_bad, n_total)."""
    P = O.ldlq_prerounding(Wt, U, What)
    s32 = np.asarray(scales, np.float32)[:, None]
    want = O.uniform_code(P, s32, L)
    codes = np.asarray(codes).astype(np.int64)
    mism = codes != want
    if not mism.any():
        return 0, 0, codes.size
    s64 = s32.astype(np.float64)
    j = np.rint(P / s64 + L / 2.0)
    bnd = (j - L / 2.0) * s64
    in_band = np.abs(P - bnd) <= BAND * np.maximum(np.abs(bnd), s64)
    adjacent = np.abs(codes - want) == 1
    bad = mism & ~(in_band & adjacent)
    return int(mism.sum()), int(bad.sum()), codes.size


def replay_e8(Wn, U, Whn, s, codes, C):
    """Conditional replay of BlockLDLQ with the E8 codebook (rows already
    normalized). A code may differ from the exact nearest codeword only when its
    distance is within the band of the best one."""
    P = O.ldlq_prerounding(Wn, U, Whn)
    m, n = P.shape
    Y = P.reshape(-1, 8)
    best, dbest = O.e8_nearest(Y, C, s)
    codes = np.asarray(codes).astype(np.int64).reshape(-1) & 0xFFFF
    mism = codes != best
    if not mism.any():
        return 0, 0, codes.size
    Cq = np.asarray(C, np.float64)
    dg = ((Y[mism] - s * Cq[codes[mism]]) ** 2).sum(axis=1)
    db = dbest[mism]
    tol = BAND * s * s * (((Y[mism] / s) ** 2).sum(axis=1) + (Cq[best[mism]] ** 2).sum(axis=1))
    bad = (dg - db) > tol
    return int(mism.sum()), int(bad.sum()), codes.size


def recon_residual(H, U, D, g=1):
    """||(I+U) D (I+U)^T - H||_F / ||H||_F in float64."""
    U = np.asarray(U, np.float64)
    n = U.shape[0]
    I = np.eye(n)
    if g == 1:
        Dm = np.diag(np.asarray(D, np.float64))
    else:
        Dm = O.block_diag_D(np.asarray(D, np.float64).reshape(n // g, g, g))
    R = (I + U) @ Dm @ (I + U).T - np.asarray(H, np.float64)
    return float(np.linalg.norm(R) / np.linalg.norm(H))


# ------------------------------------------------------------------ E8 global scale

def e8_scale_is_argmin(Wn, C, choice, ncand=32, tol=1e-5, index=None):
    """Whether candidate ``choice`` of the E8 global scale is the argmin (to a
    relative ``tol``) of the exact nearest-codeword squared error over all
    8-vectors of the row-normalized weights ``Wn``, the oracle's
    ``e8_scale_search`` rule. Exact errors are computed for the claimed
    candidate and for every candidate a lower bound cannot rule out; the bound
    per vector y at scale s is max(dist(y, s E8)^2, s^2 max(0, |y/s| - R)^2):
    the codebook is a subset of the lattice and of the ball of radius R (its
    largest norm). Returns (ok, info) with info[c] = ("exact" | "bound", value)."""
    Y = np.asarray(Wn, np.float64).reshape(-1, 8)
    C = np.asarray(C, np.float64)
    index = O.E8Index(C) if index is None else index
    cand = O.e8_scale_candidates(ncand)
    R = float(np.sqrt((C * C).sum(axis=1).max()))
    ynorm = np.sqrt((Y * Y).sum(axis=1))
    info = {}
    best = float(O.e8_nearest(Y, C, cand[choice], index)[1].sum())
    info[choice] = ("exact", best)
    ok = True
    for c in range(ncand):
        if c == choice:
            continue
        s = cand[c]
        rad = (s * np.maximum(ynorm / s - R, 0.0)) ** 2
        lb = float(rad.sum())
        if lb < best * (1 - tol):
            Z = O.e8_decode(Y / s)
            lb = float(np.maximum(((Y - s * Z) ** 2).sum(axis=1), rad).sum())
        if lb >= best * (1 - tol):
            info[c] = ("bound", lb)
            continue
        v = float(O.e8_nearest(Y, C, s, index)[1].sum())
        info[c] = ("exact", v)
        if v < best * (1 - tol):
            ok = False
    return ok, info


# ------------------------------------------------------------------ independent end-to-end run

def _first_diff(a, b):
    """First column where rows of a and b differ (a.shape[1] where none)."""
    d = a != b
    k = np.argmax(d, axis=1)
    return np.where(d.any(axis=1), k, a.shape[1])


def compare_independent_run(gpu, ref, g=1, L=None, C=None, band=BAND, loss_tol=1e-4):
    """The GPU's pass against the oracle's own pass on the same inputs.

    Both runs follow LDLQ exactly, with their own factors (float32 on the GPU,
    float64 in the oracle), so a row's decisions may part at a column where the
    pre-rounding value lies next to a decision boundary; from there each run
    follows another valid path. The rule (derived, not tuned):

      * rows whose codes agree everywhere: loss within ``loss_tol`` relative;
      * a row that diverges first at column (group) k*: the two pre-rounding
        values at k* must lie within the first-order bound that the measured
        differences of W~, U and the scale allow, and that bound must place a
        decision boundary between them (an explained near-tie). Its loss up to
        k* agrees to ``loss_tol``; after k* both are non-negative tails
        sum_k eta_k D_k eta_k^T of valid runs, so the row's loss difference is
        at most the larger tail;
      * the total loss: |l_gpu - l_oracle| <= loss_tol l_oracle + sum over
        diverged rows of max(tail_gpu, tail_oracle). With no diverged row this
        is loss_tol on the total.

    gpu: dict with Wt, H, U, D, scales, codes, What_t (numpy, GPU outputs);
    ref: the dict of ``O.quantize_layer``. Scalar grid: g = 1 and L levels;
    E8: g = 8 and the codebook C. Returns a dict of counts and losses; raises
    AssertionError when the rule fails."""
    Wg = np.asarray(gpu["Wt"], np.float64)
    Ug = np.asarray(gpu["U"], np.float64)
    Hg = np.asarray(gpu["H"], np.float64)
    Wo, Uo, Ho = ref["Wt"], ref["U"], ref["Ht"]
    m, n = Wg.shape
    if g == 1:
        sg = np.asarray(gpu["scales"], np.float32).astype(np.float64)
        so = np.asarray(ref["scales"], np.float32).astype(np.float64)
        rg = np.ones(m)
        ro = np.ones(m)
        Dg = np.asarray(gpu["D"], np.float64)
        Do = np.asarray(ref["D"], np.float64)
    else:
        sc = np.asarray(gpu["scales"], np.float32).astype(np.float64)
        sg = np.full(m, sc[0])
        rg = sc[1:]
        so = np.full(m, float(np.float32(ref["scale"])))
        ro = np.asarray(ref["rms"], np.float64)
        Dg = np.asarray(gpu["D"], np.float64).reshape(n // 8, 8, 8)
        Do = np.asarray(ref["D"], np.float64)
    Whg = np.asarray(gpu["What_t"], np.float64)
    Who = ref["What_t"]
    cg = np.asarray(gpu["codes"]).astype(np.int64)
    co = np.asarray(ref["codes"]).astype(np.int64)
    if g == 8:
        cg &= 0xFFFF
    # each side's pre-rounding targets (normalized domain for E8)
    Pg = O.ldlq_prerounding(Wg / rg[:, None], Ug, Whg / rg[:, None])
    Po = O.ldlq_prerounding(Wo / ro[:, None], Uo, Who / ro[:, None])
    # per-column (group) loss terms: rms^2 eta_K D_K eta_K^T
    if g == 1:
        tg = (Pg - Whg) ** 2 * Dg[None, :]
        to = (Po - Who) ** 2 * Do[None, :]
    else:
        eg = (Pg - Whg / rg[:, None]).reshape(m, n // 8, 8)
        eo = (Po - Who / ro[:, None]).reshape(m, n // 8, 8)
        tg = np.einsum("rka,kab,rkb->rk", eg, Dg, eg) * (rg * rg)[:, None]
        to = np.einsum("rka,kab,rkb->rk", eo, Do, eo) * (ro * ro)[:, None]
    Eg = Whg - Wg
    Eo = Who - Wo
    lg = np.einsum("ij,ij->i", Eg @ Hg, Eg)
    lo = np.einsum("ij,ij->i", Eo @ Ho, Eo)
    # divergence: the scale (candidate) first, then the codes
    same_scale = np.abs(sg - so) <= 1e-6 * so
    kstar = _first_diff(cg, co)
    kstar = np.where(same_scale, kstar, 0)
    ncol = cg.shape[1]
    agree = kstar == ncol
    assert np.allclose(lg[agree], lo[agree], rtol=loss_tol, atol=0), \
        np.abs(lg[agree] / lo[agree] - 1).max()
    bound_extra = 0.0
    div = np.nonzero(~agree)[0]
    dW = np.abs(Wg / rg[:, None] - Wo / ro[:, None])
    dU = np.abs(Ug - Uo)
    for r in div:
        k = int(kstar[r])
        if same_scale[r]:
            lo_c, hi_c = k * g, (k + 1) * g
            # first-order bound on |P_gpu - P_oracle| at the diverging column
            # from the measured input differences (earlier decisions agree)
            e_g = (Wg[r, :lo_c] - Whg[r, :lo_c]) / rg[r]
            e_o = (Wo[r, :lo_c] - Who[r, :lo_c]) / ro[r]
            dp_bound = (dW[r, lo_c:hi_c] + np.abs(e_g - e_o) @ np.abs(Uo[:lo_c, lo_c:hi_c])
                        + np.abs(e_g) @ dU[:lo_c, lo_c:hi_c])
            dp = np.abs(Pg[r, lo_c:hi_c] - Po[r, lo_c:hi_c])
            assert np.all(dp <= dp_bound * (1 + 1e-6) + 1e-12), (r, k, dp, dp_bound)
            s = so[r]
            if g == 1:
                a, b = int(cg[r, k]), int(co[r, k])
                assert abs(a - b) == 1, (r, k, a, b)
                bnd = (min(a, b) + 1 - L / 2.0) * s  # the boundary between the two levels
                slack = dp_bound[0] + band * max(abs(bnd), s)
                assert abs(Pg[r, k] - bnd) <= slack and abs(Po[r, k] - bnd) <= slack, (r, k)
            else:
                ca, cb = C[cg[r, k]], C[co[r, k]]
                p = Po[r, lo_c:hi_c]
                gap = ((p - s * ca) ** 2).sum() - ((p - s * cb) ** 2).sum()
                # the gap is linear in p: it changes by at most 2 s |c_a - c_b| |dp|
                slack = 2 * s * np.linalg.norm(ca - cb) * np.linalg.norm(dp_bound) \
                    + band * s * s * (((p / s) ** 2).sum() + (cb ** 2).sum())
                assert -slack <= gap <= slack, (r, k, gap, slack)
        pre_g = tg[r, :k].sum()
        pre_o = to[r, :k].sum()
        assert abs(pre_g - pre_o) <= loss_tol * pre_o + 1e-9 * lo[r], (r, k, pre_g, pre_o)
        bound_extra += max(tg[r, k:].sum(), to[r, k:].sum())
    tot_g, tot_o = float(lg.sum()), float(lo.sum())
    assert abs(tot_g - tot_o) <= loss_tol * tot_o + bound_extra, (tot_g, tot_o, bound_extra)
    if len(div):
        # after a legitimate near-tie neither run is favoured: the diverged rows'
        # loss differences show no bias beyond six times their own spread
        d = lg[div] - lo[div]
        assert abs(d.sum()) <= 6.0 * np.sqrt((d * d).sum()) + loss_tol * lo[div].sum(), \
            (d.sum(), np.sqrt((d * d).sum()))
    return {"rows": m, "diverged": int(len(div)), "scale_diverged": int((~same_scale).sum()),
            "loss_gpu": tot_g, "loss_oracle": tot_o, "extra_bound": bound_extra}
