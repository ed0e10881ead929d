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
