"""CPU oracle for the QuIP-family layer-quantization pass.

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The HIP library
never calls it and shares no code with it; the only thing both sides consume in
common is the seeded input generator in ``workloads``.

Plain numpy in float64 throughout, except the scalar grid's rounding
decision: the pages fix no precision for it, so it is taken in the kernel's
(a float32 pre-rounding value divided by a float32 scale) and both sides decide
an integer code in the same precision. Away from a decision boundary that
decision is the exact nearest level (pinned).

Sources (cited by title and section; the section headings of the QuIP page
were lost in extraction, so the names below are the paper's own section names):

* [QuIP] "QuIP: 2-Bit Quantization of Large Language Models With Guarantees"
  (Chee, Cai, Kuleshov, De Sa, 2023).
* [QuIP#] "QuIP#: Even Better LLM Quantization with Hadamard Incoherence and
  Lattice Codebooks" (Tseng et al., 2024), abstract.
* [QTIP] "QTIP: Quantization with Trellises and Incoherence Processing",
  summary page, "Key results" and "Builds on".

Pins: every public function here is checked in ``tests/test_oracle_pins.py``
against closed forms, textbook routines, brute force or a value the pages
print. Where the pages leave a point open, the function that needs it states
the reading it takes.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64
F32 = np.float32


class NotPositiveDefinite(ArithmeticError):
    """Raised by the LDL factorizations; ``index`` is the first failing pivot
    (the first column of the failing block for the block form)."""

    def __init__(self, index: int):
        super().__init__(f"matrix is not positive definite at pivot {index}")
        self.index = index


# --------------------------------------------------------------------------
# a1 / a2: proxy Hessian and damping
# --------------------------------------------------------------------------

def proxy_hessian(X) -> np.ndarray:
    """H = E[x x^T] over the calibration vectors (the rows of X), i.e.
    X^T X / N. [QuIP] "Adaptive Rounding Step": H is the second moment of the
    layer inputs drawn from the calibration set."""
    X = np.asarray(X, dtype=F64)
    return X.T @ X / X.shape[0]


def damp(H, alpha: float) -> np.ndarray:
    """H + alpha * mean(diag H) * I. [QuIP] "Experiments / Methods": the OPTQ
    preprocessing added for numerical stability."""
    H = np.asarray(H, dtype=F64)
    n = H.shape[0]
    return H + alpha * (np.trace(H) / n) * np.eye(n)


# --------------------------------------------------------------------------
# a3 / a4: incoherence processing
# --------------------------------------------------------------------------

def sylvester(n: int) -> np.ndarray:
    """The natural-order Sylvester Hadamard matrix: H_1 = [1],
    H_2k = [[H_k, H_k], [H_k, -H_k]]."""
    if n < 1 or n & (n - 1):
        raise ValueError("Sylvester Hadamard matrices exist for powers of two only")
    Hm = np.ones((1, 1), dtype=F64)
    while Hm.shape[0] < n:
        Hm = np.block([[Hm, Hm], [Hm, -Hm]])
    return Hm


def fwht(A, axis: int = -1) -> np.ndarray:
    """Unnormalized fast Walsh-Hadamard transform along ``axis``: returns
    H_n x for every vector x along that axis, with H_n the natural-order
    Sylvester matrix. One butterfly (a, b) -> (a + b, a - b) per pair and bit."""
    X = np.array(A, dtype=F64, copy=True)
    X = np.moveaxis(X, axis, -1).copy()
    n = X.shape[-1]
    if n < 1 or n & (n - 1):
        raise ValueError("FWHT length must be a power of two")
    shape = X.shape
    h = 1
    while h < n:
        Y = X.reshape(-1, n // (2 * h), 2, h)
        a = Y[:, :, 0, :].copy()
        b = Y[:, :, 1, :].copy()
        Y[:, :, 0, :] = a + b
        Y[:, :, 1, :] = a - b
        h *= 2
    return np.moveaxis(X.reshape(shape), -1, axis)


def rht(A, signs, side: str) -> np.ndarray:
    """Randomized Hadamard transform, [QuIP#] abstract (the orthogonal
    multiplications of [QuIP] "Incoherence Processing" done with a random-sign
    Hadamard matrix). With S = diag(signs) and Q = H_d S / sqrt(d):
    side="left" returns Q A (mixes rows, d = rows);
    side="right" returns A Q^T (mixes columns, d = cols)."""
    A = np.asarray(A, dtype=F64)
    s = np.asarray(signs, dtype=F64)
    if side == "left":
        return fwht(A * s[:, None], axis=0) / np.sqrt(A.shape[0])
    if side == "right":
        return fwht(A * s[None, :], axis=1) / np.sqrt(A.shape[1])
    raise ValueError(side)


def rht_inv(A, signs, side: str) -> np.ndarray:
    """Inverse of ``rht``: left returns Q^T A, right returns A Q."""
    A = np.asarray(A, dtype=F64)
    s = np.asarray(signs, dtype=F64)
    if side == "left":
        return fwht(A, axis=0) * s[:, None] / np.sqrt(A.shape[0])
    if side == "right":
        return fwht(A, axis=1) * s[None, :] / np.sqrt(A.shape[1])
    raise ValueError(side)


def kron_apply(A, K1, K2, side: str, inverse: bool = False) -> np.ndarray:
    """Multiplication by the Kronecker product Q = K1 (x) K2 of two orthogonal
    factors, [QuIP] "Introduction" and "Conclusion" (pre- and post-processing by
    a Kronecker product of random orthogonal matrices). Row-major index
    i = a*q + b. side="left": Q A (or Q^T A when inverse); side="right":
    A Q^T (or A Q when inverse). Computed as (K1 (x) K2) vec(M) = vec(K1 M K2^T)."""
    A = np.asarray(A, dtype=F64)
    K1 = np.asarray(K1, dtype=F64)
    K2 = np.asarray(K2, dtype=F64)
    if inverse:
        K1, K2 = K1.T, K2.T
    p, q = K1.shape[0], K2.shape[0]
    if side == "left":
        r, c = A.shape
        if p * q != r:
            raise ValueError("p*q must equal the number of rows")
        T = A.reshape(p, q, c)
        out = np.einsum("ij,jbc->ibc", K1, T)
        out = np.einsum("kb,ibc->ikc", K2, out)
        return out.reshape(r, c)
    if side == "right":
        r, c = A.shape
        if p * q != c:
            raise ValueError("p*q must equal the number of columns")
        T = A.reshape(r, p, q)
        out = np.einsum("ij,rjb->rib", K1, T)
        out = np.einsum("kb,rib->rik", K2, out)
        return out.reshape(r, c)
    raise ValueError(side)


def permute_gather(A, rows=None, cols=None) -> np.ndarray:
    """out[i][j] = A[rows[i]][cols[j]] (an absent index list is the identity).
    With P_p the permutation matrix (P_p x)_i = x_{p(i)}, this is
    P_rows A P_cols^T."""
    A = np.asarray(A)
    out = A if rows is None else A[np.asarray(rows, dtype=np.int64), :]
    return out if cols is None else out[:, np.asarray(cols, dtype=np.int64)]


def permute_scatter(A, rows=None, cols=None) -> np.ndarray:
    """out[rows[i]][cols[j]] = A[i][j]: the inverse of ``permute_gather``,
    i.e. P_rows^T A P_cols."""
    A = np.asarray(A)
    out = np.empty_like(A)
    r = np.arange(A.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    c = np.arange(A.shape[1]) if cols is None else np.asarray(cols, dtype=np.int64)
    out[np.ix_(r, c)] = A
    return out


def diag_order(H) -> np.ndarray:
    """LDLQ-RG's quantization order, [QuIP] "Experiments / Methods" (the
    weights re-ordered by diag(H)): column indices by decreasing H_jj, equal
    values in increasing index (a reading: the pages give no direction or tie
    rule). Position k of the result is the column quantized k-th."""
    d = np.diag(np.asarray(H, dtype=F64))
    return np.array(sorted(range(d.size), key=lambda j: (-d[j], j)), dtype=np.int32)


def incoherence_side(A, side: str, spec: dict, inverse: bool = False) -> np.ndarray:
    """One side of incoherence processing with either a sign vector
    (``{"signs": s}``, RHT) or two Kronecker factors (``{"A": K1, "B": K2}``),
    optionally composed with a random permutation ``"perm": p`` of the
    coordinates ([QuIP] "Further Ablation", Table 5: a permutation step inside
    the fast orthogonal multiplication). With K the sign/Kronecker transform
    the side's orthogonal matrix is Q = K P_p: the coordinates are permuted
    first, then mixed. Left: Q A (inverse Q^T A); right: A Q^T (inverse A Q)."""
    perm = spec.get("perm")
    if not inverse and perm is not None:
        A = permute_gather(A, rows=perm) if side == "left" else permute_gather(A, cols=perm)
    if "signs" in spec:
        out = (rht_inv if inverse else rht)(A, spec["signs"], side)
    else:
        out = kron_apply(A, spec["A"], spec["B"], side, inverse=inverse)
    if inverse and perm is not None:
        out = permute_scatter(out, rows=perm) if side == "left" else permute_scatter(out, cols=perm)
    return out


def incoherence_H(H, right_spec: dict) -> np.ndarray:
    """H~ = V H V^T, [QuIP] "Incoherence Processing". V is the transform on the
    input (column) side of W, so the same spec as W's right side."""
    T = incoherence_side(H, "right", right_spec)  # H V^T
    return incoherence_side(T, "left", right_spec)  # V H V^T


def incoherence_W(W, left_spec: dict, right_spec: dict) -> np.ndarray:
    """W~ = U W V^T, [QuIP] "Incoherence Processing"."""
    return incoherence_side(incoherence_side(W, "right", right_spec), "left", left_spec)


def incoherence_W_inv(Wt, left_spec: dict, right_spec: dict) -> np.ndarray:
    """Post-processing W = U^T W~ V, the inverse of ``incoherence_W``."""
    return incoherence_side(incoherence_side(Wt, "left", left_spec, inverse=True),
                            "right", right_spec, inverse=True)


# --------------------------------------------------------------------------
# a5: LDL factorization H = (I + U) D (I + U)^T, U strictly upper
# --------------------------------------------------------------------------

def udu(H, g: int = 1):
    """H = (I + U) D (I + U)^T with U strictly (block-)upper triangular and D
    diagonal (g = 1) or block diagonal with g x g blocks, by the direct
    recursion from the last column down to the first:

        D_K  = H_KK - sum_{J>K} U_KJ D_J U_KJ^T
        U_IK = (H_IK - sum_{J>K} U_IJ D_J U_KJ^T) D_K^{-1}      (I < K)

    This is the factor LDLQ needs ([QuIP] "Adaptive Rounding Step" and
    "Experiments / Methods", where QuIP's rounding is named LDLQ; block form:
    [QTIP] "Builds on", BlockLDLQ). Raises NotPositiveDefinite at the first
    pivot (block) that is not positive definite.
    Returns (U, D): U is n x n, D is (n,) for g = 1 or (n/g, g, g)."""
    H = np.asarray(H, dtype=F64)
    n = H.shape[0]
    if H.shape != (n, n):
        raise ValueError("H must be square")
    if g < 1 or n % g:
        raise ValueError("g must divide n")
    U = np.zeros((n, n), dtype=F64)
    if g == 1:
        D = np.zeros(n, dtype=F64)
        for k in range(n - 1, -1, -1):
            t = U[k, k + 1:] * D[k + 1:]
            d = H[k, k] - U[k, k + 1:] @ t
            if not d > 0:
                raise NotPositiveDefinite(k)
            D[k] = d
            if k:
                U[:k, k] = (H[:k, k] - U[:k, k + 1:] @ t) / d
        return U, D
    nb = n // g
    D = np.zeros((nb, g, g), dtype=F64)
    UD = np.zeros((n, n), dtype=F64)  # columns J hold U[:, J] D_J once J is final
    for K in range(nb - 1, -1, -1):
        lo, hi = K * g, (K + 1) * g
        S = UD[:hi, hi:] @ U[lo:hi, hi:].T
        DK = H[lo:hi, lo:hi] - S[lo:hi]
        try:
            np.linalg.cholesky(DK)
        except np.linalg.LinAlgError:
            raise NotPositiveDefinite(lo) from None
        D[K] = DK
        if lo:
            U[:lo, lo:hi] = np.linalg.solve(DK.T, (H[:lo, lo:hi] - S[:lo]).T).T
        UD[:, lo:hi] = U[:, lo:hi] @ DK
    return U, D


def udu_cholesky(H, g: int = 1):
    """The same factorization through the library Cholesky routine of the
    reversed matrix (J H J = L L^T, C = J L J upper with H = C C^T). Used at
    sizes where the direct recursion is too slow; pinned against ``udu``."""
    H = np.asarray(H, dtype=F64)
    n = H.shape[0]
    try:
        L = np.linalg.cholesky(H[::-1, ::-1])
    except np.linalg.LinAlgError:
        raise NotPositiveDefinite(-1) from None
    C = L[::-1, ::-1]
    if g == 1:
        d = np.diag(C).copy()
        U = np.triu(C / d[None, :], 1)
        return U, d * d
    nb = n // g
    D = np.zeros((nb, g, g), dtype=F64)
    U = np.zeros((n, n), dtype=F64)
    for K in range(nb):
        lo, hi = K * g, (K + 1) * g
        Ck = C[lo:hi, lo:hi]
        D[K] = Ck @ Ck.T
        if lo:
            U[:lo, lo:hi] = np.linalg.solve(Ck.T, C[:lo, lo:hi].T).T
    return U, D


def block_diag_D(D) -> np.ndarray:
    """Dense (block-)diagonal matrix from the D returned by ``udu``."""
    D = np.asarray(D, dtype=F64)
    if D.ndim == 1:
        return np.diag(D)
    nb, g, _ = D.shape
    out = np.zeros((nb * g, nb * g), dtype=F64)
    for K in range(nb):
        out[K * g:(K + 1) * g, K * g:(K + 1) * g] = D[K]
    return out


# --------------------------------------------------------------------------
# a6: scalar grid and per-row scale
# --------------------------------------------------------------------------

def uniform_code(x, s, L: int) -> np.ndarray:
    """Nearest point of the L-level midrise grid {(k - (L-1)/2) s}: the code is
    clamp(floor(x/s + L/2), 0, L-1), ties at a decision boundary going up.
    [QuIP] "Adaptive Rounding Step": rounding to a finite grid. The pages fix no
    precision for this decision, so it is taken in the kernel's: float32 x,
    float32 s, IEEE division and add. Away from a boundary (farther than a few
    float32 ulps of x/s) this is the exact nearest level of the float64 x; the
    pins check both that and the tie rule."""
    t = np.asarray(x, dtype=F32) / np.asarray(s, dtype=F32)
    k = np.floor(t + F32(L / 2))
    return np.clip(k, 0, L - 1).astype(np.int64)


def uniform_level(code, s, L: int) -> np.ndarray:
    """Grid value (k - (L-1)/2) * s, in float64 from the float32 scale."""
    return (np.asarray(code, dtype=F64) - (L - 1) / 2.0) * np.asarray(np.asarray(s, dtype=F32), dtype=F64)


def uniform_scale_candidates(amax, L: int, ncand: int = 32) -> np.ndarray:
    """Candidate steps s_c = s_max * 16^(-c/(ncand-1)), c = 0..ncand-1, with
    s_max = max|w| / ((L-1)/2) the step whose outer levels reach the largest
    weight. (32 log-spaced candidates; the range is a reading.)"""
    smax = np.asarray(amax, dtype=F64) / ((L - 1) / 2.0)
    c = np.arange(ncand, dtype=F64)
    return smax[..., None] * 16.0 ** (-c / (ncand - 1))


def uniform_scale_search(W, L: int, ncand: int = 32):
    """Per-row step minimizing the row's nearest-rounding MSE over the
    candidates (ties to the smaller candidate index; an all-zero row gets
    s = 1). Returns (s, choice, mse) with mse the (m, ncand) table."""
    W = np.asarray(W, dtype=F64)
    m = W.shape[0]
    amax = np.abs(W).max(axis=1)
    cand = uniform_scale_candidates(amax, L, ncand)
    mse = np.zeros((m, ncand), dtype=F64)
    for c in range(ncand):
        sc = cand[:, c:c + 1]
        with np.errstate(divide="ignore", invalid="ignore"):
            k = uniform_code(W, sc, L)
            err = W - uniform_level(k, sc, L)
        mse[:, c] = (err * err).sum(axis=1)
    choice = np.argmin(mse, axis=1)
    s = cand[np.arange(m), choice]
    zero = amax == 0
    s[zero] = 1.0
    choice[zero] = 0
    return s, choice, mse


# --------------------------------------------------------------------------
# a7: LDLQ / BlockLDLQ
# --------------------------------------------------------------------------

def uniform_quantizer(scales, L: int):
    """Quantizer for ``ldlq``: per-row float32 scales, L levels."""
    s32 = np.asarray(scales, dtype=F32)

    def q(P, K):
        codes = uniform_code(P, s32[:, None], L)
        return codes, uniform_level(codes, s32[:, None], L)

    return q


def ldlq(W, U, quantize, g: int = 1):
    """Adaptive rounding with linear feedback: columns (groups of g columns)
    are visited in natural order and

        W^_K = Q(W_K + (W - W^)_{:,<K} U_{<K,K}),

    i.e. W^ = Q(W + (W - W^) U) with U strictly (block-)upper. With U from
    H = (I+U) D (I+U)^T this is LDLQ, [QuIP] "Adaptive Rounding Step" and
    "Conclusion" (optimal among rounding methods with linear feedback); g > 1 is
    BlockLDLQ, [QTIP] "Builds on". Unblocked: one group at a time.
    ``quantize(P, K) -> (codes, values)`` rounds an (m, g) block.
    Returns (codes, W^): codes is (m, n) for a scalar quantizer returning an
    (m, 1) block and (m, n/g) for a vector quantizer returning one code per row."""
    W = np.asarray(W, dtype=F64)
    U = np.asarray(U, dtype=F64)
    m, n = W.shape
    What = np.zeros((m, n), dtype=F64)
    E = np.zeros((m, n), dtype=F64)
    codes = []
    for K in range(n // g):
        lo, hi = K * g, (K + 1) * g
        P = W[:, lo:hi] + E[:, :lo] @ U[:lo, lo:hi]
        c, v = quantize(P, K)
        What[:, lo:hi] = v
        E[:, lo:hi] = W[:, lo:hi] - v
        codes.append(np.asarray(c).reshape(m, -1))
    return np.concatenate(codes, axis=1), What


def ldlq_prerounding(W, U, What) -> np.ndarray:
    """P = W + (W - W^) U for a given W^ (conditional replay: the pre-rounding
    values LDLQ sees when its earlier decisions were W^). Because U is strictly
    upper, column K of P only uses columns before K."""
    W = np.asarray(W, dtype=F64)
    return W + (W - np.asarray(What, dtype=F64)) @ np.asarray(U, dtype=F64)


def optq(W, H, quantize):
    """OPTQ (formerly GPTQ) as [QuIP] "Related Work" describes it: over the
    columns in a fixed order, round the column to nearest, then move the
    not-yet-rounded weights by the error scaled so as to minimize the proxy
    loss given the rounded ones (the optimal-brain-surgeon update, with the
    inverse Hessian of the remaining coordinates kept by Schur complements).
    Independent of ``udu``/``ldlq``; used to pin LDLQ == OPTQ ([QuIP]
    "Introduction", "Experiments / Methods")."""
    W = np.asarray(W, dtype=F64)
    m, n = W.shape
    P = W.copy()
    Hinv = np.linalg.inv(np.asarray(H, dtype=F64))
    What = np.zeros((m, n), dtype=F64)
    codes = []
    for k in range(n):
        c, v = quantize(P[:, k:k + 1], k)
        v = np.asarray(v, dtype=F64)[:, 0]
        What[:, k] = v
        codes.append(np.asarray(c).reshape(m))
        err = (P[:, k] - v) / Hinv[k, k]
        P[:, k + 1:] -= np.outer(err, Hinv[k, k + 1:])
        Hinv[k + 1:, k + 1:] -= np.outer(Hinv[k + 1:, k], Hinv[k, k + 1:]) / Hinv[k, k]
    return np.stack(codes, axis=1), What


# --------------------------------------------------------------------------
# a9: proxy loss
# --------------------------------------------------------------------------

def proxy_loss(W, What, H) -> float:
    """l(W^) = tr((W^ - W) H (W^ - W)^T), [QuIP] "Introduction" and "Adaptive
    Rounding Step"."""
    E = np.asarray(What, dtype=F64) - np.asarray(W, dtype=F64)
    return float(np.einsum("ij,ij->", E @ np.asarray(H, dtype=F64), E))


# --------------------------------------------------------------------------
# a8: E8 lattice codebook and nearest codeword
# --------------------------------------------------------------------------

def e8_points(max_norm2: int = 12) -> np.ndarray:
    """All points of E8 = D8 u (D8 + 1/2) with squared norm <= max_norm2, in
    doubled coordinates (integers v = 2x). D8: integer x with even sum.
    D8 + 1/2: all coordinates in Z + 1/2 with even sum."""
    r = int(np.floor(np.sqrt(max_norm2)))
    ints = np.arange(-2 * r, 2 * r + 1, 2, dtype=np.int16)
    halves = np.arange(-2 * r - 1, 2 * r + 2, 2, dtype=np.int16)
    halves = halves[halves * halves <= 4 * max_norm2]
    out = []
    for vals in (ints, halves):
        grids = np.meshgrid(*([vals] * 8), indexing="ij")
        V = np.stack([gr.reshape(-1) for gr in grids], axis=1)
        V = V[(V.astype(np.int32) ** 2).sum(axis=1) <= 4 * max_norm2]
        # sum(x) = sum(v)/2 must be even  <=>  sum(v) = 0 mod 4
        V = V[(V.sum(axis=1) % 4) == 0]
        out.append(V)
    return np.concatenate(out, axis=0)


def e8_codebook(size: int = 65536) -> np.ndarray:
    """The ``size`` smallest-norm points of E8, ordered by (squared norm, then
    coordinates ascending as reals, first coordinate most significant). The
    code of a point is its position. ([QuIP#] abstract: E8-lattice codebooks;
    the ordering rule is the workload's.) Returns float64 (size, 8)."""
    V = e8_points(12)
    norm = (V.astype(np.int32) ** 2).sum(axis=1)
    order = np.lexsort(tuple(V[:, j] for j in range(7, -1, -1)) + (norm,))
    if size > len(order):
        raise ValueError("codebook larger than the enumerated shells")
    return V[order[:size]].astype(F64) / 2.0


def e8_nearest_bruteforce(Y, C, s: float, chunk: int = 2048):
    """argmin_c ||y - s c||^2 over the codebook rows (lowest index on ties),
    evaluated as s^2 ||c||^2 - 2 s <y, c> in float64. Returns (codes, dist)
    with dist the full squared distance."""
    Y = np.asarray(Y, dtype=F64)
    C = np.asarray(C, dtype=F64)
    c2 = (C * C).sum(axis=1) * (s * s)
    codes = np.empty(len(Y), dtype=np.int64)
    dist = np.empty(len(Y), dtype=F64)
    for i in range(0, len(Y), chunk):
        y = Y[i:i + chunk]
        d = c2[None, :] - 2.0 * s * (y @ C.T)
        k = np.argmin(d, axis=1)
        codes[i:i + chunk] = k
        dist[i:i + chunk] = d[np.arange(len(y)), k] + (y * y).sum(axis=1)
    return codes, dist


def _nearest_D8(y):
    f = np.rint(y)
    odd = (f.sum(axis=1) % 2) != 0
    if odd.any():
        yo, fo = y[odd], f[odd]
        delta = yo - fo
        j = np.argmax(np.abs(delta), axis=1)
        rows = np.arange(len(yo))
        step = np.where(delta[rows, j] >= 0, 1.0, -1.0)
        fo[rows, j] += step
        f[odd] = fo
    return f


def e8_decode(Y) -> np.ndarray:
    """Nearest point of the whole E8 lattice (Conway and Sloane's decoder:
    nearest point of D8 and of D8 + 1/2, keep the closer)."""
    Y = np.asarray(Y, dtype=F64)
    a = _nearest_D8(Y)
    b = _nearest_D8(Y - 0.5) + 0.5
    da = ((Y - a) ** 2).sum(axis=1)
    db = ((Y - b) ** 2).sum(axis=1)
    return np.where((da <= db)[:, None], a, b)


class E8Index:
    """Position of a lattice point in the codebook (or -1), and an exact
    nearest-neighbour structure over the codebook for the points whose nearest
    lattice point lies outside it."""

    def __init__(self, C):
        self.C = np.asarray(C, dtype=F64)
        V = np.rint(self.C * 2).astype(np.int64)
        self.keys = self._key(V)
        self.order = np.argsort(self.keys)
        self.sorted = self.keys[self.order]
        self._tree = None

    def nearest_exact(self, P):
        """Exact nearest codeword of every row of P (unscaled units): a k-d tree
        query (scipy's cKDTree, exact Euclidean search) when scipy is present,
        else the exhaustive search. Equally near codewords may resolve to either."""
        P = np.asarray(P, dtype=F64)
        if len(P) == 0:
            return np.zeros(0, dtype=np.int64)
        try:
            from scipy.spatial import cKDTree
        except ImportError:  # pragma: no cover
            return e8_nearest_bruteforce(P, self.C, 1.0)[0]
        if self._tree is None:
            self._tree = cKDTree(self.C)
        _, idx = self._tree.query(P, k=1, workers=-1)
        return np.asarray(idx, dtype=np.int64)

    @staticmethod
    def _key(V):
        k = np.zeros(len(V), dtype=np.int64)
        for j in range(8):
            k = k * 64 + (V[:, j] + 32)
        return k

    def lookup(self, P) -> np.ndarray:
        V = np.rint(np.asarray(P, dtype=F64) * 2).astype(np.int64)
        if np.abs(V).max(initial=0) >= 32:
            far = np.abs(V).max(axis=1) >= 32
        else:
            far = np.zeros(len(V), bool)
        V = np.clip(V, -31, 31)
        k = self._key(V)
        pos = np.searchsorted(self.sorted, k)
        pos = np.minimum(pos, len(self.sorted) - 1)
        hit = (self.sorted[pos] == k) & ~far
        return np.where(hit, self.order[pos], -1)


def e8_nearest(Y, C, s: float, index: E8Index | None = None):
    """Exact nearest codeword, fast: decode y/s on the whole lattice; when that
    lattice point belongs to the codebook it is also the nearest codeword (the
    codebook is a subset of the lattice). Otherwise search the codebook exactly
    (``E8Index.nearest_exact``). Ties between equally near codewords may resolve
    differently from ``e8_nearest_bruteforce``; the pins compare distances there."""
    Y = np.asarray(Y, dtype=F64)
    index = E8Index(C) if index is None else index
    Z = e8_decode(Y / s)
    codes = index.lookup(Z)
    miss = codes < 0
    if miss.any():
        codes[miss] = index.nearest_exact(Y[miss] / s)
    Cq = np.asarray(C, dtype=F64)[codes]
    dist = ((Y - s * Cq) ** 2).sum(axis=1)
    return codes, dist


def row_rms(W) -> np.ndarray:
    """Root mean square of every row, sqrt(sum_j w_j^2 / n) (1 for an all-zero
    row): the factor by which the E8 configuration normalizes each row of the
    incoherent weights to unit RMS before the global scale is chosen (a reading;
    [QuIP#] abstract, E8-lattice codebooks)."""
    W = np.asarray(W, dtype=F64)
    r = np.sqrt((W * W).mean(axis=1))
    return np.where(r > 0, r, 1.0)


def e8_scale_candidates(ncand: int = 32) -> np.ndarray:
    """Global scales 0.5 * 4^(c/(ncand-1)), c = 0..ncand-1 (a reading)."""
    return 0.5 * 4.0 ** (np.arange(ncand, dtype=F64) / (ncand - 1))


def e8_scale_search(Wn, C, ncand: int = 32, nearest=None):
    """Global scale minimizing the nearest-codeword MSE of all 8-vectors of
    the (row-normalized) weights. Returns (s, choice, sse per candidate)."""
    Wn = np.asarray(Wn, dtype=F64)
    Y = Wn.reshape(-1, 8)
    cand = e8_scale_candidates(ncand)
    if nearest is None:
        index = E8Index(C)
        sse = np.array([e8_nearest(Y, C, s, index)[1].sum() for s in cand])
    else:
        sse = np.array([nearest(Y, C, s)[1].sum() for s in cand])
    choice = int(np.argmin(sse))
    return cand[choice], choice, sse


def e8_quantizer(C, s: float, nearest=None):
    """Quantizer for ``ldlq`` with g = 8: nearest scaled codeword per row."""
    C = np.asarray(C, dtype=F64)
    nearest = e8_nearest if nearest is None else nearest
    index = E8Index(C) if nearest is e8_nearest else None

    def q(P, K):
        if index is not None:
            codes, _ = e8_nearest(P, C, s, index)
        else:
            codes, _ = nearest(P, C, s)
        return codes, s * C[codes]

    return q


# --------------------------------------------------------------------------
# Inference with the quantized layer
# --------------------------------------------------------------------------

def code_container_bits(bits: int) -> int:
    """Bits each code occupies in the packed format: the smallest of 2, 4, 8
    that holds `bits` (so that a code never straddles a byte)."""
    if not 1 <= bits <= 8:
        raise ValueError("bits must be in 1..8")
    return 2 if bits <= 2 else (4 if bits <= 4 else 8)


def pack_codes(codes, bits: int) -> np.ndarray:
    """Row-wise packed codes: code j of a row occupies bits
    [(j w) mod 8, (j w) mod 8 + w) of byte (j w) / 8 of that row (w the
    container width, least significant bits first); a row takes
    ceil(n w / 8) bytes. Written out element by element."""
    codes = np.asarray(codes, dtype=np.int64)
    m, n = codes.shape
    w = code_container_bits(bits)
    per = 8 // w
    nbytes = (n + per - 1) // per
    out = np.zeros((m, nbytes), dtype=np.uint8)
    for r in range(m):
        for j in range(n):
            c = int(codes[r, j])
            if not 0 <= c < (1 << bits):
                raise ValueError("code out of range")
            out[r, j // per] |= np.uint8(c << ((j % per) * w))
    return out


def unpack_codes(packed, n: int, bits: int) -> np.ndarray:
    """Inverse of ``pack_codes`` for rows of n codes."""
    packed = np.asarray(packed, dtype=np.uint8)
    w = code_container_bits(bits)
    per = 8 // w
    j = np.arange(n)
    return ((packed[:, j // per].astype(np.int64) >> ((j % per) * w)) & ((1 << w) - 1))


def qmatvec_rht(codes, scales, L: int, signs_left, signs_right, x) -> np.ndarray:
    """Product of the quantized layer with a full-precision vector at
    inference: [QuIP] "Experiments", "Throughput Comparison" (a
    quantized-matrix full-precision-vector product with the incoherence
    transforms applied around it), with random-sign Hadamard sides ([QuIP#]
    abstract). With W^~ the dequantized incoherent weights (code - (L-1)/2) s_r
    and the transforms of ``rht`` (Q_L on the m side, Q_R on the n side), the
    layer in the original basis is W^ = Q_L^T W^~ Q_R, and y = W^ x is taken
    as x' = Q_R x, y' = W^~ x', y = Q_L^T y' (the vectors as rows below)."""
    x = np.asarray(x, dtype=F64)
    xp = rht(x[None, :], signs_right, "right")[0]
    yp = uniform_level(codes, np.asarray(scales)[:, None], L) @ xp
    return rht_inv(yp[None, :], signs_left, "right")[0]


# --------------------------------------------------------------------------
# Trellis-coded quantization with a bitshift trellis ([QTIP] summary)
# --------------------------------------------------------------------------

TCQ_LCG_MUL = 1664525       # the multiplier and increment of the classic
TCQ_LCG_ADD = 1013904223    # 32-bit linear congruential generator (Numerical Recipes)
TCQ_SUM_MEAN = 510.0        # four uniform bytes: mean 4 * 255 / 2
TCQ_SUM_STD = float(np.sqrt(4.0 * (256.0 ** 2 - 1.0) / 12.0))  # and standard deviation


def tcq_code_constants(scale: float = 1.0):
    """(alpha, beta) as float32: reconstruction = fma(bytesum, alpha, beta)."""
    a = F32(scale / TCQ_SUM_STD)
    b = F32(-TCQ_SUM_MEAN * scale / TCQ_SUM_STD)
    return a, b


def tcq_code(states, scale: float = 1.0) -> np.ndarray:
    """The reconstruction value of each trellis state: a computed pseudorandom
    Gaussian code in the sense of [QTIP] (values generated from the state by a
    few integer instructions, no stored codebook; the page names such codes
    but gives no formula, so this one is a reading): one multiply-add of the
    32-bit LCG, h = (1664525 s + 1013904223) mod 2^32, then the sum of h's four
    bytes (an Irwin-Hall approximation of a Gaussian), centred and scaled to
    unit variance times ``scale``. The last step is one float32 fused
    multiply-add, fma(sum, alpha, beta), reproduced exactly here (the float64
    product and sum are exact; one rounding to float32)."""
    st = np.asarray(states, dtype=np.uint64)
    h = (st * np.uint64(TCQ_LCG_MUL) + np.uint64(TCQ_LCG_ADD)) & np.uint64(0xFFFFFFFF)
    bsum = sum(((h >> np.uint64(8 * i)) & np.uint64(0xFF)) for i in range(4)).astype(F64)
    a, b = tcq_code_constants(scale)
    return (bsum * F64(a) + F64(b)).astype(F32)


def tcq_next_state(s, bits_in, L: int, k: int):
    """The bitshift trellis: the next state shifts the L-bit state left by k
    and brings in k new bits, so consecutive states share L - k bits ([QTIP]
    summary: decoding is parallel and stateless, each value depends only on a
    window of L bits of the stream)."""
    return ((int(s) << k) | int(bits_in)) & ((1 << L) - 1)


def tcq_viterbi(x, L: int, k: int, scale: float = 1.0):
    """Trellis-coded quantization of the sequence x (length T): the state
    sequence s_0..s_{T-1} of the bitshift trellis (s_0 free, every later state
    reachable from the previous one) minimizing sum_t (x_t - c(s_t))^2, with
    c = ``tcq_code``. Dynamic programming over time (Viterbi) in float64: the
    best cost of ending in state s' at step t is the best cost over its 2^k
    predecessors p = (s' >> k) + a 2^(L-k) at step t-1, plus the distortion of
    s'. Ties go to the lowest a and, at the end, to the lowest state.
    Returns (states, cost)."""
    x = np.asarray(x, dtype=F64)
    T = x.size
    S = 1 << L
    G = 1 << (L - k)
    c = tcq_code(np.arange(S), scale).astype(F64)
    cost = (x[0] - c) ** 2
    back = np.zeros((T, G), dtype=np.int64)
    for t in range(1, T):
        pred = cost.reshape(1 << k, G)  # pred[a, m] = cost of state m + a G
        a = np.argmin(pred, axis=0)     # first minimum: the lowest a
        best = pred[a, np.arange(G)]
        back[t] = a
        # state s' = m 2^k + b continues from group m
        cost = np.repeat(best, 1 << k) + (x[t] - c) ** 2
    s = int(np.argmin(cost))
    total = float(cost[s])
    states = np.zeros(T, dtype=np.int64)
    for t in range(T - 1, 0, -1):
        states[t] = s
        m = s >> k
        s = m + int(back[t, m]) * G
    states[0] = s
    return states, total


def tcq_path_cost(x, states, scale: float = 1.0) -> float:
    """sum_t (x_t - c(s_t))^2 in float64 for a given state sequence."""
    x = np.asarray(x, dtype=F64)
    return float(((x - tcq_code(states, scale).astype(F64)) ** 2).sum())


def tcq_path_is_valid(states, L: int, k: int) -> bool:
    """Every state follows from the previous one by the bitshift rule."""
    mask = (1 << L) - 1
    st = np.asarray(states, dtype=np.int64)
    return bool(np.all((st >= 0) & (st <= mask)) and
                np.all(((st[:-1] << k) & mask) == (st[1:] & ~((1 << k) - 1) & mask)))


# --------------------------------------------------------------------------
# The whole pass (small layers)
# --------------------------------------------------------------------------

def quantize_layer(W, X, left_spec: dict, right_spec: dict, *, quant: str = "uniform",
                   bits: int = 2, g: int = 1, alpha: float = 0.01, ncand: int = 32,
                   codebook=None, use_cholesky: bool = False, rg_order: bool = False) -> dict:
    """Hessian -> damping -> incoherence -> LDL -> scale -> LDLQ -> post-processing,
    returning every intermediate. ``quant`` is "uniform" (2^bits-level grid,
    per-row scale) or "e8" (rows of W~ normalized to unit RMS, one global scale,
    BlockLDLQ with g = 8).

    ``rg_order``: LDLQ-RG's re-ordering by diag(H) ([QuIP] "Experiments /
    Methods"; its further greedy passes are not described there and are not
    done). The order r = ``diag_order(H~)`` is taken after incoherence
    processing; H~ and W~ become P_r H~ P_r^T and W~ P_r^T, the LDL, the scales,
    LDLQ, the codes and W^~ are in that order, and the post-processing scatters
    W^~'s columns back (W^~ P_r) before the inverse transforms. "Ht", "Wt" and
    "What_t" are returned in the quantization order, with "order"."""
    H = damp(proxy_hessian(X), alpha)
    Ht = incoherence_H(H, right_spec)
    Wt = incoherence_W(W, left_spec, right_spec)
    order = None
    if rg_order:
        order = diag_order(Ht)
        Ht = permute_gather(Ht, rows=order, cols=order)
        Wt = permute_gather(Wt, cols=order)
    U, D = (udu_cholesky if use_cholesky else udu)(Ht, g)
    out = {"H": H, "Ht": Ht, "Wt": Wt, "U": U, "D": D, "order": order}
    if quant == "uniform":
        L = 1 << bits
        s, choice, _ = uniform_scale_search(Wt, L, ncand)
        s32 = s.astype(F32)
        codes, What_t = ldlq(Wt, U, uniform_quantizer(s32, L), g=1)
        out.update(scales=s32, scale_choice=choice, codes=codes)
    elif quant == "e8":
        C = e8_codebook() if codebook is None else np.asarray(codebook, dtype=F64)
        rms = row_rms(Wt)
        Wn = Wt / rms[:, None]
        s, choice, _ = e8_scale_search(Wn, C, ncand)
        codes, Whn = ldlq(Wn, U, e8_quantizer(C, float(F32(s))), g=8)
        What_t = Whn * rms[:, None]
        out.update(scale=s, rms=rms, scale_choice=choice, codes=codes)
    else:
        raise ValueError(quant)
    out["What_t"] = What_t
    back = What_t if order is None else permute_scatter(What_t, cols=order)
    out["What"] = incoherence_W_inv(back, left_spec, right_spec)
    out["loss_t"] = proxy_loss(Wt, What_t, Ht)
    out["loss"] = proxy_loss(W, out["What"], H)
    return out
