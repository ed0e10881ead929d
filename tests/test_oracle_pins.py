"""Pins of the CPU oracle against things other than itself: closed forms,
textbook routines, brute force, hand-worked examples and values the pages
print. A plausible slip anywhere in the oracle (a dropped term, a wrong sign or
index, a transposed operand) fails at least one of these."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle as O
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rng(seed):
    return np.random.default_rng(seed)


def spd(seed, n, N=None, col_sigma=1.0):
    r = rng(seed)
    N = 3 * n if N is None else N
    X = r.standard_normal((N, n)) * np.exp(col_sigma * r.standard_normal(n))[None, :]
    return O.damp(O.proxy_hessian(X), 0.01)


# ---------------------------------------------------------------- a1 / a2

def test_hessian_matches_sum_of_outer_products_loop():
    X = rng(1).standard_normal((5, 3))
    H = [[0.0] * 3 for _ in range(3)]
    for t in range(5):
        for i in range(3):
            for j in range(3):
                H[i][j] += X[t, i] * X[t, j]
    H = np.array(H) / 5
    assert np.allclose(O.proxy_hessian(X), H, rtol=0, atol=1e-14)


def test_hessian_symmetric_psd():
    X = rng(2).standard_normal((50, 20)).astype(np.float32)
    H = O.proxy_hessian(X)
    assert np.array_equal(H, H.T)
    assert np.linalg.eigvalsh(H).min() > -1e-12


def test_damping_closed_form():
    H = O.proxy_hessian(rng(3).standard_normal((40, 7)))
    Hd = O.damp(H, 0.01)
    off = ~np.eye(7, dtype=bool)
    assert np.array_equal(Hd[off], H[off])
    shift = 0.01 * np.mean(np.diag(H))
    assert np.allclose(np.diag(Hd) - np.diag(H), shift, rtol=1e-14, atol=0)


# ---------------------------------------------------------------- a3 / a4

@pytest.mark.parametrize("n", [1, 2, 4, 8, 64, 256])
def test_sylvester_closed_form_entries(n):
    Hn = O.sylvester(n)
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i & j)
    assert np.array_equal(Hn, (-1.0) ** pc)
    assert np.array_equal(Hn @ Hn.T, n * np.eye(n))


@pytest.mark.parametrize("n", [1, 2, 8, 128, 1024])
def test_fwht_equals_dense_sylvester(n):
    A = rng(n).standard_normal((3, n))
    assert np.allclose(O.fwht(A, axis=1), A @ O.sylvester(n).T, rtol=0, atol=1e-10)
    assert np.allclose(O.fwht(A.T, axis=0), O.sylvester(n) @ A.T, rtol=0, atol=1e-10)


def test_fwht_rejects_non_power_of_two():
    with pytest.raises(ValueError):
        O.fwht(np.zeros((2, 12)))


@pytest.mark.parametrize("side", ["left", "right"])
def test_rht_is_the_random_sign_hadamard_matrix(side):
    r = rng(7)
    A = r.standard_normal((64, 32))
    d = 64 if side == "left" else 32
    s = np.where(r.random(d) < 0.5, -1.0, 1.0)
    Q = O.sylvester(d) @ np.diag(s) / np.sqrt(d)
    assert np.allclose(Q @ Q.T, np.eye(d), atol=1e-14)
    want = Q @ A if side == "left" else A @ Q.T
    assert np.allclose(O.rht(A, s, side), want, atol=1e-12)
    assert np.allclose(O.rht_inv(O.rht(A, s, side), s, side), A, atol=1e-12)
    if side == "right":  # Parseval: row norms preserved
        assert np.allclose(np.linalg.norm(O.rht(A, s, side), axis=1), np.linalg.norm(A, axis=1))


@pytest.mark.parametrize("side", ["left", "right"])
def test_kron_equals_dense_kron(side):
    r = rng(11)
    K1 = wl.haar_orthogonal(r, 4).astype(np.float64)
    K2 = wl.haar_orthogonal(r, 6).astype(np.float64)
    Q = np.kron(K1, K2)
    A = r.standard_normal((24, 24))
    want = Q @ A if side == "left" else A @ Q.T
    got = O.kron_apply(A, K1, K2, side)
    assert np.allclose(got, want, atol=1e-12)
    back = O.kron_apply(got, K1, K2, side, inverse=True)
    # the float32-drawn factors are orthogonal to ~1e-7; the inverse uses the transposes
    assert np.allclose(back, A @ (Q.T @ Q) if side == "right" else (Q.T @ Q) @ A, atol=1e-12)


def test_trace_invariance_and_loss_in_both_domains():
    r = rng(12)
    W = r.standard_normal((16, 32))
    H = spd(13, 32)
    left = {"signs": np.where(r.random(16) < 0.5, -1.0, 1.0)}
    K1 = np.linalg.qr(r.standard_normal((4, 4)))[0]
    K2 = np.linalg.qr(r.standard_normal((8, 8)))[0]
    right = {"A": K1, "B": K2}
    Wt = O.incoherence_W(W, left, right)
    Ht = O.incoherence_H(H, right)
    assert np.isclose(np.trace(Wt @ Ht @ Wt.T), np.trace(W @ H @ W.T), rtol=1e-12)
    What_t = Wt + 0.1 * r.standard_normal(Wt.shape)
    What = O.incoherence_W_inv(What_t, left, right)
    assert np.isclose(O.proxy_loss(Wt, What_t, Ht), O.proxy_loss(W, What, H), rtol=1e-11)
    assert np.allclose(O.incoherence_W_inv(Wt, left, right), W, atol=1e-12)


# ---------------------------------------------------------------- a5

@pytest.mark.parametrize("g", [1, 8])
def test_udu_reconstructs(g):
    H = spd(21, 64)
    U, D = O.udu(H, g)
    n = 64
    I = np.eye(n)
    rec = (I + U) @ O.block_diag_D(D) @ (I + U).T
    assert np.abs(rec - H).max() / np.abs(H).max() < 1e-12
    # strictly (block-)upper
    mask = np.triu(np.ones((n, n), bool), 1)
    if g > 1:
        blk = np.arange(n) // g
        mask = blk[:, None] < blk[None, :]
    assert np.all(U[~mask] == 0)


def test_udu_diagonal_H():
    d = np.arange(1.0, 9.0)
    U, D = O.udu(np.diag(d))
    assert np.all(U == 0) and np.array_equal(D, d)
    Hb = np.kron(np.eye(4), np.array([[2.0, 0.5], [0.5, 1.0]]))
    U, D = O.udu(Hb, 2)
    assert np.all(U == 0) and np.allclose(D, np.array([[2.0, 0.5], [0.5, 1.0]]))


def test_udu_pivots_are_inverse_cholesky_diagonal():
    # H^-1 = R^T R with R upper (textbook Cholesky of the inverse) => D_kk = 1/R_kk^2
    H = spd(22, 48)
    R = np.linalg.cholesky(np.linalg.inv(H)).T
    _, D = O.udu(H)
    assert np.allclose(D, 1.0 / np.diag(R) ** 2, rtol=1e-10)


@pytest.mark.parametrize("g", [1, 8])
def test_udu_cholesky_route_matches_recursion(g):
    H = spd(23, 96)
    U1, D1 = O.udu(H, g)
    U2, D2 = O.udu_cholesky(H, g)
    assert np.allclose(U1, U2, atol=1e-10)
    assert np.allclose(D1, D2, rtol=1e-10, atol=1e-12)


def test_udu_not_positive_definite_index():
    H = spd(24, 16)
    H[9, :] = 0
    H[:, 9] = 0  # a zero column: pivot 9 is the last one to see it (working down from 15)
    with pytest.raises(O.NotPositiveDefinite) as e:
        O.udu(H)
    assert e.value.index == 9
    with pytest.raises(O.NotPositiveDefinite) as e:
        O.udu(H, 8)
    assert e.value.index == 8


# ---------------------------------------------------------------- a6

def test_grid_codes_ties_go_up():
    s = np.float32(0.37)
    codes = O.uniform_code(np.array([-1.0, 0.0, 1.0], np.float32) * s, s, 4)
    assert codes.tolist() == [1, 2, 3]
    assert O.uniform_code(np.array([-100.0, 100.0]), 1.0, 4).tolist() == [0, 3]


@pytest.mark.parametrize("L", [4, 8, 16])
def test_grid_code_is_nearest_level(L):
    x = rng(L).uniform(-L, L, 5000)
    s = 0.9
    k = O.uniform_code(x, s, L)
    levels = (np.arange(L) - (L - 1) / 2) * np.float64(np.float32(s))
    dist = np.abs(x[:, None] - levels[None, :])
    best = dist.min(axis=1)
    assert np.all(np.abs(dist[np.arange(len(x)), k] - best) <= 1e-6)


@pytest.mark.parametrize("L", [4, 8, 16])
def test_scale_search_lands_on_max_1960_optimum(L):
    ref = golden("max1960_uniform_gaussian.json")["levels"][str(L)]
    W = wl.gaussian_rows(L, 4, 1 << 16)
    s, choice, mse = O.uniform_scale_search(W, L)
    step = 16.0 ** (1 / 31) - 1  # relative spacing of the candidates (~9.4%)
    assert np.all(np.abs(s / ref["step"] - 1) <= step)
    per_weight = mse[np.arange(4), choice] / W.shape[1]
    assert np.allclose(per_weight, ref["mse"], rtol=0.05)


def test_scale_search_table_is_brute_force_mse():
    W = rng(31).standard_normal((3, 40))
    L = 8
    s, choice, mse = O.uniform_scale_search(W, L)
    amax = np.abs(W).max(axis=1)
    for r in range(3):
        for c in (0, 7, 31):
            sc = amax[r] / 3.5 * 16.0 ** (-c / 31)
            lv = (np.arange(L) - 3.5) * np.float64(np.float32(sc))
            e = np.min(np.abs(W[r][:, None] - lv[None, :]), axis=1)
            assert np.isclose(mse[r, c], (e * e).sum(), rtol=1e-6)
        assert choice[r] == int(np.argmin(mse[r]))


def test_scale_search_zero_row():
    s, choice, _ = O.uniform_scale_search(np.zeros((2, 8)), 4)
    assert s.tolist() == [1.0, 1.0]


# ---------------------------------------------------------------- a7

def test_ldlq_worked_example():
    gd = golden("ldlq_worked_2col.json")
    H = np.array(gd["H"])
    W = np.array(gd["W"])
    U, D = O.udu(H)
    assert np.isclose(U[0, 1], gd["U01"]) and np.allclose(D, gd["D"])
    q = O.uniform_quantizer(np.array([gd["scale"]]), gd["levels"])
    codes, What = O.ldlq(W, U, q)
    assert codes[0].tolist() == gd["ldlq_codes"]
    assert np.allclose(What[0], gd["ldlq_What"])
    assert np.allclose(O.ldlq_prerounding(W, U, What)[0], gd["ldlq_prerounding"])
    assert np.isclose(O.proxy_loss(W, What, H), gd["ldlq_loss"])
    near = O.uniform_code(W, np.float32(gd["scale"]), gd["levels"])
    assert near[0].tolist() == gd["nearest_codes"]
    assert np.isclose(O.proxy_loss(W, O.uniform_level(near, 1.0, 4), H), gd["nearest_loss"])


def test_ldlq_with_diagonal_H_is_nearest_rounding():
    W = rng(41).standard_normal((32, 64)) * 2
    H = np.diag(rng(42).uniform(0.5, 2.0, 64))
    U, D = O.udu(H)
    s, _, _ = O.uniform_scale_search(W, 4)
    codes, _ = O.ldlq(W, U, O.uniform_quantizer(s, 4))
    assert np.array_equal(codes, O.uniform_code(W, s.astype(np.float32)[:, None], 4))


@pytest.mark.parametrize("L", [4, 8])
def test_ldlq_equals_optq(L):
    H = spd(43, 64, N=80)
    W = rng(44).standard_normal((48, 64))
    s, _, _ = O.uniform_scale_search(W, L)
    q = O.uniform_quantizer(s, L)
    U, _ = O.udu(H)
    c1, w1 = O.ldlq(W, U, q)
    c2, w2 = O.optq(W, H, q)
    assert np.array_equal(c1, c2)
    assert np.allclose(w1, w2, atol=1e-12)


def test_ldlq_prerounding_replays_the_sweep():
    H = spd(45, 32)
    W = rng(46).standard_normal((8, 32))
    U, _ = O.udu(H)
    seen = []
    s = np.full(8, 0.7)
    base = O.uniform_quantizer(s, 4)

    def q(P, K):
        seen.append(P[:, 0].copy())
        return base(P, K)

    _, What = O.ldlq(W, U, q)
    assert np.allclose(np.stack(seen, axis=1), O.ldlq_prerounding(W, U, What), atol=1e-12)


@pytest.mark.parametrize("m", [2, 3])
def test_ldlq_not_better_than_brute_force_optimum(m):
    r = rng(50 + m)
    n, L, s = 4, 4, 0.75  # exactly representable in float32
    levels = (np.arange(L) - 1.5) * s
    for trial in range(5):
        W = r.standard_normal((m, n))
        for diagonal in (False, True):
            H = np.diag(r.uniform(0.5, 2, n)) if diagonal else spd(60 + trial, n, N=6)
            U, _ = O.udu(H)
            _, What = O.ldlq(W, U, O.uniform_quantizer(np.full(m, s), L))
            best = 0.0
            for row in range(m):
                cand = np.array(list(itertools.product(levels, repeat=n)))
                E = cand - W[row]
                best += np.min(np.einsum("ij,jk,ik->i", E, H, E))
            got = O.proxy_loss(W, What, H)
            assert got >= best - 1e-12
            if diagonal:
                assert np.isclose(got, best, rtol=1e-12)


@pytest.mark.parametrize("g", [1, 8])
def test_loss_identity_sum_of_pivots_times_residuals(g):
    n = 64
    H = spd(70, n)
    W = rng(71).standard_normal((16, n))
    U, D = O.udu(H, g)
    if g == 1:
        q = O.uniform_quantizer(np.full(16, 0.6), 4)
    else:
        q = O.e8_quantizer(O.e8_codebook(), 0.9)
    _, What = O.ldlq(W, U, q, g=g)
    eta = What - O.ldlq_prerounding(W, U, What)
    if g == 1:
        ident = float((D * (eta * eta).sum(axis=0)).sum())
    else:
        ident = sum(np.trace(eta[:, K * g:(K + 1) * g] @ D[K] @ eta[:, K * g:(K + 1) * g].T)
                    for K in range(n // g))
    assert np.isclose(ident, O.proxy_loss(W, What, H), rtol=1e-10)


def test_block_ldlq_brute_force_with_small_codebook():
    # BlockLDLQ with g = 2 and a 9-point 2-D codebook, on 2 x 4 problems.
    C = np.array([[a, b] for a in (-1.0, 0.0, 1.0) for b in (-1.0, 0.0, 1.0)])

    def nearest(P, Cb, s):
        d = ((P[:, None, :] - s * Cb[None, :, :]) ** 2).sum(axis=2)
        k = np.argmin(d, axis=1)
        return k, d[np.arange(len(P)), k]

    r = rng(80)
    for trial in range(4):
        W = r.standard_normal((2, 4))
        for blockdiag in (False, True):
            if blockdiag:
                # blocks c_K * I: the per-block loss is c_K times the Euclidean
                # distance, so the nearest codeword per block is optimal
                H = np.diag(np.repeat(r.uniform(0.5, 2.0, 2), 2))
            else:
                H = spd(100 + trial, 4, N=5)
            U, D = O.udu(H, 2)
            codes, What = O.ldlq(W, U, O.e8_quantizer(C, 0.7, nearest=nearest), g=2)
            best = 0.0
            for row in range(2):
                cand = np.array([np.concatenate([0.7 * C[i], 0.7 * C[j]]) for i in range(9) for j in range(9)])
                E = cand - W[row]
                best += np.min(np.einsum("ij,jk,ik->i", E, H, E))
            got = O.proxy_loss(W, What, H)
            assert got >= best - 1e-12
            if blockdiag:
                assert np.isclose(got, best, rtol=1e-12)
                want = np.stack([nearest(W[:, 0:2], C, 0.7)[0], nearest(W[:, 2:4], C, 0.7)[0]], axis=1)
                assert np.array_equal(codes, want)


# ---------------------------------------------------------------- a9

def test_proxy_loss_row_loop():
    r = rng(110)
    W = r.standard_normal((3, 5))
    What = r.standard_normal((3, 5))
    H = spd(111, 5)
    want = sum(float((What[i] - W[i]) @ H @ (What[i] - W[i])) for i in range(3))
    assert np.isclose(O.proxy_loss(W, What, H), want, rtol=1e-13)


# ---------------------------------------------------------------- a8 (E8)

def sigma3(k):
    return sum(d ** 3 for d in range(1, k + 1) if k % d == 0)


def test_e8_shell_counts_theta_series():
    V = O.e8_points(12)
    norm2 = (V.astype(np.int64) ** 2).sum(axis=1)  # doubled coords: 4 * |x|^2
    counts = np.bincount(norm2 // 4, minlength=13)
    assert counts[0] == 1
    for k in range(1, 7):
        assert counts[2 * k] == 240 * sigma3(k)
        assert counts[2 * k - 1] == 0
    assert np.all(norm2 % 8 == 0)  # every E8 vector has even squared norm


def test_e8_codebook_structure():
    C = O.e8_codebook()
    assert C.shape == (65536, 8)
    assert np.all(C[0] == 0)
    V = np.rint(C * 2).astype(np.int64)
    assert np.array_equal(V / 2.0, C)
    same_parity = np.all(V % 2 == (V[:, :1] % 2), axis=1)
    assert np.all(same_parity)  # all-integer or all-half-integer
    assert np.all((V.sum(axis=1) // 2) % 2 == 0)  # even coordinate sum
    assert len(np.unique(V, axis=0)) == 65536
    n2 = (V ** 2).sum(axis=1) // 4
    assert np.all(np.diff(n2) >= 0)
    assert np.sum(n2 <= 10) == 1 + sum(240 * sigma3(k) for k in range(1, 6))  # 56881
    assert np.sum(n2 == 12) == 65536 - 56881  # 8655 of the 60480 points of norm 12
    shell = V[n2 == 12]
    for a, b in zip(shell[:-1], shell[1:]):  # lexicographic inside the shell
        assert tuple(a) < tuple(b)
        break
    keys = [tuple(v) for v in shell]
    assert keys == sorted(keys)
    # the kept part of the norm-12 shell is its lexicographically smallest 8655 points
    full12 = O.e8_points(12)
    f12 = full12[(full12.astype(np.int64) ** 2).sum(axis=1) == 48]
    rest = sorted(tuple(v) for v in f12)
    assert keys == rest[:8655]


def test_e8_decoder_is_the_nearest_lattice_point():
    pts = O.e8_points(12).astype(np.float64) / 2
    Y = rng(120).standard_normal((300, 8)) * 0.8
    Z = O.e8_decode(Y)
    d = ((Y[:, None, :] - pts[None, :, :]) ** 2).sum(axis=2).min(axis=1)
    dz = ((Y - Z) ** 2).sum(axis=1)
    assert np.all(dz <= d + 1e-12)  # never worse than any enumerated lattice point
    inside = (Z * Z).sum(axis=1) <= 12  # the enumeration holds every point of norm <= 12
    assert inside.mean() > 0.9
    assert np.allclose(dz[inside], d[inside], atol=1e-12)


@pytest.mark.parametrize("s", [0.6, 1.0, 1.5])
def test_e8_fast_nearest_equals_exhaustive(s):
    C = O.e8_codebook()
    Y = rng(121).standard_normal((3000, 8))
    k1, d1 = O.e8_nearest_bruteforce(Y, C, s)
    k2, d2 = O.e8_nearest(Y, C, s)
    assert np.allclose(d1, d2, rtol=0, atol=1e-10)
    assert np.mean(k1 == k2) > 0.999


def test_e8_codebook_mse_against_printed_gaussian_bounds():
    gd = golden("qtip_gaussian_2bit_mse.json")
    assert abs(2.0 ** (-2 * gd["bits_per_weight"]) - gd["bound_printed"]) <= 5e-4 + 1e-12
    scalar = golden("max1960_uniform_gaussian.json")["levels"]["4"]["mse"]
    C = O.e8_codebook()
    assert np.log2(len(C)) / 8 == gd["bits_per_weight"]
    Y = wl.gaussian_rows(5, 512, 64)  # 4096 Gaussian 8-vectors
    s, choice, sse = O.e8_scale_search(Y, C)
    mse = sse[choice] / Y.size
    assert mse >= 2.0 ** -4  # distortion-rate bound
    assert mse < scalar  # an 8-D lattice codebook beats the best 2-bit scalar grid
    assert 0 < choice < 31  # the optimum is inside the candidate range


# ---------------------------------------------------------------- end to end

def test_quantize_layer_end_to_end_c1():
    L = wl.make_layer("c1")
    r = O.quantize_layer(L.W, L.X, L.left, L.right, quant="uniform", bits=2)
    assert np.isclose(r["loss_t"], r["loss"], rtol=1e-10)
    # incoherence + LDLQ beats nearest rounding without incoherence (the paper's claim)
    s, _, _ = O.uniform_scale_search(L.W, 4)
    near = O.uniform_level(O.uniform_code(L.W, s.astype(np.float32)[:, None], 4), s[:, None], 4)
    assert r["loss"] < O.proxy_loss(L.W, near, r["H"])
    assert r["codes"].shape == (256, 256) and r["codes"].min() >= 0 and r["codes"].max() <= 3


def test_workloads_are_deterministic_and_shaped():
    a = wl.make_layer("c1")
    b = wl.make_layer("c1")
    assert np.array_equal(a.W, b.W) and np.array_equal(a.X, b.X)
    assert a.W.dtype == np.float32 and a.X.shape == (2048, 256)
    assert set(np.unique(a.left["signs"]).tolist()) == {-1.0, 1.0}
    frac = np.mean(np.abs(a.W) > 5)
    assert 0.002 < frac < 0.02  # ~1% outliers x10


# ---------------------------------------------------------------- inference product

def test_pack_codes_matches_handwritten_bytes():
    for case in golden("packed_codes_example.json")["cases"]:
        codes = np.array(case["codes"])
        got = O.pack_codes(codes, case["bits"])
        assert got.tolist() == case["packed"]
        assert O.unpack_codes(got, codes.shape[1], case["bits"]).tolist() == case["codes"]


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 8])
def test_pack_codes_round_trip(bits):
    codes = rng(bits).integers(0, 1 << bits, size=(7, 37))
    assert np.array_equal(O.unpack_codes(O.pack_codes(codes, bits), 37, bits), codes)


@pytest.mark.parametrize("m,n,bits", [(64, 32, 2), (16, 128, 3), (32, 64, 4)])
def test_qmatvec_rht_equals_the_dense_layer(m, n, bits):
    r = rng(m + n + bits)
    L = 1 << bits
    codes = r.integers(0, L, size=(m, n))
    scales = np.exp(r.standard_normal(m)).astype(np.float32)
    sl = r.choice([-1.0, 1.0], m)
    sr = r.choice([-1.0, 1.0], n)
    x = r.standard_normal(n)
    y = O.qmatvec_rht(codes, scales, L, sl, sr, x)
    What_t = O.uniform_level(codes, scales[:, None], L)
    tol = 1e-12 * np.abs(What_t).sum(axis=1).max() * np.abs(x).max()
    # the pass's own post-processing: the inverse two-sided transform of the matrix
    What = O.incoherence_W_inv(What_t, {"signs": sl}, {"signs": sr})
    assert np.allclose(y, What @ x, rtol=0, atol=tol)
    # explicit matrices: Q = H diag(s) / sqrt(d), W^ = Q_L^T W^~ Q_R
    QL = O.sylvester(m) * sl[None, :] / np.sqrt(m)
    QR = O.sylvester(n) * sr[None, :] / np.sqrt(n)
    assert np.allclose(y, QL.T @ What_t @ QR @ x, rtol=0, atol=tol)


# ---------------------------------------------------------------- QuIP variants: permutations

def perm_matrix(p):
    """(P x)_i = x_{p(i)}: row i of P is e_{p(i)}."""
    return np.eye(len(p))[np.asarray(p)]


def test_permute_gather_and_scatter_are_permutation_matrix_products():
    r = rng(41)
    A = r.standard_normal((5, 7))
    pr = r.permutation(5)
    pc = r.permutation(7)
    Pr, Pc = perm_matrix(pr), perm_matrix(pc)
    assert np.array_equal(O.permute_gather(A, pr, pc), Pr @ A @ Pc.T)
    assert np.array_equal(O.permute_scatter(A, pr, pc), Pr.T @ A @ Pc)
    assert np.array_equal(O.permute_scatter(O.permute_gather(A, pr, pc), pr, pc), A)
    assert np.array_equal(O.permute_gather(A, cols=pc), A @ Pc.T)
    assert np.array_equal(O.permute_gather(A, rows=pr), Pr @ A)
    # element by element for one entry
    assert O.permute_gather(A, pr, pc)[2, 3] == A[pr[2], pc[3]]
    assert O.permute_scatter(A, pr, pc)[pr[2], pc[3]] == A[2, 3]


@pytest.mark.parametrize("kind", ["rht", "kron"])
@pytest.mark.parametrize("side", ["left", "right"])
def test_permutation_inside_the_orthogonal_multiply_is_K_times_P(kind, side):
    r = rng(43)
    d = 16 if kind == "rht" else 12
    if kind == "rht":
        s = np.where(r.random(d) < 0.5, -1.0, 1.0)
        K = O.sylvester(d) @ np.diag(s) / np.sqrt(d)
        spec = {"signs": s}
    else:
        K1 = np.linalg.qr(r.standard_normal((3, 3)))[0]
        K2 = np.linalg.qr(r.standard_normal((4, 4)))[0]
        K = np.kron(K1, K2)
        spec = {"A": K1, "B": K2}
    spec["perm"] = r.permutation(d)
    Q = K @ perm_matrix(spec["perm"])
    assert np.allclose(Q @ Q.T, np.eye(d), atol=1e-13)
    A = r.standard_normal((d, d)) if side == "left" else r.standard_normal((5, d))
    want = Q @ A if side == "left" else A @ Q.T
    got = O.incoherence_side(A, side, spec)
    assert np.allclose(got, want, atol=1e-12)
    inv_want = Q.T @ A if side == "left" else A @ Q
    assert np.allclose(O.incoherence_side(A, side, spec, inverse=True), inv_want, atol=1e-12)
    # without the permutation the result differs (the step is not a no-op)
    plain = {k: v for k, v in spec.items() if k != "perm"}
    assert not np.allclose(O.incoherence_side(A, side, plain), want)


def test_diag_order_hand_worked_with_ties():
    # diag 2, 5, 5, 1, 3 -> decreasing, equal values by index: 1, 2, 4, 0, 3
    H = np.diag([2.0, 5.0, 5.0, 1.0, 3.0])
    assert O.diag_order(H).tolist() == [1, 2, 4, 0, 3]


def test_diag_order_is_the_rank_count():
    r = rng(47)
    d = r.integers(0, 6, 40).astype(np.float64)  # many ties
    H = np.diag(d) + 0.01 * np.ones((40, 40))
    o = O.diag_order(H)
    hd = np.diag(H)
    # position of j = #{i : d_i > d_j} + #{i < j : d_i == d_j}
    for j in range(40):
        rank = int(np.sum(hd > hd[j]) + np.sum(hd[:j] == hd[j]))
        assert o[rank] == j
    assert sorted(o.tolist()) == list(range(40))


def test_rg_order_pass_loss_in_both_domains_and_sorted_diagonal():
    cfg = wl.custom_config("rg", 901, 16, 32, 256, left=wl.RHT, right=wl.KRON(4, 8, perm=True),
                           bits=2, rg_order=True)
    L = wl.make_layer(cfg)
    assert sorted(L.right["perm"].tolist()) == list(range(32))
    r = O.quantize_layer(L.W, L.X, L.left, L.right, quant="uniform", bits=2, rg_order=True)
    dg = np.diag(r["Ht"])
    assert np.all(np.diff(dg) <= 0)
    # a wrong scatter back would scramble W^ and break this equality (the
    # float32-drawn Kronecker factors are orthogonal to ~1e-7 only)
    assert np.isclose(r["loss_t"], r["loss"], rtol=1e-6)
    # the order is a relabelling: H~ in quantization order is P_r H~ P_r^T
    Ht0 = O.incoherence_H(r["H"], L.right)
    assert np.allclose(r["Ht"], perm_matrix(r["order"]) @ Ht0 @ perm_matrix(r["order"]).T)


def test_rg_order_on_an_already_sorted_diagonal_changes_nothing():
    r = rng(53)
    n = 16
    # column scales halving from column to column: diag(H) falls by ~4x per
    # column, far beyond the sampling noise of 64 calibration rows
    Xc = r.standard_normal((64, n)) * 0.5 ** np.arange(n)[None, :]
    W = r.standard_normal((6, n))
    ident = {"A": np.eye(1), "B": np.eye(n)}  # identity transform: diag(H~) = diag(H)
    a = O.quantize_layer(W, Xc, {"A": np.eye(1), "B": np.eye(6)}, ident, bits=2)
    b = O.quantize_layer(W, Xc, {"A": np.eye(1), "B": np.eye(6)}, ident, bits=2, rg_order=True)
    assert np.array_equal(b["order"], np.arange(n))
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["What"], b["What"])
    # reversed column scales: the order is reversed, and the pass equals the
    # natural-order pass on the column-reversed layer, scattered back
    Xr = Xc[:, ::-1].copy()
    c = O.quantize_layer(W[:, ::-1].copy(), Xr, {"A": np.eye(1), "B": np.eye(6)}, ident, bits=2,
                         rg_order=True)
    assert np.array_equal(c["order"], np.arange(n)[::-1])
    assert np.array_equal(c["codes"], a["codes"])
    assert np.allclose(c["What"], a["What"][:, ::-1], atol=1e-12)


# ---------------------------------------------------------------- trellis-coded quantization

def test_tcq_code_hand_worked_values():
    g = golden("tcq_code_worked.json")
    for case in g["cases"]:
        h = int(case["h_hex"], 16)
        assert [(h >> (8 * i)) & 0xFF for i in range(4)] == case["bytes"]
        assert sum(case["bytes"]) == case["sum"]
        want = (case["sum"] - 510) / g["std"]
        got = float(O.tcq_code([case["state"]])[0])
        assert abs(got - want) <= 2e-7 * max(1.0, abs(want)), (case, got, want)


def test_tcq_code_is_unit_gaussian_like():
    c = O.tcq_code(np.arange(1 << 16)).astype(np.float64)
    assert abs(c.mean()) < 0.01 and abs(c.var() - 1.0) < 0.01
    assert c.min() > -3.5 and c.max() < 3.5  # Irwin-Hall with 4 terms: bounded by 3.46
    c2 = O.tcq_code(np.arange(1 << 16), 2.0).astype(np.float64)
    assert np.allclose(c2, 2 * c, rtol=2e-7, atol=1e-7)


def _tcq_brute(x, L, k):
    """Minimum over every valid state sequence, by enumeration."""
    T = len(x)
    c = O.tcq_code(np.arange(1 << L)).astype(np.float64)
    best, arg = np.inf, None
    for s0 in range(1 << L):
        for bits in itertools.product(range(1 << k), repeat=T - 1):
            st = [s0]
            for b in bits:
                st.append(O.tcq_next_state(st[-1], b, L, k))
            v = float(((np.asarray(x) - c[st]) ** 2).sum())
            if v < best:
                best, arg = v, st
    return best, arg


@pytest.mark.parametrize("L,k,T", [(4, 2, 4), (3, 1, 7), (5, 2, 3)])
def test_tcq_viterbi_equals_brute_force(L, k, T):
    x = rng(61 + L + T).standard_normal(T) * 1.3
    st, cost = O.tcq_viterbi(x, L, k)
    best, _ = _tcq_brute(x, L, k)
    assert np.isclose(cost, best, rtol=1e-12, atol=1e-12)
    assert O.tcq_path_is_valid(st, L, k)
    assert np.isclose(O.tcq_path_cost(x, st), cost, rtol=1e-12)


def test_tcq_single_step_and_memoryless_special_cases():
    x = rng(67).standard_normal(9)
    c = O.tcq_code(np.arange(1 << 6)).astype(np.float64)
    # T = 1: the nearest of all 2^L codes (lowest state on ties)
    st, cost = O.tcq_viterbi(x[:1], 6, 2)
    assert st[0] == int(np.argmin((x[0] - c) ** 2))
    # k = L: no shared bits, every step picks its own nearest code
    st, cost = O.tcq_viterbi(x, 6, 6)
    assert np.isclose(cost, ((x[:, None] - c[None, :]) ** 2).min(axis=1).sum(), rtol=1e-12)


def test_tcq_path_validity_check():
    assert O.tcq_path_is_valid([5, (5 << 2 | 3) & 15, ((5 << 2 | 3) & 15) << 2 & 15], 4, 2)
    assert O.tcq_path_is_valid([5, 6], 4, 2)  # 6 = (5 << 2 | 2) mod 16
    assert not O.tcq_path_is_valid([5, 9], 4, 2)  # 9 keeps bits 2-3 = 2, not 1
    assert not O.tcq_path_is_valid([5, 16], 4, 2)  # outside the 4-bit states


def test_tcq_gaussian_mse_between_bound_and_best_scalar():
    # 2 bits per weight (+ (L - k)/T for the free first state) on i.i.d. N(0,1):
    # no code beats the distortion-rate bound 2^(-2R); the trellis beats Max's
    # optimal 4-level scalar quantizer (0.1175)
    L, k, T = 10, 2, 64
    X = wl.gaussian_rows(5, 24, T).astype(np.float64)
    mse = np.mean([O.tcq_viterbi(x, L, k)[1] for x in X]) / T
    R = k + (L - k) / T
    assert 2.0 ** (-2 * R) <= mse < 0.1175, mse


# ---------------------------------------------------------------- grid decision vs exact nearest

@pytest.mark.parametrize("L", [2, 4, 8, 16])
def test_float32_grid_decision_is_the_exact_nearest_level_off_the_boundaries(L):
    # The decision is taken in float32 (the pages fix no precision); away from
    # the decision boundaries it must be the exact nearest level of the float64
    # value, found here by comparing distances to every level in float64.
    r = rng(200 + L)
    s32 = np.float32(0.7311)
    s = np.float64(s32)
    x = r.uniform(-(L + 1) * s, (L + 1) * s, 20000)
    bnd = (np.arange(1, L) - L / 2.0) * s  # midpoints between adjacent levels
    near = (bnd[None, :] + np.outer(np.array([-1.0, 1.0]) * 1e-6, np.maximum(np.abs(bnd), s))).ravel()
    x = np.concatenate([x, near])
    levels = (np.arange(L) - (L - 1) / 2.0) * s
    d = np.abs(x[:, None] - levels[None, :])
    exact = np.argmin(d, axis=1)
    got = O.uniform_code(x, s32, L)
    far = np.min(np.abs(x[:, None] - bnd[None, :]), axis=1) > 1e-7 * np.maximum(np.abs(x), s)
    assert far.sum() > 19000
    assert np.array_equal(got[far], exact[far])
    # on an exact boundary the tie goes up (to the larger level)
    b = np.float32(bnd[L // 2 - 1]) if L > 2 else np.float32(0.0)
    assert O.uniform_code(np.array([b]), s32, L)[0] == L // 2


# ---------------------------------------------------------------- E8 configuration pass

def test_row_rms_hand_worked_and_loop():
    gd = golden("row_rms_worked.json")
    rows = np.array(gd["rows"])
    assert O.row_rms(rows).tolist() == gd["rms"]
    W = rng(300).standard_normal((7, 24))
    W[3] = 0.0
    loop = []
    for r in range(7):
        acc = 0.0
        for j in range(24):
            acc += W[r, j] * W[r, j]
        loop.append(np.sqrt(acc / 24) if acc > 0 else 1.0)
    assert np.allclose(O.row_rms(W), loop, rtol=1e-14, atol=0)


def _identity_kron(d):
    # Q = I_p (x) I_q = I: a side whose transform leaves the matrix unchanged
    p = 8 if d % 8 == 0 else 1
    return {"A": np.eye(p), "B": np.eye(d // p)}


def test_quantize_layer_e8_with_block_diagonal_H_is_groupwise_nearest():
    # With identity transforms and an H that is block diagonal in 8 x 8 blocks,
    # the block LDL has U = 0, so BlockLDLQ gets no feedback: every group is
    # rounded to the nearest scaled codeword of the row-normalized weights, the
    # scale is the argmin of the exhaustive nearest-codeword error, and the
    # result is rescaled by each row's RMS.
    m, n = 24, 64
    r = rng(301)
    X = np.zeros((8 * 40, n))
    for g in range(n // 8):  # each calibration row lives in one column group
        X[40 * g:40 * (g + 1), 8 * g:8 * (g + 1)] = r.standard_normal((40, 8)) * np.exp(r.standard_normal(8))
    W = r.standard_normal((m, n)) * np.exp(0.5 * r.standard_normal(m))[:, None]
    C = O.e8_codebook()
    out = O.quantize_layer(W, X, _identity_kron(m), _identity_kron(n), quant="e8", g=8, codebook=C)
    assert np.array_equal(out["Ht"], out["H"]) and np.array_equal(out["Wt"], W)
    assert np.abs(out["U"]).max() == 0.0
    rms = np.sqrt((W * W).mean(axis=1))
    assert np.allclose(out["rms"], rms, rtol=1e-14)
    Wn = W / rms[:, None]
    s_bf, c_bf, sse_bf = O.e8_scale_search(Wn, C, nearest=O.e8_nearest_bruteforce)
    assert out["scale_choice"] == c_bf and out["scale"] == s_bf
    s32 = float(np.float32(s_bf))
    k_bf, d_bf = O.e8_nearest_bruteforce(Wn.reshape(-1, 8), C, s32)
    codes = out["codes"].reshape(-1)
    d_got = ((Wn.reshape(-1, 8) - s32 * C[codes]) ** 2).sum(axis=1)
    assert np.allclose(d_got, d_bf, rtol=0, atol=1e-12)
    assert np.mean(codes == k_bf) > 0.99
    assert np.allclose(out["What_t"], rms[:, None] * s32 * C[out["codes"]].reshape(m, n), rtol=1e-14)


def test_quantize_layer_e8_loss_identity_round_trip_and_both_domains():
    # A general small layer (random-sign Hadamard sides): the loss is the same
    # in both domains; W^~ / rms is exactly the scaled codewords; and the loss
    # equals sum_r rms_r^2 sum_K eta_K D_K eta_K^T with eta = P - W^~/rms the
    # residual of each group's rounding (P the pre-rounding targets).
    m, n = 16, 64
    r = rng(302)
    W = r.standard_normal((m, n))
    W[r.random((m, n)) < 0.02] *= 10
    X = r.standard_normal((256, n)) * np.exp(r.standard_normal(n))[None, :]
    left = {"signs": r.choice([-1.0, 1.0], m)}
    right = {"signs": r.choice([-1.0, 1.0], n)}
    C = O.e8_codebook()
    out = O.quantize_layer(W, X, left, right, quant="e8", g=8, codebook=C)
    assert np.isclose(out["loss"], out["loss_t"], rtol=1e-9)
    rms = out["rms"]
    s32 = float(np.float32(out["scale"]))
    Whn = out["What_t"] / rms[:, None]
    assert np.allclose(Whn, s32 * C[out["codes"]].reshape(m, n), rtol=1e-14, atol=1e-15)
    Wn = out["Wt"] / rms[:, None]
    P = O.ldlq_prerounding(Wn, out["U"], Whn)
    eta = (P - Whn).reshape(m, n // 8, 8)
    blk = np.einsum("rka,kab,rkb->r", eta, out["D"], eta)
    assert np.isclose((rms * rms * blk).sum(), out["loss_t"], rtol=1e-9)
    # the scale is the argmin of the exhaustive search on the normalized W~
    s_bf, c_bf, _ = O.e8_scale_search(Wn, C, nearest=O.e8_nearest_bruteforce)
    assert out["scale_choice"] == c_bf


def test_e8_nearest_exact_fallback_matches_exhaustive_far_outside_the_codebook():
    # Far from the origin the nearest lattice point is outside the codebook, so
    # every code comes from the exact codebook search.
    C = O.e8_codebook()
    Y = rng(303).standard_normal((400, 8)) * 3.0
    idx = O.E8Index(C)
    miss = idx.lookup(O.e8_decode(Y / 0.5)) < 0
    assert miss.mean() > 0.9
    k1, d1 = O.e8_nearest_bruteforce(Y, C, 0.5)
    k2, d2 = O.e8_nearest(Y, C, 0.5, idx)
    assert np.allclose(d1, d2, rtol=0, atol=1e-10)
