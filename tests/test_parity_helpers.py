"""CPU checks of the comparison rules the GPU parity tests apply (tests/parity.py),
on runs of the oracle itself: a run must pass against itself, a run whose
factors were rounded to float32 (what the GPU does) must pass with its
divergences explained, and planted mistakes must fail."""
import numpy as np
import pytest

import oracle as O
import workloads as wl
from tests import parity as P


def _f32_run(ref, L):
    """The oracle's LDLQ redone from float32 copies of H~ and W~ with the factors
    of the float32 H~ rounded to float32: the inputs a float32 pass works with."""
    Ht = ref["Ht"].astype(np.float32)
    Wt = ref["Wt"].astype(np.float32)
    U, D = O.udu_cholesky(Ht.astype(np.float64), 1)
    U32, D32 = U.astype(np.float32), D.astype(np.float32)
    s = np.asarray(ref["scales"], np.float32)
    codes, What = O.ldlq(Wt, U32, O.uniform_quantizer(s, L), g=1)
    return {"Wt": Wt, "H": Ht, "U": U32, "D": D32, "scales": s, "codes": codes,
            "What_t": What.astype(np.float32)}


@pytest.fixture(scope="module")
def c1_runs():
    L = wl.make_layer("c1")
    ref = O.quantize_layer(L.W, L.X, L.left, L.right, quant="uniform", bits=2)
    return ref, _f32_run(ref, 4)


def test_independent_run_rule_passes_a_run_against_itself(c1_runs):
    ref, _ = c1_runs
    gpu = {"Wt": ref["Wt"], "H": ref["Ht"], "U": ref["U"], "D": ref["D"], "scales": ref["scales"],
           "codes": ref["codes"], "What_t": ref["What_t"]}
    st = P.compare_independent_run(gpu, ref, g=1, L=4)
    assert st["diverged"] == 0 and st["extra_bound"] == 0.0


def test_independent_run_rule_explains_float32_factor_divergence(c1_runs):
    ref, run = c1_runs
    st = P.compare_independent_run(run, ref, g=1, L=4)
    assert st["rows"] == 256


def test_independent_run_rule_rejects_a_wrong_code(c1_runs):
    ref, run = c1_runs
    bad = dict(run)
    codes = run["codes"].copy()
    r, k = 5, 100
    codes[r, k] = (codes[r, k] + 2) % 4  # not an adjacent level, and not a near-tie
    bad["codes"] = codes
    with pytest.raises(AssertionError):
        P.compare_independent_run(bad, ref, g=1, L=4)


def test_independent_run_rule_rejects_a_loss_drift(c1_runs):
    ref, run = c1_runs
    bad = dict(run)
    bad["H"] = run["H"] * np.float32(1.001)  # every row's loss 1e-3 too large
    with pytest.raises(AssertionError):
        P.compare_independent_run(bad, ref, g=1, L=4)


def test_e8_scale_argmin_check_against_exhaustive_search():
    C = O.e8_codebook()
    Wn = wl.gaussian_rows(9, 64, 64)
    s, choice, sse = O.e8_scale_search(Wn, C, nearest=O.e8_nearest_bruteforce)
    ok, info = P.e8_scale_is_argmin(Wn, C, choice)
    assert ok
    assert abs(info[choice][1] - sse[choice]) <= 1e-9 * sse[choice]
    for c, (kind, v) in info.items():
        assert v <= sse[c] * (1 + 1e-9)  # bounds never exceed the exact error
        if kind == "exact":
            assert abs(v - sse[c]) <= 1e-9 * sse[c]
    worse = int(np.argsort(sse)[3])
    assert not P.e8_scale_is_argmin(Wn, C, worse)[0]
