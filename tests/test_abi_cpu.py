"""The C-ABI library on the host: it loads, exports every symbol the header
declares, and rejects bad arguments before anything is enqueued (these calls
never reach the GPU). The host-side E8 codebook builder is compared with the
oracle's independent enumeration."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "quip.h")

Q = pytest.importorskip("post_weight_quantization_quip_amd", reason="libquip.so not built")
N = Q.native


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:quip_status|int32_t|const char\*)\s+(quip_\w+)\s*\(", text, re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_symbols()
    assert len(names) >= 20
    for name in names:
        assert hasattr(N.lib, name), name
        assert name in N.SYMBOLS, f"{name} has no binding"


def test_version_and_status_strings():
    assert N.lib.quip_version() == 10000
    assert N.lib.quip_status_string(0) == b"QUIP_OK"
    assert N.lib.quip_status_string(3) == b"QUIP_ERR_NOT_PD"


def fake(addr=0x1000):
    return ctypes.c_void_p(addr)


def test_rht_validation():
    lib = N.lib
    st = lib.quip_rht(fake(), fake(), 4, 12, 12, fake(), N.RIGHT, None)
    assert st == N.QUIP_ERR_SHAPE  # 12 is not a power of two
    assert b"power of two" in lib.quip_last_error()
    assert lib.quip_rht(None, fake(), 4, 16, 16, fake(), N.RIGHT, None) == N.QUIP_ERR_ARG
    assert lib.quip_rht(fake(), fake(), 4, 16, 8, fake(), N.RIGHT, None) == N.QUIP_ERR_ARG  # ld < cols
    assert lib.quip_rht(fake(), fake(), 4, 16, 16, fake(0x1004), N.RIGHT, None) == N.QUIP_ERR_ARG
    assert lib.quip_rht(fake(), fake(), 4, 16, 16, fake(), 7, None) == N.QUIP_ERR_ARG
    assert lib.quip_rht(fake(), fake(), 3, 16, 16, fake(), N.LEFT, None) == N.QUIP_ERR_SHAPE
    assert lib.quip_rht(fake(), fake(), 4, 32768, 32768, fake(), N.RIGHT, None) == N.QUIP_ERR_SHAPE
    assert lib.quip_rht2(fake(), fake(), 4, 12, 12, fake(), fake(), None) == N.QUIP_ERR_SHAPE


def test_kron_validation():
    lib = N.lib
    ws = ctypes.c_size_t(0)
    assert lib.quip_kron_orth_workspace(10, 24, ctypes.byref(ws)) == 0 and ws.value >= 240 * 4
    assert lib.quip_kron_orth(fake(), fake(), 10, 24, 24, fake(), 4, fake(), 5, N.RIGHT, fake(0x10000),
                              1 << 20, None) == N.QUIP_ERR_SHAPE  # 4*5 != 24
    assert lib.quip_kron_orth(fake(), fake(), 10, 24, 24, fake(), 4, fake(), 6, N.RIGHT, None,
                              0, None) == N.QUIP_ERR_WORKSPACE
    assert lib.quip_kron_orth(fake(), fake(), 10, 24, 24, fake(), 4, fake(), 6, N.RIGHT, fake(0x10010),
                              1 << 20, None) == N.QUIP_ERR_WORKSPACE  # misaligned
    assert lib.quip_kron_orth(fake(), fake(), 10, 24, 24, fake(), 0, fake(), 6, N.RIGHT, fake(0x10000),
                              1 << 20, None) == N.QUIP_ERR_SHAPE


def test_ldl_validation():
    lib = N.lib
    ws = ctypes.c_size_t(0)
    assert lib.quip_ldl_workspace(64, 8, ctypes.byref(ws)) == 0 and ws.value >= 64 * 64 * 4
    assert lib.quip_ldl_workspace(60, 8, ctypes.byref(ws)) == N.QUIP_ERR_SHAPE
    assert lib.quip_ldl(fake(), 64, 64, 3, fake(), fake(), fake(), fake(0x10000), 1 << 30, None) == N.QUIP_ERR_ARG
    assert lib.quip_ldl(fake(), 60, 64, 8, fake(), fake(), fake(), fake(0x10000), 1 << 30, None) == N.QUIP_ERR_SHAPE
    assert lib.quip_ldl(fake(), 64, 32, 1, fake(), fake(), fake(), fake(0x10000), 1 << 30, None) == N.QUIP_ERR_ARG
    assert lib.quip_ldl(fake(), 64, 64, 1, fake(), fake(), None, fake(0x10000), 1 << 30, None) == N.QUIP_ERR_ARG
    assert lib.quip_ldl(fake(), 64, 64, 1, fake(), fake(), fake(), fake(0x10000), 16, None) == N.QUIP_ERR_WORKSPACE


def test_ldlq_and_scales_validation():
    lib = N.lib
    q = N.quantizer(N.Q_UNIFORM, 2)
    big = fake(0x100000)
    st = lib.quip_ldlq(fake(), 4, 16, 16, fake(), fake(), 8, 8, ctypes.byref(q), fake(), fake(), None,
                       None, None, None, big, 1 << 40, None)
    assert st == N.QUIP_ERR_ARG  # scalar grid with g = 8
    qe = N.quantizer(N.Q_E8, 2)
    st = lib.quip_ldlq(fake(), 4, 20, 20, fake(), fake(), 8, 8, ctypes.byref(qe), fake(), fake(), None,
                       fake(), None, None, big, 1 << 40, None)
    assert st == N.QUIP_ERR_SHAPE  # n % 8
    st = lib.quip_ldlq(fake(), 4, 16, 16, fake(), fake(), 8, 8, ctypes.byref(qe), fake(), fake(), None,
                       None, None, None, big, 1 << 40, None)
    assert st == N.QUIP_ERR_ARG  # no codebook
    q9 = N.quantizer(N.Q_UNIFORM, 9)
    st = lib.quip_ldlq(fake(), 4, 16, 16, fake(), fake(), 1, 8, ctypes.byref(q9), fake(), fake(), None,
                       None, None, None, big, 1 << 40, None)
    assert st == N.QUIP_ERR_UNSUPPORTED
    qb = N.quantizer(N.Q_UNIFORM, 2, 1)
    assert lib.quip_scales(fake(), 4, 16, 16, ctypes.byref(qb), fake(), None, None, big, 1 << 40,
                           None) == N.QUIP_ERR_ARG  # n_cand < 2
    st = lib.quip_ldlq(fake(), 4, 16, 16, fake(), fake(), 1, 4, ctypes.byref(q), fake(), fake(), None,
                       None, None, None, big, 1 << 40, None)
    assert st == N.QUIP_ERR_SHAPE  # B < 8
    st = lib.quip_ldlq(fake(), 4, 16, 16, fake(), None, 1, 8, ctypes.byref(q), fake(), fake(), None,
                       None, fake(), None, big, 1 << 40, None)
    assert st == N.QUIP_ERR_ARG  # per-row loss needs D


def test_hessian_and_loss_validation():
    lib = N.lib
    assert lib.quip_hessian(fake(), -1, 4, 4, fake(), 4, 0, None, 0, None) == N.QUIP_ERR_ARG
    assert lib.quip_hessian(fake(), 8, 4, 3, fake(), 4, 0, None, 0, None) == N.QUIP_ERR_ARG
    assert lib.quip_hessian(fake(), 8, 4, 4, fake(), 4, 0, fake(0x10008), 64, None) == N.QUIP_ERR_ARG  # misaligned ws
    assert lib.quip_hessian_finalize(fake(), 4, 4, 0, 0.01, fake(0x10000), 256, None) == N.QUIP_ERR_ARG
    assert lib.quip_hessian_finalize(fake(), 4, 4, 8, -1.0, fake(0x10000), 256, None) == N.QUIP_ERR_ARG
    assert lib.quip_hessian_finalize(fake(), 4, 4, 8, 0.01, fake(0x10000), 8, None) == N.QUIP_ERR_WORKSPACE
    assert lib.quip_proxy_loss(fake(), fake(), 4, 4, 4, fake(), 4, None, fake(0x10000), 1 << 20,
                               None) == N.QUIP_ERR_ARG


def test_e8_codebook_matches_oracle_enumeration():
    cb = Q.quip_e8_codebook().numpy().astype(np.float64)
    assert np.array_equal(cb, O.e8_codebook())
    assert N.lib.quip_e8_codebook(None) == N.QUIP_ERR_ARG


def test_e8_codebook_shells_hold_negations_in_reverse_order():
    """The structure the E8 search's symmetric layout assumes of this codebook
    (the GPU checks the pairing again on every call and falls back to the
    plain search when it fails): the zero vector first, then the full shells of
    squared norm 2, 4, 6, 8, 10 (the theta series' 240, 2160, 6720, 17520,
    30240), each holding the negation of its i-th point at its (S - 1 - i)-th
    place, then the first 8655 points of the norm-12 shell."""
    cb = Q.quip_e8_codebook().numpy().astype(np.float64)
    norms = (cb * cb).sum(1)
    assert np.all(cb[0] == 0)
    a = 1
    for norm, size in zip((2, 4, 6, 8, 10), (240, 2160, 6720, 17520, 30240)):
        shell = cb[a:a + size]
        assert np.all(norms[a:a + size] == norm)
        assert np.array_equal(shell[::-1], -shell)
        a += size
    assert a == 56881
    assert np.all(norms[a:] == 12) and len(norms) - a == 8655


def test_packed_codes_and_inference_product_validation():
    lib = N.lib
    # row sizes: 2-, 4- or 8-bit containers
    assert [Q.quip_packed_row_bytes(13, b) for b in (1, 2, 3, 4, 5, 8)] == [4, 4, 7, 7, 13, 13]
    out = ctypes.c_int64(0)
    assert lib.quip_packed_row_bytes(13, 0, ctypes.byref(out)) == N.QUIP_ERR_ARG
    assert lib.quip_packed_row_bytes(0, 2, ctypes.byref(out)) == N.QUIP_ERR_ARG
    assert lib.quip_pack_codes(fake(), 4, 16, 8, 2, fake(), None) == N.QUIP_ERR_ARG  # ldc < n
    assert lib.quip_pack_codes(fake(), 4, 16, 16, 9, fake(), None) == N.QUIP_ERR_ARG
    assert lib.quip_pack_codes(fake(), 4, 16, 16, 2, None, None) == N.QUIP_ERR_ARG
    ws = ctypes.c_size_t(0)
    assert lib.quip_qmatvec_rht_workspace(4096, 4096, ctypes.byref(ws)) == N.QUIP_OK
    assert ws.value >= 4 * (4096 + 4096)
    big = fake(0x100000)

    def call(m, n, bits, x=fake(), wsp=big, wsb=1 << 20):
        return lib.quip_qmatvec_rht(fake(), m, n, bits, fake(), fake(), fake(), x, fake(), wsp, wsb,
                                    None)
    assert call(6, 1024, 2) == N.QUIP_ERR_SHAPE        # m not a power of two
    assert call(64, 512, 2) == N.QUIP_ERR_SHAPE        # n below 1024
    assert call(64, 32768, 2) == N.QUIP_ERR_SHAPE      # n above 16384
    assert call(64, 1024, 0) == N.QUIP_ERR_ARG         # bits
    assert call(64, 1024, 2, x=None) == N.QUIP_ERR_ARG
    assert call(64, 1024, 2, x=fake(0x1004)) == N.QUIP_ERR_ARG  # x not 16-byte aligned
    assert call(64, 1024, 2, wsb=16) == N.QUIP_ERR_WORKSPACE
    assert call(64, 1024, 2, wsp=fake(0x100010)) == N.QUIP_ERR_WORKSPACE  # not 256-byte aligned


def test_permute_and_diag_order_validation():
    lib = N.lib
    A, O_ = fake(0x1000), fake(0x100000)
    assert lib.quip_permute(A, 8, O_, 8, 0, 8, None, None, 0, None) == N.QUIP_OK  # empty
    assert lib.quip_permute(A, 8, O_, 8, -1, 8, None, None, 0, None) == N.QUIP_ERR_ARG
    assert lib.quip_permute(None, 8, O_, 8, 4, 8, None, None, 0, None) == N.QUIP_ERR_ARG
    assert lib.quip_permute(A, 4, O_, 8, 4, 8, None, None, 0, None) == N.QUIP_ERR_ARG  # lda < cols
    assert lib.quip_permute(A, 8, O_, 8, 4, 8, None, None, 2, None) == N.QUIP_ERR_ARG  # scatter flag
    assert lib.quip_permute(A, 8, fake(0x1010), 8, 4, 8, None, None, 0, None) == N.QUIP_ERR_ARG
    assert lib.quip_permute(A, 40000, O_, 40000, 1, 40000, None, fake(0x5000), 0,
                            None) == N.QUIP_ERR_SHAPE
    ws = ctypes.c_size_t(0)
    assert lib.quip_diag_order_workspace(4096, ctypes.byref(ws)) == N.QUIP_OK
    assert ws.value >= 4 * 4096 * 8
    assert lib.quip_diag_order_workspace(0, ctypes.byref(ws)) == N.QUIP_ERR_ARG
    assert lib.quip_diag_order(A, 16, 8, fake(), fake(0x100000), 1 << 20, None) == N.QUIP_ERR_ARG
    assert lib.quip_diag_order(A, 16, 16, None, fake(0x100000), 1 << 20, None) == N.QUIP_ERR_ARG
    assert lib.quip_diag_order(A, 16, 16, fake(), fake(0x100000), 4, None) == N.QUIP_ERR_WORKSPACE


def test_tcq_validation():
    lib = N.lib
    ws = ctypes.c_size_t(0)
    assert lib.quip_tcq_workspace(4096, 256, 15, ctypes.byref(ws)) == N.QUIP_OK
    assert ws.value >= 2048 * 256 * 2048  # back-pointers of one 2048-row round
    assert lib.quip_tcq_workspace(4096, 256, 16, ctypes.byref(ws)) == N.QUIP_ERR_UNSUPPORTED
    assert lib.quip_tcq_workspace(0, 256, 12, ctypes.byref(ws)) == N.QUIP_ERR_ARG
    big = fake(0x100000)

    def call(L=12, k=2, scale=1.0, X=fake(), ldx=256, lds=256, xh=fake(), ldq=256, wsb=1 << 40):
        return lib.quip_tcq_quantize(X, 8, 256, ldx, L, k, scale, fake(), lds, xh, ldq, fake(), big,
                                     wsb, None)
    assert call(k=3) == N.QUIP_ERR_UNSUPPORTED
    assert call(L=3) == N.QUIP_ERR_UNSUPPORTED
    assert call(scale=0.0) == N.QUIP_ERR_ARG
    assert call(scale=float("inf")) == N.QUIP_ERR_ARG
    assert call(X=None) == N.QUIP_ERR_ARG
    assert call(ldx=100) == N.QUIP_ERR_ARG
    assert call(lds=100) == N.QUIP_ERR_ARG
    assert call(ldq=100) == N.QUIP_ERR_ARG
    assert call(wsb=16) == N.QUIP_ERR_WORKSPACE


def test_peak_probe_validation():
    lib = N.lib
    assert lib.quip_peak_copy(fake(), fake(0x100000), -1, None) == N.QUIP_ERR_ARG
    assert lib.quip_peak_copy(None, fake(0x100000), 16, None) == N.QUIP_ERR_ARG
    assert lib.quip_peak_copy(fake(0x1004), fake(0x100000), 16, None) == N.QUIP_ERR_ARG  # misaligned
    assert lib.quip_peak_copy(fake(0x1000), fake(0x1010), 16, None) == N.QUIP_ERR_ARG  # overlap
    assert lib.quip_peak_copy(fake(), fake(0x100000), 0, None) == N.QUIP_OK  # nothing to do
    assert lib.quip_peak_compute(3, 10, fake(), None, None) == N.QUIP_ERR_ARG
    assert lib.quip_peak_compute(0, 0, fake(), None, None) == N.QUIP_ERR_ARG
    assert lib.quip_peak_compute(1, 10, None, None, None) == N.QUIP_ERR_ARG


def test_empty_sizes_are_rejected_before_any_launch():
    # a layer, a transform or a trellis of no rows or columns is an argument
    # error (the permutation and the copy probe treat it as nothing to do)
    lib = N.lib
    sz = ctypes.c_size_t(0)
    assert lib.quip_ldl_workspace(0, 1, ctypes.byref(sz)) == N.QUIP_ERR_SHAPE
    assert lib.quip_tcq_workspace(0, 8, 8, ctypes.byref(sz)) == N.QUIP_ERR_ARG
    assert lib.quip_tcq_workspace(4, 0, 8, ctypes.byref(sz)) == N.QUIP_ERR_ARG
    assert lib.quip_diag_order_workspace(0, ctypes.byref(sz)) == N.QUIP_ERR_ARG
    assert lib.quip_proxy_loss_workspace(0, 8, ctypes.byref(sz)) == N.QUIP_ERR_ARG
    assert lib.quip_qmatvec_rht_workspace(0, 1024, ctypes.byref(sz)) == N.QUIP_ERR_ARG
    assert lib.quip_rht(fake(), fake(), 0, 16, 16, fake(), N.RIGHT, None) == N.QUIP_ERR_ARG
    assert lib.quip_hessian_workspace(0, 0, ctypes.byref(sz)) == N.QUIP_ERR_ARG
