"""ctypes binding of libquip (include/quip.h): argument marshalling only.

Every function takes torch tensors that already live on the GPU, passes their
device pointers, sizes and leading dimensions to the C ABI together with the
current HIP stream, and raises ``QuipError`` on a non-OK status. Workspaces
are sized by the library's own queries and allocated through torch's caching
allocator. No arithmetic of the pass happens here: if the library is missing,
importing this module fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("QUIP_LIB", os.path.join(_HERE, "libquip.so"))

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libquip.so not found at {LIB_PATH}; build it with "
        "`python post_weight_quantization_quip_amd/build.py` (hipcc, gfx950)")

lib = ctypes.CDLL(LIB_PATH)

c_i64 = ctypes.c_int64
c_int = ctypes.c_int
c_f = ctypes.c_float
c_vp = ctypes.c_void_p
c_sz = ctypes.c_size_t

QUIP_OK, QUIP_ERR_ARG, QUIP_ERR_SHAPE, QUIP_ERR_NOT_PD, QUIP_ERR_HIP, QUIP_ERR_UNSUPPORTED, \
    QUIP_ERR_WORKSPACE = range(7)
LEFT, RIGHT = 0, 1
Q_UNIFORM, Q_E8 = 0, 1
SCALE_COMPUTE, SCALE_GIVEN = 0, 1


class Quantizer(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("bits", ctypes.c_int32), ("n_cand", ctypes.c_int32),
                ("scale_mode", ctypes.c_int32)]


SYMBOLS = {
    "quip_version": (ctypes.c_int32, []),
    "quip_status_string": (ctypes.c_char_p, [c_int]),
    "quip_last_error": (ctypes.c_char_p, []),
    "quip_hessian_workspace": (c_int, [c_i64, c_i64, ctypes.POINTER(c_sz)]),
    "quip_hessian": (c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_int, c_vp, c_sz, c_vp]),
    "quip_hessian_finalize": (c_int, [c_vp, c_i64, c_i64, c_i64, c_f, c_vp, c_sz, c_vp]),
    "quip_rht": (c_int, [c_vp, c_vp, c_i64, c_i64, c_i64, c_vp, c_int, c_vp]),
    "quip_rht_inv": (c_int, [c_vp, c_vp, c_i64, c_i64, c_i64, c_vp, c_int, c_vp]),
    "quip_rht2": (c_int, [c_vp, c_vp, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp]),
    "quip_rht2_inv": (c_int, [c_vp, c_vp, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp]),
    "quip_kron_orth_workspace": (c_int, [c_i64, c_i64, ctypes.POINTER(c_sz)]),
    "quip_kron_orth": (c_int, [c_vp, c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_i64, c_int,
                               c_vp, c_sz, c_vp]),
    "quip_kron_orth_inv": (c_int, [c_vp, c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_i64,
                                   c_int, c_vp, c_sz, c_vp]),
    "quip_ldl_workspace": (c_int, [c_i64, c_i64, ctypes.POINTER(c_sz)]),
    "quip_ldl": (c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_sz, c_vp]),
    "quip_scales_workspace": (c_int, [c_i64, c_i64, ctypes.POINTER(Quantizer), ctypes.POINTER(c_sz)]),
    "quip_scales": (c_int, [c_vp, c_i64, c_i64, c_i64, ctypes.POINTER(Quantizer), c_vp, c_vp, c_vp,
                            c_vp, c_sz, c_vp]),
    "quip_ldlq_workspace": (c_int, [c_i64, c_i64, c_i64, c_i64, ctypes.POINTER(Quantizer),
                                    ctypes.POINTER(c_sz)]),
    "quip_ldlq": (c_int, [c_vp, c_i64, c_i64, c_i64, c_vp, c_vp, c_i64, c_i64,
                          ctypes.POINTER(Quantizer), c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_sz,
                          c_vp]),
    "quip_proxy_loss_workspace": (c_int, [c_i64, c_i64, ctypes.POINTER(c_sz)]),
    "quip_proxy_loss": (c_int, [c_vp, c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_vp, c_sz,
                                c_vp]),
    "quip_e8_codebook": (c_int, [c_vp]),
    "quip_packed_row_bytes": (c_int, [c_i64, ctypes.c_int32, ctypes.POINTER(c_i64)]),
    "quip_pack_codes": (c_int, [c_vp, c_i64, c_i64, c_i64, ctypes.c_int32, c_vp, c_vp]),
    "quip_qmatvec_rht_workspace": (c_int, [c_i64, c_i64, ctypes.POINTER(c_sz)]),
    "quip_qmatvec_rht": (c_int, [c_vp, c_i64, c_i64, ctypes.c_int32, c_vp, c_vp, c_vp, c_vp, c_vp,
                                 c_vp, c_sz, c_vp]),
    "quip_qmatvec_rht_noalloc": (c_int, [c_vp, c_i64, c_i64, ctypes.c_int32, c_vp, c_vp, c_vp, c_vp,
                                         c_vp, c_vp]),
    "quip_permute": (c_int, [c_vp, c_i64, c_vp, c_i64, c_i64, c_i64, c_vp, c_vp, ctypes.c_int32,
                             c_vp]),
    "quip_diag_order_workspace": (c_int, [c_i64, ctypes.POINTER(c_sz)]),
    "quip_diag_order": (c_int, [c_vp, c_i64, c_i64, c_vp, c_vp, c_sz, c_vp]),
    "quip_tcq_workspace": (c_int, [c_i64, c_i64, ctypes.c_int32, ctypes.POINTER(c_sz)]),
    "quip_tcq_quantize": (c_int, [c_vp, c_i64, c_i64, c_i64, ctypes.c_int32, ctypes.c_int32, c_f,
                                  c_vp, c_i64, c_vp, c_i64, c_vp, c_vp, c_sz, c_vp]),
    "quip_peak_copy": (c_int, [c_vp, c_vp, c_i64, c_vp]),
    "quip_peak_compute": (c_int, [ctypes.c_int32, c_i64, c_vp, ctypes.POINTER(ctypes.c_double), c_vp]),
    "quip_timing_enable": (c_int, [c_int]),
    "quip_timing_reset": (c_int, []),
    "quip_timing_report": (c_int, [ctypes.c_char_p, c_sz, ctypes.POINTER(c_sz)]),
}

for _name, (_res, _args) in SYMBOLS.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class QuipError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib.quip_last_error().decode() or lib.quip_status_string(status).decode()
        super().__init__(f"{where}: {lib.quip_status_string(status).decode()}: {msg}")
        self.status = status


def _check(st: int, where: str):
    if st != QUIP_OK:
        raise QuipError(st, where)


def _p(t):
    return None if t is None else c_vp(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return c_vp(s.cuda_stream)


def _ld(t: torch.Tensor) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError("expected a row-major 2-D tensor (unit column stride)")
    return t.stride(0)


def _workspace(nbytes: int, device) -> torch.Tensor | None:
    if nbytes == 0:
        return None
    ws = torch.empty(nbytes + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    return ws[off:off + nbytes]


def _ws_query(fn, *args) -> int:
    out = c_sz(0)
    _check(fn(*args, ctypes.byref(out)), fn.__name__)
    return out.value


def version() -> int:
    return lib.quip_version()


# ---------------------------------------------------------------- entry points

def quip_hessian(X: torch.Tensor, H: torch.Tensor, accumulate: bool = False, stream=None, ws=None):
    N, n = X.shape
    if ws is None:
        need = _ws_query(lib.quip_hessian_workspace, N, n)
        ws = _workspace(need, X.device) if need > 0 else None
    _check(lib.quip_hessian(_p(X), N, n, _ld(X), _p(H), _ld(H), int(accumulate), _p(ws),
                            0 if ws is None else ws.numel(), _stream(stream)),
           "quip_hessian")


def quip_hessian_finalize(H: torch.Tensor, N_total: int, alpha: float, stream=None, ws=None):
    n = H.shape[0]
    ws = _workspace(256, H.device) if ws is None else ws
    _check(lib.quip_hessian_finalize(_p(H), n, n if H.dim() == 1 else _ld(H), N_total, alpha,
                                     _p(ws), ws.numel(), _stream(stream)),
           "quip_hessian_finalize")


def quip_rht(A, out, signs, side: int, stream=None):
    r, c = A.shape
    _check(lib.quip_rht(_p(A), _p(out), r, c, _ld(A), _p(signs), side, _stream(stream)), "quip_rht")


def quip_rht_inv(A, out, signs, side: int, stream=None):
    r, c = A.shape
    _check(lib.quip_rht_inv(_p(A), _p(out), r, c, _ld(A), _p(signs), side, _stream(stream)),
           "quip_rht_inv")


def quip_rht2(A, out, signs_left, signs_right, stream=None):
    r, c = A.shape
    _check(lib.quip_rht2(_p(A), _p(out), r, c, _ld(A), _p(signs_left), _p(signs_right),
                         _stream(stream)), "quip_rht2")


def quip_rht2_inv(A, out, signs_left, signs_right, stream=None):
    r, c = A.shape
    _check(lib.quip_rht2_inv(_p(A), _p(out), r, c, _ld(A), _p(signs_left), _p(signs_right),
                             _stream(stream)), "quip_rht2_inv")


def _kron(fn, A, out, F1, F2, side, stream, ws):
    r, c = A.shape
    if ws is None:
        ws = _workspace(_ws_query(lib.quip_kron_orth_workspace, r, c), A.device)
    _check(fn(_p(A), _p(out), r, c, _ld(A), _p(F1), F1.shape[0], _p(F2), F2.shape[0], side, _p(ws),
              0 if ws is None else ws.numel(), _stream(stream)), fn.__name__)


def quip_kron_orth(A, out, F1, F2, side: int, stream=None, ws=None):
    _kron(lib.quip_kron_orth, A, out, F1, F2, side, stream, ws)


def quip_kron_orth_inv(A, out, F1, F2, side: int, stream=None, ws=None):
    _kron(lib.quip_kron_orth_inv, A, out, F1, F2, side, stream, ws)


def quip_ldl(H, g: int, U, D, info, stream=None, ws=None):
    n = H.shape[0]
    if ws is None:
        ws = _workspace(_ws_query(lib.quip_ldl_workspace, n, g), H.device)
    _check(lib.quip_ldl(_p(H), n, _ld(H), g, _p(U), _p(D), _p(info), _p(ws), ws.numel(),
                        _stream(stream)), "quip_ldl")


def quantizer(kind: int, bits: int, n_cand: int = 32, scale_mode: int = SCALE_COMPUTE) -> Quantizer:
    return Quantizer(kind, bits, n_cand, scale_mode)


def quip_scales(W, q: Quantizer, scales, mse_out=None, codebook=None, stream=None, ws=None):
    m, n = W.shape
    if ws is None:
        ws = _workspace(_ws_query(lib.quip_scales_workspace, m, n, ctypes.byref(q)), W.device)
    _check(lib.quip_scales(_p(W), m, n, _ld(W), ctypes.byref(q), _p(scales), _p(mse_out),
                           _p(codebook), _p(ws), 0 if ws is None else ws.numel(), _stream(stream)),
           "quip_scales")


def quip_ldlq(W, U, D, g: int, B: int, q: Quantizer, scales, codes, What=None, codebook=None,
              row_loss=None, loss=None, stream=None, ws=None):
    m, n = W.shape
    if ws is None:
        ws = _workspace(_ws_query(lib.quip_ldlq_workspace, m, n, g, B, ctypes.byref(q)), W.device)
    _check(lib.quip_ldlq(_p(W), m, n, _ld(W), _p(U), _p(D), g, B, ctypes.byref(q), _p(scales),
                         _p(codes), _p(What), _p(codebook), _p(row_loss), _p(loss), _p(ws),
                         ws.numel(), _stream(stream)),
           "quip_ldlq")


def quip_proxy_loss(W, What, H, loss, stream=None, ws=None):
    m, n = W.shape
    if _ld(W) != _ld(What):
        raise ValueError("W and What must share a leading dimension")
    if ws is None:
        ws = _workspace(_ws_query(lib.quip_proxy_loss_workspace, m, n), W.device)
    _check(lib.quip_proxy_loss(_p(W), _p(What), m, n, _ld(W), _p(H), _ld(H), _p(loss), _p(ws),
                               ws.numel(), _stream(stream)), "quip_proxy_loss")


def quip_e8_codebook() -> torch.Tensor:
    """The 65536 x 8 codebook in host memory (float32)."""
    out = torch.empty((65536, 8), dtype=torch.float32)
    _check(lib.quip_e8_codebook(c_vp(out.data_ptr())), "quip_e8_codebook")
    return out


def quip_packed_row_bytes(n: int, bits: int) -> int:
    out = c_i64(0)
    _check(lib.quip_packed_row_bytes(n, bits, ctypes.byref(out)), "quip_packed_row_bytes")
    return out.value


def quip_pack_codes(codes, bits: int, packed, stream=None):
    m, n = codes.shape
    _check(lib.quip_pack_codes(_p(codes), m, n, _ld(codes), bits, _p(packed), _stream(stream)),
           "quip_pack_codes")


def quip_qmatvec_rht(packed, n: int, bits: int, scales, signs_left, signs_right, x, y,
                     stream=None, ws=None):
    m = scales.numel()
    if ws is None:
        ws = _workspace(_ws_query(lib.quip_qmatvec_rht_workspace, m, n), x.device)
    _check(lib.quip_qmatvec_rht(_p(packed), m, n, bits, _p(scales), _p(signs_left),
                                _p(signs_right), _p(x), _p(y), _p(ws),
                                0 if ws is None else ws.numel(), _stream(stream)),
           "quip_qmatvec_rht")


def quip_qmatvec_rht_noalloc(packed, n: int, bits: int, scales, signs_left, signs_right, x, y,
                             stream=None):
    """quip_qmatvec_rht with its scratch in the library's static device array:
    no workspace, no allocation (calls that overlap on one GPU race)."""
    m = scales.numel()
    _check(lib.quip_qmatvec_rht_noalloc(_p(packed), m, n, bits, _p(scales), _p(signs_left),
                                        _p(signs_right), _p(x), _p(y), _stream(stream)),
           "quip_qmatvec_rht_noalloc")


def quip_permute(A, out, row_index=None, col_index=None, scatter: bool = False, stream=None):
    """Gather out = A[row_index][:, col_index], or scatter out[row_index][:, col_index] = A
    (int32 index tensors on the device; None is the identity)."""
    r, c = A.shape
    _check(lib.quip_permute(_p(A), _ld(A), _p(out), _ld(out), r, c, _p(row_index), _p(col_index),
                            int(scatter), _stream(stream)), "quip_permute")


def quip_diag_order(H, order, stream=None, ws=None):
    """order = the columns of H by decreasing H[j][j], ties by index (int32)."""
    n = H.shape[0]
    if ws is None:
        ws = _workspace(_ws_query(lib.quip_diag_order_workspace, n), H.device)
    _check(lib.quip_diag_order(_p(H), n, _ld(H), _p(order), _p(ws), 0 if ws is None else ws.numel(),
                               _stream(stream)), "quip_diag_order")


def quip_tcq_quantize(X, L: int, states, cost, Xhat=None, k: int = 2, scale: float = 1.0,
                      stream=None, ws=None):
    """Bitshift-trellis quantization of the rows of X: states (uint16, rows x T),
    the row minima (float32), optionally the values c(states)."""
    rows, T = X.shape
    if ws is None:
        ws = _workspace(_ws_query(lib.quip_tcq_workspace, rows, T, L), X.device)
    _check(lib.quip_tcq_quantize(_p(X), rows, T, _ld(X), L, k, scale, _p(states), _ld(states),
                                 _p(Xhat), _ld(Xhat) if Xhat is not None else T, _p(cost), _p(ws),
                                 0 if ws is None else ws.numel(), _stream(stream)),
           "quip_tcq_quantize")


def quip_peak_copy(src, dst, stream=None) -> None:
    """dst = src (float32, same size, device): the HBM copy probe."""
    if src.numel() != dst.numel():
        raise ValueError("quip_peak_copy: src and dst sizes differ")
    _check(lib.quip_peak_copy(_p(src), _p(dst), src.numel(), _stream(stream)), "quip_peak_copy")


def quip_peak_compute(kind: int, iters: int, out, stream=None) -> float:
    """One launch of the compute probe (0: fp32 MFMA, 1: f16 MFMA, 2: fp32
    vector FMA); returns its flop count."""
    flops = ctypes.c_double(0.0)
    _check(lib.quip_peak_compute(kind, iters, _p(out), ctypes.byref(flops), _stream(stream)),
           "quip_peak_compute")
    return flops.value


def timing_enable(on: bool = True) -> None:
    """Per-kernel event timing inside the library (measurement support)."""
    _check(lib.quip_timing_enable(int(on)), "quip_timing_enable")


def timing_reset() -> None:
    _check(lib.quip_timing_reset(), "quip_timing_reset")


def timing_report() -> dict:
    """{kernel family: (launches, total_ms, flops, bytes)} since the last reset."""
    need = c_sz(0)
    _check(lib.quip_timing_report(None, 0, ctypes.byref(need)), "quip_timing_report")
    buf = ctypes.create_string_buffer(need.value + 64)
    _check(lib.quip_timing_report(buf, len(buf), ctypes.byref(need)), "quip_timing_report")
    out = {}
    for line in buf.value.decode().splitlines():
        name, count, ms, flops, nbytes = line.split()
        out[name] = (int(count), float(ms), float(flops), float(nbytes))
    return out
