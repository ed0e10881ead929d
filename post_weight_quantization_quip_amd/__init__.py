"""QuIP-family layer quantization on AMD Instinct MI355X (gfx950).

The pass (proxy Hessian, incoherence processing, LDL, LDLQ / BlockLDLQ, proxy
loss) runs in hand-written HIP kernels behind the C ABI in include/quip.h
(libquip.so). This package is the thin Python binding over that ABI.
"""
from . import _native as native  # noqa: F401  (fails loudly if libquip.so is missing)
from ._native import (LEFT, RIGHT, Q_E8, Q_UNIFORM, SCALE_COMPUTE, SCALE_GIVEN,  # noqa: F401
                      QuipError, quantizer, quip_e8_codebook, quip_hessian,
                      quip_hessian_finalize, quip_kron_orth, quip_kron_orth_inv, quip_ldl,
                      quip_diag_order, quip_ldlq, quip_pack_codes, quip_packed_row_bytes,
                      quip_peak_compute, quip_peak_copy, quip_permute, quip_proxy_loss,
                      quip_qmatvec_rht, quip_qmatvec_rht_noalloc, quip_rht, quip_rht2, quip_rht2_inv, quip_rht_inv,
                      quip_scales, quip_tcq_quantize, timing_enable, timing_report, timing_reset)
from .pipeline import LayerPass, SideSpec, apply_side, apply_two_sided, quantize_layer  # noqa: F401

__all__ = [
    "LEFT", "RIGHT", "Q_E8", "Q_UNIFORM", "SCALE_COMPUTE", "SCALE_GIVEN", "QuipError", "quantizer",
    "quip_e8_codebook", "quip_hessian", "quip_hessian_finalize", "quip_kron_orth",
    "quip_kron_orth_inv", "quip_ldl", "quip_diag_order", "quip_peak_compute", "quip_peak_copy", "quip_permute", "quip_ldlq", "quip_pack_codes", "quip_packed_row_bytes",
    "quip_proxy_loss", "quip_qmatvec_rht", "quip_qmatvec_rht_noalloc", "quip_rht", "quip_rht2",
    "quip_rht2_inv", "quip_rht_inv", "quip_scales", "quip_tcq_quantize", "LayerPass", "SideSpec", "apply_side",
    "apply_two_sided", "quantize_layer", "timing_enable", "timing_report", "timing_reset",
]
