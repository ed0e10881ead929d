"""The whole layer pass, driven through the C ABI.

Order of the calls (every step runs in libquip's kernels; this module only
allocates buffers once and sequences the calls on one HIP stream):

  quip_hessian -> quip_hessian_finalize          H = X^T X / N + damping
  quip_rht2 / quip_kron_orth (right, then left)   H~ = V H V^T   (in place)
  quip_rht2 / quip_kron_orth                      W~ = U W V^T
  quip_ldl                                        H~ = (I+U) D (I+U)^T
  quip_ldlq                                       scales, codes, W^~ and the proxy
                                                  loss tr((W^~ - W~) H~ (W^~ - W~)^T)
                                                  per row and summed
  quip_rht2_inv / quip_kron_orth_inv              W^ = U^T W^~ V

Variants ([QuIP] "Further Ablation" and "Experiments / Methods"):
  * a side with a permutation p: its transform is K P_p. quip_permute gathers
    the coordinates before the transform (H on both sides, W on that side)
    and scatters them back after the inverse transform;
  * rg_order (LDLQ-RG's order): quip_diag_order gives the order of decreasing
    diag(H~); quip_permute gathers H~ (both sides) and W~'s columns in that
    order before the LDL, and scatters W^~'s columns back before the inverse
    transforms. H, Wt, What_t, codes and scales stay in quantization order.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

from . import _native as N


@dataclass
class SideSpec:
    """Incoherence transform of one side: random signs (RHT) or two factors."""

    signs: torch.Tensor | None = None
    F1: torch.Tensor | None = None
    F2: torch.Tensor | None = None
    perm: torch.Tensor | None = None  # int32: coordinates permuted before the transform

    @property
    def is_rht(self) -> bool:
        return self.signs is not None

    @staticmethod
    def from_numpy(spec: dict, device) -> "SideSpec":
        perm = None
        if spec.get("perm") is not None:
            perm = torch.as_tensor(spec["perm"], dtype=torch.int32).to(device).contiguous()
        if "signs" in spec:
            return SideSpec(signs=torch.as_tensor(spec["signs"], dtype=torch.float32).to(device),
                            perm=perm)
        return SideSpec(F1=torch.as_tensor(spec["A"], dtype=torch.float32).to(device).contiguous(),
                        F2=torch.as_tensor(spec["B"], dtype=torch.float32).to(device).contiguous(),
                        perm=perm)


def apply_side(A: torch.Tensor, out: torch.Tensor, side: int, spec: SideSpec, inverse: bool,
               ws=None, stream=None):
    if spec.is_rht:
        (N.quip_rht_inv if inverse else N.quip_rht)(A, out, spec.signs, side, stream=stream)
    else:
        (N.quip_kron_orth_inv if inverse else N.quip_kron_orth)(A, out, spec.F1, spec.F2, side,
                                                                stream=stream, ws=ws)


def apply_two_sided(A, out, left: SideSpec, right: SideSpec, inverse: bool, ws=None, stream=None):
    """out = Q_L A Q_R^T (inverse: Q_L^T A Q_R)."""
    if left.is_rht and right.is_rht:
        (N.quip_rht2_inv if inverse else N.quip_rht2)(A, out, left.signs, right.signs, stream=stream)
        return
    if not inverse:
        apply_side(A, out, N.RIGHT, right, False, ws, stream)
        apply_side(out, out, N.LEFT, left, False, ws, stream)
    else:
        apply_side(A, out, N.LEFT, left, True, ws, stream)
        apply_side(out, out, N.RIGHT, right, True, ws, stream)


@dataclass
class LayerPass:
    """Preallocated buffers for repeated passes over layers of one shape."""

    m: int
    n: int
    left: SideSpec
    right: SideSpec
    quant: str = "uniform"
    bits: int = 2
    B: int = 128
    g: int = 1
    alpha: float = 0.01
    n_cand: int = 32
    device: str = "cuda"
    codebook: torch.Tensor | None = None
    rg_order: bool = False
    buffers: dict = field(default_factory=dict)

    def __post_init__(self):
        m, n, dev = self.m, self.n, self.device
        f32 = dict(dtype=torch.float32, device=dev)
        b = self.buffers
        b["H"] = torch.empty((n, n), **f32)
        b["Wt"] = torch.empty((m, n), **f32)
        b["U"] = torch.empty((n, n), **f32)
        b["D"] = torch.empty((n * 8,) if self.g == 8 else (n,), **f32)
        b["info"] = torch.zeros(1, dtype=torch.int32, device=dev)
        if self.quant == "uniform":
            self.q = N.quantizer(N.Q_UNIFORM, self.bits, self.n_cand, N.SCALE_COMPUTE)
            b["scales"] = torch.empty(m, **f32)
            b["codes"] = torch.empty((m, n), dtype=torch.uint8, device=dev)
        else:
            self.q = N.quantizer(N.Q_E8, 2, self.n_cand, N.SCALE_COMPUTE)
            b["scales"] = torch.empty(m + 1, **f32)
            b["codes"] = torch.empty((m, n // 8), dtype=torch.int16, device=dev)
            if self.codebook is None:
                self.codebook = N.quip_e8_codebook().to(dev)
        b["What_t"] = torch.empty((m, n), **f32)
        b["What"] = torch.empty((m, n), **f32)
        b["loss"] = torch.zeros(1, dtype=torch.float64, device=dev)
        b["row_loss"] = torch.zeros(m, dtype=torch.float64, device=dev)
        self.side_perm = self.left.perm is not None or self.right.perm is not None
        if self.right.perm is not None or self.rg_order:
            b["Htmp"] = torch.empty((n, n), **f32)
        if self.side_perm or self.rg_order:
            b["Wtmp"] = torch.empty((m, n), **f32)
        if self.rg_order:
            b["order"] = torch.empty(n, dtype=torch.int32, device=dev)
            b["ws_order"] = N._workspace(N._ws_query(N.lib.quip_diag_order_workspace, n), dev)
        # workspaces, sized once
        need = [256]
        need.append(N._ws_query(N.lib.quip_ldl_workspace, n, self.g))
        import ctypes
        need.append(N._ws_query(N.lib.quip_ldlq_workspace, m, n, self.g, self.B, ctypes.byref(self.q)))
        need.append(N._ws_query(N.lib.quip_kron_orth_workspace, max(m, n), max(m, n)))
        b["ws"] = N._workspace(max(need), dev)

    def _hessian_ws(self, n_rows: int):
        """Workspace for the split leftover tiles of X^T X; kept for the largest
        calibration size seen (allocated on the first pass of that size)."""
        need = N._ws_query(N.lib.quip_hessian_workspace, n_rows, self.n)
        ws = self.buffers.get("ws_h")
        if need > 0 and (ws is None or ws.numel() < need):
            ws = N._workspace(need, self.device)
            self.buffers["ws_h"] = ws
        return ws if need > 0 else None

    def run(self, W: torch.Tensor, X: torch.Tensor, events: dict | None = None, stream=None,
            with_loss: bool = True) -> dict:
        """One pass. ``events`` (optional) receives torch.cuda.Event pairs per phase."""
        b = self.buffers
        ws = b["ws"]

        def mark(name):
            if events is not None:
                ev = torch.cuda.Event(enable_timing=True)
                ev.record(stream)
                events.setdefault(name, []).append(ev)

        mark("hessian")
        N.quip_hessian(X, b["H"], accumulate=False, stream=stream, ws=self._hessian_ws(X.shape[0]))
        N.quip_hessian_finalize(b["H"], X.shape[0], self.alpha, stream=stream, ws=ws)
        mark("incoherence_H")
        rp = self.right.perm
        if rp is not None:  # V = K P: permute both sides of H, then transform
            N.quip_permute(b["H"], b["Htmp"], rp, rp, stream=stream)
            apply_two_sided(b["Htmp"], b["H"], self.right, self.right, False, ws, stream)
        else:
            apply_two_sided(b["H"], b["H"], self.right, self.right, False, ws, stream)
        if self.rg_order:
            N.quip_diag_order(b["H"], b["order"], stream=stream, ws=b["ws_order"])
            N.quip_permute(b["H"], b["Htmp"], b["order"], b["order"], stream=stream)
            b["H"], b["Htmp"] = b["Htmp"], b["H"]
        mark("incoherence_W")
        if self.side_perm:
            N.quip_permute(W, b["Wtmp"], self.left.perm, rp, stream=stream)
            apply_two_sided(b["Wtmp"], b["Wt"], self.left, self.right, False, ws, stream)
        else:
            apply_two_sided(W, b["Wt"], self.left, self.right, False, ws, stream)
        if self.rg_order:
            N.quip_permute(b["Wt"], b["Wtmp"], None, b["order"], stream=stream)
            b["Wt"], b["Wtmp"] = b["Wtmp"], b["Wt"]
        mark("ldl")
        N.quip_ldl(b["H"], self.g, b["U"], b["D"], b["info"], stream=stream, ws=ws)
        mark("ldlq")
        # the proxy loss comes out of the rounding (per row and summed)
        N.quip_ldlq(b["Wt"], b["U"], b["D"], self.g, self.B, self.q, b["scales"], b["codes"],
                    b["What_t"], self.codebook, row_loss=b["row_loss"] if with_loss else None,
                    loss=b["loss"] if with_loss else None, stream=stream, ws=ws)
        mark("postprocess")
        src = b["What_t"]
        if self.rg_order:  # back to the transformed basis's column order
            N.quip_permute(src, b["Wtmp"], None, b["order"], scatter=True, stream=stream)
            src = b["Wtmp"]
        apply_two_sided(src, b["What"], self.left, self.right, True, ws, stream)
        if self.side_perm:  # undo the permutations of the sides: P_L^T (.) P_R
            N.quip_permute(b["What"], b["Wtmp"], self.left.perm, rp, scatter=True, stream=stream)
            b["What"], b["Wtmp"] = b["Wtmp"], b["What"]
        mark("end")
        return b


def quantize_layer(W: torch.Tensor, X: torch.Tensor, left: dict, right: dict, **kw) -> dict:
    """Convenience wrapper: one pass with fresh buffers. ``left``/``right`` are
    the workload dicts ({"signs": ...} or {"A": ..., "B": ...})."""
    dev = W.device
    lp = LayerPass(W.shape[0], W.shape[1], SideSpec.from_numpy(left, dev),
                   SideSpec.from_numpy(right, dev), device=dev, **kw)
    out = lp.run(W, X)
    info = int(out["info"].item())
    if info:
        raise N.QuipError(N.QUIP_ERR_NOT_PD, f"quip_ldl: pivot {info - 1} is not positive")
    return out
