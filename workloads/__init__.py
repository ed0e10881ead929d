"""Seeded synthetic layers for the QuIP-family layer-quantization pass.

This module only draws random numbers. It holds none of the method's
arithmetic (no Hessian, no transform, no factorization, no rounding), so
both the CPU oracle and the HIP path may consume it. Every random quantity
the method needs (the Rademacher sign vectors of the randomized Hadamard
transform, the Haar-random Kronecker factors) is drawn here and handed to
both sides as an input.

Stand-in note: the QuIP paper (Chee et al., "Experiments / Setup") quantizes
OPT and Llama 2 layers with 128 C4 segments of 2048 tokens as calibration
data. No model, dataset or checkpoint is available here, so these generators
stand in for them with the shapes of attention and MLP projections and with
heavy-tailed columns and outlier weights (the situation the paper's
incoherence processing is meant to fix).

Seeding: every array is drawn from
``np.random.default_rng(np.random.SeedSequence([20261203, cfg_id, stream]))``
with one stream per quantity (see ``STREAMS``). Large arrays are drawn
directly in float32; the float32 arrays are the definition of the workload.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

ROOT_SEED = 20261203

STREAMS = {
    "w_base": 0,
    "w_row_sigma": 1,
    "w_outlier": 2,
    "x_base": 3,
    "x_col_scale": 4,
    "sign_left": 5,
    "sign_right": 6,
    "kron_left_a": 7,
    "kron_left_b": 8,
    "kron_right_a": 9,
    "kron_right_b": 10,
    "perm_left": 11,
    "perm_right": 12,
}


def rng_for(cfg_id: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([ROOT_SEED, int(cfg_id), int(stream)]))


@dataclass(frozen=True)
class Side:
    """How one side of W is made incoherent: ``("rht",)`` or ``("kron", p, q)``;
    ``perm``: a random permutation of the coordinates before the transform."""

    kind: str
    p: int = 0
    q: int = 0
    perm: bool = False

    def __post_init__(self):
        if self.kind not in ("rht", "kron", "none"):
            raise ValueError(self.kind)


RHT = Side("rht")


def KRON(p: int, q: int, perm: bool = False) -> Side:
    return Side("kron", p, q, perm)


@dataclass(frozen=True)
class LayerConfig:
    name: str
    cfg_id: int
    m: int  # rows of W (outputs)
    n: int  # columns of W (inputs) = Hessian side
    N: int  # calibration rows of X
    left: Side
    right: Side
    quant: str  # "uniform" or "e8"
    bits: int
    B: int  # lazy block size of the LDLQ sweep
    g: int = 1  # group size (8 for the E8 block variant)
    alpha: float = 0.01
    w_outlier_p: float = 0.01
    w_outlier_mult: float = 10.0
    w_row_sigma: float = 0.0  # log-normal sigma of per-row std (0: none)
    x_col_sigma: float = 1.0  # log-normal sigma of per-column scale of X
    rg_order: bool = False  # quantize the columns in decreasing diag(H~) order
    description: str = ""


CONFIGS = {
    "c1": LayerConfig("c1", 1, 256, 256, 2048, RHT, RHT, "uniform", 2, 32,
                      description="tiny layer 256x256, 2-bit, RHT both sides, B=32"),
    "c2": LayerConfig("c2", 2, 4096, 4096, 4096, RHT, RHT, "uniform", 2, 128,
                      w_outlier_p=0.005, w_outlier_mult=20.0, w_row_sigma=0.5, x_col_sigma=1.5,
                      description="attention projection 4096x4096, 2-bit, RHT both sides, B=128"),
    "c3a": LayerConfig("c3a", 31, 11008, 4096, 8192, KRON(64, 172), RHT, "uniform", 3, 128,
                       description="MLP 11008x4096, 3-bit, Kron 64x172 left, RHT right"),
    "c3b": LayerConfig("c3b", 32, 4096, 11008, 8192, RHT, KRON(64, 172), "uniform", 3, 128,
                       description="MLP 4096x11008, 3-bit, RHT left, Kron 64x172 right"),
    "c4a": LayerConfig("c4a", 41, 8192, 8192, 16384, RHT, RHT, "uniform", 4, 256,
                       description="large 8192x8192, 4-bit, RHT both sides, B=256"),
    "c4b": LayerConfig("c4b", 42, 28672, 8192, 16384, KRON(128, 224), RHT, "uniform", 4, 256,
                       description="large 28672x8192, 4-bit, Kron 128x224 left, RHT right"),
    "c4c": LayerConfig("c4c", 43, 8192, 28672, 16384, RHT, KRON(128, 224), "uniform", 4, 256,
                       description="large 8192x28672, 4-bit, RHT left, Kron 128x224 right"),
    "c3p": LayerConfig("c3p", 33, 4096, 11008, 8192, RHT, KRON(64, 172, perm=True), "uniform", 3,
                       128, rg_order=True,
                       description="MLP 4096x11008, 3-bit, RHT left, Kron 64x172 right with a random "
                                   "permutation, LDLQ-RG order"),
    "c5": LayerConfig("c5", 5, 4096, 4096, 4096, RHT, RHT, "e8", 2, 128, g=8,
                      description="vector BlockLDLQ 4096x4096, E8 2^16 codebook, g=8, B=128"),
}


@dataclass
class Layer:
    cfg: LayerConfig
    W: np.ndarray  # m x n float32
    X: np.ndarray  # N x n float32
    left: dict = field(default_factory=dict)  # {"signs": (m,)} or {"A": p x p, "B": q x q}
    right: dict = field(default_factory=dict)  # {"signs": (n,)} or {"A": .., "B": ..}


def rademacher(rng: np.random.Generator, n: int) -> np.ndarray:
    """Independent +-1 with probability 1/2 each, as float32."""
    return np.where(rng.random(n) < 0.5, -1.0, 1.0).astype(np.float32)


def haar_orthogonal(rng: np.random.Generator, p: int) -> np.ndarray:
    """A Haar-distributed p x p orthogonal matrix: Q of the QR of a Gaussian
    matrix with the signs of diag(R) folded into Q (Mezzadri, 2007). Drawn in
    float64 and returned as float32; the float32 matrix is what both sides use."""
    Z = rng.standard_normal((p, p))
    Q, R = np.linalg.qr(Z)
    Q = Q * np.sign(np.diag(R))[None, :]
    return Q.astype(np.float32)


def weights(cfg: LayerConfig, m: Optional[int] = None, n: Optional[int] = None) -> np.ndarray:
    m = cfg.m if m is None else m
    n = cfg.n if n is None else n
    W = rng_for(cfg.cfg_id, STREAMS["w_base"]).standard_normal((m, n), dtype=np.float32)
    if cfg.w_row_sigma > 0:
        sig = np.exp(cfg.w_row_sigma * rng_for(cfg.cfg_id, STREAMS["w_row_sigma"]).standard_normal(m))
        W *= sig.astype(np.float32)[:, None]
    if cfg.w_outlier_p > 0:
        mask = rng_for(cfg.cfg_id, STREAMS["w_outlier"]).random((m, n), dtype=np.float32) < cfg.w_outlier_p
        W[mask] *= np.float32(cfg.w_outlier_mult)
    return W


def activations(cfg: LayerConfig, N: Optional[int] = None, n: Optional[int] = None) -> np.ndarray:
    N = cfg.N if N is None else N
    n = cfg.n if n is None else n
    X = rng_for(cfg.cfg_id, STREAMS["x_base"]).standard_normal((N, n), dtype=np.float32)
    col = np.exp(cfg.x_col_sigma * rng_for(cfg.cfg_id, STREAMS["x_col_scale"]).standard_normal(n))
    X *= col.astype(np.float32)[None, :]
    return X


def random_permutation(rng: np.random.Generator, n: int) -> np.ndarray:
    """A uniformly random permutation of 0..n-1, as int32."""
    return rng.permutation(n).astype(np.int32)


def side_inputs(cfg: LayerConfig, side: Side, dim: int, which: str) -> dict:
    if side.kind == "rht":
        out = {"signs": rademacher(rng_for(cfg.cfg_id, STREAMS[f"sign_{which}"]), dim)}
    elif side.kind == "kron":
        if side.p * side.q != dim:
            raise ValueError(f"kron {side.p}x{side.q} does not match dimension {dim}")
        out = {"A": haar_orthogonal(rng_for(cfg.cfg_id, STREAMS[f"kron_{which}_a"]), side.p),
               "B": haar_orthogonal(rng_for(cfg.cfg_id, STREAMS[f"kron_{which}_b"]), side.q)}
    else:
        return {}
    if side.perm:
        out["perm"] = random_permutation(rng_for(cfg.cfg_id, STREAMS[f"perm_{which}"]), dim)
    return out


def make_layer(name_or_cfg, with_x: bool = True) -> Layer:
    cfg = CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    W = weights(cfg)
    X = activations(cfg) if with_x else np.zeros((0, cfg.n), np.float32)
    return Layer(cfg, W, X,
                 side_inputs(cfg, cfg.left, cfg.m, "left"),
                 side_inputs(cfg, cfg.right, cfg.n, "right"))


def custom_config(name: str, cfg_id: int, m: int, n: int, N: int, *, left: Side = RHT,
                  right: Side = RHT, quant: str = "uniform", bits: int = 2, B: int = 32,
                  g: int = 1, **kw) -> LayerConfig:
    """A small ad-hoc layer with the config-1 generator (ragged shapes, edge cases)."""
    return LayerConfig(name, cfg_id, m, n, N, left, right, quant, bits, B, g, **kw)


def gaussian_rows(seed: int, m: int, n: int) -> np.ndarray:
    """i.i.d. N(0,1) float32 rows (the Gaussian-source benchmarks)."""
    return np.random.default_rng(np.random.SeedSequence([ROOT_SEED, 9000, seed])).standard_normal(
        (m, n), dtype=np.float32)


def uniform_rows(seed: int, m: int, n: int, lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(np.random.SeedSequence([ROOT_SEED, 9200, seed]))
    return rng.uniform(lo, hi, size=(m, n)).astype(np.float32)
