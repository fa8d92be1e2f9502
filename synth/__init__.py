"""Seeded synthetic inputs for the attention forward pass.

This module only *makes inputs*: it draws seeded random numbers and encodes
them in the storage formats the kernels read (fp32, bf16 bit patterns, and the
fp32 draws that the int8 quantiser consumes).  It holds none of the method's
arithmetic (no scores, no softmax, no quantisation), so both the FP64 oracle
side and the HIP side can take their inputs from it without sharing any part
of the computation they are compared on.

Workload shapes follow the pages' two model families: GPT-2-small attention
(12 heads, head_dim 64, the "Why Low-Precision Transformer Training Fails"
page, Figure 2) and Llama-2-7B attention (32 heads, head_dim 128, cited by
"Is Flash Attention Stable?", reference list).  No dataset or trained weight
is used: i.i.d. N(0,1) draws stand in for activations, and a shared rank-4
component stands in for the similar low-rank representations that the
"Why Low-Precision Transformer Training Fails" page describes (core claim;
Figure 4).
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, Optional

import numpy as np

__all__ = [
    "Config", "CONFIGS", "make_inputs", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "input_digest", "Inputs",
]


@dataclasses.dataclass(frozen=True)
class Config:
    """One attention forward workload (per-head Q, K, V in R^{N x d})."""
    name: str
    batch: int
    heads: int
    seq_len: int
    head_dim: int
    causal: bool
    dtype: str          # "f32" | "bf16" | "int8"  (type of Q and K as stored)
    p_bf16: bool        # default P rounding mode for this workload
    seed: int
    kind: str = "iid"   # "iid" | "lowrank4"
    description: str = ""

    @property
    def shape(self):
        return (self.batch, self.heads, self.seq_len, self.head_dim)

    def flops(self) -> float:
        """MFMA contraction flops over visible (query, key) pairs (QK^T + PV)."""
        b, h, n, d = self.shape
        if self.causal:
            return 2.0 * b * h * d * n * (n + 1)
        return 4.0 * b * h * n * n * d

    def scaled(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS: Dict[str, Config] = {
    "c1": Config("c1", 1, 1, 256, 64, False, "f32", False, 1, "iid",
                 "single head, fp32 I/O, non-causal, scale 1/sqrt(64)"),
    "c2": Config("c2", 8, 12, 1024, 64, True, "bf16", True, 2, "iid",
                 "GPT-2-small attention shape, causal, bf16"),
    "c3": Config("c3", 4, 32, 4096, 128, True, "bf16", True, 3, "iid",
                 "Llama-2-7B attention shape, causal, bf16, P rounded to bf16"),
    "c4": Config("c4", 1, 32, 16384, 128, True, "bf16", True, 4, "lowrank4",
                 "long sequence, Q/K share a rank-4 component, causal, bf16"),
    "c5": Config("c5", 4, 32, 2048, 128, False, "int8", True, 5, "iid",
                 "int8 Q/K with per-row fp32 scales, bf16 V, non-causal"),
}


# ---------------------------------------------------------------------------
# storage encodings
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Encode float32 values as bfloat16 bit patterns (uint16).

    IEEE round-to-nearest-even on the upper 16 bits of the binary32 pattern;
    NaN stays NaN (quiet, sign kept); overflow rounds to +-inf.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded = rounded.copy()
        rounded[nan] = ((u[nan] >> np.uint32(16)).astype(np.uint16)
                        | np.uint16(0x0040))
    return rounded


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def input_digest(*arrays: Optional[np.ndarray]) -> str:
    h = hashlib.sha256()
    for a in arrays:
        if a is None:
            h.update(b"none")
        else:
            a = np.ascontiguousarray(a)
            h.update(str(a.dtype).encode() + str(a.shape).encode())
            h.update(a.tobytes())
    return h.hexdigest()


@dataclasses.dataclass
class Inputs:
    """Encoded inputs of one workload.

    q, k: float32 arrays when ``cfg.dtype == "f32"``; bf16 bit patterns
    (uint16) when "bf16"; for "int8" they are the float32 draws that the int8
    quantiser turns into codes and per-row scales (each side runs its own
    quantiser on these).  v is float32 for "f32", bf16 bits otherwise.
    """
    cfg: Config
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray

    @property
    def v_is_bf16(self) -> bool:
        return self.v.dtype == np.uint16

    def digest(self) -> str:
        return input_digest(self.q, self.k, self.v)


def _normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def make_inputs(cfg: Config, seed: Optional[int] = None, *,
                lowrank_shared_coeffs: bool = True) -> Inputs:
    """Draw the workload's Q, K, V with numpy PCG64 seeded by ``seed``.

    Draw order: Q, K, V for i.i.d. workloads; for "lowrank4": the 128x4 basis
    draw, the coefficients, the Q noise, the K noise, then V.
    ``lowrank_shared_coeffs=False`` draws separate coefficients for Q and K
    (same basis) instead of one component shared by both.
    """
    seed = cfg.seed if seed is None else seed
    rng = np.random.default_rng(seed)
    shape = cfg.shape
    b, h, n, d = shape
    if cfg.kind == "iid":
        q = _normal(rng, shape)
        k = _normal(rng, shape)
        v = _normal(rng, shape)
    elif cfg.kind == "lowrank4":
        basis_draw = rng.standard_normal(size=(d, 4))
        u, _ = np.linalg.qr(basis_draw)              # d x 4, orthonormal cols
        u = u.astype(np.float32)
        cq = _normal(rng, (b, h, n, 4))
        ck = cq if lowrank_shared_coeffs else _normal(rng, (b, h, n, 4))
        eq = _normal(rng, shape)
        ek = _normal(rng, shape)
        comp_q = np.float32(3.0) * (cq @ u.T)
        comp_k = comp_q if lowrank_shared_coeffs else np.float32(3.0) * (ck @ u.T)
        q = np.float32(0.9) * comp_q + np.float32(0.1) * eq
        k = np.float32(0.9) * comp_k + np.float32(0.1) * ek
        del eq, ek, comp_q, comp_k
        v = _normal(rng, shape)
    else:
        raise ValueError(f"unknown input kind {cfg.kind!r}")
    q = np.ascontiguousarray(q, dtype=np.float32)
    k = np.ascontiguousarray(k, dtype=np.float32)
    if cfg.dtype == "f32":
        return Inputs(cfg, q, k, np.ascontiguousarray(v, dtype=np.float32))
    if cfg.dtype == "bf16":
        return Inputs(cfg, f32_to_bf16_bits(q), f32_to_bf16_bits(k),
                      f32_to_bf16_bits(v))
    if cfg.dtype == "int8":
        return Inputs(cfg, q, k, f32_to_bf16_bits(v))
    raise ValueError(f"unknown dtype {cfg.dtype!r}")


def small(cfg: Config, *, batch=None, heads=None, seq_len=None, head_dim=None,
          causal=None) -> Config:
    """A reduced copy of ``cfg`` (same dtype, kind, seed) for fast parity runs."""
    kw = {}
    for key, val in (("batch", batch), ("heads", heads), ("seq_len", seq_len),
                     ("head_dim", head_dim), ("causal", causal)):
        if val is not None:
            kw[key] = val
    return cfg.scaled(**kw)
