"""Seeded synthetic workloads for the RAM-Net layer recurrence.

This module only draws random numbers and stores them in the layer's input
dtypes.  It holds none of the layer's arithmetic, so both the HIP path and the
CPU oracle can consume what it produces without sharing any method code.

Workload shapes follow the RAM-Net project page (muoncat.github.io/ramnet_web):
M = 1024 = 4^5 slots with 20 address scores ("Product Softmax" paragraph),
Top-8/16/32 ("state access" paragraph) and d_v = 64, the split under which the
340M state-access figure works out.  The pages measure model quality on public
suites that need trained weights; these random inputs stand in only for the
layer's tensor shapes and value distributions.

Draw order (numpy PCG64 per seed, C-order [B,T,H,*], float32 standard normals):
q logits, k logits, v, gamma, gate logits g, then S0, m0 and pos0 when the
workload asks for them.  Logits are scaled by the workload's sigma.  bf16
inputs are rounded to nearest-even and kept as float32 arrays whose values are
exactly representable in bf16, so any consumer widens them without loss.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    d_p: int
    U: int
    K: int
    d_v: int
    in_dtype: str          # "f32" | "bf16"   (q, k, v, gamma, g)
    state_dtype: str       # "f32" | "bf16"   (S and out; mass is always f32)
    logit_sigma: float
    seed: int
    cape: int = 1
    s0_sigma: float = 0.0  # 0: zero initial state
    m0_uniform: Optional[tuple] = None  # (lo, hi) or None for zero mass
    pos0_max: int = 0      # pos0[b] ~ U{0..pos0_max}; 0 means all zero
    steps: int = 0         # >0: decode workload, T == 1 per step
    eps_gsu: float = 1e-6
    eps_norm: float = 1e-6

    @property
    def M(self) -> int:
        return self.d_p ** self.U

    @property
    def L(self) -> int:
        """Address logits per key or query: U * d_p."""
        return self.U * self.d_p

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: a tiny CPU-fast case, the 340M-like Top-8 prefill, the
# Top-32 prefill with an LDS-sized bf16 state, batched decode from a
# pre-filled state, and the 4^8-slot large-state prefill.
WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", B=1, T=256, H=1, d_p=4, U=5, K=8, d_v=64,
                     in_dtype="f32", state_dtype="f32", logit_sigma=1.0,
                     seed=0),
    "prefill_top8": Workload("prefill_top8", B=8, T=4096, H=8, d_p=4, U=5,
                             K=8, d_v=64, in_dtype="bf16", state_dtype="f32",
                             logit_sigma=1.5, seed=1),
    "prefill_top32": Workload("prefill_top32", B=4, T=8192, H=8, d_p=4, U=5,
                              K=32, d_v=64, in_dtype="bf16",
                              state_dtype="bf16", logit_sigma=1.5, seed=2),
    "decode": Workload("decode", B=256, T=1, H=16, d_p=4, U=5, K=16, d_v=128,
                       in_dtype="bf16", state_dtype="bf16", logit_sigma=1.5,
                       seed=3, s0_sigma=0.1, m0_uniform=(0.5, 1.5),
                       pos0_max=4095, steps=1024),
    "large_state": Workload("large_state", B=2, T=32768, H=16, d_p=4, U=8,
                            K=32, d_v=64, in_dtype="bf16", state_dtype="bf16",
                            logit_sigma=2.0, seed=4),
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); float32 out."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    nan = np.isnan(x)
    out = r.astype(np.uint32).view(np.float32)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    x = x.astype(np.float32, copy=False)
    return round_bf16(x) if dtype == "bf16" else np.ascontiguousarray(x)


def make_inputs(w: Workload, seed: Optional[int] = None,
                B: Optional[int] = None, T: Optional[int] = None,
                H: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw one batch of layer inputs (and the initial state) for `w`.

    B, T, H may be overridden to cut a smaller case with the same
    distributions.  Returns float32 arrays (values representable in their
    declared dtype) plus int32 pos0.
    """
    B = w.B if B is None else B
    T = w.T if T is None else T
    H = w.H if H is None else H
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    L, dv = w.L, w.d_v

    def normal(shape, sigma=1.0):
        a = rng.standard_normal(size=shape, dtype=np.float32)
        if sigma != 1.0:
            a *= np.float32(sigma)
        return a

    out = {}
    out["q"] = _store(normal((B, T, H, L), w.logit_sigma), w.in_dtype)
    out["k"] = _store(normal((B, T, H, L), w.logit_sigma), w.in_dtype)
    out["v"] = _store(normal((B, T, H, dv)), w.in_dtype)
    out["gamma"] = _store(normal((B, T, H)), w.in_dtype)
    out["g"] = _store(normal((B, T, H, dv)), w.in_dtype)
    M = w.M
    if w.s0_sigma > 0:
        out["S0"] = _store(normal((B, H, M, dv), w.s0_sigma), w.state_dtype)
    else:
        out["S0"] = np.zeros((B, H, M, dv), np.float32)
    if w.m0_uniform is not None:
        lo, hi = w.m0_uniform
        out["m0"] = (lo + (hi - lo) * rng.random(size=(B, H, M),
                                                 dtype=np.float32)).astype(np.float32)
    else:
        out["m0"] = np.zeros((B, H, M), np.float32)
    if w.pos0_max > 0:
        out["pos0"] = rng.integers(0, w.pos0_max + 1, size=(B,), dtype=np.int32)
    else:
        out["pos0"] = np.zeros((B,), np.int32)
    return out


def make_decode_step(w: Workload, step: int, B: Optional[int] = None,
                     H: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Per-step decode inputs q, k, v, gamma, g, each [B, H, *], drawn from
    PCG64([seed, step]) in the same order as make_inputs."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    rng = np.random.Generator(np.random.PCG64([w.seed, step]))
    L, dv = w.L, w.d_v

    def normal(shape, sigma=1.0):
        a = rng.standard_normal(size=shape, dtype=np.float32)
        if sigma != 1.0:
            a *= np.float32(sigma)
        return a

    return {
        "q": _store(normal((B, H, L), w.logit_sigma), w.in_dtype),
        "k": _store(normal((B, H, L), w.logit_sigma), w.in_dtype),
        "v": _store(normal((B, H, dv)), w.in_dtype),
        "gamma": _store(normal((B, H)), w.in_dtype),
        "g": _store(normal((B, H, dv)), w.in_dtype),
    }


# ---------------------------------------------------------------- whole layer
#
# Token activations and projection weights for a layer with its dense
# projections.  Two kinds:
#   grid  x = i/8 with i uniform on [-8, 8]; weights = j * 2^-e with j uniform
#         on [-8, 8] and 2^-e the power of two that puts the projected logits
#         near the workload's sigma (values near 1).  Every dot product is a
#         short sum of dyadic numbers, exact in fp32 in any order.
#   gauss x ~ N(0, 1), weights ~ N(0, sigma^2 / d_model), both bf16.
# alpha: "pow2" draws alpha_h from {0, fp32(ln 2), -fp32(ln 2)}, whose e^alpha
# round to 1, 2 and 1/2 in fp32; "general" draws alpha_h ~ U(-1, 1); None
# leaves it out.
# Draw order (PCG64([seed, 17])): x, w_q, w_k, w_v, w_g, w_gamma, w_o, alpha.

LN2_F32 = float(np.float32(np.log(2.0)))


def make_layer_weights(w: Workload, d_model: int, seed: Optional[int] = None,
                       B: Optional[int] = None, T: Optional[int] = None,
                       H: Optional[int] = None, kind: str = "grid",
                       alpha: Optional[str] = "pow2") -> Dict[str, np.ndarray]:
    B = w.B if B is None else B
    T = w.T if T is None else T
    H = w.H if H is None else H
    rng = np.random.Generator(np.random.PCG64([w.seed if seed is None else seed, 17]))
    L, dv, D = w.L, w.d_v, d_model

    if kind == "grid":
        def step(sigma):  # std of i/8 * j * s is about 3 s per term
            return 2.0 ** np.round(np.log2(sigma / (3.0 * np.sqrt(D))))

        def mat(shape, sigma):
            return (rng.integers(-8, 9, size=shape) * step(sigma)).astype(np.float32)
        x = (rng.integers(-8, 9, size=(B, T, D)) / 8.0).astype(np.float32)
    elif kind == "gauss":
        def mat(shape, sigma):
            return round_bf16(rng.standard_normal(size=shape, dtype=np.float32)
                              * np.float32(sigma / np.sqrt(D)))
        x = round_bf16(rng.standard_normal(size=(B, T, D), dtype=np.float32))
    else:
        raise ValueError(kind)
    out = {"x": x,
           "w_q": mat((D, H * L), w.logit_sigma),
           "w_k": mat((D, H * L), w.logit_sigma),
           "w_v": mat((D, H * dv), 1.0),
           "w_g": mat((D, H * dv), 1.0),
           "w_gamma": mat((D, H), 1.0)}
    if kind == "grid":
        out["w_o"] = (rng.integers(-8, 9, size=(H * dv, D))
                      * 2.0 ** np.round(np.log2(1.0 / (3.0 * np.sqrt(H * dv))))).astype(np.float32)
    else:
        out["w_o"] = round_bf16(rng.standard_normal(size=(H * dv, D), dtype=np.float32)
                                * np.float32(1.0 / np.sqrt(H * dv)))
    if alpha == "pow2":
        out["alpha"] = (rng.integers(-1, 2, size=H) * LN2_F32).astype(np.float32)
    elif alpha == "general":
        out["alpha"] = rng.uniform(-1.0, 1.0, size=H).astype(np.float32)
    elif alpha is not None:
        raise ValueError(alpha)
    return out
