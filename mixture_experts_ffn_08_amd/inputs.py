"""Seeded synthetic inputs for one mixture-of-experts feed-forward layer.

This module is the only code shared by the CPU oracle and the HIP path.  It
holds layer shapes and random-number recipes and none of the layer's own
arithmetic: no routing, no softmax, no expert maths.

Recipe (every shape, seed 0 unless a caller asks otherwise):

* token matrix x[T][d] ~ N(0, 1);
* router weight W_r[E][d] ~ N(0, 1/d);
* expert e: gate[e][F][d] and up[e][F][d] ~ N(0, 1/d), down[e][d][F] ~ N(0, 1/F);
* shared expert (when F_shared > 0): same, with F_shared in place of F;
* for the skewed DeepSeek-V3-shaped layer, a per-expert logit bias
  b_e = 2.0 * ln(z_{r(e)}) with Zipf weights z_r = r^-1.1 (r = 1..E) and r(e)
  a seeded random permutation of the experts.

Values are drawn as float32 N(0,1), scaled by fan_in^-1/2 in float32 and, for
bf16 shapes, rounded to bfloat16 with round-to-nearest-even.  bf16 tensors are
returned as their uint16 bit patterns; ``bf16_bits_to_f32`` widens them
exactly.

Weights are stored (out_features, in_features), the order torch.nn.Linear
keeps them in: the router of both code listings on the pages (ML Interview
Notes "Mixture of Experts: Sparse FFNs, Routers, and Shared Experts", the
Router class; The Residual Stream "Mixture of Experts: More Parameters, Same
FLOPs", section "An MoE tiny GPT") is an nn.Linear(d, E) held as (E, d).  The
Residual Stream listing stacks the expert matrices as gate (E, d, F), up
(E, d, F), down (E, F, d); the tensors here are those transposed per expert,
so h @ gate[e] of that listing is h @ gate[e].T here.

Each tensor, and each expert's matrices, come from their own counter-keyed
numpy stream (SeedSequence spawn keys), so any one expert can be regenerated
alone and the order of generation does not matter.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

# Score modes, numbered as in include/moe.h.
SOFTMAX_THEN_TOPK = 0
TOPK_THEN_SOFTMAX = 1
SIGMOID_THEN_TOPK = 2

# Stream keys.
_X, _W_ROUTER, _BIAS_PERM, _EXPERT, _SHARED, _SELECT_BIAS = 0, 1, 2, 3, 4, 5
_GATE, _UP, _DOWN = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """One MoE layer workload.

    dtype   "f32" or "bf16": storage type of x, all weights, activations and y.
    T       tokens; d model width; E routed experts; k experts per token;
    F       routed expert hidden width; F_shared shared expert width (0 = none).
    mode    SOFTMAX_THEN_TOPK, TOPK_THEN_SOFTMAX or SIGMOID_THEN_TOPK; renorm
            applies to the first.
    phi     capacity factor, or None for dropless routing.
    zipf_bias  add the skewed per-expert logit bias described above.
    alpha   weight of the balance term.
    select_bias  standard deviation of a seeded per-expert selection-only bias
            (normal, float32); 0 = none.
    """

    name: str
    dtype: str
    T: int
    d: int
    E: int
    k: int
    F: int
    F_shared: int
    mode: int
    renorm: bool
    phi: Optional[float]
    zipf_bias: bool
    alpha: float = 0.01
    select_bias: float = 0.0

    def with_(self, **kw) -> "LayerShape":
        return dataclasses.replace(self, **kw)

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


SHAPES = {
    # Tiny fp32 layer, top-2 of 8, softmax over the chosen two.
    "tiny_f32": LayerShape("tiny_f32", "f32", 64, 64, 8, 2, 128, 0,
                           TOPK_THEN_SOFTMAX, False, None, False),
    # Mixtral-8x7B-shaped: 8 experts of width 14336, top-2, softmax over the chosen two.
    "mixtral": LayerShape("mixtral", "bf16", 4096, 4096, 8, 2, 14336, 0,
                          TOPK_THEN_SOFTMAX, False, None, False),
    "mixtral_cap": LayerShape("mixtral_cap", "bf16", 4096, 4096, 8, 2, 14336, 0,
                              TOPK_THEN_SOFTMAX, False, 1.25, False),
    # Qwen2-57B-A14B-shaped: 64 experts, top-8, softmax over all, no renormalization,
    # one always-on shared expert of width 20480.
    "qwen2": LayerShape("qwen2", "bf16", 8192, 3584, 64, 8, 2560, 20480,
                        SOFTMAX_THEN_TOPK, False, None, False),
    # Qwen3-30B-A3B-shaped: 128 experts of width 768, top-8, softmax over all then
    # renormalized over the chosen eight; prefill and decode batch sizes.
    "qwen3_prefill": LayerShape("qwen3_prefill", "bf16", 16384, 2048, 128, 8, 768, 0,
                                SOFTMAX_THEN_TOPK, True, None, False),
    "qwen3_decode": LayerShape("qwen3_decode", "bf16", 64, 2048, 128, 8, 768, 0,
                               SOFTMAX_THEN_TOPK, True, None, False),
    # DeepSeek-V3-shaped: 256 experts of width 2048, top-8, renormalized, one shared
    # expert of width 2048, Zipf-skewed router.
    "dsv3_skew": LayerShape("dsv3_skew", "bf16", 8192, 7168, 256, 8, 2048, 2048,
                            SOFTMAX_THEN_TOPK, True, None, True),
}


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(seed: int, key: tuple, shape: tuple, fan_in: int, dtype: str) -> np.ndarray:
    a = _rng(seed, *key).standard_normal(shape, dtype=np.float32)
    if fan_in != 1:
        a *= np.float32(fan_in ** -0.5)
    return f32_to_bf16_bits(a) if dtype == "bf16" else a


def as_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values of a tensor as float32 (bf16 bits widened, f32 returned as is)."""
    return bf16_bits_to_f32(a) if dtype == "bf16" else np.ascontiguousarray(a, dtype=np.float32)


class LayerInputs:
    """Seeded inputs of one layer.  x, w_router and bias are generated eagerly;
    expert weights on demand (``expert(e)``, ``experts()``), since the largest
    shape holds 22.5 GB of them."""

    def __init__(self, shape: LayerShape, seed: int = 0):
        self.shape, self.seed = shape, seed
        s = shape
        self.x = _normal(seed, (_X,), (s.T, s.d), 1, s.dtype)
        self.w_router = _normal(seed, (_W_ROUTER,), (s.E, s.d), s.d, s.dtype)
        self.bias = zipf_logit_bias(s.E, seed) if s.zipf_bias else None
        self.select_bias = (None if s.select_bias == 0 else
                            (_rng(seed, _SELECT_BIAS).standard_normal(s.E, dtype=np.float32) *
                             np.float32(s.select_bias)).astype(np.float32))

    def expert(self, e: int):
        """(gate[F][d], up[F][d], down[d][F]) of routed expert e."""
        s = self.shape
        return (_normal(self.seed, (_EXPERT, e, _GATE), (s.F, s.d), s.d, s.dtype),
                _normal(self.seed, (_EXPERT, e, _UP), (s.F, s.d), s.d, s.dtype),
                _normal(self.seed, (_EXPERT, e, _DOWN), (s.d, s.F), s.F, s.dtype))

    def shared(self):
        """(gate[F_s][d], up[F_s][d], down[d][F_s]) of the shared expert, or None."""
        s = self.shape
        if s.F_shared <= 0:
            return None
        return (_normal(self.seed, (_SHARED, _GATE), (s.F_shared, s.d), s.d, s.dtype),
                _normal(self.seed, (_SHARED, _UP), (s.F_shared, s.d), s.d, s.dtype),
                _normal(self.seed, (_SHARED, _DOWN), (s.d, s.F_shared), s.F_shared, s.dtype))

    def experts(self, sink=None, threads: Optional[int] = None):
        """Generate every routed expert.  With ``sink(e, gate, up, down)`` each
        expert is handed over and dropped (bounded host memory); without, the
        stacked arrays (gate[E][F][d], up[E][F][d], down[E][d][F]) are returned."""
        s = self.shape
        threads = threads or min(16, os.cpu_count() or 1)
        out = None
        if sink is None:
            dt = np.uint16 if s.dtype == "bf16" else np.float32
            out = (np.empty((s.E, s.F, s.d), dt), np.empty((s.E, s.F, s.d), dt),
                   np.empty((s.E, s.d, s.F), dt))

        def one(e):
            g, u, dn = self.expert(e)
            if sink is None:
                out[0][e], out[1][e], out[2][e] = g, u, dn
            else:
                sink(e, g, u, dn)

        with ThreadPoolExecutor(threads) as ex:
            for _ in ex.map(one, range(s.E)):
                pass
        return out


def zipf_logit_bias(E: int, seed: int = 0) -> np.ndarray:
    """b_e = 2.0 * ln(r(e)^-1.1), r(e) in 1..E a seeded permutation; float32."""
    rank = _rng(seed, _BIAS_PERM).permutation(E) + 1
    return (2.0 * (-1.1) * np.log(rank.astype(np.float64))).astype(np.float32)
