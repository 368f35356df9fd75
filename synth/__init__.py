"""Seeded synthetic inputs for the group-quantized MoE FFN layer.

This module is the one piece of code shared by the CPU oracle's tests and the
GPU path's tests and benchmark.  It only *draws* inputs: fp32 expert weights,
bf16 router weights, bf16 activations and per-expert router offsets.  It holds
none of the layer's arithmetic (no quantisation, routing, permutation, FFN or
combine); each side implements those on its own.

Every tensor is drawn from ``numpy.random.default_rng(SeedSequence(key))``
with a key ``[seed, workload_id, layer, tensor_id, index]`` so that any single
expert, or any single token batch, can be regenerated on its own.  That lets a
test rebuild just the experts a sampled token routes to.

The workload shapes stand in for the model classes the pages run: 35B-A3B
MoE models routing 8 of 128/256 experts (Krasis update, "Latest results
(v1.0)"), a 125B model routing 10 of 512 experts (Qwen 3.8 Flash Next on an
RTX 3060, introduction; Qwen-tin, "Memory layout and performance") and
per-part mixed 4/6/8-bit HQQ precision (Krasis update, "Latest updates").
No trained weights or text are used: all values are synthetic.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get_workload",
    "T_ROUTER", "T_GATE", "T_UP", "T_DOWN", "T_ACT", "T_RANK", "T_BITS", "T_LOGITS",
    "rng_for", "expert_weight_f32", "expert_weights_f32", "router_weight_bf16",
    "activations_bf16", "router_bias", "direct_logits_f32", "layer_bits",
    "f32_to_bf16_bits_input",
]

# tensor ids used in the seed key
T_ROUTER, T_GATE, T_UP, T_DOWN = 0, 1, 2, 3
T_ACT, T_RANK, T_BITS, T_LOGITS = 7, 8, 9, 10

WEIGHT_STD = np.float32(0.02)  # expert and router weights ~ N(0, 0.02)
GROUP = 64                      # quantisation group along the input dimension


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int                 # workload id in the seed key
    H: int                   # hidden size
    I: int                   # expert intermediate size
    E: int                   # routed experts
    k: int                   # experts per token
    S: int                   # always-on shared experts (0 or 1)
    bits: int                # 4/6/8, or 0 for per-layer mixed
    tokens: tuple            # token-batch sizes of the workload
    bias: Optional[str] = None   # None | "zipf" | "hot"
    layers: int = 1
    bits_mix: tuple = ()     # (#4-bit, #6-bit, #8-bit) layers when bits == 0
    steps: int = 1
    seed: int = 0

    @property
    def n_mats(self) -> int:
        return self.E + self.S


WORKLOADS = {w.name: w for w in [
    # single layer, hidden 2048, 128 experts, intermediate 512, top-8, 4-bit
    Workload("moe_h2048_e128_k8_b4", 1, 2048, 512, 128, 8, 0, 4, (1, 16)),
    # decode, 256 experts + 1 shared expert, 4-bit
    Workload("moe_h2048_e256_k8_s1_b4", 2, 2048, 512, 256, 8, 1, 4, (1, 4, 8)),
    # prefill chunks on the 128-expert shapes, 6-bit, Zipf(1.1) router offsets
    Workload("moe_h2048_e128_k8_b6_zipf", 3, 2048, 512, 128, 8, 0, 6, (512, 2048, 4096), "zipf"),
    # wide MoE, hidden 4096, 512 experts, intermediate 768, top-10, 10% hot experts
    Workload("moe_h4096_e512_k10_b4_hot", 4, 4096, 768, 512, 10, 0, 4, (1, 8192), "hot"),
    # the same prefill chunks on the 256-expert + 1-shared shapes (the decode
    # layer's), 6-bit, Zipf(1.1) router offsets
    Workload("moe_h2048_e256_k8_s1_b6_zipf", 6, 2048, 512, 256, 8, 1, 6, (512, 2048, 4096), "zipf"),
    # 48 stacked blocks (RMSNorm -> 128-expert MoE -> residual), mixed 4/6/8-bit
    Workload("stack48_h2048_e128_k8_mixed", 5, 2048, 512, 128, 8, 0, 0, (1,), None,
             layers=48, bits_mix=(24, 14, 10), steps=256),
]}


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]


def rng_for(w: Workload, layer: int, tensor_id: int, index: int = 0, extra: Sequence[int] = ()):
    key = [w.seed, w.wid, layer, tensor_id, index, *extra]
    return np.random.default_rng(np.random.SeedSequence(key))


def f32_to_bf16_bits_input(a: np.ndarray) -> np.ndarray:
    """Store drawn fp32 values as bf16 bit patterns (round to nearest even).

    This only fixes the storage type of generated inputs.  NaN never occurs in
    drawn data and is not handled.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _proj_shape(w: Workload, proj: int):
    # gate/up map H -> I ([I, H]); down maps I -> H ([H, I]); rows are outputs
    return (w.I, w.H) if proj in (T_GATE, T_UP) else (w.H, w.I)


def expert_weight_f32(w: Workload, layer: int, proj: int, e: int, out: Optional[np.ndarray] = None):
    """fp32 N(0, 0.02) weight of one projection of expert ``e`` (row = output)."""
    shape = _proj_shape(w, proj)
    if out is None:
        out = np.empty(shape, np.float32)
    g = rng_for(w, layer, proj, e)
    g.standard_normal(out=out, dtype=np.float32)
    out *= WEIGHT_STD
    return out


def expert_weights_f32(w: Workload, layer: int, proj: int, experts: Sequence[int],
                       out: Optional[np.ndarray] = None, threads: Optional[int] = None):
    """Stack of ``expert_weight_f32`` for several experts, drawn on a thread pool."""
    experts = list(experts)
    shape = _proj_shape(w, proj)
    if out is None:
        out = np.empty((len(experts),) + shape, np.float32)
    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if threads <= 1 or len(experts) <= 1:
        for i, e in enumerate(experts):
            expert_weight_f32(w, layer, proj, e, out[i])
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda ie: expert_weight_f32(w, layer, proj, ie[1], out[ie[0]]),
                        enumerate(experts)))
    return out


def router_weight_bf16(w: Workload, layer: int = 0) -> np.ndarray:
    """Router weight [E, H] as bf16 bits, drawn N(0, 0.02) in fp32."""
    a = rng_for(w, layer, T_ROUTER).standard_normal((w.E, w.H), dtype=np.float32) * WEIGHT_STD
    return f32_to_bf16_bits_input(a)


def activations_bf16(w: Workload, T: int, batch: int = 0, layer: int = 0) -> np.ndarray:
    """Token activations [T, H] as bf16 bits, drawn N(0, 1) in fp32."""
    a = rng_for(w, layer, T_ACT, batch, extra=(T,)).standard_normal((T, w.H), dtype=np.float32)
    return f32_to_bf16_bits_input(a)


def router_bias(w: Workload, layer: int = 0) -> Optional[np.ndarray]:
    """Per-expert router-logit offset [E] fp32 that skews expert load, or None.

    zipf: expert e gets prior mass proportional to rank[e]^-1.1, rank a seeded
      permutation of 1..E, i.e. an offset of -1.1*ln(rank[e]).
    hot:  floor(E/10) seeded experts share 80% of the prior softmax mass and
      the rest share 20%: offsets ln(0.8/n_hot) and ln(0.2/(E-n_hot)).
    """
    if w.bias is None:
        return None
    perm = rng_for(w, layer, T_RANK).permutation(w.E)
    if w.bias == "zipf":
        rank = (perm + 1).astype(np.float64)
        return (-1.1 * np.log(rank)).astype(np.float32)
    if w.bias == "hot":
        n_hot = w.E // 10
        b = np.full(w.E, math.log(0.2 / (w.E - n_hot)), np.float64)
        b[perm[:n_hot]] = math.log(0.8 / n_hot)
        return b.astype(np.float32)
    raise ValueError(w.bias)


def hot_experts(w: Workload, layer: int = 0) -> np.ndarray:
    perm = rng_for(w, layer, T_RANK).permutation(w.E)
    return np.sort(perm[: w.E // 10])


def direct_logits_f32(w: Workload, T: int, batch: int = 0) -> np.ndarray:
    """Router logits drawn U(0, 1) directly, for selection tests on given logits."""
    return rng_for(w, 0, T_LOGITS, batch, extra=(T,)).random((T, w.E), dtype=np.float32)


def layer_bits(w: Workload) -> list:
    """Bit width of each layer.  Mixed workloads assign exact counts of 4/6/8-bit
    layers by a seeded permutation; others use ``w.bits`` everywhere."""
    if w.bits:
        return [w.bits] * w.layers
    n4, n6, n8 = w.bits_mix
    assert n4 + n6 + n8 == w.layers
    perm = rng_for(w, 0, T_BITS).permutation(w.layers)
    bits = [0] * w.layers
    for i, l in enumerate(perm):
        bits[l] = 4 if i < n4 else (6 if i < n4 + n6 else 8)
    return bits
