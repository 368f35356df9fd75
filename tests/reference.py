"""Whole-layer references for the GPU parity tests: the oracle's result and,
next to it, the oracle's rounding variant of the GPU path (bf16 h; bf16
weights at prefill) with per-element bounds from tests/tolerance.py, built
expert by expert on a thread pool so that full-size batches (every token of
an 8192-token chunk) finish in a minute.

Routing follows the oracle on the GPU's fp32 logits (the tests check the
GPU's logits against the oracle's own and its selection bit for bit).
Experts are quantised by the oracle from the seeded draws.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
import synth
from tests import tolerance as tol

PROJ = {"gate": synth.T_GATE, "up": synth.T_UP, "down": synth.T_DOWN}
# moe_qgemm_prefill runs routed experts with at most PREFILL_GEMV_MAX
# assignments in the batch through the GEMV (decode) arithmetic instead of the
# matrix cores, when the batch has at least PREFILL_GEMV_MIN such experts
PREFILL_GEMV_MAX = 2
PREFILL_GEMV_MIN = 64


def _threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def expert_mats(w: synth.Workload, layer: int, e: int, bits):
    b = bits if isinstance(bits, dict) else {k: bits for k in PROJ}
    return {name: oracle.quantize(synth.expert_weight_f32(w, layer, tid, e), b[name]) for name, tid in PROJ.items()}


class LayerReference:
    """Reference of one layer call on token rows x (bf16 bits [T, H]) routed
    from logits [T, E]: path "prefill" or "decode".  Per assignment (in
    assignment order a = t (k+S) + j): y (the exact oracle's), yv / dyv (the
    variant and its bound), hv / dhv; per token: out (exact), outv / doutv.
    """

    def __init__(self, w: synth.Workload, x_bits, logits, path: str, layer: int = 0, bits=None,
                 residual_bits=None, norm_eps=None, threads=None, batch_counts=None):
        """norm_eps: x_bits is a residual stream; the block is
        x + moe(RMSNorm(x)) (residual_bits must then be None).  batch_counts:
        assignments per expert in the whole GPU batch (when x holds a subset
        of its tokens), which decides the prefill path per expert."""
        self.w = w
        T = x_bits.shape[0]
        x_dev = None
        if norm_eps is not None:
            residual_bits = x_bits
            xr = oracle.bf16_to_f32(x_bits).astype(np.float64)
            x_dev = tol.rmsnorm_flip(xr, norm_eps)
            x_bits = oracle.rmsnorm_bf16(x_bits, norm_eps)
        k, S, E, H, I = w.k, w.S, w.E, w.H, w.I
        kS = k + S
        bits = bits or w.bits
        self.idx = oracle.select_topk(logits, k)
        self.wt = oracle.topk_weights(logits, self.idx)
        counts, offsets, sorted_a, inverse = oracle.permute(self.idx, E, S)
        self.counts, self.offsets, self.sorted, self.inverse = counts, offsets, sorted_a, inverse
        x = oracle.bf16_to_f32(x_bits).astype(np.float64)
        A = T * kS
        self.y = np.zeros((A, H), np.float32)
        self.yv = np.zeros((A, H), np.float32)
        self.dyv = np.zeros((A, H), np.float32)
        self.hv = np.zeros((A, I), np.float32)
        self.dhv = np.zeros((A, I), np.float32)
        work = [e for e in range(E + S) if counts[e]]
        bc = counts if batch_counts is None else np.asarray(batch_counts)
        small = (bc[:E] > 0) & (bc[:E] <= PREFILL_GEMV_MAX)
        on_gemv = small if small.sum() >= PREFILL_GEMV_MIN else np.zeros(E, bool)

        def one(e):
            lo, hi = offsets[e], offsets[e + 1]
            a = sorted_a[lo:hi]
            xe = x[a // kS]
            mats = expert_mats(w, layer, e, bits)
            dense = [oracle.dequant(*mats[p]) for p in ("gate", "up", "down")]
            y = oracle.expert_ffn(xe, *dense)
            if path == "prefill" and e < E and on_gemv[e]:
                hv, dhv, yv, dyv = tol.decode_ffn(xe, mats, bits)
                dyv = dyv + 2.0 ** -8 * (np.abs(yv) + dyv)          # y stored in bf16
            elif path == "prefill":
                hv, dhv, yv, dyv = tol.prefill_ffn(xe, mats)
            else:
                hv, dhv, yv, dyv = tol.decode_ffn(xe, mats, bits, None if x_dev is None else x_dev[a // kS])
            up = lambda v: (v * (1 + 2.0 ** -20)).astype(np.float32)   # fp32 storage, rounded up
            self.y[a] = y
            self.yv[a] = yv
            self.dyv[a] = up(dyv)
            self.hv[a] = hv
            self.dhv[a] = up(dhv)

        from threadpoolctl import threadpool_limits
        with threadpool_limits(1), ThreadPoolExecutor(threads or _threads()) as ex:
            list(ex.map(one, work))
        res = None if residual_bits is None else oracle.bf16_to_f32(residual_bits).astype(np.float64)
        y3 = self.y.astype(np.float64).reshape(T, kS, H)
        self.out = oracle.combine(y3, self.wt, S) + (0 if res is None else res)
        self.outv, self.doutv = tol.combine_bound(self.wt, self.yv.astype(np.float64).reshape(T, kS, H),
                                                  self.dyv.astype(np.float64).reshape(T, kS, H), S, residual=res)


def check_bounded(name, got, want, bound, exact_frac=None, exact_where=None):
    """|got - want| <= bound everywhere; where exact_where, bit-equal.
    Returns the largest used fraction of the bound."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    err = np.abs(got - want)
    bad = err > bound
    assert not bad.any(), (f"{name}: {int(bad.sum())} of {bad.size} elements outside the bound; "
                           f"worst err {err[bad].max():.3e} bound there {bound[bad][np.argmax(err[bad])]:.3e}")
    if exact_where is not None:
        neq = (got != want) & exact_where
        assert not neq.any(), f"{name}: {int(neq.sum())} elements differ where no rounding flip is possible"
    used = err / np.where(bound > 0, bound, 1)
    return float(used.max()) if used.size else 0.0
