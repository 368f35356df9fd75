"""Step-by-step oracle of the quantised MoE FFN layer (NumPy, CPU).

TEST INFRASTRUCTURE ONLY -- see the package docstring.  Each function states
the step it implements.  Parity status: every function here is pinned by the
CPU tests in ``tests/test_oracle_*.py`` (closed forms, special cases, brute
force and library routines); none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_to_f32", "f32_to_bf16", "quantize", "pack", "unpack", "dequant",
    "router_logits", "select_topk", "topk_weights", "assignment_experts",
    "permute", "expert_ffn", "combine", "QuantLayer", "moe_layer",
    "rmsnorm_bf16", "residual_bf16", "silu", "shrink_lp", "group_mean", "hqq_refine",
    "kv_encode", "kv_decode",
]

GROUP = 64


# --------------------------------------------------------------------------
# bf16 storage type
# --------------------------------------------------------------------------
def bf16_to_f32(u16: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> fp32 value (exact: the bits are the top half)."""
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(a) -> np.ndarray:
    """fp32 (or fp64, first rounded to fp32) -> bf16 bits, round to nearest even.

    fp64 inputs are rounded straight to bf16 by going through the exact fp64
    value: a double is first split so that no double rounding happens.
    """
    a = np.asarray(a)
    if a.dtype == np.float64:
        # round fp64 to bf16 directly: scale by the bf16 ulp at each value
        out = np.empty(a.shape, np.uint16)
        flat = a.reshape(-1)
        res = out.reshape(-1)
        m, ex = np.frexp(flat)              # flat = m * 2**ex, 0.5 <= |m| < 1
        r = np.rint(m * 256.0) / 256.0       # 8 significant bits, ties to even
        v = np.ldexp(r, ex).astype(np.float32)  # exact: 8-bit significand
        res[:] = (v.view(np.uint32) >> 16).astype(np.uint16)
        return out
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


# --------------------------------------------------------------------------
# quantised weight format
# --------------------------------------------------------------------------
def quantize(w: np.ndarray, bits: int, group: int = GROUP):
    """HQQ-style affine group quantisation of ``w`` [N, K] along K.

    The format stores an unsigned code q per weight and one fp16 scale s and
    fp16 zero z per group of ``group`` consecutive inputs of a row, so that
    the weight is recovered as (q - z) * s (Krasis update, "Latest results
    (v1.0)": HQQ 4/6/8-bit expert weights).  The pages give no solver; this
    is the min-max start that HQQ refines, in fp32:
        s  = (max - min) / (2^b - 1)          fp32, then rounded to fp16
        z  = -min / s16                       fp32, then rounded to fp16
        q  = clip(rint(w / s16 + z16), 0, 2^b - 1)   rint = ties to even
    A group whose fp16 scale is zero (constant group, or a range too small
    for fp16) stores s16 = 1, z16 = fp16(-min) and q = 0.
    Returns q [N, K] uint8, s16 [N, K/group] fp16, z16 [N, K/group] fp16.
    """
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    qmax = np.float32(2 ** bits - 1)
    wg = w.reshape(N, K // group, group)
    mn = wg.min(axis=2)
    mx = wg.max(axis=2)
    s = (mx - mn) / qmax
    s16 = s.astype(np.float16)
    degenerate = s16 == np.float16(0)
    s16 = np.where(degenerate, np.float16(1), s16)
    z16 = (-mn / s16.astype(np.float32)).astype(np.float16)
    v = wg / s16.astype(np.float32)[..., None] + z16.astype(np.float32)[..., None]
    q = np.clip(np.rint(v), np.float32(0), qmax)
    q[degenerate] = 0
    return q.astype(np.uint8).reshape(N, K), s16, z16


# --------------------------------------------------------------------------
# HQQ zero-point refinement (the step that produces the format's z)
# --------------------------------------------------------------------------
# The pages only name HQQ (Krasis update, "Latest results (v1.0)" and "Latest
# updates"); the solver is the published half-quadratic one (Badri & Shaji,
# "Half-Quadratic Quantization of Large Machine Learning Models", 2023),
# restated here from its description: with the scale s held, the zero z of a
# group minimises the lp error (p < 1) of the reconstruction, split with an
# auxiliary residual e and solved by alternating the two closed-form
# sub-problems while the coupling weight beta grows by kappa each round.
#
# Precision.  The codes are those of the quantiser (fp32, as ``quantize``).
# Everything else is real arithmetic carried in fp64: the residual
# r = w - (q - z) s is exact in fp64 (w is fp32, q an integer, z and s fp16
# values), the shrink and the zero sub-problem are evaluated in fp64, and a
# group's means are its fp64 sum divided by 64.  A mean is stored as an fp16
# zero, rounded once from fp64; the fp64 sum's rounding (a few fp64 ulps of
# the sum, whatever the order of the additions) is 2^-40 of an fp16 step, so
# the stored zero is the one the exact mean gives except where that mean
# falls within such a distance of an fp16 rounding boundary.  The solver's
# parameters are single-precision numbers (lp, beta, kappa as fp32).

def shrink_lp(x: np.ndarray, beta, p) -> np.ndarray:
    """Proximal step of the lp penalty (p <= 1), generalised soft threshold:
    sign(x) * max(|x| - |x|^(p-1) / beta, 0), in fp64.  At x = 0 and p < 1
    the threshold is infinite and the result 0."""
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    with np.errstate(divide="ignore"):
        t = np.power(a, np.float64(p) - 1.0) / np.float64(beta)
    return np.copysign(np.maximum(a - t, 0.0), x)


def group_mean(x: np.ndarray) -> np.ndarray:
    """Mean over the last axis: the fp64 sum of the values divided by their
    count (its rounding does not depend on the summation order beyond a few
    fp64 ulps)."""
    x = np.asarray(x, np.float64)
    return x.sum(axis=-1) / x.shape[-1]


def hqq_refine(w: np.ndarray, bits: int, lp: float = 0.7, beta: float = 10.0, kappa: float = 1.01,
               iters: int = 20, group: int = GROUP, trace: bool = False):
    """Min-max quantisation (``quantize``) followed by HQQ's zero-point
    refinement, group by group with s fixed.  One round, from the group's
    current fp16 zero z:
        q  = clip(rint(w / s + z), 0, 2^b - 1)          (codes for z, fp32)
        r  = w - (q - z) s;  E = mean |r|               (its error)
        stop if E is not below the group's best so far; else keep z as best
        e  = shrink_lp(r, beta, lp)                     (residual sub-problem)
        z  = fp16(mean(q - (w - e) / s))                (zero sub-problem)
        beta = beta * kappa
    The group keeps the zero of its lowest error and the codes for it, so its
    mean absolute error never exceeds the min-max one.  The stopping test is
    taken per group: the objective is a sum over groups whose variables are
    disjoint, so each group's test is the published whole-tensor test applied
    to that group's own part of the objective.  Groups whose fp16 scale is
    zero keep the min-max result.  Returns q, s16, z16 as ``quantize``; with
    ``trace`` also a list, per round, of (z [N, K/64], E [N, K/64], active)
    as the round found them."""
    if group != 64:
        raise ValueError("the refinement runs on groups of 64")
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    q0, s16, z16 = quantize(w, bits, group)
    qmax = np.float32(2 ** bits - 1)
    wg = w.reshape(N, K // group, group)
    degenerate = ((wg.max(axis=2) - wg.min(axis=2)) / qmax).astype(np.float16) == np.float16(0)
    sf = s16.astype(np.float32)[..., None]
    sd = sf.astype(np.float64)
    wd = wg.astype(np.float64)
    z = z16.astype(np.float32)
    zb = z.copy()
    best = np.full(z.shape, np.inf, np.float64)
    active = ~degenerate
    p = np.float64(np.float32(lp))
    b = np.float64(np.float32(beta))
    kap = np.float64(np.float32(kappa))
    rounds = []
    for _ in range(iters):
        if not active.any():
            break
        qv = np.clip(np.rint(wg / sf + z[..., None]), np.float32(0), qmax)
        r = wd - (qv.astype(np.float64) - z[..., None].astype(np.float64)) * sd
        E = group_mean(np.abs(r))
        if trace:
            rounds.append((z.copy(), E.copy(), active.copy()))
        active = active & (E < best)
        best = np.where(active, E, best)
        zb = np.where(active, z, zb)
        e = shrink_lp(r, b, p)
        znew = group_mean(qv.astype(np.float64) - (wd - e) / sd)
        z = np.where(active, znew.astype(np.float16).astype(np.float32), z)
        b = b * kap
    q = np.clip(np.rint(wg / sf + zb[..., None]), np.float32(0), qmax)
    q[degenerate] = 0
    out = (q.astype(np.uint8).reshape(N, K), s16, zb.astype(np.float16))
    return out + (rounds,) if trace else out


# --------------------------------------------------------------------------
# group-quantised KV-cache codec (the same format on bf16 cache rows)
# --------------------------------------------------------------------------
# Krasis update, "Latest updates": the KV cache is also stored in 4- and 6-bit
# group-quantised form (checked for accuracy against bf16).  The reading here:
# the weight format of ``quantize``/``pack`` applied to rows of the cache
# (one row = one token's vector of one head; groups of 64 along it), rows
# stored one after the other in the packed byte order of ``pack``.

def kv_encode(x_bf16: np.ndarray, bits: int):
    """bf16 rows [R, D] -> (packed codes [R, D*bits/8] uint8, s16 [R, D/64],
    z16 [R, D/64]): min-max quantisation (``quantize``) of the exact fp32
    values of the bf16 inputs, packed by ``pack``."""
    x = bf16_to_f32(x_bf16)
    q, s16, z16 = quantize(x, bits)
    return pack(q, bits), s16, z16


def kv_decode(packed: np.ndarray, s16: np.ndarray, z16: np.ndarray, bits: int, D: int) -> np.ndarray:
    """Inverse map: codes unpacked, dequantised as (q - z) * s in fp32
    (``dequant``), rounded to bf16 (ties to even) -> bf16 bits [R, D]."""
    return f32_to_bf16(dequant(unpack(packed, bits, D), s16, z16))


def pack(q: np.ndarray, bits: int) -> np.ndarray:
    """Pack codes [N, K] into rows of K*bits/8 bytes.

    4-bit: code 2i in the low nibble of byte i, code 2i+1 in the high nibble.
    6-bit: codes 4i..4i+3 form the 24-bit little-endian word
           c0 | c1<<6 | c2<<12 | c3<<18 stored in bytes 3i, 3i+1, 3i+2.
    8-bit: one byte per code.
    """
    q = np.asarray(q, dtype=np.uint8)
    N, K = q.shape
    if bits == 8:
        return q.copy()
    if bits == 4:
        lo = q[:, 0::2]
        hi = q[:, 1::2]
        return (lo | (hi << 4)).astype(np.uint8)
    if bits == 6:
        c = q.reshape(N, K // 4, 4).astype(np.uint32)
        word = c[..., 0] | (c[..., 1] << 6) | (c[..., 2] << 12) | (c[..., 3] << 18)
        out = np.empty((N, K // 4, 3), np.uint8)
        out[..., 0] = word & 0xFF
        out[..., 1] = (word >> 8) & 0xFF
        out[..., 2] = (word >> 16) & 0xFF
        return out.reshape(N, K * 3 // 4)
    raise ValueError("bits must be 4, 6 or 8")


def unpack(packed: np.ndarray, bits: int, K: int) -> np.ndarray:
    """Inverse of ``pack``: rows of K*bits/8 bytes -> codes [N, K] uint8."""
    p = np.asarray(packed, dtype=np.uint8)
    N = p.shape[0]
    if bits == 8:
        return p.copy()
    if bits == 4:
        q = np.empty((N, K), np.uint8)
        q[:, 0::2] = p & 0x0F
        q[:, 1::2] = p >> 4
        return q
    if bits == 6:
        b = p.reshape(N, K // 4, 3).astype(np.uint32)
        word = b[..., 0] | (b[..., 1] << 8) | (b[..., 2] << 16)
        q = np.empty((N, K // 4, 4), np.uint8)
        for j in range(4):
            q[..., j] = (word >> (6 * j)) & 0x3F
        return q.reshape(N, K)
    raise ValueError("bits must be 4, 6 or 8")


def dequant(q: np.ndarray, s16: np.ndarray, z16: np.ndarray, group: int = GROUP) -> np.ndarray:
    """Recover fp32 weights: w = (q - z) * s per group, two fp32 roundings."""
    N, K = q.shape
    qf = q.astype(np.float32).reshape(N, K // group, group)
    d = (qf - z16.astype(np.float32)[..., None]) * s16.astype(np.float32)[..., None]
    return d.reshape(N, K)


# --------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------
def router_logits(x_bf16: np.ndarray, wr_bf16: np.ndarray, bias=None) -> np.ndarray:
    """Router logits [T, E] = x . Wr^T (+ per-expert offset), as fp32.

    The dot products are taken in fp64 and rounded once to fp32; the offset,
    when given, is added in fp32 and so shifts both selection and weights.
    """
    x = bf16_to_f32(x_bf16).astype(np.float64)
    wr = bf16_to_f32(wr_bf16).astype(np.float64)
    L = (x @ wr.T).astype(np.float32)
    if bias is not None:
        L = L + np.asarray(bias, dtype=np.float32)[None, :]
    return L


def select_topk(L: np.ndarray, k: int) -> np.ndarray:
    """Top-k experts per token on fp32 logits (Qwen 3.8 Flash Next on an
    RTX 3060, introduction: top-10 routing over 512 experts).

    Largest logit first; equal logits go lower expert index first, and -0.0
    equals +0.0 -- exactly a stable descending sort.  Returns int32 [T, k].
    """
    L = np.asarray(L, dtype=np.float32)
    order = np.argsort(-L, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def topk_weights(L: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Routing weights: softmax over all experts, kept on the selected k and
    renormalised over them.  That equals a softmax over the k selected logits,
    computed here in fp64 relative to the largest (the first) of them."""
    Ls = np.take_along_axis(np.asarray(L, dtype=np.float32), idx.astype(np.int64), axis=1)
    Ls = Ls.astype(np.float64)
    e = np.exp(Ls - Ls[:, :1])
    return e / e.sum(axis=1, keepdims=True)


def assignment_experts(idx: np.ndarray, E: int, S: int) -> np.ndarray:
    """Expert of each assignment a = t*(k+S)+j: the routed expert idx[t, j]
    for j < k, shared expert E + (j - k) for j >= k.  Returns [T*(k+S)]."""
    T, k = idx.shape
    ids = np.empty((T, k + S), np.int64)
    ids[:, :k] = idx
    for j in range(S):
        ids[:, k + j] = E + j
    return ids.reshape(-1)


def permute(idx: np.ndarray, E: int, S: int = 0):
    """Group assignments by expert: histogram, exclusive scan, stable scatter.

    Returns counts [E+S], offsets [E+S+1], sorted [A] (assignment ids grouped
    by expert, ascending assignment id within an expert) and inverse [A]
    (position of each assignment in ``sorted``); all int32.
    """
    ids = assignment_experts(idx, E, S)
    counts = np.bincount(ids, minlength=E + S)
    offsets = np.zeros(E + S + 1, np.int64)
    np.cumsum(counts, out=offsets[1:])
    sorted_a = np.argsort(ids, kind="stable")
    inverse = np.empty_like(sorted_a)
    inverse[sorted_a] = np.arange(ids.size)
    return (counts.astype(np.int32), offsets.astype(np.int32),
            sorted_a.astype(np.int32), inverse.astype(np.int32))


# --------------------------------------------------------------------------
# expert FFN, combine
# --------------------------------------------------------------------------
def silu(g):
    return g / (1.0 + np.exp(-g))


def expert_ffn(x: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray, h_bf16: bool = False,
               w_bf16: bool = False) -> np.ndarray:
    """SwiGLU expert: h = silu(Wg x) * (Wu x); y = Wd h.  fp64.

    x [n, H]; wg, wu [I, H]; wd [H, I] (dequantised fp32 weights).  The
    activation sits on the gate; gate and up share the input x (Raon-1-mini
    on an RTX 5070 Ti, optimisation table: projections sharing an input).
    With ``h_bf16`` the intermediate h is rounded to bf16 (nearest even)
    before the down projection: the variant in which h is stored in bf16
    between the two projections.  With ``w_bf16`` the dequantised weights
    are rounded to bf16 (nearest even) first: the variant in which the
    products are taken on bf16 matrix units.  Everything else stays fp64.
    """
    x = np.asarray(x, dtype=np.float64)
    if w_bf16:
        wg, wu, wd = (bf16_to_f32(f32_to_bf16(np.asarray(m, np.float32))) for m in (wg, wu, wd))
    g = x @ np.asarray(wg, np.float64).T
    u = x @ np.asarray(wu, np.float64).T
    h = silu(g) * u
    if h_bf16:
        h = bf16_to_f32(f32_to_bf16(h)).astype(np.float64)
    return h @ np.asarray(wd, np.float64).T


def combine(y: np.ndarray, w: np.ndarray, S: int = 0) -> np.ndarray:
    """out[t] = sum_{j<k} w[t,j] * y[t,j] + sum_{j>=k} y[t,j], ascending j, fp64.

    y [T, k+S, H]; w [T, k].  Shared experts enter with weight one."""
    T, kS, H = y.shape
    k = kS - S
    out = np.zeros((T, H), np.float64)
    for j in range(k):
        out += w[:, j:j + 1] * y[:, j, :]
    for j in range(k, kS):
        out += y[:, j, :]
    return out


class QuantLayer:
    """Quantised MoE layer for the oracle: expert weights held as q/s/z.

    ``experts`` maps expert id (routed 0..E-1, shared E..E+S-1) to a dict with
    keys gate/up/down, each a (q, s16, z16) triple.  It may be a lazy mapping
    (any object with ``__getitem__``) so that full-size layers only build the
    experts a test touches.
    """

    def __init__(self, H, I, E, k, S, experts, group=GROUP):
        self.H, self.I, self.E, self.k, self.S = H, I, E, k, S
        self.experts = experts
        self.group = group
        self._cache = {}

    def dense(self, e):
        if e not in self._cache:
            ex = self.experts[e]
            self._cache[e] = tuple(dequant(*ex[p], group=self.group) for p in ("gate", "up", "down"))
        return self._cache[e]


def moe_layer(layer: QuantLayer, x_bf16: np.ndarray, wr_bf16=None, bias=None, logits=None, h_bf16=False,
              w_bf16=False):
    """Forward pass of one MoE FFN layer, step by step.

    1. router logits (or given fp32 ``logits``), 2. top-k selection,
    3. renormalised softmax weights, 4. permutation of assignments to
    experts, 5. per-expert SwiGLU FFN over that expert's tokens,
    6. weighted combine.  Returns a dict of every intermediate; ``out`` is the
    fp64 layer output [T, H] before any rounding to bf16.  ``h_bf16`` and
    ``w_bf16`` as in expert_ffn.
    """
    T = x_bf16.shape[0]
    k, E, S, H = layer.k, layer.E, layer.S, layer.H
    if logits is None:
        logits = router_logits(x_bf16, wr_bf16, bias)
    logits = np.asarray(logits, dtype=np.float32)
    idx = select_topk(logits, k)
    w = topk_weights(logits, idx)
    counts, offsets, sorted_a, inverse = permute(idx, E, S)
    x = bf16_to_f32(x_bf16).astype(np.float64)
    kS = k + S
    y = np.zeros((T * kS, H), np.float64)
    for e in range(E + S):
        lo, hi = offsets[e], offsets[e + 1]
        if hi == lo:
            continue
        a = sorted_a[lo:hi]
        wg, wu, wd = layer.dense(e)
        y[a] = expert_ffn(x[a // kS], wg, wu, wd, h_bf16, w_bf16)
    out = combine(y.reshape(T, kS, H), w, S)
    return dict(logits=logits, idx=idx, w=w, counts=counts, offsets=offsets,
                sorted=sorted_a, inverse=inverse, y=y, out=out)


# --------------------------------------------------------------------------
# stacked blocks: RMSNorm -> MoE -> residual
# --------------------------------------------------------------------------
def rmsnorm_bf16(x_bf16: np.ndarray, eps: float = 1e-6, gamma=None) -> np.ndarray:
    """n = x / sqrt(mean(x^2) + eps) * gamma, fp64, rounded to bf16 bits."""
    x = bf16_to_f32(x_bf16).astype(np.float64)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    n = x * r
    if gamma is not None:
        n = n * bf16_to_f32(gamma).astype(np.float64)
    return f32_to_bf16(n)


def residual_bf16(x_bf16: np.ndarray, moe_out: np.ndarray) -> np.ndarray:
    """x <- bf16(x + bf16(moe_out)): the block output is rounded to bf16,
    added to the bf16 residual stream and the sum rounded once to bf16."""
    o = bf16_to_f32(f32_to_bf16(np.asarray(moe_out, np.float64))).astype(np.float64)
    return f32_to_bf16(bf16_to_f32(x_bf16).astype(np.float64) + o)
