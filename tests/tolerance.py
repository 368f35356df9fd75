"""Per-element error bounds of the GPU expert FFN against the oracle's
rounding variants, derived from the arithmetic the kernels perform.

Rounding-error model.  Each fp32 addition or product the kernels round
errs by at most u |v| (u = 2^-24, v the exact value being rounded); R such
errors, independent and mean-zero, sum to at most lam u sqrt(R) P, where P
bounds every |v|, except with probability at most 2 exp(-lam^2 (1-u)^2 / 2)
(Higham & Mary, "A new approach to probabilistic rounding error analysis",
SIAM J. Sci. Comput. 2019).  lam = 8 puts that probability below 3e-14 per
element, so a test of 10^8 elements fails by chance with probability below
3e-6.  P is taken from the partial sums the kernel's own summation order
forms, computed here exactly from the oracle's values.

What each path computes (and so what the bounds cover):

* Prefill (grouped GEMM on bf16 matrix cores): every weight is
  bf16(fp32((q - z) s)) -- the oracle's dequantised weight rounded once to
  bf16, exactly -- and every product of bf16 values is exact in fp32.  The
  K products of an output are summed in fp32, 64 inputs (a quantisation
  group) per K-slice, slices in ascending order, in any order inside a
  slice: every partial sum is within the slice's sum |terms| of the sum at
  the slice's start, so P = max over slice starts of |partial sum| + max
  over slices of their sum |terms|, and R = K (a factor 2 on the bound
  leaves room for the matrix unit's internal rounding).  h = silu(g) u in
  fp32, rounded to bf16; y likewise over I, rounded to bf16.  Oracle
  variant: expert_ffn(w_bf16=True, h_bf16=True) in fp64.
* Decode (grouped GEMV): per group of 64 inputs two fp32 accumulators take
  the exact products (OFF + q) x of the even and of the odd input pairs
  (OFF = 128 at 4 and 6 bits, 0 at 8 bits); then s ((a0 + a1) - (z + OFF)
  sum(x)) is added to the output in fp32, group after group.  Its weights
  are thus (q - z) s exactly; the oracle's are that value rounded to fp32
  (relative 2^-24 per weight, a separate deterministic term).  h = silu(g) u
  in fp32, rounded to bf16; y the same scheme over I with h, kept in fp32.
  Oracle variant: expert_ffn(h_bf16=True) in fp64.

The one discontinuous step is the rounding of h to bf16: where the GPU's
h before rounding and the oracle's lie on opposite sides of a bf16 rounding
boundary, the two bf16 values differ by one bf16 spacing.  That can only
happen where a boundary lies within the bound on the difference of the
unrounded values; rounding_flip names those elements, and everywhere else
the GPU's bf16 h equals the oracle's bit for bit.

SiLU: the kernels evaluate g * rcp(1 + exp2(-g log2 e)); its relative error
is below (|g| + 16) u.

Test infrastructure: uses the oracle's dequantisation and rounding only.
"""
from __future__ import annotations

import numpy as np

import oracle

LAM = 8.0
U32 = 2.0 ** -24
GROUP = 64


def prob_bound(R, P) -> np.ndarray:
    """lam u sqrt(R) P: R roundings of values at most P."""
    return LAM * U32 * np.sqrt(R) * P


def bf16(a) -> np.ndarray:
    """fp64 values rounded to bf16 (nearest even), as fp64."""
    return oracle.bf16_to_f32(oracle.f32_to_bf16(np.asarray(a, np.float64))).astype(np.float64)


def bf16_spacing(a) -> np.ndarray:
    """Distance between consecutive bf16 values at |a| (normal range)."""
    a = np.maximum(np.abs(np.asarray(a, np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def rounding_flip(pre, delta) -> np.ndarray:
    """Largest |bf16(p) - bf16(pre)| over |p - pre| <= delta: zero where no
    bf16 rounding boundary lies within delta of pre, else one spacing (plus
    delta, for deltas as large as a spacing)."""
    a = np.abs(np.asarray(pre, np.float64))
    sp = bf16_spacing(a)
    e2 = 2.0 ** np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    k = np.floor(a / sp)
    d = np.minimum(np.abs(a - (k + 0.5) * sp), np.abs(a - (k - 0.5) * sp))
    d = np.minimum(d, np.abs(a - (e2 - sp / 4)))       # boundary just below the binade
    return np.where(d <= delta, sp + delta, 0.0)


def silu(g):
    return g / (1.0 + np.exp(-g))


def dsilu(g):
    s = 1.0 / (1.0 + np.exp(-g))
    return s * (1.0 + g * (1.0 - s))


def slice_peak(x, w, chunk=GROUP):
    """Bound on |every partial sum| of sum_k x_k w_k summed slice by slice
    (chunk inputs each, ascending, any order inside a slice): max over slice
    boundaries of |partial sum| plus max over slices of sum |terms|.  x [n, K],
    w [N, K] -> [n, N]."""
    n, K = x.shape
    S = np.zeros((n, w.shape[0]))
    peak = np.zeros_like(S)
    tmax = np.zeros_like(S)
    for c in range(K // chunk):
        sl = slice(c * chunk, (c + 1) * chunk)
        tmax = np.maximum(tmax, np.abs(x[:, sl]) @ np.abs(w[:, sl]).T)
        S = S + x[:, sl] @ w[:, sl].T
        peak = np.maximum(peak, np.abs(S))
    return peak + tmax


def _h_stage(g, dg, u, du):
    """The oracle's bf16 h and the bound on |h_gpu - h_oracle| after both
    round to bf16 (zero where that rounding cannot differ)."""
    hpre = silu(g) * u
    dh = np.abs(dsilu(g) * u) * dg + np.abs(silu(g)) * du + dg * du + (np.abs(g) + 16) * U32 * np.abs(hpre)
    return bf16(hpre), rounding_flip(hpre, dh)


# --------------------------------------------------------------------------
# prefill
# --------------------------------------------------------------------------
def _mfma_dot(x, x_dev, w):
    """Value, and bound, of x . w^T summed in fp32 slice by slice (bf16
    inputs, exact products); x_dev bounds |x_gpu - x| per element."""
    K = x.shape[1]
    val = x @ w.T
    P = slice_peak(x, w) + x_dev @ np.abs(w).T
    return val, 2 * prob_bound(K, P) + x_dev @ np.abs(w).T


def prefill_ffn(x, expert):
    """Oracle h and y (weights and h rounded to bf16, y before its own
    rounding) with per-element bounds: (h, dh, y, dy), dy including the bf16
    rounding of the GPU's y.  x: fp64 token rows [n, H]; expert: {"gate" |
    "up" | "down": (q, s16, z16)}."""
    wg, wu, wd = (bf16(oracle.dequant(*expert[p])) for p in ("gate", "up", "down"))
    zero = np.zeros_like(x)
    g, dg = _mfma_dot(x, zero, wg)
    u, du = _mfma_dot(x, zero, wu)
    h, dh = _h_stage(g, dg, u, du)
    y, dacc = _mfma_dot(h, dh, wd)
    return h, dh, y, dacc + 2.0 ** -8 * (np.abs(y) + dacc)


# --------------------------------------------------------------------------
# decode
# --------------------------------------------------------------------------
def _gemv_dot(x, x_dev, mat, bits):
    """Value (oracle weights, fp64) and bound of the decode kernels' group
    scheme for x . w^T; x_dev bounds |x_gpu - x| per element."""
    q, s16, z16 = mat
    N, K = q.shape
    n = x.shape[0]
    ng = K // GROUP
    w = oracle.dequant(q, s16, z16).astype(np.float64)
    off = 128.0 if bits in (4, 6) else 0.0
    s = s16.astype(np.float64)
    zc = np.abs(z16.astype(np.float64)) + off
    val = x @ w.T
    xa = np.abs(x) + x_dev
    # per group: the accumulators' partial sums over the even and the odd
    # pairs of (off + q) x, the correction (z + off) sum(x), the group value
    peak_a = np.zeros((n, N))
    peak_out = np.zeros((n, N))
    out = np.zeros((n, N))
    for c in range(ng):
        sl = slice(c * GROUP, (c + 1) * GROUP)
        xc = x[:, sl].reshape(n, GROUP // 2, 2)
        wc = (off + q[:, sl].astype(np.float64)).reshape(N, GROUP // 2, 2)
        pairs = np.einsum("njt,ijt->nij", xc, wc)                  # [n, N, 32]
        a0 = np.cumsum(pairs[..., 0::2], axis=-1)
        a1 = np.cumsum(pairs[..., 1::2], axis=-1)
        A = a0[..., -1] + a1[..., -1]
        corr = zc[:, c][None, :] * x[:, sl].sum(1)[:, None]
        pk = np.maximum(np.maximum(np.abs(a0).max(-1), np.abs(a1).max(-1)), np.maximum(np.abs(A), np.abs(corr)))
        peak_a = np.maximum(peak_a, s[:, c][None, :] * (pk + np.abs(A - corr)))
        out = out + x[:, sl] @ w[:, sl].T
        peak_out = np.maximum(peak_out, np.abs(out))
    R = ng * (GROUP + 4) + ng
    bound = prob_bound(R, np.maximum(peak_a, peak_out) + x_dev @ np.abs(w).T)
    bound = bound + U32 * (xa @ np.abs(w).T) + x_dev @ np.abs(w).T
    return val, bound


def decode_ffn(x, expert, bits, x_dev=None):
    """Oracle h and y (h rounded to bf16) with per-element bounds for the
    decode path: (h, dh, y, dy), y kept unrounded as the kernels keep it.
    bits: {"gate" | "up" | "down": b} or one width; x_dev bounds |x_gpu - x|
    per element when the GPU's input may differ (a normalised row)."""
    b = bits if isinstance(bits, dict) else {k: bits for k in ("gate", "up", "down")}
    zero = np.zeros_like(x) if x_dev is None else x_dev
    g, dg = _gemv_dot(x, zero, expert["gate"], b["gate"])
    u, du = _gemv_dot(x, zero, expert["up"], b["up"])
    h, dh = _h_stage(g, dg, u, du)
    y, dy = _gemv_dot(h, dh, expert["down"], b["down"])
    return h, dh, y, dy


def rmsnorm_flip(x, eps):
    """Bound on |n_gpu - n_oracle| for n = bf16(x / sqrt(mean(x^2) + eps)):
    the kernels sum the squares in fp32 (all terms positive, so the sum
    bounds every partial sum) and scale in fp32; zero where the bf16
    rounding cannot differ.  x: fp64 values of bf16 rows [T, H]."""
    H = x.shape[1]
    npre = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True) + eps)
    return rounding_flip(npre, np.abs(npre) * (prob_bound(H, 1.0) + 8 * U32))


# --------------------------------------------------------------------------
# combine
# --------------------------------------------------------------------------
def combine_bound(w, y, dy, S=0, w_rel=1e-5, residual=None):
    """Oracle out and the bound on |out_gpu - out_oracle| for out =
    bf16(sum_j w_j y_j + shared y [+ residual]): y [T, kS, H] the oracle's,
    dy their bounds, w [T, k] the oracle's weights (the GPU's within w_rel
    relative); residual (bf16 values [T, H]) is added in fp32 to the bf16 of
    the sum and rounded again."""
    T, kS, H = y.shape
    k = kS - S
    ww = np.ones((T, kS))
    ww[:, :k] = w
    wabs = np.abs(ww)[..., None]
    wdev = np.zeros((T, kS, 1))
    wdev[:, :k, 0] = w_rel * np.abs(w)
    out = (ww[..., None] * y).sum(1)
    b = (wabs * dy).sum(1) + (wdev * (np.abs(y) + dy)).sum(1) + prob_bound(kS + 2, (wabs * (np.abs(y) + dy)).sum(1))
    b = b + 2.0 ** -8 * (np.abs(out) + b)
    if residual is not None:
        out = out + residual
        b = b + 2.0 ** -8 * (np.abs(out) + b)
    return out, b
