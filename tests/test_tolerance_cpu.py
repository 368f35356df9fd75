"""The derived per-element bounds of tests/tolerance.py against fp32
emulations of the two paths' arithmetic (CPU, no GPU): an emulation that
follows the kernel's steps stays inside the bound; the bound is tight (a
few times the bf16 rounding the output itself needs); an emulation with a
planted mistake (a dropped K-slice of one tile, a code off by one in a
group) leaves it."""
import numpy as np

import oracle
from tests import tolerance as tol

f32 = np.float32


def _expert(rng, H, I, bits):
    mats = {}
    for name, (N, K) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
        w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
        mats[name] = oracle.quantize(w, bits)
    return mats


def _bf16(a):
    return oracle.bf16_to_f32(oracle.f32_to_bf16(np.asarray(a, np.float32)))


def _silu32(g):
    g = g.astype(np.float32)
    return (g * (f32(1) / (f32(1) + np.exp2(-g * f32(1.4426950408889634))))).astype(np.float32)


def _seq_dot32(x, w, step=16):
    """fp32 sums of exact products, accumulated step by step along K."""
    acc = np.zeros((x.shape[0], w.shape[0]), np.float32)
    for k0 in range(0, x.shape[1], step):
        part = (x[:, k0:k0 + step].astype(np.float64) @ w[:, k0:k0 + step].T.astype(np.float64)).astype(np.float32)
        acc = (acc + part).astype(np.float32)
    return acc


def _emulate_prefill(x, mats, drop_slice=None):
    """The prefill path in fp32: bf16 weights, sums over K 16 at a time in
    ascending order, h and y rounded to bf16.  Returns (h, y)."""
    wg, wu, wd = (_bf16(oracle.dequant(*mats[p])) for p in ("gate", "up", "down"))
    if drop_slice is not None:
        wg = wg.copy()
        wg[:, drop_slice * 64:(drop_slice + 1) * 64] = 0
    g = _seq_dot32(x, wg)
    u = _seq_dot32(x, wu)
    h = _bf16(_silu32(g) * u)
    return h.astype(np.float64), _bf16(_seq_dot32(h, wd)).astype(np.float64)


def _group_dot32(x, q, s16, z16, off):
    """The decode kernels' scheme: per group, two fp32 accumulators of
    (off + q) x over the even and the odd input pairs, then
    s ((a0 + a1) - (z + off) sum(x)) added in fp32; groups in order."""
    n, K = x.shape
    acc = np.zeros((n, q.shape[0]), np.float32)
    for c in range(K // 64):
        sl = slice(64 * c, 64 * c + 64)
        a = [np.zeros_like(acc), np.zeros_like(acc)]
        for j, k in enumerate(range(sl.start, sl.stop, 2)):
            p = (x[:, k:k + 2].astype(np.float64) @ (off + q[:, k:k + 2].astype(np.float64)).T).astype(np.float32)
            a[j & 1] = (a[j & 1] + p).astype(np.float32)
        xs = x[:, sl].astype(np.float32).sum(1, dtype=np.float32)[:, None]
        s = s16[:, c].astype(np.float32)[None, :]
        zc = (z16[:, c].astype(np.float32) + f32(off))[None, :]
        acc = (acc + s * ((a[0] + a[1]) - zc * xs)).astype(np.float32)
    return acc


def _emulate_decode(x, mats, bits, bump=None):
    off = 128.0 if bits in (4, 6) else 0.0
    mg = mats["gate"]
    if bump is not None:
        q = mg[0].copy()
        q[bump] = q[bump] + 1 if q[bump] < 2 ** bits - 1 else q[bump] - 1
        mg = (q, mg[1], mg[2])
    g = _group_dot32(x, *mg, off)
    u = _group_dot32(x, *mats["up"], off)
    h = _bf16(_silu32(g) * u)
    return h.astype(np.float64), _group_dot32(h, *mats["down"], off).astype(np.float64)


def _check_h(h_emu, h, dh):
    """Outside the at-risk set the bf16 h equal bit for bit; inside, within the bound."""
    safe = dh == 0
    assert np.array_equal(h_emu[safe], h[safe])
    assert np.all(np.abs(h_emu - h) <= dh + (h_emu == h) * 0)


def test_prefill_bound_holds_and_is_tight():
    rng = np.random.default_rng(31)
    H, I = 512, 256
    mats = _expert(rng, H, I, 4)
    x = _bf16(rng.standard_normal((24, H))).astype(np.float64)
    h, dh, y, dy = tol.prefill_ffn(x, mats)
    h_emu, emu = _emulate_prefill(x, mats)
    _check_h(h_emu, h, dh)
    assert np.mean(dh > 0) < 0.35                    # most h cannot flip: they must be bit-exact
    assert np.all(np.abs(emu - y) <= dy)
    # tight: for most elements within a few bf16 roundings of y (2^-8 |y|), a
    # third of the 2e-2 bar everywhere
    assert np.median(dy / (2.0 ** -8 * np.abs(y))) < 3
    assert np.max(dy) < 2e-2 / 3 * np.max(np.abs(y))
    # a dropped K-slice of the gate projection: h and y leave their bounds
    h_bad, bad = _emulate_prefill(x, mats, drop_slice=3)
    assert np.any(np.abs(h_bad - h) > dh) and np.any(np.abs(bad - y) > dy)


def test_decode_bound_holds_and_is_tight():
    for bits in (4, 6, 8):
        rng = np.random.default_rng(40 + bits)
        H, I = 512, 256
        mats = _expert(rng, H, I, bits)
        x = _bf16(rng.standard_normal((6, H))).astype(np.float64)
        h, dh, y, dy = tol.decode_ffn(x, mats, bits)
        h_emu, emu = _emulate_decode(x, mats, bits)
        _check_h(h_emu, h, dh)
        assert np.mean(dh > 0) < 0.75, (bits, np.mean(dh > 0))
        assert np.all(np.abs(emu - y) <= dy), bits
        # the sums of (128 + q) x cancel the offset afterwards, which the bound
        # must cover: still well inside the 2e-2 bar
        assert np.max(dy) < 2e-2 / 2 * np.max(np.abs(y)), bits
        # a code off by one in one group of the gate projection (every token): h leaves its bound
        h_bad, bad = _emulate_decode(x, mats, bits, bump=(5, 70))
        assert np.any(np.abs(h_bad - h) > dh), bits


def test_rounding_flip():
    """The h rounding analysis: values whose rounding cannot change get 0,
    values next to a rounding boundary get one spacing."""
    sp = 2.0 ** -7                        # bf16 spacing in [1, 2)
    pre = np.array([1.0, 1.0 + sp / 2, 1.0 + sp / 2 + 1e-9, 1.0 + 0.25 * sp, 2.0 - sp / 2])
    d = np.full(pre.shape, 1e-6)
    got = tol.rounding_flip(pre, d)
    assert got[0] == 0                    # 1.0: the nearest boundaries are 1 - 2^-9 and 1 + 2^-8
    assert got[1] > 0 and got[2] > 0 and got[4] > 0
    assert got[3] == 0
