"""Pins that tie the CPU oracle to something other than itself.

Each ``pin_*`` function raises AssertionError when the oracle (module ``o``)
disagrees with a hand-derived example, a closed form, a special case that
reduces to a library routine, an invariant, or brute force on tiny inputs.
The CPU tests call them on the real oracle; the mutation tests call them
after planting a mistake in the oracle and expect them to fail.
"""
from __future__ import annotations

import itertools
import json
import math
import os
import struct

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _f32_from_hex(hs):
    return np.array([struct.unpack(">f", bytes.fromhex(h))[0] for h in hs], np.float32)


def _f16_from_hex(hs):
    return np.array([int(h, 16) for h in hs], np.uint16).view(np.float16)


# --------------------------------------------------------------------------
# quantisation format
# --------------------------------------------------------------------------
def pin_quant_golden(o):
    """Hand-derived worked examples (tests/golden/quant_examples.json)."""
    d = _golden("quant_examples.json")
    for ex in d["examples"]:
        w = _f32_from_hex(ex["w_f32_hex"])[None, :]
        q, s16, z16 = o.quantize(w, ex["bits"], group=ex["group"])
        assert q.tolist() == [ex["q"]], (ex["name"], q)
        assert s16.view(np.uint16).tolist() == [[int(h, 16) for h in ex["s16_hex"]]], ex["name"]
        assert z16.view(np.uint16).tolist() == [[int(h, 16) for h in ex["z16_hex"]]], ex["name"]
        d32 = o.dequant(q, s16, z16, group=ex["group"])
        assert d32.tolist() == [ex["dequant"]], ex["name"]
        p = o.pack(q, ex["bits"])
        assert bytes(p.reshape(-1)).hex() == ex["packed_hex"], ex["name"]
    for v in d["packing_vectors"]:
        q = np.array([v["q"]], np.uint8)
        p = o.pack(q, v["bits"])
        assert bytes(p.reshape(-1)).hex() == v["packed_hex"], v
        assert o.unpack(p, v["bits"], q.shape[1]).tolist() == q.tolist(), v


def pin_quant_error_bound(o, bits, seed=0, N=64, K=512, group=64):
    """Closed-form bound on |w - (q - z) s| for min-max quantisation.

    With z* = -min/s16 the exact zero, v = w/s16 + z16 lies within
    |z16 - z*| + qmax |s/s16 - 1| of [0, qmax], so rint and clipping move it
    at most 1/2 + that much; fp32 rounding adds a few ulps of |w|.  Every
    non-constant group also uses both end codes 0 and qmax.
    """
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    q, s16, z16 = o.quantize(w, bits, group=group)
    qmax = 2 ** bits - 1
    assert q.dtype == np.uint8 and q.max() <= qmax
    wg = w.reshape(N, K // group, group).astype(np.float64)
    mn, mx = wg.min(-1), wg.max(-1)
    s = (mx - mn) / qmax
    sf = s16.astype(np.float64)
    zstar = -mn / sf
    slack = np.abs(z16.astype(np.float64) - zstar) + qmax * np.abs(s / sf - 1.0)
    bound = sf * (0.5 + slack) + 4 * 2.0 ** -24 * (np.abs(wg).max(-1) + sf * qmax)
    err = np.abs(o.dequant(q, s16, z16, group=group).astype(np.float64).reshape(wg.shape) - wg)
    assert np.all(err <= bound[..., None]), float((err - bound[..., None]).max())
    # the quantiser is relative to the group's own range
    assert np.all(np.abs(s / sf - 1.0) <= 2.0 ** -11)
    qg = q.reshape(N, K // group, group)
    assert np.all(qg.min(-1) == 0) and np.all(qg.max(-1) == qmax)


def pin_quant_on_grid(o, bits, seed=1, N=16, K=256, group=64):
    """Weights built exactly on a power-of-two grid, (q0 - z0) * 2^-e, with
    both end codes in every group, quantise back to exactly (q0, 2^-e, z0)."""
    rng = np.random.default_rng(seed)
    qmax = 2 ** bits - 1
    G = K // group
    q0 = rng.integers(0, qmax + 1, (N, G, group))
    q0[:, :, 0] = 0
    q0[:, :, 1] = qmax
    for r in range(N):          # move the end codes around the group
        for g in range(G):
            rng.shuffle(q0[r, g])
    z0 = rng.integers(0, qmax + 1, (N, G))
    e = rng.integers(5, 12, (N, G))
    s0 = np.ldexp(1.0, -e)
    w = ((q0 - z0[..., None]) * s0[..., None]).astype(np.float32).reshape(N, K)
    q, s16, z16 = o.quantize(w, bits, group=group)
    assert np.array_equal(q.reshape(N, G, group), q0.astype(np.uint8))
    assert np.array_equal(s16.astype(np.float64), s0)
    assert np.array_equal(z16.astype(np.float64), z0.astype(np.float64))
    assert np.array_equal(o.dequant(q, s16, z16, group=group), w)


def pin_pack_exhaustive(o):
    """Every byte pattern round-trips through unpack/pack, and every code
    tuple through pack/unpack, for 4-, 6- and 8-bit."""
    allb = np.arange(256, dtype=np.uint8)[None, :]
    for bits in (4, 8):
        K = 256 * 8 // bits
        q = o.unpack(allb, bits, K)
        assert q.max() < 2 ** bits
        assert np.array_equal(o.pack(q, bits), allb)
    pairs = np.array(list(itertools.product(range(16), repeat=2)), np.uint8).reshape(1, -1)
    assert np.array_equal(o.unpack(o.pack(pairs, 4), 4, pairs.shape[1]), pairs)
    # all 2^24 three-byte words of 6-bit packing
    words = np.arange(1 << 24, dtype=np.uint32)
    b = np.stack([(words & 0xFF), (words >> 8) & 0xFF, (words >> 16) & 0xFF], -1).astype(np.uint8)
    b = b.reshape(1, -1)
    q = o.unpack(b, 6, (1 << 24) * 4)
    assert q.max() <= 63
    assert np.array_equal(o.pack(q, 6), b)
    # the four codes of word w are its 6-bit fields, lowest first
    qq = q.reshape(-1, 4).astype(np.uint32)
    assert np.array_equal(qq[:, 0] | (qq[:, 1] << 6) | (qq[:, 2] << 12) | (qq[:, 3] << 18), words)


# --------------------------------------------------------------------------
# routing
# --------------------------------------------------------------------------
def pin_routing_golden(o):
    d = _golden("routing_examples.json")
    for ex in d["topk"]:
        L = np.array(ex["logits"], np.float32)
        idx = o.select_topk(L, ex["k"])
        assert idx.tolist() == ex["idx"], ex
        if "weights" in ex:
            w = o.topk_weights(L, idx)
            assert np.allclose(w, ex["weights"], rtol=1e-15, atol=0), (w, ex)
    for ex in d["permute"]:
        c, off, srt, inv = o.permute(np.array(ex["idx"], np.int32), ex["E"], ex["S"])
        assert c.tolist() == ex["counts"]
        assert off.tolist() == ex["offsets"]
        assert srt.tolist() == ex["sorted"]
        assert inv.tolist() == ex["inverse"]


def _brute_topk(row, k):
    """The unique k-subset S with, for i in S and j not in S, L_i > L_j or
    (L_i == L_j and i < j); listed by (-L_i, i)."""
    E = len(row)
    found = []
    for S in itertools.combinations(range(E), k):
        Sset = set(S)
        ok = all((row[i] > row[j]) or (row[i] == row[j] and i < j)
                 for i in S for j in range(E) if j not in Sset)
        if ok:
            found.append(S)
    assert len(found) == 1
    return sorted(found[0], key=lambda i: (-row[i], i))


def pin_topk_bruteforce(o, trials=300, seed=2):
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        E = int(rng.integers(1, 9))
        k = int(rng.integers(1, E + 1))
        L = rng.integers(-2, 3, (1, E)).astype(np.float32)   # many ties
        if rng.random() < 0.3:
            L = L * np.float32(0.0)                      # mixes -0.0 and +0.0
        got = o.select_topk(L, k)[0].tolist()
        assert got == _brute_topk([float(v) for v in L[0]], k), (L, k, got)


def pin_weights(o, seed=3):
    """Weights sum to one; with k = E they are scipy's full softmax; adding a
    constant to every logit leaves them unchanged."""
    import scipy.special
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((32, 16)).astype(np.float32)
    for k in (1, 3, 16):
        idx = o.select_topk(L, k)
        w = o.topk_weights(L, idx)
        assert np.allclose(w.sum(1), 1.0, atol=1e-12, rtol=0)
        assert np.all(np.diff(w, axis=1) <= 0)           # descending logits
    idx = o.select_topk(L, 16)
    full = scipy.special.softmax(L.astype(np.float64), axis=1)
    assert np.allclose(o.topk_weights(L, idx), np.take_along_axis(full, idx.astype(np.int64), 1),
                       rtol=1e-12, atol=0)
    Li = rng.integers(-8, 8, (8, 10)).astype(np.float32)
    idx = o.select_topk(Li, 4)
    assert np.allclose(o.topk_weights(Li + np.float32(32.0), idx), o.topk_weights(Li, idx),
                       rtol=1e-12, atol=0)


def _brute_permute(idx, E, S):
    T, k = idx.shape
    ids = []
    for t in range(T):
        for j in range(k + S):
            ids.append(int(idx[t, j]) if j < k else E + j - k)
    counts = [0] * (E + S)
    for e in ids:
        counts[e] += 1
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    fill = list(offsets[:-1])
    srt = [0] * len(ids)
    for a, e in enumerate(ids):
        srt[fill[e]] = a
        fill[e] += 1
    inv = [0] * len(ids)
    for p, a in enumerate(srt):
        inv[a] = p
    return counts, offsets, srt, inv


def pin_permute_bruteforce(o, trials=100, seed=4):
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        E = int(rng.integers(1, 20))
        k = int(rng.integers(1, min(E, 6) + 1))
        S = int(rng.integers(0, 2))
        T = int(rng.integers(0, 12))
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32) \
            if T else np.zeros((0, k), np.int32)
        got = [a.tolist() for a in o.permute(idx, E, S)]
        assert got == list(_brute_permute(idx, E, S)), (idx, E, S)


# --------------------------------------------------------------------------
# expert FFN and layer
# --------------------------------------------------------------------------
def _f32(v):
    return float(np.float32(v))


def _brute_layer(x_bits, wr_bits, bias, dense, E, k, S):
    """Scalar-loop layer in Python floats (fp64) from dequantised weights."""
    def bf(u):
        return struct.unpack("<f", struct.pack("<I", int(u) << 16))[0]
    T, H = x_bits.shape
    x = [[bf(x_bits[t, h]) for h in range(H)] for t in range(T)]
    wr = [[bf(wr_bits[e, h]) for h in range(H)] for e in range(E)]
    outs = []
    for t in range(T):
        logits = []
        for e in range(E):
            acc = 0.0
            for h in range(H):
                acc += x[t][h] * wr[e][h]
            l = _f32(acc)
            if bias is not None:
                l = _f32(l + float(bias[e]))
            logits.append(l)
        sel = sorted(range(E), key=lambda e: (-logits[e], e))[:k]
        ex = [math.exp(logits[e] - logits[sel[0]]) for e in sel]
        tot = sum(ex)
        experts = [(e, v / tot) for e, v in zip(sel, ex)] + [(E + j, 1.0) for j in range(S)]
        out = [0.0] * H
        for e, wgt in experts:
            wg, wu, wd = dense[e]
            I = wg.shape[0]
            hvec = []
            for i in range(I):
                g = sum(float(wg[i, h]) * x[t][h] for h in range(H))
                u = sum(float(wu[i, h]) * x[t][h] for h in range(H))
                hvec.append(g / (1.0 + math.exp(-g)) * u)
            for n in range(H):
                yv = sum(float(wd[n, i]) * hvec[i] for i in range(I))
                out[n] += wgt * yv
        outs.append(out)
    return np.array(outs)


def tiny_layer(o, bits, E=2, S=0, H=8, I=8, group=8, seed=5, k=1, T=3, with_bias=False):
    rng = np.random.default_rng(seed)
    experts = {}
    for e in range(E + S):
        ex = {}
        for name, shape in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
            w = (rng.standard_normal(shape) * 0.5).astype(np.float32)
            ex[name] = o.quantize(w, bits, group=group)
        experts[e] = ex
    layer = o.QuantLayer(H, I, E, k, S, experts, group=group)
    x = rng.standard_normal((T, H)).astype(np.float32)
    x_bits = ((x.view(np.uint32) + 0x8000) >> 16).astype(np.uint16)   # any bf16 values will do
    wr = rng.standard_normal((E, H)).astype(np.float32)
    wr_bits = ((wr.view(np.uint32) + 0x8000) >> 16).astype(np.uint16)
    bias = rng.standard_normal(E).astype(np.float32) if with_bias else None
    return layer, x_bits, wr_bits, bias


def pin_layer_bruteforce(o):
    """Whole layer vs scalar loops on 2-4 expert, 8-dim layers, all bit widths."""
    for bits in (4, 6, 8):
        for (E, k, S, with_bias) in ((2, 1, 0, False), (2, 2, 0, True), (3, 2, 1, True), (4, 3, 1, False)):
            layer, x, wr, bias = tiny_layer(o, bits, E=E, S=S, k=k, with_bias=with_bias,
                                            seed=bits * 10 + E)
            got = o.moe_layer(layer, x, wr, bias)["out"]
            dense = {e: layer.dense(e) for e in range(E + S)}
            ref = _brute_layer(x, wr, bias, dense, E, k, S)
            assert np.allclose(got, ref, rtol=1e-11, atol=1e-12), (bits, E, k, S)


def _torch_ffn(x, wg, wu, wd):
    import torch
    xt = torch.tensor(x, dtype=torch.float64)
    g = xt @ torch.tensor(np.asarray(wg, np.float64)).T
    u = xt @ torch.tensor(np.asarray(wu, np.float64)).T
    return ((torch.nn.functional.silu(g) * u) @ torch.tensor(np.asarray(wd, np.float64)).T).numpy()


def pin_layer_special_cases(o, seed=6):
    """k = E is the dense softmax mixture; E = k = 1 is one quantised SwiGLU
    FFN; a shared expert adds its FFN with weight one; permuting the order of
    the experts changes nothing.  FFNs here come from torch (fp64)."""
    import scipy.special
    rng = np.random.default_rng(seed)
    H, I, group = 128, 64, 64
    for bits in (4, 6, 8):
        E, S = 5, 1
        experts = {}
        for e in range(E + S):
            experts[e] = {n: o.quantize((rng.standard_normal(sh) * 0.05).astype(np.float32), bits)
                          for n, sh in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I)))}
        x = (rng.standard_normal((6, H))).astype(np.float32)
        xb = ((x.view(np.uint32) + 0x8000) >> 16).astype(np.uint16)
        xf = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        wr = ((rng.standard_normal((E, H)) * 0.1).astype(np.float32).view(np.uint32) + 0x8000) >> 16
        wr = wr.astype(np.uint16)
        dense = {e: tuple(o.dequant(*experts[e][p]) for p in ("gate", "up", "down")) for e in experts}
        ffn = {e: _torch_ffn(xf, *dense[e]) for e in experts}
        # k = E: dense mixture
        layer = o.QuantLayer(H, I, E, E, 0, experts)
        r = o.moe_layer(layer, xb, wr)
        p = scipy.special.softmax(r["logits"].astype(np.float64), axis=1)
        mix = sum(p[:, e:e + 1] * ffn[e] for e in range(E))
        assert np.allclose(r["out"], mix, rtol=1e-10, atol=1e-13)
        # shared expert adds its FFN with weight one
        layer2 = o.QuantLayer(H, I, E, 2, 0, experts)
        layer3 = o.QuantLayer(H, I, E, 2, 1, experts)
        d = o.moe_layer(layer3, xb, wr)["out"] - o.moe_layer(layer2, xb, wr)["out"]
        assert np.allclose(d, ffn[E], rtol=1e-10, atol=1e-13)
        # E = k = 1
        one = o.QuantLayer(H, I, 1, 1, 0, {0: experts[3]})
        r1 = o.moe_layer(one, xb, wr[3:4])
        assert np.array_equal(r1["w"], np.ones((6, 1)))
        assert np.allclose(r1["out"], ffn[3], rtol=1e-12, atol=1e-14)
        # permutation of expert order
        perm = rng.permutation(E)
        bias = rng.standard_normal(E).astype(np.float32)
        lay_a = o.QuantLayer(H, I, E, 3, 1, experts)
        exp_b = {i: experts[int(perm[i])] for i in range(E)}
        exp_b[E] = experts[E]
        lay_b = o.QuantLayer(H, I, E, 3, 1, exp_b)
        ra = o.moe_layer(lay_a, xb, wr, bias)
        rb = o.moe_layer(lay_b, xb, wr[perm], bias[perm])
        assert np.allclose(ra["out"], rb["out"], rtol=1e-12, atol=1e-14)
        assert np.array_equal(perm[rb["idx"]], ra["idx"])


def pin_on_grid_layer(o, seed=7):
    """Weights on the quantisation grid dequantise exactly, so the layer's
    FFN output equals torch's fp64 FFN of the original weights."""
    rng = np.random.default_rng(seed)
    H, I, bits = 128, 64, 4
    experts, orig = {}, {}
    for e in range(2):
        ex, og = {}, {}
        for n, (N, K) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
            q0 = rng.integers(0, 16, (N, K // 64, 64))
            q0[:, :, 0], q0[:, :, 1] = 0, 15
            z0 = rng.integers(0, 16, (N, K // 64))
            w = ((q0 - z0[..., None]) * 2.0 ** -6).astype(np.float32).reshape(N, K)
            ex[n] = o.quantize(w, bits)
            og[n] = w
        experts[e], orig[e] = ex, og
    x = rng.standard_normal((4, H)).astype(np.float32)
    xb = ((x.view(np.uint32) + 0x8000) >> 16).astype(np.uint16)
    xf = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    layer = o.QuantLayer(H, I, 1, 1, 1, {0: experts[0], 1: experts[1]})
    wr = np.zeros((1, H), np.uint16)
    r = o.moe_layer(layer, xb, wr)
    ref = _torch_ffn(xf, orig[0]["gate"], orig[0]["up"], orig[0]["down"]) + \
        _torch_ffn(xf, orig[1]["gate"], orig[1]["up"], orig[1]["down"])
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-14)


def pin_bf16_and_norm(o, seed=8):
    """bf16 rounding equals torch's; RMSNorm of a constant vector is the
    closed form c / sqrt(c^2 + eps); residual add rounds once."""
    import torch
    rng = np.random.default_rng(seed)
    a = np.concatenate([rng.standard_normal(10000).astype(np.float32) * 10.0 ** rng.integers(-20, 20, 10000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 3.0e38], np.float32)])
    a = a.astype(np.float32)
    ref = torch.tensor(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(o.f32_to_bf16(a), ref)
    assert np.array_equal(o.bf16_to_f32(ref), torch.tensor(a).to(torch.bfloat16).float().numpy())
    # fp64 -> bf16 rounds once (no detour through fp32)
    d = np.array([1.0 + 2.0 ** -8 + 2.0 ** -40, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8], np.float64)
    assert o.bf16_to_f32(o.f32_to_bf16(d)).tolist() == [1.0078125, 1.0, 1.015625]
    for c in (0.5, 3.0, -2.0, 1e-3):
        xb = o.f32_to_bf16(np.full((1, 64), c, np.float32))
        cb = float(o.bf16_to_f32(xb)[0, 0])
        expect = o.f32_to_bf16(np.array([cb / math.sqrt(cb * cb + 1e-6)], np.float64))[0]
        assert np.all(o.rmsnorm_bf16(xb) == expect)
    x = rng.standard_normal((4, 256)).astype(np.float32)
    xb = o.f32_to_bf16(x)
    ref = torch.nn.functional.rms_norm(torch.tensor(o.bf16_to_f32(xb), dtype=torch.float64), (256,), eps=1e-6)
    got = o.bf16_to_f32(o.rmsnorm_bf16(xb)).astype(np.float64)
    assert np.allclose(got, ref.numpy(), rtol=2.0 ** -8, atol=0)
    one = o.f32_to_bf16(np.array([[1.0, 1.0]], np.float32))
    # the block output is rounded to bf16 first (2^-8 + 2^-20 -> 2^-8), then
    # 1 + 2^-8 is a tie that goes to even (1.0); 1 + 1.5 ulp goes to 1 + 2 ulp
    r = o.residual_bf16(one, np.array([[2.0 ** -8 + 2.0 ** -20, 2.0 ** -7 + 2.0 ** -8]]))
    assert o.bf16_to_f32(r)[0].tolist() == [1.0, 1.015625]


def pin_ffn_bf16_h(o, seed=9):
    """h_bf16 rounds h = silu(g) u to bf16 before the down projection: torch's
    own silu and bf16 conversion of the same h give the same y, and the change
    from the fp64 FFN stays within the rounding bound 2^-9 sum_i |Wd||h|."""
    import torch
    rng = np.random.default_rng(seed)
    n, H, I = 5, 64, 48
    x = rng.standard_normal((n, H))
    wg, wu = (rng.standard_normal((I, H)) * 0.3).astype(np.float32), (rng.standard_normal((I, H)) * 0.3).astype(np.float32)
    wd = (rng.standard_normal((H, I)) * 0.3).astype(np.float32)
    xt = torch.tensor(x, dtype=torch.float64)
    h = torch.nn.functional.silu(xt @ torch.tensor(wg, dtype=torch.float64).T) * (xt @ torch.tensor(wu, dtype=torch.float64).T)
    hb = h.float().to(torch.bfloat16).double()
    ref = (hb @ torch.tensor(wd, dtype=torch.float64).T).numpy()
    got = o.expert_ffn(x, wg, wu, wd, h_bf16=True)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-14)
    exact = o.expert_ffn(x, wg, wu, wd)
    bound = 2.0 ** -9 * (np.abs(h.numpy()) @ np.abs(wd.astype(np.float64)).T)
    assert np.all(np.abs(got - exact) <= bound * (1 + 1e-9))
    assert not np.array_equal(got, exact)


def pin_ffn_bf16_w(o, seed=10):
    """w_bf16 rounds the dequantised fp32 weights to bf16 before the
    products: torch's fp32 -> bf16 conversion of the same weights, with h
    rounded as well, gives the same y; weights that are bf16 values already
    (a power-of-two grid) are left as they are; otherwise the result moves
    from the fp64 FFN."""
    import torch
    rng = np.random.default_rng(seed)
    n, H, I = 6, 64, 48
    x = rng.standard_normal((n, H))
    wg, wu, wd = ((rng.standard_normal(sh) * 0.3).astype(np.float32) for sh in ((I, H), (I, H), (H, I)))
    tb = lambda a: torch.tensor(a).to(torch.bfloat16).double()       # fp32 -> bf16, nearest even
    xt = torch.tensor(x, dtype=torch.float64)
    h = torch.nn.functional.silu(xt @ tb(wg).T) * (xt @ tb(wu).T)
    hb = torch.tensor(o.bf16_to_f32(o.f32_to_bf16(h.numpy())), dtype=torch.float64)
    ref = (hb @ tb(wd).T).numpy()
    got = o.expert_ffn(x, wg, wu, wd, h_bf16=True, w_bf16=True)
    assert np.allclose(got, ref, rtol=1e-12, atol=1e-14)
    assert not np.allclose(got, o.expert_ffn(x, wg, wu, wd, h_bf16=True), rtol=1e-6, atol=0)
    grid = [((rng.integers(-8, 8, sh)) * 2.0 ** -5).astype(np.float32) for sh in ((I, H), (I, H), (H, I))]
    assert np.array_equal(o.expert_ffn(x, *grid, w_bf16=True), o.expert_ffn(x, *grid))


# --------------------------------------------------------------------------
# HQQ zero-point refinement
# --------------------------------------------------------------------------
def pin_shrink_closed_form(o):
    """The lp shrink on values where it is exact by hand: p = 1 is the soft
    threshold sign(x) max(|x| - 1/beta, 0); p = 1/2 subtracts |x|^(-1/2)/beta."""
    x = np.array([3, -3, 0.125, -0.125, 0, 0.25], np.float32)
    assert np.array_equal(o.shrink_lp(x, 4.0, 1.0), np.array([2.75, -2.75, 0, 0, 0, 0], np.float32))
    x = np.array([4, 0.25, -16, 0.0625, 0], np.float32)
    assert np.array_equal(o.shrink_lp(x, 1.0, 0.5), np.array([3.5, 0, -15.75, 0, 0], np.float32))
    # large |x|: the threshold vanishes relative to x
    assert o.shrink_lp(np.array([1e6], np.float32), 1e3, 0.7)[0] == 1e6 - 1e6 ** -0.3 / 1e3
    # fp64 throughout: a residual of 2^-30 with p = 1 and beta = 2^40 keeps 2^-30 - 2^-40
    assert o.shrink_lp(np.array([2.0 ** -30]), 2.0 ** 40, 1.0)[0] == 2.0 ** -30 - 2.0 ** -40


def pin_group_mean(o):
    """A group's mean is its fp64 sum over the count: exact on values an
    fp32 sum loses (2^24 + 1 + 1 - 2^24 = 2, where a pairwise fp32 tree gives
    1 and a left-to-right fp32 sum 0), the same in any order of the values,
    and the exact mean of integers."""
    x = np.zeros(64, np.float32)
    x[:4] = [2.0 ** 24, 1, 1, -2.0 ** 24]
    assert o.group_mean(x) == 2 / 64
    rng = np.random.default_rng(20)
    y = (rng.standard_normal((50, 64)) * 100).astype(np.float32)
    for _ in range(3):
        perm = rng.permutation(64)
        assert np.array_equal(o.group_mean(y).astype(np.float16), o.group_mean(y[:, perm]).astype(np.float16))
    n = rng.integers(-1000, 1000, size=(50, 64))
    assert np.array_equal(o.group_mean(n.astype(np.float32)), n.sum(1) / 64)


def pin_hqq_golden(o):
    """The refinement's trajectory on a group worked by hand
    (tests/golden/hqq_trajectory.json): every round's zero and error, the
    round it stops at (the zero stops moving once the fp16 step exceeds the
    shrink threshold), the kept zero and its codes."""
    with open(os.path.join(GOLDEN, "hqq_trajectory.json")) as fh:
        g = json.load(fh)
    w = np.array([1.0, 16.0] + [4.25] * 31 + [8.375] * 31, np.float32)[None, :]
    codes = np.array([0, 15] + [3] * 31 + [7] * 31, np.uint8)[None, :]
    for case in g["cases"]:
        q, s16, z16, rounds = o.hqq_refine(w, g["group"]["bits"], lp=case["lp"], beta=case["beta"],
                                          kappa=case["kappa"], iters=case["iters"], trace=True)
        zs = [float(r[0][0, 0]) for r in rounds if r[2][0, 0]]
        Es = [float(r[1][0, 0]) for r in rounds if r[2][0, 0]]
        assert zs == case["z_rounds"], (zs, case["z_rounds"])
        assert Es == case["E_rounds"], (Es, case["E_rounds"])
        assert float(z16[0, 0]) == case["z_final"] and float(s16[0, 0]) == 1.0
        assert np.array_equal(q, codes)


def _group_mae(o, w, q, s16, z16):
    d = o.dequant(q, s16, z16)
    N, K = w.shape
    return np.abs(w.astype(np.float64) - d).reshape(N, K // 64, 64).mean(-1)


def pin_hqq_refine(o, bits, seed=21, N=64, K=512):
    """The refinement: no rounds -> the min-max result; an exactly
    representable group stays as it is (error 0); no group's error grows;
    over seeded N(0, 0.02) weights the mean absolute error falls by a margin
    (measured 3.7 / 3.5 / 2.2 % at 4 / 6 / 8 bits)."""
    rng = np.random.default_rng(seed + bits)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    q0, s0, z0 = o.quantize(w, bits)
    q1, s1, z1 = o.hqq_refine(w, bits, iters=0)
    assert np.array_equal(q0, q1) and np.array_equal(s0.view(np.uint16), s1.view(np.uint16))
    assert np.array_equal(z0.view(np.uint16), z1.view(np.uint16))
    # on the grid: w = (q* - z*) s with both code ends present
    qmax = 2 ** bits - 1
    qs = rng.integers(0, qmax + 1, size=(8, 64))
    qs[:, 0], qs[:, 1] = 0, qmax
    wg = ((qs - 3.5) * 2.0 ** -7).astype(np.float32)
    qg, sg, zg = o.hqq_refine(wg, bits)
    assert np.array_equal(qg, qs) and np.all(sg == np.float16(2.0 ** -7)) and np.all(zg == np.float16(3.5))
    # never worse, better on average
    q2, s2, z2 = o.hqq_refine(w, bits)
    assert np.array_equal(s2.view(np.uint16), s0.view(np.uint16))
    e0 = _group_mae(o, w, q0, s0, z0)
    e2 = _group_mae(o, w, q2, s2, z2)
    assert np.all(e2 <= e0 * (1 + 1e-6))
    assert e2.mean() <= e0.mean() * (1 - (0.01 if bits == 8 else 0.02)), (e0.mean(), e2.mean())
    # the codes are those of the stored zero
    v = w.reshape(N, K // 64, 64) / s2.astype(np.float32)[..., None] + z2.astype(np.float32)[..., None]
    assert np.array_equal(np.clip(np.rint(v), 0, qmax).astype(np.uint8).reshape(N, K), q2)


def pin_hqq_least_squares_round(o, bits=4, seed=22, N=64, K=512):
    """With beta -> 0 the residual is shrunk to zero and the zero update is
    the least-squares zero for the current codes, mean(q - w / s) (the
    minimiser of sum (w - (q - z) s)^2 over z).  After one such round a group
    keeps either its min-max zero or that one (to one fp16 ulp), the latter
    only where it lowers the error."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    q0, s0, z0 = o.quantize(w, bits)
    q1, s1, z1 = o.hqq_refine(w, bits, lp=1.0, beta=1e-30, kappa=1.0, iters=2)
    wg = w.reshape(N, K // 64, 64).astype(np.float64)
    sf = s0.astype(np.float64)[..., None]
    zls = np.mean(q0.reshape(N, K // 64, 64) - wg / sf, axis=-1)
    moved = z1 != z0
    ulp = np.spacing(np.abs(zls).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(z1.astype(np.float64) - zls)[moved] <= ulp[moved])
    assert moved.mean() > 0.1
    e0 = _group_mae(o, w, q0, s0, z0)
    e1 = _group_mae(o, w, q1, s1, z1)
    assert np.all(e1[moved] < e0[moved])


# --------------------------------------------------------------------------
# KV-cache codec
# --------------------------------------------------------------------------
def pin_kv_codec(o, seed=23):
    """The codec on bf16 rows: values on a power-of-two grid whose ends are
    the group's min and max come back exactly; any row comes back within half
    a quantisation step plus one bf16 rounding; the packed bytes of 4-bit rows
    hold code 2i in the low nibble of byte i (hand-built row)."""
    rng = np.random.default_rng(seed)
    for bits in (4, 6, 8):
        qmax = 2 ** bits - 1
        q = rng.integers(0, qmax + 1, size=(16, 128))
        q[:, 0], q[:, 1], q[:, 64], q[:, 65] = 0, qmax, 0, qmax
        x = o.f32_to_bf16(((q - 5) * 2.0 ** -6).astype(np.float32))
        p, s16, z16 = o.kv_encode(x, bits)
        assert p.shape == (16, 128 * bits // 8) and np.all(s16 == np.float16(2.0 ** -6)) and np.all(z16 == 5)
        assert np.array_equal(o.kv_decode(p, s16, z16, bits, 128), x)
        y = o.f32_to_bf16((rng.standard_normal((32, 192)) * 3).astype(np.float32))
        p, s16, z16 = o.kv_encode(y, bits)
        back = o.bf16_to_f32(o.kv_decode(p, s16, z16, bits, 192)).astype(np.float64)
        yf = o.bf16_to_f32(y).astype(np.float64)
        step = np.repeat(s16.astype(np.float64), 64, axis=1)
        # half a step, widened by the fp16 rounding of s and z (<= (2^bits - 1) 2^-10 steps)
        assert np.all(np.abs(back - yf) <= (0.5 + (2 ** bits - 1) * 2.0 ** -10) * step + 2.0 ** -8 * np.abs(back) + 1e-30)
    # 4-bit byte order by hand: codes 0..15 then 15..0 repeated
    codes = np.tile(np.r_[np.arange(16), np.arange(15, -1, -1)], 2)
    x = o.f32_to_bf16((codes * 0.5).astype(np.float32))[None, :]
    p, s16, z16 = o.kv_encode(x, 4)
    assert s16[0, 0] == np.float16(0.5) and z16[0, 0] == 0
    assert list(p[0, :8]) == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    # decoding rounds to the nearest bf16: 8-bit code 103 with s = 5/512 and
    # z = 0 is 515/512 = 1.005859375, nearer 1 + 2^-7 (bf16 0x3F81) than 1
    pk = np.zeros((1, 64), np.uint8)
    pk[0, 0] = 103
    out = o.kv_decode(pk, np.array([[5 / 512]], np.float16), np.zeros((1, 1), np.float16), 8, 64)
    assert out[0, 0] == 0x3F81 and np.all(out[0, 1:] == 0)
