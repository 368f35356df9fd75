"""Plant plausible mistakes in the oracle (on the CPU) and check that at
least one pin catches each of them.  This is how we know the pins constrain
the oracle rather than echo it."""
import numpy as np
import pytest

import oracle
import oracle.moe as om
from tests import pins

_quantize, _pack, _permute, _expert_ffn = om.quantize, om.pack, om.permute, om.expert_ffn


def _fails(fn, *a, **kw):
    try:
        fn(*a, **kw)
    except AssertionError:
        return True
    return False


def _quantize_zero_from_max(w, bits, group=64):
    # mistake: zero taken from the maximum instead of the minimum
    w = np.asarray(w, np.float32)
    N, K = w.shape
    qmax = np.float32(2 ** bits - 1)
    wg = w.reshape(N, K // group, group)
    mn, mx = wg.min(2), wg.max(2)
    s16 = ((mx - mn) / qmax).astype(np.float16)
    s16 = np.where(s16 == 0, np.float16(1), s16)
    z16 = (mx / s16.astype(np.float32)).astype(np.float16)
    q = np.clip(np.rint(wg / s16.astype(np.float32)[..., None] + z16.astype(np.float32)[..., None]), 0, qmax)
    return q.astype(np.uint8).reshape(N, K), s16, z16


def _quantize_trunc(w, bits, group=64):
    # mistake: truncation instead of round-to-nearest-even
    q, s16, z16 = _quantize(w, bits, group)
    N, K = q.shape
    wg = np.asarray(w, np.float32).reshape(N, K // group, group)
    v = wg / s16.astype(np.float32)[..., None] + z16.astype(np.float32)[..., None]
    q2 = np.clip(np.floor(v), 0, 2 ** bits - 1).astype(np.uint8).reshape(N, K)
    return q2, s16, z16


def _pack_swapped_nibbles(q, bits):
    if bits == 4:
        q = np.asarray(q, np.uint8)
        return (q[:, 1::2] | (q[:, 0::2] << 4)).astype(np.uint8)
    return _pack(q, bits)


def _dequant_plus_zero(q, s16, z16, group=64):
    # mistake: sign of the zero flipped
    N, K = q.shape
    qf = q.astype(np.float32).reshape(N, K // group, group)
    return ((qf + z16.astype(np.float32)[..., None]) * s16.astype(np.float32)[..., None]).reshape(N, K)


def _select_last_index_wins(L, k):
    # mistake: ties broken towards the higher expert index
    L = np.asarray(L, np.float32)
    E = L.shape[1]
    order = np.argsort(-L[:, ::-1], axis=1, kind="stable")
    return (E - 1 - order[:, :k]).astype(np.int32)


def _weights_full_softmax_no_renorm(L, idx):
    # mistake: softmax over all experts, not renormalised over the selected
    L64 = np.asarray(L, np.float64)
    p = np.exp(L64 - L64.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    return np.take_along_axis(p, idx.astype(np.int64), 1)


def _permute_unstable(idx, E, S=0):
    counts, offsets, srt, inv = _permute(idx, E, S)
    srt = srt.copy()
    for e in range(E + S):       # mistake: descending order inside an expert
        srt[offsets[e]:offsets[e + 1]] = srt[offsets[e]:offsets[e + 1]][::-1]
    inv = np.empty_like(srt)
    inv[srt] = np.arange(srt.size)
    return counts, offsets, srt, inv


def _ffn_silu_on_up(x, wg, wu, wd, h_bf16=False, w_bf16=False):
    x = np.asarray(x, np.float64)
    g = x @ np.asarray(wg, np.float64).T
    u = x @ np.asarray(wu, np.float64).T
    return (g * om.silu(u)) @ np.asarray(wd, np.float64).T


def _ffn_transposed_down(x, wg, wu, wd, h_bf16=False, w_bf16=False):
    x = np.asarray(x, np.float64)
    g = x @ np.asarray(wg, np.float64).T
    u = x @ np.asarray(wu, np.float64).T
    return (om.silu(g) * u) @ np.asarray(wd, np.float64).T[::-1]   # mistake: rows reversed


def _ffn_rounds_up_not_h(x, wg, wu, wd, h_bf16=False, w_bf16=False):
    # mistake: the bf16 rounding applied to the up projection instead of h
    x = np.asarray(x, np.float64)
    g = x @ np.asarray(wg, np.float64).T
    u = x @ np.asarray(wu, np.float64).T
    if h_bf16:
        u = om.bf16_to_f32(om.f32_to_bf16(u)).astype(np.float64)
    return (om.silu(g) * u) @ np.asarray(wd, np.float64).T


def _ffn_w_truncated(x, wg, wu, wd, h_bf16=False, w_bf16=False):
    # mistake: the bf16 weights truncated instead of rounded to nearest even
    if w_bf16:
        wg, wu, wd = (om.bf16_to_f32((np.asarray(m, np.float32).view(np.uint32) >> 16).astype(np.uint16))
                      for m in (wg, wu, wd))
    return _expert_ffn(x, wg, wu, wd, h_bf16)


def _combine_drop_shared(y, w, S=0):
    # mistake: the shared experts' outputs are left out
    T, kS, H = y.shape
    out = np.zeros((T, H))
    for j in range(kS - S):
        out += w[:, j:j + 1] * y[:, j, :]
    return out


def _rmsnorm_no_eps(x_bf16, eps=1e-6, gamma=None):
    x = om.bf16_to_f32(x_bf16).astype(np.float64)
    return om.f32_to_bf16(x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True)))


def _residual_no_block_rounding(x_bf16, moe_out):
    return om.f32_to_bf16(om.bf16_to_f32(x_bf16).astype(np.float64) + np.asarray(moe_out, np.float64))


def _shrink_identity(x, beta, p):
    # mistake: the residual is not shrunk at all
    return np.asarray(x, np.float64)


def _mean_fp32_left_to_right(x):
    # mistake: the group's mean summed left to right in fp32
    x = np.asarray(x, np.float32)
    acc = np.zeros(x.shape[:-1], np.float32)
    for i in range(x.shape[-1]):
        acc = (acc + x[..., i]).astype(np.float32)
    return (acc / np.float32(x.shape[-1])).astype(np.float64)


def _hqq_variant(sign=1.0, keep_best=True, max_rounds=None):
    """The refinement with one plausible mistake planted (the rest as the
    oracle states it)."""
    def refine(w, bits, lp=0.7, beta=10.0, kappa=1.01, iters=20, group=64, trace=False):
        w = np.asarray(w, np.float32)
        N, K = w.shape
        q0, s16, z16 = _quantize(w, bits, group)
        qmax = np.float32(2 ** bits - 1)
        wg = w.reshape(N, K // group, group)
        sf = s16.astype(np.float32)[..., None]
        sd, wd = sf.astype(np.float64), wg.astype(np.float64)
        z = z16.astype(np.float32)
        zb, best, active = z.copy(), np.full(z.shape, np.inf), np.ones(z.shape, bool)
        b, p, kap = np.float64(np.float32(beta)), np.float64(np.float32(lp)), np.float64(np.float32(kappa))
        rounds = []
        n = iters if max_rounds is None else min(iters, max_rounds)
        for _ in range(n):
            if not active.any():
                break
            qv = np.clip(np.rint(wg / sf + z[..., None]), 0, qmax)
            r = wd - (qv.astype(np.float64) - z[..., None]) * sd
            E = om.group_mean(np.abs(r))
            rounds.append((z.copy(), E.copy(), active.copy()))
            if keep_best:
                active = active & (E < best)
                best = np.where(active, E, best)
                zb = np.where(active, z, zb)
            e = om.shrink_lp(r, b, p)
            znew = om.group_mean(qv + sign * (-(wd - e) / sd))
            z = np.where(active, znew.astype(np.float16).astype(np.float32), z)
            if not keep_best:
                zb = z
            b = b * kap
        q = np.clip(np.rint(wg / sf + zb[..., None]), 0, qmax)
        out = (q.astype(np.uint8).reshape(N, K), s16, zb.astype(np.float16))
        return out + (rounds,) if trace else out
    return refine


_hqq_zero_sign_flipped = _hqq_variant(sign=-1.0)     # mistake: z = mean(q + (w - e) / s)
_hqq_keeps_last = _hqq_variant(keep_best=False)      # mistake: the last zero, not the best one
_hqq_round_cap = _hqq_variant(max_rounds=5)          # mistake: at most 5 rounds whatever iters says
_hqq_zero_sign_flipped.__name__ = "_hqq_zero_sign_flipped"
_hqq_keeps_last.__name__ = "_hqq_keeps_last"
_hqq_round_cap.__name__ = "_hqq_round_cap"


def _kv_decode_truncating(packed, s16, z16, bits, D):
    # mistake: the decoded value truncated to bf16 instead of rounded
    d = om.dequant(om.unpack(packed, bits, D), s16, z16).astype(np.float32)
    return (d.view(np.uint32) >> 16).astype(np.uint16)


MUTANTS = [
    ("quantize", _quantize_zero_from_max, [pins.pin_quant_golden, lambda o: pins.pin_quant_error_bound(o, 4)]),
    ("quantize", _quantize_trunc, [pins.pin_quant_golden, lambda o: pins.pin_quant_error_bound(o, 6)]),
    ("pack", _pack_swapped_nibbles, [pins.pin_quant_golden]),
    ("dequant", _dequant_plus_zero, [pins.pin_quant_golden, lambda o: pins.pin_quant_on_grid(o, 8)]),
    ("select_topk", _select_last_index_wins, [pins.pin_routing_golden, pins.pin_topk_bruteforce]),
    ("topk_weights", _weights_full_softmax_no_renorm, [pins.pin_routing_golden, pins.pin_weights]),
    ("permute", _permute_unstable, [pins.pin_routing_golden, pins.pin_permute_bruteforce]),
    ("expert_ffn", _ffn_silu_on_up, [pins.pin_layer_bruteforce, pins.pin_layer_special_cases]),
    ("expert_ffn", _ffn_transposed_down, [pins.pin_layer_bruteforce, pins.pin_on_grid_layer]),
    ("expert_ffn", _ffn_rounds_up_not_h, [pins.pin_ffn_bf16_h]),
    ("expert_ffn", _ffn_w_truncated, [pins.pin_ffn_bf16_w]),
    ("combine", _combine_drop_shared, [pins.pin_layer_bruteforce, pins.pin_layer_special_cases]),
    ("rmsnorm_bf16", _rmsnorm_no_eps, [pins.pin_bf16_and_norm]),
    ("residual_bf16", _residual_no_block_rounding, [pins.pin_bf16_and_norm]),
    ("shrink_lp", _shrink_identity, [pins.pin_shrink_closed_form, lambda o: pins.pin_hqq_refine(o, 4)]),
    ("shrink_lp", _shrink_identity, [pins.pin_hqq_golden]),
    ("group_mean", _mean_fp32_left_to_right, [pins.pin_group_mean]),
    ("hqq_refine", _hqq_zero_sign_flipped, [pins.pin_hqq_least_squares_round, pins.pin_hqq_golden]),
    ("hqq_refine", _hqq_keeps_last, [lambda o: pins.pin_hqq_refine(o, 6), pins.pin_hqq_golden]),
    ("hqq_refine", _hqq_round_cap, [pins.pin_hqq_golden]),
    ("kv_decode", _kv_decode_truncating, [pins.pin_kv_codec]),
]


@pytest.mark.parametrize("name,mutant,checks", MUTANTS,
                         ids=[f"{m[0]}:{m[1].__name__}" for m in MUTANTS])
def test_pins_catch_planted_mistake(monkeypatch, name, mutant, checks):
    monkeypatch.setattr(om, name, mutant)
    monkeypatch.setattr(oracle, name, mutant)
    for check in checks:
        assert _fails(check, oracle), f"pin {check} did not catch mutant {mutant.__name__}"
