"""GPU parity of the whole MoE layer (route -> permute -> decode or prefill
expert FFN -> combine) against the oracle, through the C ABI.

The oracle is routed from the GPU's fp32 logits (its selection on given
logits is checked bit for bit elsewhere), and the GPU logits themselves are
checked against the oracle's.  Layer outputs must satisfy
max|gpu - oracle| / (max|oracle| + 1e-6) <= 2e-2 on the bf16 output against
the fp64 oracle.  The decode path keeps fp32 arithmetic except for h, which
it stores in bf16 between the projections; against the oracle variant that
rounds h the same way it is also held to the tighter DECODE_TOL.
Full-size workloads compare sampled tokens (tokens are independent in a MoE
layer, so the oracle's result for a token subset is exact)."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import bf16_tensor, gpu_layer, oracle_layer, rel_err, to_bits

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

SPEC_TOL = 2e-2
# Against the oracle variant that rounds h to bf16 as the decode path does,
# the only differences left are fp32 accumulation (~1e-6) and the h values
# whose fp32 and fp64 results fall on opposite sides of a bf16 rounding
# boundary: each such h moves by one bf16 ulp (2^-8 relative).  A few h in
# 10^3 do (fp32 error ~1e-5 relative against a 2^-8 spacing), so y stays
# within 2e-3 of max|y|, and the bf16 output within one bf16 half-ulp
# (2^-8 relative) plus 1e-3.
DECODE_TOL = 2.0 ** -8 + 1e-3
DECODE_Y_TOL = 2e-3


@pytest.fixture(scope="module")
def bq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_expert_amd as m
    return m


_LAYERS = {}


def layer_for(bq, name, bits=None):
    key = (name, bits)
    if key not in _LAYERS:
        if len(_LAYERS) >= 2:     # keep device memory bounded
            _LAYERS.clear()
            torch.cuda.empty_cache()
        w = synth.get_workload(name)
        q = gpu_layer(w, bits=bits)
        wr = bf16_tensor(synth.router_weight_bf16(w))
        bias = synth.router_bias(w)
        bt = None if bias is None else torch.from_numpy(bias).cuda()
        _LAYERS[key] = (w, bq.MoELayer(q, wr, bt, T_max=1), oracle_layer(w, bits=bits))
    return _LAYERS[key]


def check_layer(bq, name, T, prefill, sample=None, bits=None, batch=0, fused=False):
    """fused: the decode layer through moe_decode_forward (no y to check)."""
    w, layer, olayer = layer_for(bq, name, bits)
    x = synth.activations_bf16(w, T, batch=batch)
    r = layer.forward(bf16_tensor(x), prefill=prefill, fused_layer=fused)
    torch.cuda.synchronize()
    logits = r["logits"].cpu().numpy()
    wr = synth.router_weight_bf16(w)
    bias = synth.router_bias(w)
    rows = np.arange(T) if sample is None else np.unique(np.linspace(0, T - 1, sample).astype(int))
    ref_logits = oracle.router_logits(x[rows], wr, bias)
    assert np.max(np.abs(logits[rows] - ref_logits)) <= 1e-5 * np.max(np.abs(ref_logits))
    ref = oracle.moe_layer(olayer, x[rows], logits=logits[rows])
    idx = r["idx"].cpu().numpy()
    assert np.array_equal(idx[rows], ref["idx"])
    wt = r["w"].cpu().numpy()
    assert np.max(np.abs(wt[rows] - ref["w"]) / ref["w"]) <= 1e-5
    out = oracle.bf16_to_f32(to_bits(r["out"]))[rows]
    err = rel_err(out, ref["out"])
    assert err <= SPEC_TOL, err
    if fused:
        ref_b = oracle.moe_layer(olayer, x[rows], logits=logits[rows], h_bf16=True)
        err_b = rel_err(out, ref_b["out"])
        assert err_b <= DECODE_TOL, err_b
        return r, err, None
    kS = w.k + w.S
    y = r["y"]
    y = (oracle.bf16_to_f32(to_bits(y)) if y.dtype == torch.bfloat16 else y.cpu().numpy())
    ya = y.reshape(T, kS, w.H)[rows].reshape(-1, w.H)
    yerr = rel_err(ya, ref["y"])
    if not prefill:
        ref_b = oracle.moe_layer(olayer, x[rows], logits=logits[rows], h_bf16=True)
        err_b, yerr_b = rel_err(out, ref_b["out"]), rel_err(ya, ref_b["y"])
        assert err_b <= DECODE_TOL and yerr_b <= DECODE_Y_TOL, (err_b, yerr_b)
        assert yerr <= SPEC_TOL, yerr
    else:
        print(f"  out err {err:.3e} y err {yerr:.3e}", flush=True)
        assert yerr <= SPEC_TOL, yerr
    return r, err, yerr


DECODE_CASES = [("moe_h2048_e128_k8_b4", 1), ("moe_h2048_e128_k8_b4", 16), ("moe_h2048_e256_k8_s1_b4", 1),
                ("moe_h2048_e256_k8_s1_b4", 4), ("moe_h2048_e256_k8_s1_b4", 8), ("moe_h4096_e512_k10_b4_hot", 1)]


@pytest.mark.parametrize("name,T", DECODE_CASES)
def test_decode_layer(bq, name, T):
    print(f"decode {name} T={T}", flush=True)
    check_layer(bq, name, T, prefill=False)


@pytest.mark.parametrize("bits", [6, 8])
@pytest.mark.parametrize("T", [1, 3, 16])
def test_decode_layer_6_8_bit(bq, bits, T):
    # the stacked workload's 6- and 8-bit layers use the 128-expert shapes
    print(f"decode 128-expert {bits}-bit T={T}", flush=True)
    check_layer(bq, "moe_h2048_e128_k8_b4", T, prefill=False, bits=bits, batch=bits)


FUSED_CASES = [("moe_h2048_e256_k8_s1_b4", 1), ("moe_h2048_e256_k8_s1_b4", 3), ("moe_h2048_e256_k8_s1_b4", 8),
               ("moe_h2048_e256_k8_s1_b4", 64), ("moe_h2048_e128_k8_b4", 16), ("moe_h2048_e128_k8_b4", 64),
               ("moe_h4096_e512_k10_b4_hot", 1), ("moe_h4096_e512_k10_b4_hot", 37)]


@pytest.mark.parametrize("name,T", FUSED_CASES)
def test_decode_forward(bq, name, T):
    """moe_decode_forward: routing inside the gate/up kernel, combine inside
    the down kernel.  At T = 64 on 128 experts most experts serve three or
    more tokens (several work items each)."""
    print(f"decode forward {name} T={T}", flush=True)
    check_layer(bq, name, T, prefill=False, fused=True, batch=5)


def test_decode_forward_verify_batches(bq):
    """Every batch the speculative-verify cost curve measures (1 .. 16 tokens
    per call on the 256-expert + shared layer), each against the oracle."""
    for T in range(1, 17):
        print(f"decode forward verify batch T={T}", flush=True)
        check_layer(bq, "moe_h2048_e256_k8_s1_b4", T, prefill=False, fused=True, batch=40 + T)


@pytest.mark.parametrize("bits", [6, 8])
@pytest.mark.parametrize("T", [2, 17])
def test_decode_forward_6_8_bit(bq, bits, T):
    print(f"decode forward 128-expert {bits}-bit T={T}", flush=True)
    check_layer(bq, "moe_h2048_e128_k8_b4", T, prefill=False, bits=bits, batch=bits, fused=True)


def test_decode_forward_matches_route_and_residual(bq):
    """The fused layer's logits, top-k ids and weights are those of
    moe_route_permute_decode bit for bit; with a residual its output is
    bf16(residual + bf16(sum)) of its own output without one."""
    w, layer, _ = layer_for(bq, "moe_h2048_e256_k8_s1_b4")
    T = 8
    x = bf16_tensor(synth.activations_bf16(w, T, batch=11))
    a = layer.forward(x, fused_layer=True)
    b = layer.forward(x, fused_layer=False, fused_route=True)
    for key in ("logits", "idx", "w"):
        assert torch.equal(a[key], b[key]), key
    res = bf16_tensor(synth.activations_bf16(w, T, batch=12))
    c = layer.forward(x, residual=res, fused_layer=True)
    expect = oracle.f32_to_bf16(oracle.bf16_to_f32(to_bits(res)) + oracle.bf16_to_f32(to_bits(a["out"])))
    assert np.array_equal(to_bits(c["out"]), expect)
    d = layer.forward(x, fused_layer=True)
    assert torch.equal(a["out"].view(torch.uint8), d["out"].view(torch.uint8))


ODD = {
    # 100 experts (two candidates per lane, 28 padding slots), H 512, I 256
    "e100": synth.Workload("odd_e100", 91, 512, 256, 100, 6, 1, 4, (1, 5)),
    # 1000 experts (16 per lane), k + S = 16 slots (the largest down block), 8-bit
    "e1000": synth.Workload("odd_e1000", 92, 1024, 256, 1000, 15, 1, 8, (3,)),
}


@pytest.mark.parametrize("name", ["e100", "e1000"])
def test_decode_forward_odd_shapes(bq, name):
    """moe_decode_forward on shapes the named workloads do not reach: expert
    counts that are not multiples of 64, the widest selection, 16 slots,
    H = 512 and 1024, I = 256."""
    w = ODD[name]
    q = gpu_layer(w)
    wr = synth.router_weight_bf16(w)
    ml = bq.MoELayer(q, bf16_tensor(wr), None, T_max=max(w.tokens))
    ol = oracle_layer(w)
    for T in w.tokens:
        print(f"decode forward {w.name} T={T}", flush=True)
        x = synth.activations_bf16(w, T, batch=2)
        r = ml.forward(bf16_tensor(x), fused_layer=True)
        torch.cuda.synchronize()
        logits = r["logits"].cpu().numpy()
        assert np.max(np.abs(logits - oracle.router_logits(x, wr, None))) <= 1e-5 * np.max(np.abs(logits))
        ref = oracle.moe_layer(ol, x, logits=logits)
        assert np.array_equal(r["idx"].cpu().numpy(), ref["idx"])
        assert np.max(np.abs(r["w"].cpu().numpy() - ref["w"]) / ref["w"]) <= 1e-5
        out = oracle.bf16_to_f32(to_bits(r["out"]))
        assert rel_err(out, ref["out"]) <= SPEC_TOL
        ref_b = oracle.moe_layer(ol, x, logits=logits, h_bf16=True)
        assert rel_err(out, ref_b["out"]) <= DECODE_TOL
    del ml, q
    torch.cuda.empty_cache()


def test_stacked_blocks(bq):
    """The stacked workload's first five blocks (6-, 4-, 4-, 4- and 8-bit):
    n = RMSNorm(x); x = bf16(x + bf16(moe(n))) per block, the GPU side with
    moe_decode_forward adding into x in place (residual and out alias), for
    three consecutive batch-1 tokens.  Each block is checked against the
    oracle on the GPU's own block input, and the final residual stream
    against the oracle's chain run from the token alone (routed on the GPU's
    logits of each block)."""
    _LAYERS.clear()
    torch.cuda.empty_cache()
    w = synth.get_workload("stack48_h2048_e128_k8_mixed")
    bits = synth.layer_bits(w)[:5]
    assert set(bits) == {4, 6, 8}
    layers = [gpu_layer(w, layer=l, bits=b) for l, b in enumerate(bits)]
    wrs = [bf16_tensor(synth.router_weight_bf16(w, layer=l)) for l in range(len(bits))]
    ols = [oracle_layer(w, layer=l, bits=b) for l, b in enumerate(bits)]
    ws = layers[0].workspace(1)
    for step in range(3):
        x0 = synth.activations_bf16(w, 1, batch=step)
        x = bf16_tensor(x0)
        xo = x0.copy()
        for l in range(len(bits)):
            before = to_bits(x)
            n = bq.moe_rmsnorm(x)
            nb = to_bits(n)
            _, logits, idx, _ = bq.moe_decode_forward(layers[l], n, wrs[l], None, ws, residual=x, out=x)
            torch.cuda.synchronize()
            lg = logits.cpu().numpy()
            blk = oracle.moe_layer(ols[l], nb, logits=lg)
            assert np.array_equal(idx.cpu().numpy(), blk["idx"])
            want = oracle.bf16_to_f32(oracle.residual_bf16(before, blk["out"])).astype(np.float64)
            got = oracle.bf16_to_f32(to_bits(x)).astype(np.float64)
            # the block output to the layer tolerance, plus one bf16 ulp of x
            # for the two roundings of the sum
            bound = 2.0 ** -7 * np.abs(want) + SPEC_TOL * np.max(np.abs(blk["out"]))
            assert np.all(np.abs(got - want) <= bound), (step, l)
            xo = oracle.residual_bf16(xo, oracle.moe_layer(ols[l], oracle.rmsnorm_bf16(xo), logits=lg)["out"])
        err = rel_err(oracle.bf16_to_f32(to_bits(x)), oracle.bf16_to_f32(xo))
        print(f"  stacked token {step}: rel err {err:.2e}", flush=True)
        assert err <= SPEC_TOL, (step, err)
    del layers
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,T,layer_bits", [("stack48_h2048_e128_k8_mixed", 1, 6), ("stack48_h2048_e128_k8_mixed", 5, 8),
                                              ("moe_h2048_e256_k8_s1_b4", 8, None)])
def test_decode_block(bq, name, T, layer_bits):
    """moe_decode_block (RMSNorm inside the router launch, in place) against
    moe_rmsnorm + moe_decode_forward(residual = out = x): bit for bit
    without shared experts; with one (run as whole rows in the gate/up launch
    instead of K slices) within the decode bound; and the block output
    against the oracle."""
    w = synth.get_workload(name)
    layer = gpu_layer(w, bits=layer_bits)
    wr = bf16_tensor(synth.router_weight_bf16(w))
    bias = synth.router_bias(w)
    bt = None if bias is None else torch.from_numpy(bias).cuda()
    ws = layer.workspace(T)
    x0 = synth.activations_bf16(w, T, batch=21)
    xa = bf16_tensor(x0)
    _, la, ia, wa = bq.moe_decode_block(layer, xa, wr, bt, ws)
    xb = bf16_tensor(x0)
    n = bq.moe_rmsnorm(xb)
    _, lb, ib, wb = bq.moe_decode_forward(layer, n, wr, bt, ws, residual=xb, out=xb)
    torch.cuda.synchronize()
    assert torch.equal(la, lb) and torch.equal(ia, ib) and torch.equal(wa, wb)
    ga = oracle.bf16_to_f32(to_bits(xa)).astype(np.float64)
    gb = oracle.bf16_to_f32(to_bits(xb)).astype(np.float64)
    ol = oracle_layer(w, bits=layer_bits)
    blk = oracle.moe_layer(ol, to_bits(n), logits=lb.cpu().numpy())
    scale = np.max(np.abs(blk["out"]))
    if w.S == 0:
        assert np.array_equal(to_bits(xa), to_bits(xb))
    else:
        assert np.all(np.abs(ga - gb) <= 2.0 ** -7 * np.abs(gb) + DECODE_TOL * scale)
    want = oracle.bf16_to_f32(oracle.residual_bf16(x0, blk["out"])).astype(np.float64)
    assert np.all(np.abs(ga - want) <= 2.0 ** -7 * np.abs(want) + SPEC_TOL * scale)
    del layer
    torch.cuda.empty_cache()


def test_stack_megakernel(bq):
    """The one-launch stacked decode (moe_stack_decode) over the stacked
    workload's first five blocks (6-, 4-, 4-, 4- and 8-bit), three tokens.
    Block by block: the megakernel's x after l blocks against block l run by
    the step-by-step path (moe_rmsnorm + moe_decode_forward) on the
    megakernel's x after l - 1 blocks and against the oracle on the same
    input; end to end against the oracle's chain."""
    _LAYERS.clear()
    torch.cuda.empty_cache()
    w = synth.get_workload("stack48_h2048_e128_k8_mixed")
    bits = synth.layer_bits(w)[:5]
    layers = [gpu_layer(w, layer=l, bits=b) for l, b in enumerate(bits)]
    wrs = [bf16_tensor(synth.router_weight_bf16(w, layer=l)) for l in range(len(bits))]
    ols = [oracle_layer(w, layer=l, bits=b) for l, b in enumerate(bits)]
    sd = bq.StackDecoder(layers, wrs)
    ws = layers[0].workspace(1)
    for step in range(3):
        x0 = synth.activations_bf16(w, 1, batch=10 + step)
        prev = x0.copy()
        xo = x0.copy()
        for l in range(1, len(bits) + 1):
            print(f"  stack megakernel token {step} blocks {l}", flush=True)
            xm = bf16_tensor(x0).reshape(-1)
            sd.run(xm, nlayers=l)
            xr = bf16_tensor(prev)
            n = bq.moe_rmsnorm(xr)
            _, logits, idx, _ = bq.moe_decode_forward(layers[l - 1], n, wrs[l - 1], None, ws, residual=xr, out=xr)
            torch.cuda.synchronize()
            got = oracle.bf16_to_f32(to_bits(xm)).astype(np.float64)
            step_path = oracle.bf16_to_f32(to_bits(xr)).reshape(-1).astype(np.float64)
            blk = oracle.moe_layer(ols[l - 1], to_bits(n), logits=logits.cpu().numpy())
            want = oracle.bf16_to_f32(oracle.residual_bf16(prev, blk["out"])).reshape(-1).astype(np.float64)
            scale = np.max(np.abs(blk["out"]))
            assert np.all(np.abs(got - want) <= 2.0 ** -7 * np.abs(want) + SPEC_TOL * scale), (step, l)
            assert np.all(np.abs(got - step_path) <= 2.0 ** -7 * np.abs(step_path) + DECODE_TOL * scale), (step, l)
            prev = to_bits(xm).reshape(1, -1)
            xo = oracle.residual_bf16(xo, oracle.moe_layer(ols[l - 1], oracle.rmsnorm_bf16(xo), wrs_np(w, l - 1))["out"])
        err = rel_err(oracle.bf16_to_f32(prev), oracle.bf16_to_f32(xo))
        print(f"  stack megakernel token {step}: end-to-end rel err {err:.2e}", flush=True)
        assert err <= SPEC_TOL, (step, err)
    # no blocks: nothing runs, x is left as it was
    x0 = synth.activations_bf16(w, 1, batch=30)
    xz = bf16_tensor(x0).reshape(-1)
    sd.run(xz, nlayers=0)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(xz), x0.reshape(-1))
    with pytest.raises(ValueError):
        sd.run(xz, nlayers=len(bits) + 1)
    assert sd.read_status() == 0     # no barrier gave up, the table matched
    del sd, layers
    torch.cuda.empty_cache()


def wrs_np(w, l):
    return synth.router_weight_bf16(w, layer=l)


@pytest.mark.parametrize("case", ["lanes", "slots", "nan_inf"])
def test_decode_select_ties_bitexact(bq, case):
    """The decode selection (both moe_route_permute_decode and the copy inside
    moe_decode_forward's gate/up kernel) on logits full of exact ties, -inf
    and NaN: ids equal the oracle's stable descending sort bit for bit.
    Ties come from repeated router rows (identical rows give identical
    logits), NaN and -inf from the bias."""
    w, layer, _ = layer_for(bq, "moe_h2048_e256_k8_s1_b4")
    base = synth.router_weight_bf16(w)[:16]
    e = np.arange(w.E)
    bias = np.zeros(w.E, np.float32)
    T = 8
    x = synth.activations_bf16(w, T, batch=13)
    if case == "lanes":        # equal values 16 experts apart (different lanes)
        wr = base[e % 16]
    elif case == "slots":      # equal values in 4 neighbouring experts, repeated every 64
        wr = base[(e // 4) % 16]
    else:                      # zero tokens: the bias alone; six numbers (ties, -inf), then NaN in index order
        wr = base[e % 16]
        x = np.zeros_like(x)
        bias[:] = np.nan
        bias[[10, 40, 77, 130, 200, 255]] = [1.0, -np.inf, 1.0, 0.0, -np.inf, 2.0]
    ml = bq.MoELayer(layer.q, bf16_tensor(np.ascontiguousarray(wr)), torch.from_numpy(bias).cuda(), T_max=T)
    xt = bf16_tensor(x)
    for fused_layer in (True, False):
        r = ml.forward(xt, fused_layer=fused_layer, fused_route=True)
        torch.cuda.synchronize()
        L = r["logits"].cpu().numpy()
        assert np.array_equal(r["idx"].cpu().numpy(), oracle.select_topk(L, w.k)), (case, fused_layer)


@pytest.mark.parametrize("T", [1, 100, 512])
def test_prefill_layer_small(bq, T):
    print(f"prefill 128-expert 6-bit zipf T={T}", flush=True)
    check_layer(bq, "moe_h2048_e128_k8_b6_zipf", T, prefill=True)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("T", [70, 300])
def test_prefill_layer_4_8_bit(bq, bits, T):
    print(f"prefill 128-expert {bits}-bit T={T}", flush=True)
    check_layer(bq, "moe_h2048_e128_k8_b4", T, prefill=True, bits=bits, batch=bits)


@pytest.mark.parametrize("T", [2048, 4096])
def test_prefill_layer_sampled(bq, T):
    print(f"prefill 128-expert 6-bit zipf T={T} (sampled)", flush=True)
    check_layer(bq, "moe_h2048_e128_k8_b6_zipf", T, prefill=True, sample=48)


@pytest.mark.parametrize("T", [130, 600])
def test_prefill_shared_expert(bq, T):
    """Prefill with a shared expert (256 routed + 1 shared, 4-bit): the
    shared expert takes every token (tiles of 128 plus a ragged one), the
    routed ones few each."""
    print(f"prefill 256-expert + shared T={T}", flush=True)
    check_layer(bq, "moe_h2048_e256_k8_s1_b4", T, prefill=True, batch=7)


def test_prefill_wide_sampled(bq):
    print("prefill 512-expert hot T=8192 (sampled)", flush=True)
    check_layer(bq, "moe_h4096_e512_k10_b4_hot", 8192, prefill=True, sample=24)


@pytest.mark.parametrize("name,T", [("moe_h2048_e256_k8_s1_b4", 64), ("moe_h2048_e128_k8_b4", 33)])
def test_decode_prefill_agree(bq, name, T):
    """Cross-check (not a pin): both paths on the same batch."""
    w, layer, _ = layer_for(bq, name)
    x = bf16_tensor(synth.activations_bf16(w, T, batch=3))
    a = oracle.bf16_to_f32(to_bits(layer.forward(x, prefill=False)["out"]))
    b = oracle.bf16_to_f32(to_bits(layer.forward(x, prefill=True)["out"]))
    assert rel_err(b, a) <= SPEC_TOL


@pytest.mark.parametrize("prefill,T", [(False, 16), (True, 700)])
def test_deterministic(bq, prefill, T):
    w, layer, _ = layer_for(bq, "moe_h2048_e128_k8_b4")
    x = bf16_tensor(synth.activations_bf16(w, T, batch=9))
    a = layer.forward(x, prefill=prefill, fused_layer=False)
    b = layer.forward(x, prefill=prefill, fused_layer=False)
    for key in ("out", "idx", "sorted", "y"):
        assert torch.equal(a[key].view(torch.uint8) if a[key].dtype == torch.bfloat16 else a[key],
                           b[key].view(torch.uint8) if b[key].dtype == torch.bfloat16 else b[key]), key


def test_empty_batch(bq):
    w, layer, _ = layer_for(bq, "moe_h2048_e128_k8_b4")
    x = torch.empty((0, w.H), dtype=torch.bfloat16, device="cuda")
    for prefill in (False, True):
        r = layer.forward(x, prefill=prefill)
        assert r["out"].shape == (0, w.H)
