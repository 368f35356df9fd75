"""GPU parity of the whole MoE layer (route -> permute -> decode or prefill
expert FFN -> combine) against the oracle, through the C ABI.

The oracle is routed from the GPU's fp32 logits (its selection on given
logits is checked bit for bit elsewhere), and the GPU logits themselves are
checked against the oracle's.  Every check holds the layer output to
max|gpu - oracle| / (max|oracle| + 1e-6) <= 2e-2 against the fp64 oracle,
and, element by element, the intermediate h, the expert outputs y and the
layer output to the bounds tests/tolerance.py derives from the kernels'
arithmetic against the oracle's rounding variant of the same path (bf16 h,
and bf16 weights at prefill): h bit for bit wherever its bf16 rounding
cannot differ.  Full-size prefill chunks are checked on every token."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import bf16_tensor, gpu_layer, oracle_layer, rel_err, to_bits
from tests import tolerance as tol
from tests.reference import LayerReference, check_bounded

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

SPEC_TOL = 2e-2


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


def gpu_h(bq, layer, r, T, fused, a_sel):
    """The GPU's h rows of assignments a_sel, from the workspace: assignment
    order after moe_decode_forward, expert-sorted order otherwise (located
    by the GPU's own inverse permutation)."""
    h = bq.workspace_h(layer.q, layer.ws, T, layer.T_max)
    hb = oracle.bf16_to_f32(to_bits(h)).astype(np.float64)
    pos = a_sel if fused else r["inverse"].cpu().numpy()[a_sel]
    return hb[pos]


def check_routing(w, x, r, rows):
    logits = r["logits"].cpu().numpy()
    wr = synth.router_weight_bf16(w)
    ref_logits = oracle.router_logits(x[rows], wr, synth.router_bias(w))
    assert np.max(np.abs(logits[rows] - ref_logits)) <= 1e-5 * np.max(np.abs(ref_logits))
    return logits[rows]


def check_against(ref, w, r, rows, T, bq, layer, fused, prefill):
    """The GPU's routing, h, y and output against a LayerReference of the
    same rows; returns (spec error, largest used fraction of the bounds)."""
    assert np.array_equal(r["idx"].cpu().numpy()[rows], ref.idx)
    wt = r["w"].cpu().numpy()[rows]
    assert np.max(np.abs(wt - ref.wt) / ref.wt) <= 1e-5
    kS = w.k + w.S
    a_sel = (rows[:, None] * kS + np.arange(kS)[None, :]).reshape(-1)
    used = {}
    used["h"] = check_bounded("h", gpu_h(bq, layer, r, T, fused, a_sel), ref.hv, ref.dhv, exact_where=ref.dhv == 0)
    if not fused:
        y = r["y"]
        y = (oracle.bf16_to_f32(to_bits(y)) if y.dtype == torch.bfloat16 else y.cpu().numpy())[a_sel]
        used["y"] = check_bounded("y", y, ref.yv, ref.dyv)
        assert rel_err(y, ref.y) <= SPEC_TOL
    out = oracle.bf16_to_f32(to_bits(r["out"]))[rows]
    used["out"] = check_bounded("out", out, ref.outv, ref.doutv)
    err = rel_err(out, ref.out)
    assert err <= SPEC_TOL, err
    at_risk = float(np.mean(ref.dhv > 0))
    print(f"  spec err {err:.2e}; bounds used: " + ", ".join(f"{k} {v:.2f}" for k, v in used.items())
          + f"; h at risk of a rounding flip {at_risk:.3f}", flush=True)
    return err, used


def check_layer(bq, name, T, prefill, sample=None, bits=None, batch=0, fused=False):
    """fused: the decode layer through moe_decode_forward (no y to check)."""
    w, layer, _ = layer_for(bq, name, bits)
    x = synth.activations_bf16(w, T, batch=batch)
    r = layer.forward(bf16_tensor(x), prefill=prefill, fused_layer=fused)
    torch.cuda.synchronize()
    rows = np.arange(T) if sample is None else np.unique(np.linspace(0, T - 1, sample).astype(int))
    logits = check_routing(w, x, r, rows)
    ref = LayerReference(w, x[rows], logits, "prefill" if prefill else "decode", bits=bits or w.bits)
    return check_against(ref, w, r, rows, T, bq, layer, fused, prefill)


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
        rows = np.arange(T)
        logits = check_routing(w, x, r, rows)
        ref = LayerReference(w, x, logits, "decode")
        check_against(ref, w, r, rows, T, bq, ml, True, False)
    del ml, q
    torch.cuda.empty_cache()


STACK_TOKENS = 16
_STACK = {}


def stack_layers(bq):
    """All 48 blocks of the stacked workload on the GPU (kept for the
    stacked tests)."""
    if not _STACK:
        _LAYERS.clear()
        torch.cuda.empty_cache()
        w = synth.get_workload("stack48_h2048_e128_k8_mixed")
        bits = synth.layer_bits(w)
        layers = [gpu_layer(w, layer=l, bits=b) for l, b in enumerate(bits)]
        wrs = [bf16_tensor(synth.router_weight_bf16(w, layer=l)) for l in range(len(bits))]
        _STACK.update(w=w, bits=bits, layers=layers, wrs=wrs)
    return _STACK["w"], _STACK["bits"], _STACK["layers"], _STACK["wrs"]


def check_block(w, l, bits, x_in, x_out, logits=None, h=None):
    """Block l (x <- x + moe(RMSNorm(x))) on the GPU's own inputs x_in
    (bf16 bits [n, H]) against the oracle, batched over the n tokens: the
    outputs x_out within the derived bound and the spec bar, the GPU's h
    (assignment order, if given) bit for bit where its rounding cannot
    differ.  Routing: the GPU's logits if given, else the oracle's own
    logits, leaving out tokens whose k-th and (k+1)-th logit are within 1e-4
    of each other (their selection may legitimately differ); returns how
    many were left out."""
    wr = synth.router_weight_bf16(w, layer=l)
    n_or = oracle.rmsnorm_bf16(x_in)
    keep = np.arange(x_in.shape[0])
    if logits is None:
        logits = oracle.router_logits(n_or, wr)
        srt = -np.sort(-logits, axis=1)
        margin = srt[:, w.k - 1] - srt[:, w.k]
        keep = np.nonzero(margin > 1e-4 * np.abs(srt[:, 0]))[0]
    else:
        # the GPU's normalised row may differ from the oracle's by one bf16
        # spacing where a rounding boundary lies within the norm's own bound
        # (tolerance.rmsnorm_flip); each such element moves logit e by up to
        # |Wr[e, i]| times that spacing, on top of the fp32 dot's rounding
        flip = tol.rmsnorm_flip(oracle.bf16_to_f32(x_in).astype(np.float64), 1e-6)
        wr_abs = np.abs(oracle.bf16_to_f32(wr).astype(np.float64))
        bound = flip @ wr_abs.T + 1e-4 * np.max(np.abs(logits))
        assert np.all(np.abs(logits - oracle.router_logits(n_or, wr)) <= bound)
    ref = LayerReference(w, x_in[keep], logits[keep], "decode", layer=l, bits=bits, norm_eps=1e-6)
    got = oracle.bf16_to_f32(x_out[keep]).astype(np.float64)
    check_bounded(f"block {l} x", got, ref.outv, ref.doutv)
    moe = ref.out - oracle.bf16_to_f32(x_in[keep])
    assert np.all(np.abs(got - ref.out) <= 2.0 ** -8 * np.abs(ref.out) + SPEC_TOL * np.max(np.abs(moe))), l
    if h is not None:
        check_bounded(f"block {l} h", h[keep].reshape(-1, w.I), ref.hv, ref.dhv, exact_where=ref.dhv == 0)
    return x_in.shape[0] - keep.size


def test_stacked_blocks(bq):
    """moe_decode_block over all 48 blocks of the stacked workload (4-, 6-
    and 8-bit layers), 16 batch-1 tokens each pushed through every block in
    turn.  Teacher-forced: block l of the oracle, batched over the tokens,
    takes the GPU's input to block l and is routed on the GPU's logits; the
    block's output, and its h read from the workspace, are held to the
    derived bounds.  The 48 blocks' outputs after the last block are also
    compared with the oracle's own chain (reported)."""
    w, bits, layers, wrs = stack_layers(bq)
    L, H, n = len(bits), w.H, STACK_TOKENS
    xs = np.zeros((L + 1, n, H), np.uint16)
    lg = torch.empty((L, n, w.E), dtype=torch.float32, device="cuda")
    hs = torch.empty((L, n, w.k, w.I), dtype=torch.bfloat16, device="cuda")
    ws = layers[0].workspace(1)
    for t in range(n):
        x0 = synth.activations_bf16(w, 1, batch=100 + t)
        xs[0, t] = x0[0]
        x = bf16_tensor(x0)
        for l in range(L):
            _, logits, _, _ = bq.moe_decode_block(layers[l], x, wrs[l], None, ws)
            lg[l, t] = logits[0]
            hs[l, t] = bq.workspace_h(layers[l], ws, 1, 1).view(w.k, w.I)
            xs[l + 1, t] = to_bits(x)[0]
    torch.cuda.synchronize()
    lgn = lg.cpu().numpy()
    hn = oracle.bf16_to_f32(to_bits(hs)).astype(np.float64)
    for l in range(L):
        if l % 8 == 0:
            print(f"  stacked blocks: block {l} of {L}", flush=True)
        check_block(w, l, bits[l], xs[l], xs[l + 1], logits=lgn[l], h=hn[l])


def test_decode_block(bq):
    """moe_decode_block (RMSNorm inside the router launch, in place) equals
    moe_rmsnorm + moe_decode_forward(residual = out = x) bit for bit without
    shared experts; with one (run as whole rows in the gate/up launch instead
    of K slices) both are held to the derived bounds."""
    for name, T, lbits in (("stack48_h2048_e128_k8_mixed", 1, 6), ("stack48_h2048_e128_k8_mixed", 5, 8),
                           ("moe_h2048_e256_k8_s1_b4", 8, None)):
        w = synth.get_workload(name)
        layer = gpu_layer(w, bits=lbits)
        wr = bf16_tensor(synth.router_weight_bf16(w))
        ws = layer.workspace(T)
        x0 = synth.activations_bf16(w, T, batch=21)
        xa = bf16_tensor(x0)
        _, la, ia, wa = bq.moe_decode_block(layer, xa, wr, None, ws)
        xb = bf16_tensor(x0)
        nb = bq.moe_rmsnorm(xb)
        _, lb, ib, wb = bq.moe_decode_forward(layer, nb, wr, None, ws, residual=xb, out=xb)
        torch.cuda.synchronize()
        assert torch.equal(la, lb) and torch.equal(ia, ib) and torch.equal(wa, wb)
        if w.S == 0:
            assert np.array_equal(to_bits(xa), to_bits(xb))
        lw = w if lbits is None else w
        for xo in (xa, xb):
            check_block(lw, 0, lbits or w.bits, x0, to_bits(xo), logits=la.cpu().numpy())
        del layer
        torch.cuda.empty_cache()


def test_stack_megakernel(bq):
    """The one-launch stacked decode (moe_stack_decode) over all 48 blocks,
    16 tokens.  Each block runs alone (a one-block table) on the token's
    state after the previous block, teacher-forced against the oracle
    (routed on its own logits; near-tie tokens left out and counted); the
    48 one-block launches in a row equal one launch of all 48 blocks bit for
    bit (the kernel adds its K slices in a fixed order).  The workspace's
    error word stays zero throughout."""
    w, bits, layers, wrs = stack_layers(bq)
    L, H, n = len(bits), w.H, STACK_TOKENS
    one = [bq.StackDecoder([layers[l]], [wrs[l]]) for l in range(L)]
    whole = bq.StackDecoder(layers, wrs)
    xs = np.zeros((L + 1, n, H), np.uint16)
    for t in range(n):
        x0 = synth.activations_bf16(w, 1, batch=300 + t)
        xs[0, t] = x0[0]
        x = bf16_tensor(x0).reshape(-1)
        for l in range(L):
            one[l].run(x)
            xs[l + 1, t] = to_bits(x)
        xw = bf16_tensor(x0).reshape(-1)
        whole.run(xw)
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(xw), xs[L, t]), t
    assert whole.read_status() == 0 and all(d.read_status() == 0 for d in one)
    skipped = 0
    for l in range(L):
        if l % 8 == 0:
            print(f"  stack megakernel: block {l} of {L}", flush=True)
        skipped += check_block(w, l, bits[l], xs[l], xs[l + 1])
    print(f"  stack megakernel: {skipped} of {L * n} block inputs left out as near ties", flush=True)
    assert skipped <= L * n // 50
    # no blocks: nothing runs, x is left as it was; more blocks than the table holds: refused
    x0 = synth.activations_bf16(w, 1, batch=30)
    xz = bf16_tensor(x0).reshape(-1)
    whole.run(xz, nlayers=0)
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(xz), x0.reshape(-1))
    with pytest.raises(ValueError):
        whole.run(xz, nlayers=L + 1)
    del one, whole


def test_stack_table_mismatch(bq):
    """A table whose header holds fewer layers than the call asks for: every
    workgroup leaves before touching a layer, x is left as it was, and the
    workspace's error word reads 2 (table mismatch) once, then 0.  A call
    with a matching table afterwards runs and reports nothing."""
    import ctypes
    w, bits, layers, wrs = stack_layers(bq)
    L = bq.lib()
    sd = bq.StackDecoder(layers[:2], wrs[:2])
    big = torch.zeros(L.moe_stack_table_bytes(4), dtype=torch.uint8, device="cuda")
    descs = (bq._LayerDesc * 2)(*[l.desc() for l in layers[:2]])
    ptrs = (ctypes.c_void_p * 2)(*[t.data_ptr() for t in wrs[:2]])
    assert L.moe_stack_table_write(descs, ptrs, 2, bq._p(big), big.numel()) == 0
    x0 = synth.activations_bf16(w, 1, batch=31)
    x = bf16_tensor(x0).reshape(-1)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = L.moe_stack_decode(ctypes.byref(sd.dims), bq._p(big), big.numel(), 3, ctypes.c_float(1e-6), bq._p(x),
                            bq._p(sd.ws), sd.ws.numel(), stream)
    assert rc == 0
    torch.cuda.synchronize()
    assert np.array_equal(to_bits(x), x0.reshape(-1))
    assert sd.read_status() == 2
    assert sd.read_status() == 0
    sd.run(x)
    torch.cuda.synchronize()
    assert sd.read_status() == 0
    assert not np.array_equal(to_bits(x), x0.reshape(-1))
    del sd, big


def test_stack_generic_shape(bq):
    """moe_stack_decode at a shape that has no compile-time instantiation of
    the kernel (the 512-expert layer: H 4096, I 768, k 10, E 512; two blocks
    with their own weights, routed without the workload's router bias), so
    the path with run-time dimensions: 4 tokens, each block teacher-forced
    against the oracle on its own logits, one-block launches equal to one
    launch of both bit for bit, error word zero."""
    _STACK.clear()
    _LAYERS.clear()
    torch.cuda.empty_cache()
    w = synth.get_workload("moe_h4096_e512_k10_b4_hot")
    L, n = 2, 4
    layers = [gpu_layer(w, layer=l) for l in range(L)]
    wrs = [bf16_tensor(synth.router_weight_bf16(w, layer=l)) for l in range(L)]
    one = [bq.StackDecoder([layers[l]], [wrs[l]]) for l in range(L)]
    whole = bq.StackDecoder(layers, wrs)
    xs = np.zeros((L + 1, n, w.H), np.uint16)
    for t in range(n):
        x0 = synth.activations_bf16(w, 1, batch=500 + t)
        xs[0, t] = x0[0]
        x = bf16_tensor(x0).reshape(-1)
        for l in range(L):
            one[l].run(x)
            xs[l + 1, t] = to_bits(x)
        xw = bf16_tensor(x0).reshape(-1)
        whole.run(xw)
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(xw), xs[L, t]), t
    assert whole.read_status() == 0 and all(d.read_status() == 0 for d in one)
    skipped = sum(check_block(w, l, w.bits, xs[l], xs[l + 1]) for l in range(L))
    print(f"  generic stack: {skipped} of {L * n} block inputs left out as near ties", flush=True)
    assert skipped <= 1
    del one, whole, layers, wrs
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
def test_prefill_layer_full(bq, T):
    """Prompt chunks of 2048 and 4096 tokens on the 128-expert 6-bit layer
    with Zipf router offsets, every token."""
    print(f"prefill 128-expert 6-bit zipf T={T} (every token)", flush=True)
    check_layer(bq, "moe_h2048_e128_k8_b6_zipf", T, prefill=True)


@pytest.mark.parametrize("T", [130, 600])
def test_prefill_shared_expert(bq, T):
    """Prefill with a shared expert (256 routed + 1 shared, 4-bit): the
    shared expert takes every token (tiles of 128 plus a ragged one), the
    routed ones few each."""
    print(f"prefill 256-expert + shared T={T}", flush=True)
    check_layer(bq, "moe_h2048_e256_k8_s1_b4", T, prefill=True, batch=7)


@pytest.mark.parametrize("T", [512, 2048, 4096])
def test_prefill_shared_6bit_full(bq, T):
    """The prefill chunks on the 256-expert + shared layer at 6 bits with
    Zipf offsets (the prompt workload read on the decode layer's shapes),
    every token."""
    print(f"prefill 256-expert + shared 6-bit zipf T={T} (every token)", flush=True)
    check_layer(bq, "moe_h2048_e256_k8_s1_b6_zipf", T, prefill=True, batch=1)


def test_prefill_wide_full(bq):
    """The 512-expert layer (10 % hot experts) at an 8192-token chunk, every
    token: 51 hot experts with ~1600 tokens each and ~320 cold ones with one
    or two."""
    print("prefill 512-expert hot T=8192 (every token)", flush=True)
    check_layer(bq, "moe_h4096_e512_k10_b4_hot", 8192, prefill=True)


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
