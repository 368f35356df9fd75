"""GPU parity of the integer and routing steps against the oracle, through
the C ABI: quantisation codes and packing (bit-exact), unpacking (bit-exact),
top-k ids on given logits (bit-exact), routing weights (<= 1e-5 relative),
router logits, permutation (bit-exact), combine and RMSNorm."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import bf16_tensor, device_codes, device_packed, device_sz, rel_err, to_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def bq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_expert_amd as m
    return m


def _sz_from_oracle(s16, z16):
    return (s16.view(np.uint16).astype(np.uint32) | (z16.view(np.uint16).astype(np.uint32) << 16))


def _weights(seed, shape):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal(shape) * 0.02).astype(np.float32)
    w2 = w.reshape(-1, 64)
    special = [lambda g: 0.37,                                   # constant group
               lambda g: np.linspace(-1, 1, 64),                 # exact end points
               lambda g: g * 1e3,                                # wide range
               lambda g: g * 1e-3,                               # narrow range: subnormal fp16 scale
               lambda g: (rng.integers(0, 16, 64) - 7) * 2.0 ** -6]   # on a power-of-two grid
    for i, f in enumerate(special[: len(w2)]):
        w2[i] = f(w2[i])
    return w


@pytest.mark.parametrize("bits", [4, 6, 8])
@pytest.mark.parametrize("shape", [(3, 64, 512), (2, 128, 192), (1, 64, 64)])
def test_quantize_bitexact(bq, bits, shape):
    w = _weights(bits * 7 + shape[1], shape)
    qw = bq.moe_quantize(torch.from_numpy(w).cuda(), bits)
    torch.cuda.synchronize()
    q, s16, z16 = oracle.quantize(w.reshape(-1, shape[-1]), bits)
    got_packed = qw.q.cpu().numpy().reshape(-1)
    assert np.array_equal(got_packed, device_packed(q, bits))
    got_sz = qw.sz.cpu().numpy().view(np.uint32).reshape(-1)
    assert np.array_equal(got_sz, device_sz(_sz_from_oracle(s16, z16)))


@pytest.mark.parametrize("bits", [4, 6, 8])
@pytest.mark.parametrize("shape", [(3, 64, 512), (2, 128, 192), (1, 64, 64)])
def test_qweight_load_bitexact(bq, bits, shape):
    """Weights quantised elsewhere enter through moe_pack + moe_qweight_load:
    the oracle's codes, packed by the library's host routine, with separate
    fp16 scale and zero arrays, land byte for byte where moe_quantize puts
    the same weights (and where the oracle's own model of the device layout
    puts them)."""
    w = _weights(bits * 11 + shape[1], shape)
    K = shape[-1]
    q, s16, z16 = oracle.quantize(w.reshape(-1, K), bits)
    packed = bq.moe_pack(q, bits)
    assert np.array_equal(packed, oracle.pack(q, bits))
    qw = bq.moe_qweight_load(torch.from_numpy(packed).cuda(), torch.from_numpy(s16).cuda(),
                             torch.from_numpy(z16).cuda(), K, bits)
    ref = bq.moe_quantize(torch.from_numpy(w).cuda(), bits)
    torch.cuda.synchronize()
    got_q = qw.q.cpu().numpy().reshape(-1)
    got_sz = qw.sz.cpu().numpy().view(np.uint32).reshape(-1)
    assert np.array_equal(got_q, ref.q.cpu().numpy().reshape(-1))
    assert np.array_equal(got_sz, ref.sz.cpu().numpy().view(np.uint32).reshape(-1))
    assert np.array_equal(got_q, device_packed(q, bits))
    assert np.array_equal(got_sz, device_sz(_sz_from_oracle(s16, z16)))
    # and the decode kernels' unpacking reads back the oracle's codes
    assert np.array_equal(bq.moe_unpack(qw.q, K, bits).cpu().numpy().reshape(-1, K), q)


def _hqq_gpu(bq, w, bits, **kw):
    qw = bq.moe_quantize_hqq(torch.from_numpy(w).cuda(), bits, **kw)
    torch.cuda.synchronize()
    return qw.q.cpu().numpy().reshape(-1), qw.sz.cpu().numpy().view(np.uint32).reshape(-1)


@pytest.mark.parametrize("bits", [4, 6, 8])
@pytest.mark.parametrize("shape", [(3, 64, 512), (1, 64, 64)])
def test_quantize_hqq_l1_bitexact(bq, bits, shape):
    """HQQ refinement with p = 1 (the soft threshold: no power function, so
    every step is an IEEE fp32 operation both sides round alike): codes and
    scale/zero words equal the oracle's bit for bit, special groups
    included."""
    w = _weights(bits * 11 + shape[1], shape)
    got_q, got_sz = _hqq_gpu(bq, w, bits, lp=1.0, beta=10.0, kappa=1.01, iters=20)
    q, s16, z16 = oracle.hqq_refine(w.reshape(-1, shape[-1]), bits, lp=1.0, beta=10.0, kappa=1.01, iters=20)
    assert np.array_equal(got_q, device_packed(q, bits))
    assert np.array_equal(got_sz, device_sz(_sz_from_oracle(s16, z16)))


@pytest.mark.parametrize("iters,beta,kappa", [(1, 10.0, 1.01), (3, 2.0, 1.5), (50, 10.0, 1.01)])
def test_quantize_hqq_l1_rounds_bitexact(bq, iters, beta, kappa):
    """Other round counts and penalty schedules, p = 1: bit-exact."""
    w = _weights(iters * 5, (2, 64, 256))
    got_q, got_sz = _hqq_gpu(bq, w, 4, lp=1.0, beta=beta, kappa=kappa, iters=iters)
    q, s16, z16 = oracle.hqq_refine(w.reshape(-1, 256), 4, lp=1.0, beta=beta, kappa=kappa, iters=iters)
    assert np.array_equal(got_q, device_packed(q, 4))
    assert np.array_equal(got_sz, device_sz(_sz_from_oracle(s16, z16)))


@pytest.mark.parametrize("bits", [4, 6, 8])
def test_quantize_hqq_no_rounds_is_minmax(bq, bits):
    w = _weights(bits * 13, (2, 64, 256))
    got_q, got_sz = _hqq_gpu(bq, w, bits, iters=0)
    qw = bq.moe_quantize(torch.from_numpy(w).cuda(), bits)
    torch.cuda.synchronize()
    assert np.array_equal(got_q, qw.q.cpu().numpy().reshape(-1))
    assert np.array_equal(got_sz, qw.sz.cpu().numpy().view(np.uint32).reshape(-1))


@pytest.mark.parametrize("bits", [4, 6, 8])
@pytest.mark.parametrize("scale", [0.02, 2.0])
def test_quantize_hqq_default_bitexact(bq, bits, scale):
    """The default solver (p = 0.7, beta 10, kappa 1.01, 20 rounds), bit for
    bit: codes and scale/zero words equal the oracle's.  Both sides form the
    residual exactly and the shrink and the means in fp64, and round a mean
    once to fp16, so the power function's last fp64 bit and the order of the
    additions cannot move a stored zero.  At weights N(0, 0.02) every
    residual is below the shrink's threshold (the rounds fit the zero by
    least squares); at N(0, 2) the shrink acts on most of them."""
    shape = (8, 128, 512)
    w = (_weights(bits * 17, shape) * np.float32(scale / 0.02)).astype(np.float32)
    N, K = shape[0] * shape[1], shape[2]
    got_q, got_sz = _hqq_gpu(bq, w, bits)
    q, s16, z16 = oracle.hqq_refine(w.reshape(N, K), bits)
    assert np.array_equal(got_q, device_packed(q, bits))
    assert np.array_equal(got_sz, device_sz(_sz_from_oracle(s16, z16)))
    # the rounds did something: zeros moved off the min-max ones
    q0, s0, z0 = oracle.quantize(w.reshape(N, K), bits)
    assert (z16 != z0).mean() > 0.2


@pytest.mark.parametrize("iters,z_final", [(4, -1.208984375), (20, -1.2373046875)])
def test_quantize_hqq_golden_group(bq, iters, z_final):
    """The hand-worked group of tests/golden/hqq_trajectory.json (s = 1,
    p = 1, beta 8, kappa 2) on the device: the stored zero after 4 rounds and
    where the refinement stops, and the codes."""
    g = np.array([1.0, 16.0] + [4.25] * 31 + [8.375] * 31, np.float32)
    w = np.tile(g, (64, 1))
    got_q, got_sz = _hqq_gpu(bq, w, 4, lp=1.0, beta=8.0, kappa=2.0, iters=iters)
    z = np.array([(int(v) >> 16) for v in got_sz], np.uint16).view(np.float16)
    assert np.all(z == np.float16(z_final)) and np.all((got_sz & 0xFFFF) == 0x3C00)
    codes = np.array([0, 15] + [3] * 31 + [7] * 31, np.uint8)
    assert np.array_equal(device_codes(got_q, 64, 64, 4), np.tile(codes, (64, 1)))


def _kv_rows(seed, R, D):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((R, D)) * 2).astype(np.float32)
    g = x.reshape(-1, 64)
    g[0] = 0.37                                          # constant group
    g[1] = np.linspace(-3, 3, 64)                        # exact end points
    g[2] *= 1e4                                          # wide range
    g[3] *= 1e-4                                         # narrow range: subnormal fp16 scale
    g[4] = (rng.integers(0, 16, 64) - 7) * 2.0 ** -5     # on a power-of-two grid
    return oracle.f32_to_bf16(x)


@pytest.mark.parametrize("bits", [4, 6, 8])
@pytest.mark.parametrize("R,D", [(5, 64), (37, 128), (64, 192)])
def test_kv_codec_bitexact(bq, bits, R, D):
    """KV-cache codec: packed codes and scale/zero words of the encoder, and
    the decoder's bf16 rows, equal the oracle's bit for bit."""
    x = _kv_rows(bits * 31 + R, R, D)
    q, sz = bq.moe_kv_encode(bf16_tensor(x), bits)
    out = bq.moe_kv_decode(q, sz, D, bits)
    torch.cuda.synchronize()
    p, s16, z16 = oracle.kv_encode(x, bits)
    assert np.array_equal(q.cpu().numpy(), p)
    assert np.array_equal(sz.cpu().numpy().view(np.uint32), _sz_from_oracle(s16, z16))
    assert np.array_equal(to_bits(out), oracle.kv_decode(p, s16, z16, bits, D))


@pytest.mark.parametrize("bits", [4, 6])
def test_kv_codec_cache_size(bq, bits):
    """At a cache's size (32768 tokens x 8 heads x 128, as bench.py --kv
    times it): sampled rows against the oracle, every row's round trip
    within half a step plus a bf16 rounding."""
    R, D = 32768 * 8, 128
    g = torch.Generator(device="cuda")
    g.manual_seed(99)
    xt = (torch.randn((R, D), generator=g, device="cuda") * 2).to(torch.bfloat16)
    q, sz = bq.moe_kv_encode(xt, bits)
    out = bq.moe_kv_decode(q, sz, D, bits)
    torch.cuda.synchronize()
    rows = np.unique(np.linspace(0, R - 1, 257).astype(int))
    x = to_bits(xt[torch.from_numpy(rows).cuda()])
    p, s16, z16 = oracle.kv_encode(x, bits)
    assert np.array_equal(q[torch.from_numpy(rows).cuda()].cpu().numpy(), p)
    assert np.array_equal(to_bits(out[torch.from_numpy(rows).cuda()]), oracle.kv_decode(p, s16, z16, bits, D))
    s = (sz & 0xFFFF).to(torch.int16).view(torch.float16).float().repeat_interleave(64, dim=1)
    err = (out.float() - xt.float()).abs()
    # half a step, widened by the fp16 rounding of s and z (each at most 2^-11 relative, times
    # 2^bits - 1 and |z| <= 2^bits - 1 steps), plus the bf16 rounding
    bound = (0.5 + (2 ** bits - 1) * 2.0 ** -10) * s + 2.0 ** -8 * out.float().abs()
    assert bool((err <= bound).all())


@pytest.mark.parametrize("bits", [4, 6, 8])
def test_unpack_bitexact(bq, bits):
    rng = np.random.default_rng(bits)
    K, rows = 2048, 64
    packed = rng.integers(0, 256, (rows, K * bits // 8), dtype=np.uint8)
    packed[0, : 256] = np.arange(256, dtype=np.uint8)
    got = bq.moe_unpack(torch.from_numpy(packed).cuda(), K, bits).cpu().numpy()
    assert np.array_equal(got, device_codes(packed.reshape(-1), rows, K, bits))


@pytest.mark.parametrize("E,k,T", [(128, 8, 16), (256, 8, 8), (512, 10, 33), (6, 3, 5), (1024, 64, 3), (8, 8, 4),
                                   (2500, 8, 7), (4096, 16, 5)])
def test_topk_on_given_logits_bitexact(bq, E, k, T):
    w = synth.Workload("t", 99, 64, 64, E, k, 0, 4, (T,))
    L = synth.direct_logits_f32(w, T)
    Lt = torch.from_numpy(L).cuda()
    _, idx, wt = bq.moe_route_topk(None, None, None, E, k, logits=Lt)
    ref = oracle.select_topk(L, k)
    assert np.array_equal(idx.cpu().numpy(), ref)
    rw = oracle.topk_weights(L, ref)
    assert np.max(np.abs(wt.cpu().numpy() - rw) / rw) <= 1e-5


def test_topk_ties_bitexact(bq):
    rng = np.random.default_rng(11)
    L = rng.integers(-3, 4, (300, 96)).astype(np.float32)
    L[:20] *= np.float32(0.0)            # rows of +-0.0 ties
    L[20, :] = 1.0                        # all equal
    L[21, :] = -np.inf                    # all -inf: index order
    L[22, ::2] = -np.inf
    Lt = torch.from_numpy(L).cuda()
    for k in (1, 5, 96):
        _, idx, _ = bq.moe_route_topk(None, None, None, 96, k, logits=Lt)
        assert np.array_equal(idx.cpu().numpy(), oracle.select_topk(L, k))


@pytest.mark.parametrize("T", [1, 16, 63, 64, 200, 4096])
@pytest.mark.parametrize("wl", ["moe_h2048_e128_k8_b4", "moe_h4096_e512_k10_b4_hot"])
def test_router_logits(bq, T, wl):
    w = synth.get_workload(wl)
    if T > 512 and w.H > 2048:
        T = 1024
    x = synth.activations_bf16(w, T, batch=5)
    wr = synth.router_weight_bf16(w)
    bias = synth.router_bias(w)
    bt = None if bias is None else torch.from_numpy(bias).cuda()
    logits, idx, wt = bq.moe_route_topk(bf16_tensor(x), bf16_tensor(wr), bt, w.E, w.k)
    ref = oracle.router_logits(x, wr, bias)
    got = logits.cpu().numpy()
    assert np.max(np.abs(got - ref)) <= 1e-5 * np.max(np.abs(ref))
    # selection on the GPU's own logits is bit-exact
    assert np.array_equal(idx.cpu().numpy(), oracle.select_topk(got, w.k))


@pytest.mark.parametrize("T,E,H", [(8192, 512, 4096), (8192, 1024, 2048), (5000, 400, 512)])
def test_router_logits_tiled(bq, T, E, H):
    """The tiled router GEMM at large batches: 128 x 64 tiles (8192 tokens x
    512 experts: 256 tiles of 128 x 128, one block a CU), 128 x 128 tiles
    (8192 x 1024: 512 of them) and ragged edges in both M and N (5000 x
    400: 40 x 7 tiles of 128 x 64), every logit against the oracle's fp64 dot products."""
    rng = np.random.default_rng(T * 7 + E)
    x = synth.f32_to_bf16_bits_input(rng.standard_normal((T, H), dtype=np.float32))
    wr = synth.f32_to_bf16_bits_input(rng.standard_normal((E, H), dtype=np.float32) * np.float32(0.02))
    logits, idx, _ = bq.moe_route_topk(bf16_tensor(x), bf16_tensor(wr), None, E, 8)
    ref = oracle.router_logits(x, wr, None)
    got = logits.cpu().numpy()
    assert np.max(np.abs(got - ref)) <= 1e-5 * np.max(np.abs(ref))
    assert np.array_equal(idx.cpu().numpy(), oracle.select_topk(got, 8))


@pytest.mark.parametrize("T,k,E,S", [(0, 8, 128, 0), (1, 8, 128, 0), (16, 8, 128, 0), (8, 8, 256, 1),
                                     (113, 8, 128, 1), (128, 8, 128, 0), (4096, 8, 128, 0), (8192, 10, 512, 0),
                                     (300, 4, 4000, 1), (2000, 2, 3, 0)])
def test_permute_bitexact(bq, T, k, E, S):
    rng = np.random.default_rng(T + E)
    if T:
        if E >= 2 * k:   # skewed: half the tokens prefer a few experts
            idx = np.stack([rng.choice(E, k, replace=False, p=None) for _ in range(T)]).astype(np.int32)
            idx[: T // 2, 0] = rng.integers(0, 3, T // 2)
            for t in range(T // 2):      # keep ids distinct within a token
                row = idx[t]
                _, first = np.unique(row, return_index=True)
                if len(first) < k:
                    free = np.setdiff1d(np.arange(E), row)
                    dup = np.setdiff1d(np.arange(k), first)
                    row[dup] = free[: len(dup)]
        else:
            idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    else:
        idx = np.zeros((0, k), np.int32)
    it = torch.from_numpy(idx).cuda() if T else torch.zeros((0, k), dtype=torch.int32, device="cuda")
    counts, offsets, srt, inv, active = bq.moe_permute(it, E, S)
    c, o, s, i = oracle.permute(idx, E, S)
    assert np.array_equal(counts.cpu().numpy(), c)
    assert np.array_equal(offsets.cpu().numpy(), o)
    assert np.array_equal(srt.cpu().numpy(), s)
    assert np.array_equal(inv.cpu().numpy(), i)
    act = active.cpu().numpy()
    nz = np.nonzero(c)[0]
    assert act[0] == len(nz) and np.array_equal(act[1:1 + len(nz)], nz)


def test_permute_counts_out_of_range_ids(bq):
    idx = np.array([[0, 1], [5, 2], [-1, 3], [2, 9]], np.int32)   # 5, -1 and 9 are outside [0, 5)
    ws = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    counts, offsets, srt, inv, active = bq.moe_permute(torch.from_numpy(idx).cuda(), 5, 0, ws=ws)
    assert bq.moe_read_status(ws) == 3
    assert counts.cpu().tolist() == [1, 1, 2, 1, 0]
    assert srt.cpu().tolist()[:5] == [0, 1, 3, 6, 5]
    assert inv.cpu().tolist() == [0, 1, -1, 2, -1, 4, 3, -1]


@pytest.mark.parametrize("T,k,S,H,dtype", [(1, 8, 0, 2048, "f32"), (8, 8, 1, 2048, "f32"), (37, 10, 0, 4096, "bf16"),
                                           (5, 3, 1, 64, "bf16")])
def test_combine(bq, T, k, S, H, dtype):
    rng = np.random.default_rng(T * H)
    y = rng.standard_normal((T * (k + S), H)).astype(np.float32)
    w = rng.random((T, k))
    w = (w / w.sum(1, keepdims=True)).astype(np.float32)
    if dtype == "bf16":
        yb = oracle.f32_to_bf16(y)
        y = oracle.bf16_to_f32(yb)
        yt = bf16_tensor(yb)
    else:
        yt = torch.from_numpy(y).cuda()
    out = bq.moe_combine(yt, torch.from_numpy(w).cuda(), k, S)
    ref = oracle.combine(y.reshape(T, k + S, H).astype(np.float64), w.astype(np.float64), S)
    got = oracle.bf16_to_f32(to_bits(out))
    assert rel_err(got, ref) <= 2.0 ** -8
    # with a residual: bf16(res + bf16(sum))
    res = oracle.f32_to_bf16(rng.standard_normal((T, H)).astype(np.float32))
    out2 = bq.moe_combine(yt, torch.from_numpy(w).cuda(), k, S, residual=bf16_tensor(res))
    ref2 = oracle.bf16_to_f32(oracle.residual_bf16(res, ref))
    got2 = oracle.bf16_to_f32(to_bits(out2))
    assert np.max(np.abs(got2 - ref2)) <= 2.0 ** -7 * np.max(np.abs(ref2))


def test_rmsnorm(bq):
    rng = np.random.default_rng(3)
    x = oracle.f32_to_bf16((rng.standard_normal((9, 2048)) * 3).astype(np.float32))
    x[0] = oracle.f32_to_bf16(np.full(2048, 0.5, np.float32))
    out = bq.moe_rmsnorm(bf16_tensor(x))
    got = to_bits(out)
    ref = oracle.rmsnorm_bf16(x)
    # fp32 arithmetic vs fp64: at most one bf16 ulp apart
    gd = oracle.bf16_to_f32(got).astype(np.float64)
    rd = oracle.bf16_to_f32(ref).astype(np.float64)
    assert np.all(np.abs(gd - rd) <= 2.0 ** -7 * np.abs(rd) + 1e-30)
    assert np.array_equal(got[0], ref[0])


@pytest.mark.parametrize("wl,T", [("moe_h2048_e128_k8_b4", 1), ("moe_h2048_e128_k8_b4", 16),
                                  ("moe_h2048_e256_k8_s1_b4", 8), ("moe_h4096_e512_k10_b4_hot", 1),
                                  ("moe_h4096_e512_k10_b4_hot", 13), ("moe_h2048_e128_k8_b6_zipf", 64)])
def test_route_permute_decode_fused(bq, wl, T):
    """The decode routing entry point (router + selection/grouping) equals the oracle's routing on the GPU's
    logits (bit for bit) and its logits match the oracle's; repeated calls on
    one workspace keep working."""
    w = synth.get_workload(wl)
    wr = bf16_tensor(synth.router_weight_bf16(w))
    bias = synth.router_bias(w)
    bt = None if bias is None else torch.from_numpy(bias).cuda()
    ws = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    for rep in range(3):
        x = synth.activations_bf16(w, T, batch=20 + rep)
        r = bq.moe_route_permute_decode(bf16_tensor(x), wr, bt, w.E, w.k, w.S, ws)
        logits = r[0].cpu().numpy()
        ref_l = oracle.router_logits(x, synth.router_weight_bf16(w), bias)
        assert np.max(np.abs(logits - ref_l)) <= 1e-5 * np.max(np.abs(ref_l))
        idx = oracle.select_topk(logits, w.k)
        assert np.array_equal(r[1].cpu().numpy(), idx)
        rw = oracle.topk_weights(logits, idx)
        assert np.max(np.abs(r[2].cpu().numpy() - rw) / rw) <= 1e-5
        c, o, s, i = oracle.permute(idx, w.E, w.S)
        for got, ref in zip(r[3:7], (c, o, s, i)):
            assert np.array_equal(got.cpu().numpy(), ref)
        act = r[7].cpu().numpy()
        nz = np.nonzero(c)[0]
        assert act[0] == len(nz) and np.array_equal(act[1:1 + len(nz)], nz)
    assert ws[0:4].cpu().numpy().view(np.int32)[0] == 0   # no bad ids


@pytest.mark.parametrize("T", [33, 65, 300])
def test_route_permute_decode_long_batch(bq, T):
    """Batches past 64 tokens take the counting branch of the grouping (the
    token masks cover 64 tokens); both branches give the oracle's permutation."""
    w = synth.Workload("route_long", 88, 512, 64, 32, 2, 1, 4, (T,))
    wr = bf16_tensor(synth.router_weight_bf16(w))
    ws = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    x = synth.activations_bf16(w, T)
    r = bq.moe_route_permute_decode(bf16_tensor(x), wr, None, w.E, w.k, w.S, ws)
    logits = r[0].cpu().numpy()
    idx = oracle.select_topk(logits, w.k)
    assert np.array_equal(r[1].cpu().numpy(), idx)
    c, o, s, i = oracle.permute(idx, w.E, w.S)
    for got, ref in zip(r[3:7], (c, o, s, i)):
        assert np.array_equal(got.cpu().numpy(), ref)
