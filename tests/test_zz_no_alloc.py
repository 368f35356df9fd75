"""moe_decode_forward_noalloc (the decode layer on the library's static
scratch, for callers that cannot allocate) against moe_decode_forward (the
same kernels on a caller's workspace), through the C ABI: outputs, logits,
routing ids and weights equal bit for bit, on two calls in a row, the second
with a smaller batch, on two layers."""
import ctypes

import numpy as np
import pytest

import synth
from tests.gpu_util import bf16_tensor, gpu_layer, to_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def bq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_expert_amd as m
    return m


def _both(bq, layer, wr, bias, x, residual=None):
    L = bq.lib()
    T = x.shape[0]
    dev = x.device
    ref = bq.moe_decode_forward(layer, x, wr, bias, layer.workspace(T, device=dev), residual=residual)
    out = torch.empty((T, layer.H), dtype=torch.bfloat16, device=dev)
    logits = torch.empty((T, layer.E), dtype=torch.float32, device=dev)
    idx = torch.empty((T, layer.k), dtype=torch.int32, device=dev)
    w = torch.empty((T, layer.k), dtype=torch.float32, device=dev)
    d = layer.desc()
    rc = L.moe_decode_forward_noalloc(ctypes.byref(d), bq._p(x), bq._p(wr), bq._p(bias), T, bq._p(residual),
                                      bq._p(logits), bq._p(idx), bq._p(w), bq._p(out),
                                      ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, L.moe_last_error().decode()
    torch.cuda.synchronize()
    return ref, (out, logits, idx, w)


@pytest.mark.parametrize("name,Ts", [("moe_h2048_e256_k8_s1_b4", (8, 3)), ("moe_h4096_e512_k10_b4_hot", (4, 1))])
def test_noalloc_matches_workspace_path(bq, name, Ts):
    w = synth.get_workload(name)
    layer = gpu_layer(w)
    wr = bf16_tensor(synth.router_weight_bf16(w))
    b = synth.router_bias(w)
    bias = None if b is None else torch.from_numpy(b).cuda()
    for call, T in enumerate(Ts):
        print(f"  noalloc {name} call {call} T={T}", flush=True)
        x = bf16_tensor(synth.activations_bf16(w, T, batch=40 + call))
        residual = bf16_tensor(synth.activations_bf16(w, T, batch=60 + call)) if call else None
        ref, got = _both(bq, layer, wr, bias, x, residual)
        for a, g in zip(ref, got):
            if a.dtype == torch.bfloat16:
                assert np.array_equal(to_bits(a), to_bits(g))
            else:
                assert torch.equal(a, g)
    del layer
    torch.cuda.empty_cache()


def test_noalloc_rejects_oversized(bq):
    """A layer and batch whose scratch exceeds the static array is refused
    before anything is enqueued."""
    L = bq.lib()
    cap = L.moe_decode_forward_noalloc_max_scratch()
    qw = bq._QWeight(4096, 4096, 4)
    d = bq._LayerDesc(4096, 1024, 1000, 1, 15, qw, qw, qw)
    assert L.moe_workspace_bytes(ctypes.byref(d), 64) > cap
    ok = ctypes.c_void_p(4096)
    assert L.moe_decode_forward_noalloc(ctypes.byref(d), ok, ok, None, 64, None, ok, ok, ok, ok, None) == -4
    assert "static scratch" in L.moe_last_error().decode()
