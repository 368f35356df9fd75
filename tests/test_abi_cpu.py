"""The C-ABI library loads on a machine without a GPU, exports every entry
point include/moeq.h declares, and rejects bad arguments on the host before
anything reaches the GPU.  No compute call is made here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moeq.h")
LIB = os.path.join(ROOT, "bit_quantized_expert_amd", "libmoeq.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmoeq.so not built")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def bq():
    import bit_quantized_expert_amd as m
    return m


def test_header_declares_the_five_steps():
    names = declared()
    for n in ("moe_route_topk", "moe_permute", "moe_qgemv_decode", "moe_qgemm_prefill", "moe_combine"):
        assert n in names


def test_every_declared_symbol_is_exported(bq):
    lib = ctypes.CDLL(LIB)
    missing = [n for n in declared() if not hasattr(lib, n)]
    assert not missing, missing


def _err(lib):
    return lib.moe_last_error().decode()


def test_host_validation(bq):
    L = bq.lib()
    P = ctypes.c_void_p
    ok = P(4096)            # any aligned non-null value: never dereferenced on error paths
    mis = P(4096 + 4)
    # moe_quantize
    assert L.moe_quantize(None, 4, 64, 4, ok, ok, None) == -1
    assert L.moe_quantize(ok, 4, 64, 5, ok, ok, None) == -2 and "bits" in _err(L)
    assert L.moe_quantize(ok, 4, 96, 4, ok, ok, None) == -2
    assert L.moe_quantize(ok, 4, 64, 4, ok, ok, None) == -2 and "multiple of 64" in _err(L)   # rows % 64
    assert L.moe_quantize(mis, 64, 64, 4, ok, ok, None) == -3
    # decode block: its own checks first
    assert L.moe_decode_block(ok, None, ok, None, 1, ctypes.c_float(1e-6), ok, ok, ok, ok, 0, None) == -1
    assert L.moe_decode_block(ok, ok, ok, None, 1, ctypes.c_float(-1.0), ok, ok, ok, ok, 0, None) == -1
    # stacked decode: argument checks before any device query or launch
    assert L.moe_stack_table_bytes(0) == 0 and L.moe_stack_table_bytes(3) == 64 + 192
    assert L.moe_stack_table_write(None, None, 2, ok, 1 << 20) == -1
    assert L.moe_stack_decode(None, ok, 1 << 20, 1, ctypes.c_float(1e-6), ok, ok, 0, None) == -1
    assert L.moe_stack_read_status(None, 0, None, None, None) == -1
    # KV codec
    assert L.moe_kv_encode(None, 4, 64, 4, ok, ok, None) == -1
    assert L.moe_kv_encode(ok, 4, 64, 5, ok, ok, None) == -2 and "bits" in _err(L)
    assert L.moe_kv_encode(ok, 4, 96, 4, ok, ok, None) == -2 and "multiple of 64" in _err(L)
    assert L.moe_kv_encode(mis, 4, 64, 4, ok, ok, None) == -3
    assert L.moe_kv_encode(ok, 0, 64, 4, ok, ok, None) == 0      # nothing to do, no launch
    assert L.moe_kv_decode(ok, None, 4, 64, 4, ok, None) == -1
    assert L.moe_kv_decode(ok, ok, -1, 64, 4, ok, None) == -1
    assert L.moe_kv_decode(ok, ok, 4, 64, 7, ok, None) == -2
    assert L.moe_kv_decode(ok, ok, 4, 64, 4, mis, None) == -3
    # moe_quantize_hqq: its own parameters, then moe_quantize's checks
    assert L.moe_quantize_hqq(ok, 64, 64, 4, 0.0, 10.0, 1.01, 20, ok, ok, None) == -1 and "lp" in _err(L)
    assert L.moe_quantize_hqq(ok, 64, 64, 4, 1.5, 10.0, 1.01, 20, ok, ok, None) == -1
    assert L.moe_quantize_hqq(ok, 64, 64, 4, 0.7, 0.0, 1.01, 20, ok, ok, None) == -1
    assert L.moe_quantize_hqq(ok, 64, 64, 4, 0.7, 10.0, 0.5, 20, ok, ok, None) == -1
    assert L.moe_quantize_hqq(ok, 64, 64, 4, 0.7, 10.0, 1.01, -1, ok, ok, None) == -1
    assert L.moe_quantize_hqq(ok, 64, 64, 4, 0.7, 10.0, 1.01, 1001, ok, ok, None) == -1
    assert L.moe_quantize_hqq(ok, 64, 64, 5, 0.7, 10.0, 1.01, 20, ok, ok, None) == -2
    assert L.moe_quantize_hqq(mis, 64, 64, 4, 0.7, 10.0, 1.01, 20, ok, ok, None) == -3
    assert L.moe_unpack(ok, 4, 64, 7, ok, None) == -2
    # routing
    assert L.moe_route_topk(ok, ok, None, 4, 64, 8, 9, ok, ok, ok, None, 0, None) == -1    # k > E
    assert L.moe_route_topk(ok, ok, None, 4, 96, 8, 2, ok, ok, ok, None, 0, None) == -2    # H % 64
    assert L.moe_route_topk(None, None, ok, 4, 64, 8, 2, ok, ok, ok, None, 0, None) == -1  # bias w/o router
    assert L.moe_route_topk(mis, ok, None, 4, 64, 8, 2, ok, ok, ok, None, 0, None) == -3
    # permute: workspace too small
    assert L.moe_permute(ok, 4, 2, 8, 0, ok, ok, ok, ok, ok, ok, 16, None) == -4
    assert L.moe_permute(ok, 4, 2, 8, 0, ok, ok, ok, ok, ok, None, 1 << 20, None) == -4
    # combine
    assert L.moe_combine(ok, 0, ok, None, 2, 2, 0, 12, ok, None) == -2
    assert L.moe_combine(ok, 3, ok, None, 2, 2, 0, 16, ok, None) == -1
    assert L.moe_rmsnorm(ok, None, 2, 16, ctypes.c_float(1e-6), ok, None) == -1   # alias
    # layer validation through the decode / prefill entries
    bad = bq._LayerDesc(2048, 512, 8, 0, 2, bq._QWeight(4096, 4096, 4), bq._QWeight(4096, 4096, 4),
                        bq._QWeight(4096, 4096, 5))
    assert L.moe_workspace_bytes(ctypes.byref(bad), 4) == 0
    assert L.moe_qgemv_decode(ctypes.byref(bad), ok, 1, ok, ok, ok, ok, ok, 1 << 30, None) == -2
    mixed = bq._LayerDesc(2048, 512, 8, 0, 2, bq._QWeight(4096, 4096, 4), bq._QWeight(4096, 4096, 6),
                          bq._QWeight(4096, 4096, 4))
    assert L.moe_qgemm_prefill(ctypes.byref(mixed), ok, 1, ok, ok, ok, ok, ok, 1 << 30, None) == -2
    good = bq._LayerDesc(2048, 512, 8, 0, 2, bq._QWeight(4096, 4096, 4), bq._QWeight(4096, 4096, 4),
                         bq._QWeight(4096, 4096, 4))
    need = L.moe_workspace_bytes(ctypes.byref(good), 16)
    assert need > 16 * 2 * 512 * 4
    assert L.moe_qgemv_decode(ctypes.byref(good), ok, 16, ok, ok, ok, ok, ok, need - 1, None) == -4
    assert "workspace" in _err(L)
    unaligned = bq._LayerDesc(2048, 512, 8, 0, 2, bq._QWeight(4096 + 8, 4096, 4), bq._QWeight(4096, 4096, 4),
                              bq._QWeight(4096, 4096, 4))
    assert L.moe_qgemv_decode(ctypes.byref(unaligned), ok, 1, ok, ok, ok, ok, ok, 1 << 30, None) == -3


def test_workspace_grows_with_batch(bq):
    L = bq.lib()
    d = bq._LayerDesc(4096, 768, 512, 0, 10, bq._QWeight(4096, 4096, 4), bq._QWeight(4096, 4096, 4),
                      bq._QWeight(4096, 4096, 4))
    a, b = L.moe_workspace_bytes(ctypes.byref(d), 1), L.moe_workspace_bytes(ctypes.byref(d), 8192)
    assert 0 < a < b
    assert b >= 8192 * 10 * 768 * 4


@pytest.mark.parametrize("bits", [4, 6, 8])
def test_pack_matches_oracle(bq, bits):
    """moe_pack (the library's host routine) writes the plain packed rows the
    oracle's pack writes, byte for byte, on random codes and on every code
    value at every position of a pack unit."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 1 << bits, size=(37, 192), dtype=np.uint8)
    assert np.array_equal(bq.moe_pack(codes, bits), oracle.pack(codes, bits))
    # each value at each of the 4 positions of a 4-code unit (covers both
    # nibbles and all four 6-bit fields)
    vals = np.arange(1 << bits, dtype=np.uint8)
    unit = np.zeros((vals.size * 4, 4), np.uint8)
    for p in range(4):
        unit[p * vals.size:(p + 1) * vals.size, p] = vals
    assert np.array_equal(bq.moe_pack(unit, bits), oracle.pack(unit, bits))


def test_pack_rejects_bad_input(bq):
    import numpy as np
    L = bq.lib()
    P = ctypes.c_void_p
    bad = np.array([[0, 16, 1, 2]], np.uint8)
    out = np.zeros(4, np.uint8)
    assert L.moe_pack(bad.ctypes.data_as(P), 1, 4, 4, out.ctypes.data_as(P)) == -1 and "exceeds" in _err(L)
    assert L.moe_pack(bad.ctypes.data_as(P), 1, 4, 5, out.ctypes.data_as(P)) == -2
    assert L.moe_pack(bad.ctypes.data_as(P), 1, 3, 8, out.ctypes.data_as(P)) == -2
    assert L.moe_pack(None, 1, 4, 8, out.ctypes.data_as(P)) == -1
    ok = P(4096)
    assert L.moe_qweight_load(ok, ok, ok, 64, 64, 5, ok, ok, None) == -2
    assert L.moe_qweight_load(ok, ok, ok, 32, 64, 4, ok, ok, None) == -2
    assert L.moe_qweight_load(ok, ok, ok, 64, 64, 4, P(4096 + 4), ok, None) == -3
    assert L.moe_qweight_load(None, ok, ok, 64, 64, 4, ok, ok, None) == -1
    assert L.moe_qweight_load(ok, ok, ok, 0, 64, 4, ok, ok, None) == 0     # nothing to do, no launch
