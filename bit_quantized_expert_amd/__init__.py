"""Python binding of libmoeq: the forward pass of a group-quantised MoE FFN
layer on MI355X (gfx950).

Argument marshalling only.  Every step of the layer runs in the HIP kernels
of ``libmoeq.so`` (built by ``python bit_quantized_expert_amd/build.py``);
PyTorch supplies device memory and the current stream.  Importing this
package without the built library raises -- there is no fallback.

Functions carry the names of the C entry points (see ``include/moeq.h``):
``moe_quantize``, ``moe_quantize_hqq``, ``moe_kv_encode``, ``moe_kv_decode``, ``moe_unpack``, ``moe_route_topk``, ``moe_permute``,
``moe_route_permute_decode``, ``moe_qgemv_decode``, ``moe_qgemm_prefill``,
``moe_combine``, ``moe_decode_forward``, ``moe_decode_block``, ``moe_rmsnorm``,
``moe_workspace_bytes``, ``moe_read_status``, ``moe_pack``, ``moe_qweight_load``
(plus ``StackDecoder`` for the stacked-decode calls and ``quantize_layer``,
which quantises a whole layer on the device from fp32 host arrays).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoeq.so")

MOEQ_Y_F32, MOEQ_Y_BF16 = 0, 1
GROUP = 64

_ERRORS = {-1: "invalid argument", -2: "unsupported", -3: "misaligned", -4: "workspace", -5: "HIP error"}


class MoeqError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libmoeq error {code} ({_ERRORS.get(code, '?')}): {msg}")
        self.code = code


class _QWeight(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("sz", ctypes.c_void_p), ("bits", ctypes.c_int)]


class _LayerDesc(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int), ("I", ctypes.c_int), ("E", ctypes.c_int), ("S", ctypes.c_int),
                ("k", ctypes.c_int), ("gate", _QWeight), ("up", _QWeight), ("down", _QWeight)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoeq.so (after torch, so both share one HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python bit_quantized_expert_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, L64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_long, ctypes.c_size_t
        sig = {
            "moe_workspace_bytes": (SZ, [P, I]),
            "moe_workspace_h": (I, [P, I, P]),
            "moe_last_error": (ctypes.c_char_p, []),
            "moe_quantize": (I, [P, L64, I, I, P, P, P]),
            "moe_quantize_hqq": (I, [P, L64, I, I, ctypes.c_float, ctypes.c_float, ctypes.c_float, I, P, P, P]),
            "moe_unpack": (I, [P, L64, I, I, P, P]),
            "moe_kv_encode": (I, [P, L64, I, I, P, P, P]),
            "moe_stack_table_bytes": (SZ, [I]),
            "moe_stack_workspace_bytes": (SZ, [P]),
            "moe_stack_table_write": (I, [P, P, I, P, SZ]),
            "moe_stack_decode": (I, [P, P, SZ, I, ctypes.c_float, P, P, SZ, P]),
            "moe_stack_read_status": (I, [P, SZ, P, P, P]),
            "moe_kv_decode": (I, [P, P, L64, I, I, P, P]),
            "moe_route_topk": (I, [P, P, P, I, I, I, I, P, P, P, P, SZ, P]),
            "moe_permute": (I, [P, I, I, I, I, P, P, P, P, P, P, SZ, P]),
            "moe_route_permute_decode": (I, [P, P, P, I, I, I, I, I, P, P, P, P, P, P, P, P, P, SZ, P]),
            "moe_qgemv_decode": (I, [P, P, I, P, P, P, P, P, SZ, P]),
            "moe_decode_forward": (I, [P, P, P, P, I, P, P, P, P, P, P, SZ, P]),
            "moe_decode_block": (I, [P, P, P, P, I, ctypes.c_float, P, P, P, P, SZ, P]),
            "moe_decode_forward_noalloc": (I, [P, P, P, P, I, P, P, P, P, P, P]),
            "moe_decode_forward_noalloc_max_scratch": (SZ, []),
            "moe_qgemm_prefill": (I, [P, P, I, P, P, P, P, P, SZ, P]),
            "moe_combine": (I, [P, I, P, P, I, I, I, I, P, P]),
            "moe_rmsnorm": (I, [P, P, I, I, ctypes.c_float, P, P]),
            "moe_read_status": (I, [P, SZ, P, P]),
            "moe_pack": (I, [P, L64, I, I, P]),
            "moe_qweight_load": (I, [P, P, P, L64, I, I, P, P, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


lib()   # fail at import time if the library is missing


def _check(rc):
    if rc != 0:
        raise MoeqError(rc, lib().moe_last_error().decode())


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t, dtype=None, name="tensor"):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


# --------------------------------------------------------------------------
# quantised weights
# --------------------------------------------------------------------------
@dataclass
class QWeight:
    """One projection of all experts: q [n_mats, N, K*bits/8] uint8 and
    sz [n_mats, N, K/64] int32 (fp16 scale | fp16 zero << 16)."""
    q: torch.Tensor
    sz: torch.Tensor
    bits: int

    def desc(self):
        return _QWeight(self.q.data_ptr(), self.sz.data_ptr(), self.bits)


def moe_quantize(w: torch.Tensor, bits: int, out: Optional[QWeight] = None, stream=None) -> QWeight:
    """Quantise fp32 weights [..., N, K] (device) along K in groups of 64."""
    _dev(w, torch.float32, "w")
    K = w.shape[-1]
    rows = w.numel() // K
    if out is None:
        q = torch.empty(w.shape[:-1] + (K * bits // 8,), dtype=torch.uint8, device=w.device)
        sz = torch.empty(w.shape[:-1] + (K // GROUP,), dtype=torch.int32, device=w.device)
        out = QWeight(q, sz, bits)
    _check(lib().moe_quantize(_p(w), rows, K, bits, _p(out.q), _p(out.sz), _stream(stream)))
    return out


def moe_pack(codes, bits: int):
    """Host codes [N, K] (uint8 numpy array, each < 2^bits) -> plain packed
    rows [N, K*bits/8] (uint8 numpy array), by the library's host routine."""
    import numpy as np
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    N, K = c.shape
    out = np.empty((N, K * bits // 8), np.uint8)
    _check(lib().moe_pack(c.ctypes.data_as(ctypes.c_void_p), N, K, bits, out.ctypes.data_as(ctypes.c_void_p)))
    return out


def moe_qweight_load(packed: torch.Tensor, scale: torch.Tensor, zero: torch.Tensor, K: int, bits: int,
                     out: Optional[QWeight] = None, stream=None) -> QWeight:
    """Plain packed codes [..., N, K*bits/8] (device uint8) with fp16 scale and
    zero [..., N, K/64] (device) -> the kernels' tiled QWeight."""
    _dev(packed, torch.uint8, "packed")
    _dev(scale, torch.float16, "scale")
    _dev(zero, torch.float16, "zero")
    rows = packed.numel() // (K * bits // 8)
    if scale.numel() != rows * (K // GROUP) or zero.numel() != scale.numel():
        raise ValueError("scale and zero must hold one value per row and group of 64")
    if out is None:
        q = torch.empty_like(packed)
        sz = torch.empty(scale.shape, dtype=torch.int32, device=packed.device)
        out = QWeight(q, sz, bits)
    _check(lib().moe_qweight_load(_p(packed), _p(scale), _p(zero), rows, K, bits, _p(out.q), _p(out.sz),
                                  _stream(stream)))
    return out


def bf16_from_bits(bits_u16, device="cuda") -> torch.Tensor:
    """bf16 tensor on the device from a numpy array of bf16 bit patterns."""
    import numpy as np
    a = np.ascontiguousarray(bits_u16, dtype=np.uint16).view(np.int16)
    return torch.from_numpy(a).to(device).view(torch.bfloat16)


def moe_quantize_hqq(w: torch.Tensor, bits: int, lp: float = 0.7, beta: float = 10.0, kappa: float = 1.01,
                     iters: int = 20, out: Optional[QWeight] = None, stream=None) -> QWeight:
    """moe_quantize with HQQ's zero-point refinement of every group."""
    _dev(w, torch.float32, "w")
    K = w.shape[-1]
    rows = w.numel() // K
    if out is None:
        q = torch.empty(w.shape[:-1] + (K * bits // 8,), dtype=torch.uint8, device=w.device)
        sz = torch.empty(w.shape[:-1] + (K // GROUP,), dtype=torch.int32, device=w.device)
        out = QWeight(q, sz, bits)
    _check(lib().moe_quantize_hqq(_p(w), rows, K, bits, lp, beta, kappa, iters, _p(out.q), _p(out.sz),
                                  _stream(stream)))
    return out


def moe_kv_encode(x: torch.Tensor, bits: int, q: Optional[torch.Tensor] = None, sz: Optional[torch.Tensor] = None,
                  stream=None):
    """bf16 cache rows [..., D] -> (packed codes [..., D*bits/8] uint8,
    scale/zero words [..., D/64] int32)."""
    _dev(x, torch.bfloat16, "x")
    D = x.shape[-1]
    rows = x.numel() // D
    if q is None:
        q = torch.empty(x.shape[:-1] + (D * bits // 8,), dtype=torch.uint8, device=x.device)
    if sz is None:
        sz = torch.empty(x.shape[:-1] + (D // GROUP,), dtype=torch.int32, device=x.device)
    _check(lib().moe_kv_encode(_p(x), rows, D, bits, _p(q), _p(sz), _stream(stream)))
    return q, sz


def moe_kv_decode(q: torch.Tensor, sz: torch.Tensor, D: int, bits: int, out: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    _dev(q, torch.uint8, "q")
    rows = q.numel() // (D * bits // 8)
    if out is None:
        out = torch.empty(q.shape[:-1] + (D,), dtype=torch.bfloat16, device=q.device)
    _check(lib().moe_kv_decode(_p(q), _p(sz), rows, D, bits, _p(out), _stream(stream)))
    return out


class StackDecoder:
    """Stacked decode of a batch-1 token through blocks of MoE layers in one
    launch (moe_stack_decode): the layers' device table is written once
    here; ``run(x)`` updates the residual stream x (bf16 [H]) in place."""

    def __init__(self, layers, w_routers, device="cuda"):
        n = len(layers)
        self.layers, self.w_routers = list(layers), list(w_routers)   # keep the weights alive
        descs = (_LayerDesc * n)(*[l.desc() for l in layers])
        wrs = (ctypes.c_void_p * n)(*[w.data_ptr() for w in w_routers])
        self.table = torch.empty(lib().moe_stack_table_bytes(n), dtype=torch.uint8, device=device)
        _check(lib().moe_stack_table_write(descs, wrs, n, _p(self.table), self.table.numel()))
        self.n = n
        self.dims = layers[0].desc()
        nbytes = lib().moe_stack_workspace_bytes(ctypes.byref(self.dims))
        if nbytes == 0:
            raise MoeqError(-2, lib().moe_last_error().decode())
        self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=device)

    def run(self, x: torch.Tensor, eps: float = 1e-6, nlayers: Optional[int] = None, stream=None) -> torch.Tensor:
        _dev(x, torch.bfloat16, "x")
        n = self.n if nlayers is None else nlayers
        if not 0 <= n <= self.n:
            raise ValueError(f"nlayers={n}: the table holds {self.n} layers")
        _check(lib().moe_stack_decode(ctypes.byref(self.dims), _p(self.table), self.table.numel(), n, eps, _p(x),
                                      _p(self.ws), self.ws.numel(), _stream(stream)))
        return x

    def read_status(self, stream=None) -> int:
        """Synchronise and return the workspace's error word (0 = none since
        the last read; bit 1: a wait gave up; bit 2: table mismatch) and
        clear it."""
        v = ctypes.c_int(0)
        _check(lib().moe_stack_read_status(_p(self.ws), self.ws.numel(), ctypes.byref(self.dims), ctypes.byref(v),
                                           _stream(stream)))
        return v.value


def moe_unpack(q: torch.Tensor, K: int, bits: int, stream=None) -> torch.Tensor:
    _dev(q, torch.uint8, "q")
    rows = q.numel() // (K * bits // 8)
    codes = torch.empty(q.shape[:-1] + (K,), dtype=torch.uint8, device=q.device)
    _check(lib().moe_unpack(_p(q), rows, K, bits, _p(codes), _stream(stream)))
    return codes


@dataclass
class QuantLayer:
    """Quantised expert weights of one MoE layer resident in HBM."""
    H: int
    I: int
    E: int
    S: int
    k: int
    gate: QWeight
    up: QWeight
    down: QWeight

    def desc(self) -> _LayerDesc:
        return _LayerDesc(self.H, self.I, self.E, self.S, self.k, self.gate.desc(), self.up.desc(),
                          self.down.desc())

    def workspace_bytes(self, T_max: int) -> int:
        return moe_workspace_bytes(self, T_max)

    def workspace(self, T_max: int, device="cuda") -> torch.Tensor:
        # zero-filled: the library's control words start (and stay) at zero
        return torch.zeros(max(256, self.workspace_bytes(T_max)), dtype=torch.uint8, device=device)


PROJECTIONS = ("gate", "up", "down")


def quantize_layer(H: int, I: int, E: int, S: int, k: int, bits, draw, device="cuda", chunk: int = 64,
                   stream=None) -> QuantLayer:
    """Quantise a layer's expert weights on the device (moe_quantize), from
    fp32 host arrays drawn ``chunk`` experts at a time: ``draw(proj, experts)``
    returns [len(experts), N, K] float32 for proj in "gate", "up" (N = I,
    K = H) and "down" (N = H, K = I).  ``bits``: one width, or a dict per
    projection."""
    n = E + S
    projs = {}
    for name in PROJECTIONS:
        b = bits[name] if isinstance(bits, dict) else bits
        N, K = (I, H) if name != "down" else (H, I)
        q = torch.empty((n, N, K * b // 8), dtype=torch.uint8, device=device)
        sz = torch.empty((n, N, K // GROUP), dtype=torch.int32, device=device)
        for e0 in range(0, n, chunk):
            es = list(range(e0, min(n, e0 + chunk)))
            wd = torch.from_numpy(draw(name, es)).to(device)
            moe_quantize(wd, b, out=QWeight(q[e0:e0 + len(es)], sz[e0:e0 + len(es)], b), stream=stream)
            del wd
        projs[name] = QWeight(q, sz, b)
    torch.cuda.synchronize()
    return QuantLayer(H, I, E, S, k, projs["gate"], projs["up"], projs["down"])


def workspace_h(layer: QuantLayer, ws: torch.Tensor, T: int, T_max: int) -> torch.Tensor:
    """The intermediate h (bf16 [T*(k+S), I]) the last expert call left in
    workspace ws (sized for T_max tokens), as a view."""
    off = ctypes.c_size_t(0)
    d = layer.desc()
    _check(lib().moe_workspace_h(ctypes.byref(d), T_max, ctypes.byref(off)))
    A = T * (layer.k + layer.S)
    return ws[off.value:off.value + A * layer.I * 2].view(torch.bfloat16).view(A, layer.I)


def moe_workspace_bytes(layer: QuantLayer, T_max: int) -> int:
    d = layer.desc()
    n = lib().moe_workspace_bytes(ctypes.byref(d), T_max)
    if n == 0:
        raise MoeqError(-1, lib().moe_last_error().decode())
    return n


# --------------------------------------------------------------------------
# the five steps
# --------------------------------------------------------------------------
def moe_route_topk(x: Optional[torch.Tensor], w_router: Optional[torch.Tensor], bias: Optional[torch.Tensor],
                   E: int, k: int, logits: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                   stream=None):
    """Router logits (or given fp32 logits when w_router is None), top-k ids
    and renormalised weights.  Returns (logits [T,E] f32, idx [T,k] i32,
    w [T,k] f32)."""
    if w_router is not None:
        _dev(x, torch.bfloat16, "x")
        _dev(w_router, torch.bfloat16, "w_router")
        T, H = x.shape
        if logits is None:
            logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    else:
        _dev(logits, torch.float32, "logits")
        T, H = logits.shape[0], 0
    if bias is not None:
        _dev(bias, torch.float32, "bias")
    dev = logits.device
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _check(lib().moe_route_topk(_p(x) if w_router is not None else None, _p(w_router), _p(bias), T, H, E, k,
                                _p(logits), _p(idx), _p(w), _p(ws), 0 if ws is None else ws.numel(),
                                _stream(stream)))
    return logits, idx, w


def permute_ws_bytes(A: int, n_experts: int) -> int:
    nblk = (A + 1023) // 1024
    return 256 + ((nblk * n_experts * 4 + 255) // 256) * 256


def moe_permute(idx: torch.Tensor, E: int, S: int, ws: Optional[torch.Tensor] = None, stream=None):
    """Group assignments by expert.  Returns (counts, offsets, sorted, inverse,
    active) int32 device tensors."""
    _dev(idx, torch.int32, "topk_idx")
    T, k = idx.shape
    A = T * (k + S)
    dev = idx.device
    counts = torch.empty(E + S, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + S + 1, dtype=torch.int32, device=dev)
    sorted_a = torch.empty(max(A, 1), dtype=torch.int32, device=dev)
    inverse = torch.empty(max(A, 1), dtype=torch.int32, device=dev)
    active = torch.empty(E + S + 1, dtype=torch.int32, device=dev)
    if ws is None:
        ws = torch.zeros(permute_ws_bytes(A, E + S), dtype=torch.uint8, device=dev)
    _check(lib().moe_permute(_p(idx), T, k, E, S, _p(counts), _p(offsets), _p(sorted_a), _p(inverse), _p(active),
                             _p(ws), ws.numel(), _stream(stream)))
    return counts, offsets, sorted_a[:A], inverse[:A], active


def fused_route_ok(T: int, H: int, E: int, k: int, S: int) -> bool:
    return T * (k + S) <= 1024 and E + S <= 1024 and k <= 64 and H in (512, 1024, 2048, 4096)


def moe_route_permute_decode(x: torch.Tensor, w_router: torch.Tensor, bias: Optional[torch.Tensor], E: int,
                             k: int, S: int, ws: torch.Tensor, stream=None):
    """moe_route_topk + moe_permute in two short launches (decode batches).  Returns
    (logits, idx, w, counts, offsets, sorted, inverse, active)."""
    _dev(x, torch.bfloat16, "x")
    _dev(w_router, torch.bfloat16, "w_router")
    T, H = x.shape
    dev = x.device
    A = T * (k + S)
    logits = torch.empty((T, E), dtype=torch.float32, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    counts = torch.empty(E + S, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + S + 1, dtype=torch.int32, device=dev)
    sorted_a = torch.empty(max(A, 1), dtype=torch.int32, device=dev)
    inverse = torch.empty(max(A, 1), dtype=torch.int32, device=dev)
    active = torch.empty(E + S + 1, dtype=torch.int32, device=dev)
    _check(lib().moe_route_permute_decode(_p(x), _p(w_router), _p(bias), T, H, E, k, S, _p(logits), _p(idx),
                                          _p(w), _p(counts), _p(offsets), _p(sorted_a), _p(inverse), _p(active),
                                          _p(ws), ws.numel(), _stream(stream)))
    return logits, idx, w, counts, offsets, sorted_a[:A], inverse[:A], active


def moe_qgemv_decode(layer: QuantLayer, x: torch.Tensor, offsets, sorted_a, active, ws: torch.Tensor,
                     y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    _dev(x, torch.bfloat16, "x")
    T = x.shape[0]
    A = T * (layer.k + layer.S)
    if y is None:
        y = torch.empty((A, layer.H), dtype=torch.float32, device=x.device)
    d = layer.desc()
    _check(lib().moe_qgemv_decode(ctypes.byref(d), _p(x), T, _p(offsets), _p(sorted_a), _p(active), _p(y),
                                  _p(ws), ws.numel(), _stream(stream)))
    return y


def decode_forward_ok(layer: QuantLayer, T: int) -> bool:
    """Whether moe_decode_forward takes this layer and batch (its documented limits)."""
    return (0 < T <= 64 and layer.E <= 1024 and layer.k + layer.S <= 16
            and layer.H in (512, 1024, 2048, 4096) and layer.gate.bits == layer.up.bits
            and (layer.I in (256, 512, 768) or (layer.I == 1024 and layer.down.bits == 4)))


def moe_decode_forward(layer: QuantLayer, x: torch.Tensor, w_router: torch.Tensor, bias: Optional[torch.Tensor],
                       ws: torch.Tensor, residual: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                       stream=None):
    """The whole decode layer in three launches.  Returns (out, logits, idx, w)."""
    _dev(x, torch.bfloat16, "x")
    _dev(w_router, torch.bfloat16, "w_router")
    T = x.shape[0]
    dev = x.device
    logits = torch.empty((T, layer.E), dtype=torch.float32, device=dev)
    idx = torch.empty((T, layer.k), dtype=torch.int32, device=dev)
    w = torch.empty((T, layer.k), dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty((T, layer.H), dtype=torch.bfloat16, device=dev)
    d = layer.desc()
    _check(lib().moe_decode_forward(ctypes.byref(d), _p(x), _p(w_router), _p(bias), T, _p(residual), _p(logits),
                                    _p(idx), _p(w), _p(out), _p(ws), ws.numel(), _stream(stream)))
    return out, logits, idx, w


def moe_decode_forward_noalloc(layer: QuantLayer, x: torch.Tensor, w_router: torch.Tensor,
                               bias: Optional[torch.Tensor], residual: Optional[torch.Tensor] = None,
                               out: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
                               idx: Optional[torch.Tensor] = None, w: Optional[torch.Tensor] = None, stream=None):
    """moe_decode_forward on the library's static scratch (no workspace);
    output tensors are allocated here unless given.  Returns (out, logits,
    idx, w)."""
    _dev(x, torch.bfloat16, "x")
    _dev(w_router, torch.bfloat16, "w_router")
    T = x.shape[0]
    dev = x.device
    if logits is None:
        logits = torch.empty((T, layer.E), dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty((T, layer.k), dtype=torch.int32, device=dev)
    if w is None:
        w = torch.empty((T, layer.k), dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty((T, layer.H), dtype=torch.bfloat16, device=dev)
    d = layer.desc()
    _check(lib().moe_decode_forward_noalloc(ctypes.byref(d), _p(x), _p(w_router), _p(bias), T, _p(residual),
                                            _p(logits), _p(idx), _p(w), _p(out), _stream(stream)))
    return out, logits, idx, w


def moe_decode_block(layer: QuantLayer, x: torch.Tensor, w_router: torch.Tensor, bias: Optional[torch.Tensor],
                     ws: torch.Tensor, eps: float = 1e-6, stream=None):
    """x <- x + moe(RMSNorm(x)) in place (three launches).  Returns (x, logits, idx, w)."""
    _dev(x, torch.bfloat16, "x")
    _dev(w_router, torch.bfloat16, "w_router")
    T = x.shape[0]
    dev = x.device
    logits = torch.empty((T, layer.E), dtype=torch.float32, device=dev)
    idx = torch.empty((T, layer.k), dtype=torch.int32, device=dev)
    w = torch.empty((T, layer.k), dtype=torch.float32, device=dev)
    d = layer.desc()
    _check(lib().moe_decode_block(ctypes.byref(d), _p(x), _p(w_router), _p(bias), T, eps, _p(logits), _p(idx), _p(w),
                                  _p(ws), ws.numel(), _stream(stream)))
    return x, logits, idx, w


def moe_qgemm_prefill(layer: QuantLayer, x: torch.Tensor, counts, offsets, sorted_a, ws: torch.Tensor,
                      y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    _dev(x, torch.bfloat16, "x")
    T = x.shape[0]
    A = T * (layer.k + layer.S)
    if y is None:
        y = torch.empty((A, layer.H), dtype=torch.bfloat16, device=x.device)
    d = layer.desc()
    _check(lib().moe_qgemm_prefill(ctypes.byref(d), _p(x), T, _p(counts), _p(offsets), _p(sorted_a), _p(y),
                                   _p(ws), ws.numel(), _stream(stream)))
    return y


def moe_combine(y: torch.Tensor, topk_w: torch.Tensor, k: int, S: int, residual: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    _dev(y, None, "y")
    dt = {torch.float32: MOEQ_Y_F32, torch.bfloat16: MOEQ_Y_BF16}[y.dtype]
    T = topk_w.shape[0]
    H = y.shape[-1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
    _check(lib().moe_combine(_p(y), dt, _p(topk_w), _p(residual), T, k, S, H, _p(out), _stream(stream)))
    return out


def moe_rmsnorm(x: torch.Tensor, gamma: Optional[torch.Tensor] = None, eps: float = 1e-6,
                out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    _dev(x, torch.bfloat16, "x")
    T, H = x.shape
    if out is None:
        out = torch.empty_like(x)
    _check(lib().moe_rmsnorm(_p(x), _p(gamma), T, H, eps, _p(out), _stream(stream)))
    return out


def moe_read_status(ws: torch.Tensor, stream=None) -> int:
    n = ctypes.c_int(0)
    _check(lib().moe_read_status(_p(ws), ws.numel(), ctypes.byref(n), _stream(stream)))
    return n.value


# --------------------------------------------------------------------------
# the whole layer
# --------------------------------------------------------------------------
DECODE_MAX_T = 64


class MoELayer:
    """A quantised MoE FFN layer with its router, run by the five calls.

    ``forward(x)`` picks the decode path (grouped GEMV) for T <= 64 tokens
    and the prefill path (grouped GEMM) above -- separate code paths for the
    two phases (Krasis update, "Overview")."""

    def __init__(self, qlayer: QuantLayer, w_router: torch.Tensor, bias: Optional[torch.Tensor] = None,
                 T_max: int = 1):
        self.q = qlayer
        self.w_router = w_router
        self.bias = bias
        self.T_max = 0
        self.ws = None
        self.reserve(T_max)

    def reserve(self, T_max: int):
        if T_max > self.T_max:
            self.ws = self.q.workspace(T_max, device=self.w_router.device)
            self.T_max = T_max

    def forward(self, x: torch.Tensor, residual: Optional[torch.Tensor] = None, stream=None, prefill=None,
                fused_route=None, fused_layer=None):
        """Decode batches (T <= 64) go through moe_decode_forward when it takes
        the layer (fused_layer=False: the five calls instead); the result then
        has no permutation arrays or expert outputs (None)."""
        T = x.shape[0]
        self.reserve(T)
        q = self.q
        use_prefill = T > DECODE_MAX_T if prefill is None else prefill
        if fused_layer is None:
            fused_layer = not use_prefill and decode_forward_ok(q, T)
        if fused_layer:
            out, logits, idx, w = moe_decode_forward(q, x, self.w_router, self.bias, self.ws, residual=residual,
                                                     stream=stream)
            return dict(out=out, logits=logits, idx=idx, w=w, counts=None, offsets=None, sorted=None,
                        inverse=None, active=None, y=None)
        if fused_route is None:
            fused_route = not use_prefill and T > 0 and fused_route_ok(T, q.H, q.E, q.k, q.S)
        if fused_route:
            logits, idx, w, counts, offsets, sorted_a, inverse, active = moe_route_permute_decode(
                x, self.w_router, self.bias, q.E, q.k, q.S, self.ws, stream=stream)
        else:
            logits, idx, w = moe_route_topk(x, self.w_router, self.bias, q.E, q.k, ws=self.ws, stream=stream)
            counts, offsets, sorted_a, inverse, active = moe_permute(idx, q.E, q.S, ws=self.ws, stream=stream)
        if use_prefill:
            y = moe_qgemm_prefill(q, x, counts, offsets, sorted_a, self.ws, stream=stream)
        else:
            y = moe_qgemv_decode(q, x, offsets, sorted_a, active, self.ws, stream=stream)
        out = moe_combine(y, w, q.k, q.S, residual=residual, stream=stream)
        return dict(out=out, logits=logits, idx=idx, w=w, counts=counts, offsets=offsets, sorted=sorted_a,
                    inverse=inverse, active=active, y=y)
