"""Shared helpers of the GPU tests: build a layer's inputs from the seeded
generator on both sides -- the HIP path quantises on the device, the oracle
quantises the same fp32 draws on the CPU -- and compare results."""
from __future__ import annotations

import numpy as np

import oracle
import synth

PROJ = {"gate": synth.T_GATE, "up": synth.T_UP, "down": synth.T_DOWN}


def bf16_tensor(bits_u16: np.ndarray, device="cuda"):
    import bit_quantized_expert_amd as bq
    return bq.bf16_from_bits(bits_u16, device)


def to_bits(t) -> np.ndarray:
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def synth_draw(w: synth.Workload, layer: int = 0):
    """draw(proj, experts) of the seeded fp32 expert weights, for
    bit_quantized_expert_amd.quantize_layer."""
    return lambda name, es: synth.expert_weights_f32(w, layer, PROJ[name], es)


def gpu_layer(w: synth.Workload, layer: int = 0, bits=None, device="cuda", chunk=64):
    """Quantise every expert's weights on the device (HIP path) from the
    seeded fp32 draws, streaming ``chunk`` experts at a time."""
    import bit_quantized_expert_amd as bq
    return bq.quantize_layer(w.H, w.I, w.E, w.S, w.k, bits or w.bits, synth_draw(w, layer), device=device,
                             chunk=chunk)


class LazyExperts:
    """Oracle-side experts: quantised by the oracle from the same fp32 draws,
    built on first use."""

    def __init__(self, w: synth.Workload, layer: int = 0, bits=None):
        self.w, self.layer, self.bits = w, layer, bits or w.bits
        self.cache = {}

    def __getitem__(self, e):
        if e not in self.cache:
            self.cache[e] = {name: oracle.quantize(synth.expert_weight_f32(self.w, self.layer, tid, e), self.bits)
                             for name, tid in PROJ.items()}
        return self.cache[e]


def oracle_layer(w: synth.Workload, layer: int = 0, bits=None) -> oracle.QuantLayer:
    return oracle.QuantLayer(w.H, w.I, w.E, w.k, w.S, LazyExperts(w, layer, bits))


# The device byte layout of packed codes (include/moeq.h, moe_qweight): in
# each chunk (32 codes at 4-bit, 16 at 6/8-bit) field n holds code
# FIELD_CODE[bits][n]; rows are tiled by 64, chunk-major inside a tile.
CHUNK_CODES = {4: 32, 6: 16, 8: 16}
FIELD_CODE = {4: [8 * (n >> 3) + 2 * (n & 3) + ((n >> 2) & 1) for n in range(32)],
              6: [0, 2, 12, 1, 3, 4, 6, 13, 5, 7, 8, 10, 14, 9, 11, 15],
              8: list(range(16))}


def device_packed(q: np.ndarray, bits: int) -> np.ndarray:
    """Device bytes of codes q [rows][K]: the oracle's packing of the
    field-ordered codes, re-laid out in 64-row tiles (flat uint8)."""
    rows, K = q.shape
    c = CHUNK_CODES[bits]
    cpr = K // c
    fields = np.asarray(q).reshape(rows, cpr, c)[:, :, FIELD_CODE[bits]].reshape(rows, K)
    packed = oracle.pack(fields, bits)
    nb = c * bits // 8
    return packed.reshape(rows // 64, 64, cpr, nb).transpose(0, 2, 1, 3).reshape(-1)


def device_codes(dev_bytes: np.ndarray, rows: int, K: int, bits: int) -> np.ndarray:
    """Inverse of device_packed: natural codes [rows][K] of device bytes."""
    c = CHUNK_CODES[bits]
    cpr = K // c
    nb = c * bits // 8
    rowmajor = np.asarray(dev_bytes).reshape(rows // 64, cpr, 64, nb).transpose(0, 2, 1, 3).reshape(rows, -1)
    fields = oracle.unpack(rowmajor, bits, K).reshape(rows, cpr, c)
    codes = np.empty_like(fields)
    codes[:, :, FIELD_CODE[bits]] = fields
    return codes.reshape(rows, K)


def device_sz(words: np.ndarray) -> np.ndarray:
    """Device order of scale/zero words [rows][K/64] (flat uint32)."""
    rows, gpr = words.shape
    return np.asarray(words).reshape(rows // 64, 64, gpr).transpose(0, 2, 1).reshape(-1)


def rel_err(gpu, ref) -> float:
    """max |gpu - ref| / (max |ref| + 1e-6)"""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(gpu - ref)) / (np.max(np.abs(ref)) + 1e-6)) if ref.size else 0.0
