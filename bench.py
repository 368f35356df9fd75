#!/usr/bin/env python3
"""Benchmark of the quantised MoE FFN layer's hot path on one MI355X.

A step is one pass of the whole layer -- router logits, top-k routing,
permutation, the expert FFN (decode grouped GEMV or prefill grouped GEMM)
and the weighted combine -- over one batch of synthetic tokens whose inputs
and weights are already resident in HBM.

The default line is the largest single-GPU workload: the 125B-class wide
layer (hidden 4096, 512 experts, intermediate 768, top-10, 10 % hot experts,
4-bit) at a prefill chunk of 8192 tokens, its roofline against the bf16
matrix-core peak.  The same layer at one decode token and the 256-expert +
shared decode layer at 8 tokens are measured in the same run and nested in
the line ("decode").

Cache-honest timing: successive steps use different copies of the layer's
weights (R replicas at distinct addresses, R * layer size >> the 256 MB
Infinity Cache) and different token batches, the way consecutive layers of
a model would, so weight bytes come from HBM.  The steps are captured in HIP
graphs (one graph holds one step per replica and batch, a second one the
remainder) and replayed: exactly --steps steps are timed.

Prints one JSON line (see the field list in the design notes).
    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME:T]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, GB/s
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "bit_quantized_expert_amd", "csrc")
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
RIDGE = PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)   # FLOP per byte where the two peaks meet
DEFAULT_WORKLOAD = "moe_h4096_e512_k10_b4_hot:8192"
# measured in the same run and nested in the default line
NESTED_DECODE = ("moe_h4096_e512_k10_b4_hot:1", "moe_h2048_e256_k8_s1_b4:8")
NESTED_STEPS, NESTED_WARMUP = 400, 50


def parse_workload(s):
    name, _, T = s.partition(":")
    w = synth.get_workload(name)
    return w, int(T) if T else w.tokens[-1]


def expert_bytes(w, bits):
    """Algorithmic bytes of one expert: three I x H matrices of codes plus an
    fp16 scale and zero per 64 weights."""
    return 3 * w.I * w.H * (bits / 8 + 4 / 64)


def kernel_sources_hash():
    """sha256 over every HIP source of the library: a counter reading taken
    on other sources no longer describes the kernels that run."""
    import hashlib
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h")):
            h.update(f.encode())
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload, T):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary (rocprofv3 FETCH_SIZE and WRITE_SIZE, each scaled by what the
    counter reads for a plain copy of known size), or None when there is no
    summary for this workload or the kernels changed since it was taken."""
    path = os.path.join(PROFILES, f"pmc_{workload}_T{T}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            k, sep, v = line.partition("=")
            if sep:
                kv[k.strip()] = v.strip()
    if kv.get("kernel_sources_sha256") != kernel_sources_hash():
        return None
    try:
        return round(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def copy_calibrate(mib):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}), flush=True)


def synth_draw(w, layer=0):
    """draw(proj, experts) of the seeded fp32 expert weights (quantize_layer)."""
    tid = {"gate": synth.T_GATE, "up": synth.T_UP, "down": synth.T_DOWN}
    return lambda name, es: synth.expert_weights_f32(w, layer, tid[name], es)


def synth_layer(bq, w, layer=0, bits=None, device="cuda"):
    """The workload's layer quantised on the device from its seeded draws."""
    return bq.quantize_layer(w.H, w.I, w.E, w.S, w.k, bits or w.bits, synth_draw(w, layer), device=device)


class Step:
    """Preallocated buffers and the ctypes calls of one layer step.

    Decode batches that moe_decode_forward takes run as that one call
    (router; routing + gate/up; down + combine); the others as
    route/permute, the expert FFN call and the combine."""

    def __init__(self, bq, layer, wr, bias, x, T, ws, y=None, out=None):
        import torch
        self.bq, self.L, self.T = bq, layer, T
        self.desc = layer.desc()
        dev = x.device
        E, S, k, H = layer.E, layer.S, layer.k, layer.H
        A = T * (k + S)
        self.x, self.wr, self.bias, self.ws = x, wr, bias, ws
        self.logits = torch.empty((T, E), dtype=torch.float32, device=dev)
        self.idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.counts = torch.empty(E + S, dtype=torch.int32, device=dev)
        self.offsets = torch.empty(E + S + 1, dtype=torch.int32, device=dev)
        self.sorted = torch.empty(A, dtype=torch.int32, device=dev)
        self.inverse = torch.empty(A, dtype=torch.int32, device=dev)
        self.active = torch.empty(E + S + 1, dtype=torch.int32, device=dev)
        self.prefill = T > bq.DECODE_MAX_T
        self.layer_fused = not self.prefill and bq.decode_forward_ok(layer, T)
        self.fused = not self.prefill and bq.fused_route_ok(T, H, E, k, S)
        # steps run one after another on one stream, so they may share these
        self.y = y if y is not None else torch.empty((A, H), dtype=torch.bfloat16 if self.prefill else torch.float32,
                                                     device=dev)
        self.out = out if out is not None else torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        self.residual = None

    def distinct_experts(self) -> int:
        """Experts the batch touched (routed ones from the top-k ids, plus the shared)."""
        import torch
        return int(torch.unique(self.idx).numel()) + self.L.S

    def route_permute(self, s):
        lib, p, L = self.bq.lib(), self.bq._p, self.L
        if self.fused:
            self.bq._check(lib.moe_route_permute_decode(
                p(self.x), p(self.wr), p(self.bias), self.T, L.H, L.E, L.k, L.S, p(self.logits), p(self.idx),
                p(self.w), p(self.counts), p(self.offsets), p(self.sorted), p(self.inverse), p(self.active),
                p(self.ws), self.ws.numel(), s))
            return
        self.bq._check(lib.moe_route_topk(p(self.x), p(self.wr), p(self.bias), self.T, L.H, L.E, L.k, p(self.logits),
                                          p(self.idx), p(self.w), p(self.ws), self.ws.numel(), s))
        self.bq._check(lib.moe_permute(p(self.idx), self.T, L.k, L.E, L.S, p(self.counts), p(self.offsets),
                                       p(self.sorted), p(self.inverse), p(self.active), p(self.ws), self.ws.numel(), s))

    def experts(self, s):
        lib, p = self.bq.lib(), self.bq._p
        d = ctypes.byref(self.desc)
        if self.prefill:
            self.bq._check(lib.moe_qgemm_prefill(d, p(self.x), self.T, p(self.counts), p(self.offsets),
                                                 p(self.sorted), p(self.y), p(self.ws), self.ws.numel(), s))
        else:
            self.bq._check(lib.moe_qgemv_decode(d, p(self.x), self.T, p(self.offsets), p(self.sorted),
                                                p(self.active), p(self.y), p(self.ws), self.ws.numel(), s))

    def combine(self, s):
        lib, p, L = self.bq.lib(), self.bq._p, self.L
        self.bq._check(lib.moe_combine(p(self.y), 1 if self.prefill else 0, p(self.w), p(self.residual), self.T, L.k,
                                       L.S, L.H, p(self.out), s))

    def decode_forward(self, s):
        lib, p = self.bq.lib(), self.bq._p
        self.bq._check(lib.moe_decode_forward(ctypes.byref(self.desc), p(self.x), p(self.wr), p(self.bias), self.T,
                                              p(self.residual), p(self.logits), p(self.idx), p(self.w),
                                              p(self.out), p(self.ws), self.ws.numel(), s))

    # the step split around the part whose duration the roofline uses: the
    # expert FFN call, or the whole fused decode call
    def pre(self, s):
        if not self.layer_fused:
            self.route_permute(s)

    def timed(self, s):
        if self.layer_fused:
            self.decode_forward(s)
        else:
            self.experts(s)

    def post(self, s):
        if not self.layer_fused:
            self.combine(s)

    def run(self, s):
        self.pre(s)
        self.timed(s)
        self.post(s)


class StackStep:
    """One token through every block of the stacked workload:
    n = RMSNorm(x); route n; experts(n); x = bf16(x + bf16(combine)) --
    moe_decode_block per block (three launches), or moe_rmsnorm and the
    block's Step where the fused decode does not apply."""

    def __init__(self, bq, layers, wrs, x, ws):
        import torch
        self.bq, self.layers, self.wrs, self.x, self.ws = bq, layers, wrs, x, ws
        self.n = torch.empty_like(x)
        self.steps = [Step(bq, L, wr, None, self.n, x.shape[0], ws) for L, wr in zip(layers, wrs)]
        for st in self.steps:      # every block adds into the residual stream x
            st.out = x
            st.residual = x

    def block(self, st, s):
        lib, p = self.bq.lib(), self.bq._p
        T, H = self.x.shape
        if st.layer_fused:
            self.bq._check(lib.moe_decode_block(ctypes.byref(st.desc), p(self.x), p(st.wr), None, T,
                                                ctypes.c_float(1e-6), p(st.logits), p(st.idx), p(st.w), p(st.ws),
                                                st.ws.numel(), s))
        else:
            self.bq._check(lib.moe_rmsnorm(p(self.x), None, T, H, ctypes.c_float(1e-6), p(self.n), s))
            st.run(s)

    def run(self, s):
        for st in self.steps:
            self.block(st, s)


def build_stack(bq, w, device):
    """All blocks of the stacked workload, each with its own weights and bit
    width (quantised on the device)."""
    import torch
    bits = synth.layer_bits(w)
    layers, wrs = [], []
    for l, b in enumerate(bits):
        layers.append(synth_layer(bq, w, layer=l, bits=b, device=device))
        wrs.append(bq.bf16_from_bits(synth.router_weight_bf16(w, layer=l), device=device))
    torch.cuda.synchronize()
    return layers, wrs, bits


def main_stack(a, w, bq, dev):
    """Stacked decode: 256 consecutive batch-1 tokens through all blocks,
    one HIP graph per token step, timed end to end."""
    import torch
    t0 = time.time()
    layers, wrs, bits = build_stack(bq, w, dev)
    n_tok = w.steps
    xs = torch.stack([bq.bf16_from_bits(synth.activations_bf16(w, 1, batch=b), device=dev) for b in range(n_tok)])
    x = torch.empty((1, w.H), dtype=torch.bfloat16, device=dev)
    ws = layers[0].workspace(1, device=dev)
    st = StackStep(bq, layers, wrs, x, ws)
    print(f"# setup {time.time() - t0:.1f}s: {w.name} layers={len(layers)} bits={bits}", file=sys.stderr, flush=True)
    s = torch.cuda.Stream()
    sp = ctypes.c_void_p(s.cuda_stream)
    with torch.cuda.stream(s):
        x.copy_(xs[0])
        st.run(sp)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        st.run(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()

    def tokens(n):
        with torch.cuda.stream(s):
            for i in range(n):
                x.copy_(xs[i % n_tok])
                graph.replay()

    tokens(min(a.warmup, n_tok))
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(s)
    tokens(n_tok)
    ev1.record(s)
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    per_tok = total_ms / n_tok
    # algorithmic bytes per token: routed experts (realised, per layer) + routers + x, out
    distinct = [ss.distinct_experts() for ss in st.steps]
    alg = sum(d * expert_bytes(w, b) for d, b in zip(distinct, bits)) + len(bits) * (w.E * w.H * 2 + 4 * w.H * 2)
    # the timed part of each block (the fused decode call, or the expert FFN
    # call) for one token, with events
    kev = []
    fused = all(ss.layer_fused for ss in st.steps)
    with torch.cuda.stream(s):
        x.copy_(xs[0])
        for ss in st.steps:
            if fused:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(s)
                st.block(ss, sp)
                e1.record(s)
            else:
                bq._check(bq.lib().moe_rmsnorm(bq._p(x), None, 1, w.H, ctypes.c_float(1e-6), bq._p(st.n), sp))
                ss.pre(sp)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(s)
                ss.timed(sp)
                e1.record(s)
                ss.post(sp)
            kev.append((e0, e1))
    torch.cuda.synchronize()
    kern_ms = sum(e0.elapsed_time(e1) for e0, e1 in kev)
    if fused:   # the whole block: norm, routers and x traffic included
        exp_bytes = alg
        kname = "moe_decode_block (RMSNorm + router; routing + gate/up; down + combine + residual), summed over the blocks of one token"
    else:
        exp_bytes = sum(d * expert_bytes(w, b) for d, b in zip(distinct, bits))
        kname = "moe_qgemv_decode (gate/up + down), summed over the blocks of one token"
    achieved = exp_bytes / (kern_ms * 1e-3) / 1e9
    res = {
        "metric": "MoE-layer tokens/s", "value": round(n_tok / (total_ms * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": n_tok, "warmup": a.warmup, "ms_per_step": round(per_tok, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "u4/u6/u8 codes x bf16 -> fp32",
        "data": "synthetic (seeded N(0,0.02) weights quantised on the GPU; N(0,1) bf16 states)",
        "config": {"workload": w.name, "blocks": len(bits), "bits_per_block": bits, "tokens_per_step": 1,
                   "hip_graph": True, "alg_bytes_per_token": round(alg),
                   "GBps_per_token_stream": round(alg / (per_tok * 1e-3) / 1e9, 1)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None, "kernel": kname,
                     "alg_bytes_per_token": round(exp_bytes), "kernel_us_per_token": round(kern_ms * 1e3, 3)},
    }
    # the same tokens through moe_stack_decode: one cooperative launch per
    # token for all blocks (eager launches: the copy of the token's state
    # and the launch, per token)
    sd = bq.StackDecoder(layers, wrs, device=dev)

    def mk_tokens(n):
        with torch.cuda.stream(s):
            for i in range(n):
                x.copy_(xs[i % n_tok])
                sd.run(x, stream=s)

    mk_tokens(min(a.warmup, n_tok))
    torch.cuda.synchronize()
    ev0.record(s)
    mk_tokens(n_tok)
    ev1.record(s)
    torch.cuda.synchronize()
    mk_total = ev0.elapsed_time(ev1)
    mev = []
    with torch.cuda.stream(s):
        for i in range(min(32, n_tok)):
            x.copy_(xs[i])
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            sd.run(x, stream=s)
            e1.record(s)
            mev.append((e0, e1))
    torch.cuda.synchronize()
    mk_kern = float(np.mean([e0.elapsed_time(e1) for e0, e1 in mev]))
    layer_path = {"value": res["value"], "ms_per_step": res["ms_per_step"], "roofline": res["roofline"]}
    mk = {"value": round(n_tok / (mk_total * 1e-3), 1), "ms_per_step": round(mk_total / n_tok, 6),
          "kernel_us_per_token": round(mk_kern * 1e3, 3),
          "achieved": round(alg / (mk_kern * 1e-3) / 1e9, 1)}
    if mk["value"] > layer_path["value"]:
        res["value"], res["ms_per_step"] = mk["value"], mk["ms_per_step"]
        res["config"]["path"] = "moe_stack_decode (one cooperative launch per token for all blocks)"
        res["config"]["hip_graph"] = False
        res["config"]["GBps_per_token_stream"] = round(alg / (mk["ms_per_step"] * 1e-3) / 1e9, 1)
        res["roofline"] = {"bound": "hbm", "achieved": mk["achieved"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": round(mk["achieved"] / PEAK_HBM_GBS, 4), "traffic": None,
                           "kernel": "moe_stack_decode (all blocks of one token, one launch)",
                           "alg_bytes_per_token": round(alg), "kernel_us_per_token": mk["kernel_us_per_token"]}
        res["layer_path"] = layer_path
    else:
        res["config"]["path"] = ("moe_decode_block per block (HIP graph)" if fused
                                 else "moe_rmsnorm + expert calls per block (HIP graph)")
        res["megakernel"] = mk
    del sd
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_stack(w, bits, a.cpu_budget)
    print(json.dumps(res), flush=True)


class OracleExperts:
    """The oracle's experts of one layer: quantised by the oracle from the
    seeded fp32 draws when first used (its load step, not timed)."""

    def __init__(self, w, layer=0, bits=None):
        self.w, self.layer, self.bits = w, layer, bits or w.bits
        self.cache = {}

    def load(self, experts, threads=None):
        import oracle
        from concurrent.futures import ThreadPoolExecutor
        tid = {"gate": synth.T_GATE, "up": synth.T_UP, "down": synth.T_DOWN}
        todo = [int(e) for e in experts if int(e) not in self.cache]

        def one(e):
            return e, {n: oracle.quantize(synth.expert_weight_f32(self.w, self.layer, t, e), self.bits)
                       for n, t in tid.items()}
        with ThreadPoolExecutor(threads or min(16, len(os.sched_getaffinity(0)))) as ex:
            for e, d in ex.map(one, todo):
                self.cache[e] = d

    def __getitem__(self, e):
        if e not in self.cache:
            self.load([e], threads=1)
        return self.cache[e]


def blas_threads():
    from threadpoolctl import threadpool_info
    return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] + [1])


def cpu_baseline_stack(w, bits, budget_s):
    import oracle
    n, t_total = 0, 0.0
    experts = [OracleExperts(w, layer=l, bits=b) for l, b in enumerate(bits)]
    wrs = [synth.router_weight_bf16(w, layer=l) for l in range(len(bits))]
    while t_total < budget_s and n < 8:
        x = synth.activations_bf16(w, 1, batch=2000 + n)
        for l in range(len(bits)):          # quantise the touched experts first (untimed load step)
            nrm = oracle.rmsnorm_bf16(x)
            L = oracle.router_logits(nrm, wrs[l])
            for e in oracle.select_topk(L, w.k)[0]:
                experts[l][int(e)]
            layer = oracle.QuantLayer(w.H, w.I, w.E, w.k, w.S, experts[l])
            t0 = time.perf_counter()
            out = oracle.moe_layer(layer, nrm, wrs[l])["out"]
            x = oracle.residual_bf16(x, out)
            t_total += time.perf_counter() - t0
        n += 1
    return {"value": n / t_total, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"{n} tokens through all {len(bits)} blocks ({t_total:.1f} s of oracle time; the per-block "
                      f"quantisation of the touched experts excluded)"}


def build_replicas(bq, w, R, device):
    """Quantise the layer once on the device, then copy it to R - 1 more
    places so consecutive steps never find their weights in a cache."""
    import torch
    base = synth_layer(bq, w, device=device)
    reps = [base]
    for _ in range(R - 1):
        cp = lambda qw: bq.QWeight(qw.q.clone(), qw.sz.clone(), qw.bits)
        reps.append(bq.QuantLayer(base.H, base.I, base.E, base.S, base.k, cp(base.gate), cp(base.up), cp(base.down)))
    torch.cuda.synchronize()
    return reps


def cpu_baseline(w, T, budget_s=20.0):
    """The oracle as it stands, timed on this host's cores on a bounded
    sample of the same workload: whole-layer forwards (routing, permutation,
    dequantisation of the touched experts, FFN, combine) of the workload's
    token batches -- or, for prefill chunks, of consecutive 16-token slices
    of the chunk -- until ~budget_s of timed CPU work.  Quantising the
    touched experts is the oracle's load step and is not timed."""
    import oracle
    wr = synth.router_weight_bf16(w)
    bias = synth.router_bias(w)
    experts = OracleExperts(w)
    slice_T = min(T, 16)
    n_tok, t_total, n_runs, b = 0, 0.0, 0, 0
    chunk = None
    while t_total < budget_s and n_runs < 64:
        if slice_T < T:      # slices of the first prefill chunk
            if chunk is None:
                chunk = synth.activations_bf16(w, T, batch=0)
            x = chunk[(b * slice_T) % T:(b * slice_T) % T + slice_T]
        else:
            x = synth.activations_bf16(w, T, batch=1000 + b)
        L = oracle.router_logits(x, wr, bias)
        experts.load(set(oracle.select_topk(L, w.k).reshape(-1).tolist()) | set(range(w.E, w.E + w.S)))
        layer = oracle.QuantLayer(w.H, w.I, w.E, w.k, w.S, experts)   # fresh dequant cache
        t0 = time.perf_counter()
        oracle.moe_layer(layer, x, wr, bias)
        t_total += time.perf_counter() - t0
        n_tok += x.shape[0]
        n_runs += 1
        b += 1
    what = (f"{n_runs} consecutive {slice_T}-token slices of the first {T}-token chunk" if slice_T < T
            else f"{n_runs} whole-layer forwards of {T} tokens")
    return {"value": n_tok / t_total, "unit": "tokens/s", "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"{what} ({n_tok} tokens, {t_total:.1f} s); "
                      f"dequantisation of the routed experts included, weight quantisation excluded; "
                      f"NumPy elementwise work single-threaded, BLAS threads as given in cores; "
                      f"host has {len(os.sched_getaffinity(0))} usable cores"}


def main_curve(a, w, bq, dev):
    """Decode cost against batch size: the whole layer (moe_decode_forward)
    at T = 1 .. 16 tokens per call, each timed like the default bench (HIP
    graph of steps over weight replicas and token batches), relative to
    T = 1 -- the price of verifying T - 1 speculated tokens with the target
    token in one call."""
    import torch
    layer_bytes = expert_bytes(w, w.bits) * w.n_mats
    R = a.replicas or max(2, min(16, math.ceil(2e9 / layer_bytes)))
    reps = build_replicas(bq, w, R, dev)
    wr = bq.bf16_from_bits(synth.router_weight_bf16(w))
    bias = synth.router_bias(w)
    bias_t = None if bias is None else torch.from_numpy(bias).to(dev)
    s = torch.cuda.Stream()
    curve = []
    for T in range(1, a.curve_max + 1):
        NB = a.batches
        xs = [bq.bf16_from_bits(synth.activations_bf16(w, T, batch=b)) for b in range(NB)]
        ws = [reps[0].workspace(T, device=dev) for _ in range(R)]
        G = max(R, NB)
        steps = [Step(bq, reps[i % R], wr, bias_t, xs[i % NB], T, ws[i % R]) for i in range(G)]
        with torch.cuda.stream(s):
            for st in steps:
                st.run(ctypes.c_void_p(s.cuda_stream))
        torch.cuda.synchronize()
        distinct = float(np.mean([st.distinct_experts() for st in steps]))
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=s):
            for st in steps:
                st.run(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        n = max(1, a.steps // G)
        with torch.cuda.stream(s):
            for _ in range(max(1, a.warmup // G)):
                graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        with torch.cuda.stream(s):
            for _ in range(n):
                graph.replay()
        e1.record(s)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (n * G)
        alg = distinct * expert_bytes(w, w.bits) + w.E * w.H * 2 + 2 * T * w.H * 2
        curve.append({"T": T, "us_per_step": round(us, 3), "distinct_experts": round(distinct, 2),
                      "alg_bytes": round(alg), "GBps": round(alg / (us * 1e-6) / 1e9, 1),
                      "fused_layer": bool(steps[0].layer_fused)})
        print(f"# T={T}: {us:.2f} us/step, {distinct:.1f} experts", file=sys.stderr, flush=True)
        del graph, steps, ws, xs
        torch.cuda.empty_cache()
    t1 = curve[0]["us_per_step"]
    for c in curve:
        c["rel_to_T1"] = round(c["us_per_step"] / t1, 3)
    print(json.dumps({"metric": "decode step time relative to one token", "workload": w.name,
                      "data": "synthetic", "curve": curve}), flush=True)


def main_hqq(a, w, bq, dev):
    """The quantisation step before the path: moe_quantize_hqq (min-max,
    then HQQ's zero refinement) against plain moe_quantize on one projection
    of every expert of the workload (gate: [E+S, I, H] fp32 N(0, 0.02) drawn
    on the device), and the mean absolute reconstruction error of each."""
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    wt = torch.randn((w.n_mats, w.I, w.H), generator=g, device=dev, dtype=torch.float32) * a.hqq_std
    bits = w.bits

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    def mae(qw):
        codes = bq.moe_unpack(qw.q, w.H, bits).float().reshape(w.n_mats * w.I, w.H // 64, 64)
        # device sz order -> [rows][K/64]: tiles of 64 rows are group-major
        sz = qw.sz.reshape(-1).view(torch.int32)
        rows = w.n_mats * w.I
        sz = sz.reshape(rows // 64, w.H // 64, 64).transpose(1, 2).reshape(rows, w.H // 64)
        s = (sz & 0xFFFF).to(torch.int16).view(torch.float16).float()
        z = ((sz >> 16) & 0xFFFF).to(torch.int16).view(torch.float16).float()
        d = (codes - z[..., None]) * s[..., None]
        return float((wt.reshape(rows, w.H // 64, 64) - d).abs().mean())

    out = bq.moe_quantize(wt, bits)
    ms_mm = timed(lambda: bq.moe_quantize(wt, bits, out=out), 5)
    err_mm = mae(out)
    outh = bq.moe_quantize_hqq(wt, bits)
    ms_h = timed(lambda: bq.moe_quantize_hqq(wt, bits, out=outh), 3)
    err_h = mae(outh)
    n = wt.numel()
    print(json.dumps({"metric": "HQQ-refined quantisation throughput", "value": round(n / (ms_h * 1e-3) / 1e9, 3),
                      "unit": "Gweights/s", "workload": w.name, "bits": bits, "weights": n,
                      "matrix": [w.n_mats, w.I, w.H], "ms_hqq": round(ms_h, 3), "ms_minmax": round(ms_mm, 3),
                      "minmax_GBps_fp32_in": round(n * 4 / (ms_mm * 1e-3) / 1e9, 1),
                      "mae_minmax": err_mm, "mae_hqq": err_h, "mae_drop": round(1 - err_h / err_mm, 4),
                      "solver": {"lp": 0.7, "beta": 10.0, "kappa": 1.01, "iters": 20}, "weight_std": a.hqq_std,
                      "zeros_moved": round(float(((outh.sz >> 16) != (out.sz >> 16)).float().mean()), 4),
                      "data": "synthetic"}),
          flush=True)


def main_kv(a, bq, dev):
    """The KV-cache codec at a cache's size: 32768 tokens x 8 heads x 128
    values (bf16 N(0, 4) drawn on the device), encode and decode timed with
    HIP events; both are HBM-bound (bf16 rows one way, codes + scale/zero
    words the other)."""
    import torch
    R, D = 32768 * 8, 128
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    x = (torch.randn((R, D), generator=g, device=dev) * 2).to(torch.bfloat16)
    res = {"metric": "KV-cache codec throughput", "rows": R, "D": D, "data": "synthetic", "codec": []}

    def timed(fn, n=20):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for bits in (4, 6, 8):
        q, sz = bq.moe_kv_encode(x, bits)
        out = bq.moe_kv_decode(q, sz, D, bits)
        ms_e = timed(lambda: bq.moe_kv_encode(x, bits, q=q, sz=sz))
        ms_d = timed(lambda: bq.moe_kv_decode(q, sz, D, bits, out=out))
        nbytes = x.numel() * 2 + q.numel() + sz.numel() * 4
        err = float((out.float() - x.float()).abs().mean())
        res["codec"].append({"bits": bits, "encode_us": round(ms_e * 1e3, 2), "decode_us": round(ms_d * 1e3, 2),
                             "bytes": nbytes, "encode_GBps": round(nbytes / (ms_e * 1e-3) / 1e9, 1),
                             "decode_GBps": round(nbytes / (ms_d * 1e-3) / 1e9, 1),
                             "encode_frac": round(nbytes / (ms_e * 1e-3) / 1e9 / PEAK_HBM_GBS, 3),
                             "decode_frac": round(nbytes / (ms_d * 1e-3) / 1e9 / PEAK_HBM_GBS, 3),
                             "mean_abs_err": err})
    print(json.dumps(res), flush=True)


def hot_share(w, steps, bq):
    """Realised routing on the hot-expert workload: the share of top-k
    selections and of routing weight that lands on the hot experts, and the
    assignments per hot and per cold expert (mean), from every step's GPU
    routing."""
    import torch
    hot = torch.from_numpy(synth.hot_experts(w)).to(steps[0].idx.device)
    sel = wt = tot_w = n_sel = 0.0
    counts = []
    for st in steps:
        m = torch.isin(st.idx.long(), hot)
        sel += float(m.sum())
        n_sel += m.numel()
        wt += float((st.w * m).sum())
        tot_w += float(st.w.sum())
        counts.append(torch.bincount(st.idx.reshape(-1).long(), minlength=w.E).float())
    c = torch.stack(counts).mean(0)
    is_hot = torch.zeros(w.E, dtype=torch.bool, device=c.device)
    is_hot[hot] = True
    return {"hot_experts": int(hot.numel()), "selections": round(sel / n_sel, 4),
            "routing_weight": round(wt / tot_w, 4),
            "assignments_per_hot_expert": round(float(c[is_hot].mean()), 1),
            "assignments_per_cold_expert": round(float(c[~is_hot].mean()), 2),
            "cold_experts_at_most_32": round(float(((c <= 32) & ~is_hot).sum()), 1)}


def measure(a, w, T, bq, dev, steps, warmup, cpu=True):
    """Time exactly ``steps`` layer steps of workload w at T tokens (after
    ``warmup`` untimed ones) and the dominant call's launches; returns the
    result line as a dict."""
    import torch
    bits = w.bits
    layer_bytes = expert_bytes(w, bits) * w.n_mats
    R = a.replicas or max(2, min(16, math.ceil(2e9 / layer_bytes)))
    t0 = time.time()
    reps = build_replicas(bq, w, R, dev)
    wr = bq.bf16_from_bits(synth.router_weight_bf16(w))
    bias = synth.router_bias(w)
    bias_t = None if bias is None else torch.from_numpy(bias).to(dev)
    NB = a.batches
    xs = [bq.bf16_from_bits(synth.activations_bf16(w, T, batch=b)) for b in range(NB)]
    ws = [reps[0].workspace(T, device=dev) for _ in range(R)]
    G = max(R, NB)    # steps per graph: every replica and batch once
    A = T * (w.k + w.S)
    prefill = T > bq.DECODE_MAX_T
    y = torch.empty((A, w.H), dtype=torch.bfloat16 if prefill else torch.float32, device=dev)
    out = torch.empty((T, w.H), dtype=torch.bfloat16, device=dev)
    steps_l = [Step(bq, reps[i % R], wr, bias_t, xs[i % NB], T, ws[i % R], y=y, out=out) for i in range(G)]
    print(f"# setup {time.time() - t0:.1f}s: {w.name} T={T} replicas={R} batches={NB} graph_steps={G}",
          file=sys.stderr, flush=True)

    s = torch.cuda.Stream()
    sp = ctypes.c_void_p(s.cuda_stream)
    with torch.cuda.stream(s):
        for st in steps_l:          # eager warm pass (also loads code objects)
            st.run(sp)
    torch.cuda.synchronize()

    # realised distinct experts per step -> algorithmic bytes
    distinct = [st.distinct_experts() for st in steps_l]
    n_dist = float(np.mean(distinct))
    # the layer's algorithmic work: each distinct expert's weights once, the
    # router rows, x in and the output out; flops of the experts and router
    bytes_8d = n_dist * expert_bytes(w, bits) + w.E * w.H * 2 + T * w.H * 2 + T * w.H * 2
    exp_flops = A * 6 * w.I * w.H
    flops_8d = exp_flops + 2 * T * w.E * w.H

    graphs = {}

    def graph_of(n, part="run"):
        if a.no_graph:
            return None
        key = (n, part)
        if key not in graphs:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for st in steps_l[:n]:
                    getattr(st, part)(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            torch.cuda.synchronize()
            graphs[key] = g
        return graphs[key]

    def run_steps(n):
        """Exactly n steps: whole graphs of G steps, then one graph of the
        remaining n % G steps (eager launches without graphs)."""
        gfull = graph_of(G) if n >= G else None
        grem = graph_of(n % G) if n % G else None
        with torch.cuda.stream(s):
            if a.no_graph:
                for i in range(n):
                    steps_l[i % G].run(sp)
                return
            for _ in range(n // G):
                gfull.replay()
            if grem is not None:
                grem.replay()

    run_steps(warmup)
    if steps % G:
        graph_of(steps % G)    # captured before the timed region
    if steps >= G:
        graph_of(G)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(s)
    run_steps(steps)
    ev1.record(s)
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    ms_per_step = total_ms / steps

    # dominant call: the expert FFN call (or the whole fused decode call),
    # timed with events on its stream around replays of a graph that holds
    # only that call for every step (the routing results it reads are those
    # of the last full pass); eager launches when graphs are off
    kg = graph_of(G, "timed")
    with torch.cuda.stream(s):
        if kg is not None:
            kg.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        nrep = max(2, min(50, steps // G))
        e0.record(s)
        for _ in range(nrep):
            if kg is not None:
                kg.replay()
            else:
                for st in steps_l:
                    st.timed(sp)
        e1.record(s)
    torch.cuda.synchronize()
    kern_ms = e0.elapsed_time(e1) / (nrep * G)

    if prefill:
        # The grouped GEMM: bound by the matrix cores when the layer's
        # arithmetic intensity (its flops over its algorithmic bytes) is above
        # the ridge of the two peaks, else by HBM.  The kernel's own bytes are
        # the layer's less the router rows (another launch reads those); the
        # h and y round trips are reported beside, not counted.
        kern_bytes = bytes_8d - w.E * w.H * 2
        tflops = exp_flops / (kern_ms * 1e-3) / 1e12
        gbps = kern_bytes / (kern_ms * 1e-3) / 1e9
        intensity = flops_8d / bytes_8d
        common = {"traffic": measured_traffic(w.name, T),
                  "kernel": "moe_qgemm_prefill (tile schedule, gate/up and down grouped GEMM kernels)",
                  "alg_flops_per_launch": exp_flops, "alg_bytes_per_launch": round(kern_bytes),
                  "h_y_round_trip_bytes": 2 * A * w.I * 2 + 2 * A * w.H * 2,
                  "layer_intensity_flop_per_byte": round(intensity, 1), "ridge_flop_per_byte": RIDGE,
                  "kernel_us": round(kern_ms * 1e3, 3),
                  "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4), "hbm_frac": round(gbps / PEAK_HBM_GBS, 4)}
        if intensity >= RIDGE:
            roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tflops / PEAK_BF16_TFLOPS, 4), **common}
        else:
            roof = {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(gbps / PEAK_HBM_GBS, 4), **common}
    else:
        fused = steps_l[0].layer_fused
        # fused: the whole layer call (router rows, x and out included)
        dec_bytes = bytes_8d if fused else n_dist * expert_bytes(w, bits) + T * w.H * 2
        achieved = dec_bytes / (kern_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": measured_traffic(w.name, T),
                "kernel": ("moe_decode_forward (router; routing + gate/up; down + combine)" if fused
                           else "moe_qgemv_decode (gate/up + down grouped GEMV kernels)"),
                "alg_bytes_per_launch": round(dec_bytes), "kernel_us": round(kern_ms * 1e3, 3)}

    res = {
        "metric": "MoE-layer tokens/s",
        "value": round(T * steps / (total_ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"u{bits} codes x bf16 -> fp32" if not prefill else f"u{bits} codes -> bf16 MFMA, fp32 acc",
        "data": "synthetic (seeded N(0,0.02) weights quantised on the GPU; N(0,1) bf16 tokens)",
        "config": {"workload": w.name, "phase": "prefill" if prefill else "decode", "tokens": T, "hidden": w.H,
                   "intermediate": w.I, "experts": w.E, "top_k": w.k, "shared": w.S, "bits": bits,
                   "weight_replicas": R, "token_batches": NB, "hip_graph": not a.no_graph,
                   "distinct_experts_per_step": round(n_dist, 2), "layer_alg_bytes": round(bytes_8d),
                   "layer_alg_flops": flops_8d,
                   "layer_GBps": round(bytes_8d / (ms_per_step * 1e-3) / 1e9, 1),
                   "layer_TFLOPs": round(flops_8d / (ms_per_step * 1e-3) / 1e12, 2)},
        "roofline": roof,
    }
    if w.bias == "hot":
        res["config"]["hot_share"] = hot_share(w, steps_l, bq)
    if cpu and not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, T, a.cpu_budget)
    del graphs, steps_l, reps, ws, xs, y, out
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    help=f"NAME:T (default {DEFAULT_WORKLOAD}, with {', '.join(NESTED_DECODE)} nested)")
    ap.add_argument("--replicas", type=int, default=0, help="weight copies (0: enough for >= 2 GB)")
    ap.add_argument("--batches", type=int, default=16)
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-nested", action="store_true", help="default line without the nested decode lines")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--kv", action="store_true", help="only time the KV-cache codec at a cache's size")
    ap.add_argument("--hqq", action="store_true",
                    help="only time the HQQ-refined quantisation of one projection of the workload")
    ap.add_argument("--hqq-std", type=float, default=0.02,
                    help="standard deviation of the weights --hqq quantises (0.02: the workloads' weights)")
    ap.add_argument("--curve-max", type=int, default=0, metavar="T",
                    help="only measure the decode layer at 1 .. T tokens per call (cost curve)")
    ap.add_argument("--copy-calibrate", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (counter calibration)")
    a = ap.parse_args()

    if a.gpus != 1:
        print(json.dumps({"error": "bench.py runs on one GPU only; --gpus must be 1 "
                                   "(the multi-GPU sharding is described in the design notes, not built)"}))
        sys.exit(2)
    if a.steps < 1 or a.warmup < 0:
        print(json.dumps({"error": "--steps must be >= 1 and --warmup >= 0"}))
        sys.exit(2)

    if a.copy_calibrate:
        return copy_calibrate(a.copy_calibrate)

    import torch
    import bit_quantized_expert_amd as bq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if a.kv:
        return main_kv(a, bq, dev)
    w, T = parse_workload(a.workload or DEFAULT_WORKLOAD)
    if w.layers > 1:
        return main_stack(a, w, bq, dev)
    if a.curve_max:
        return main_curve(a, w, bq, dev)
    if a.hqq:
        return main_hqq(a, w, bq, dev)
    res = measure(a, w, T, bq, dev, a.steps, a.warmup)
    if a.workload is None and not a.no_nested:
        res["decode"] = []
        for spec in NESTED_DECODE:
            wd, Td = parse_workload(spec)
            r = measure(a, wd, Td, bq, dev, NESTED_STEPS, NESTED_WARMUP, cpu=False)
            res["decode"].append({k: r[k] for k in ("value", "unit", "steps", "ms_per_step", "config", "roofline")})
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
