"""CPU oracle for the forward pass of a group-quantised MoE FFN layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, links or runs
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` use it.  It shares no code with the HIP library.

It is a plain, slow, step-by-step NumPy implementation of what the layer
computes.  Floating point work downstream of dequantisation is done in fp64;
the dequantised weights themselves are fp32, as the layer defines them.

Sources (the pages are prose about runtimes, not code):
  * Krasis update (Qwen3.6-35B-A3B on a 3070 laptop), "Latest results (v1.0)"
    and "Latest updates": expert weights stored as HQQ 4-, 6- and 8-bit
    group-quantised values, mixed per part of the model; prefill and decode
    handled by separate paths ("Overview").
  * Qwen 3.8 Flash Next on an RTX 3060, introduction; Qwen-tin, "Memory layout
    and performance": top-k routing, 10 of 512 experts per token; a prefill
    batch touches nearly every expert.
  * Raon-1-mini on a 16 GB RTX 5070 Ti, optimisation table: projections that
    share one input are run together (gate and up here).

What the pages leave open (group size, fp16 scale/zero, min-max quantiser,
packing order, SwiGLU form, tie-break, renormalisation, shared expert) is
fixed by the readings listed in the design notes; each function below states
the reading it implements.
"""
from .moe import *  # noqa: F401,F403
from .moe import __all__  # noqa: F401
