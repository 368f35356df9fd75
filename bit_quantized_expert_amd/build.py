"""Build libmoeq.so (the HIP kernels and their C ABI) for gfx950 with hipcc.

    python bit_quantized_expert_amd/build.py [-j N] [--save-temps] [-D NAME[=VALUE] ...] [--out PATH]

(Run it by path: importing the package itself needs the built library.)

Each ``csrc/*.hip`` is compiled to an object under ``_build/`` in parallel and
the objects are linked into ``bit_quantized_expert_amd/libmoeq.so``.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoeq.so")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# Sources whose kernels count their own outstanding loads (explicit
# s_waitcnt vmcnt(N) on global -> LDS loads): scratch traffic would add
# vector-memory operations the counts do not know about, so these must
# compile without any scratch use.
NO_SCRATCH = {"prefill.hip"}


def _check_no_scratch(src, out):
    import re
    bad = []
    name = None
    for line in out.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) != 0:
            bad.append(name)
    if bad:
        raise RuntimeError(f"{src}: kernels use scratch memory (register spills): {bad}")


def _compile(src, save_temps=False, defines=(), build_dir=BUILD):
    obj = os.path.join(build_dir, os.path.basename(src)[:-4] + ".o")
    cmd = [hipcc(), *FLAGS, *[f"-D{d}" for d in defines], "-c", src, "-o", obj]
    if os.path.basename(src) in NO_SCRATCH:
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    if save_temps:
        cmd.insert(1, "--save-temps")
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=build_dir)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)   # host pass does not know the feature
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if os.path.basename(src) in NO_SCRATCH:
        _check_no_scratch(src, out)
        import re
        out = "\n".join(l for l in out.splitlines()
                        if "remark:" not in l and not re.match(r"^\s*\d*\s*\|", l))
    return obj, out


def build(jobs: int = 8, save_temps: bool = False, verbose: bool = False, defines=(), out: str = LIB) -> str:
    """Compile every source and link the library at ``out``; ``defines``
    (NAME or NAME=VALUE) are passed to every compile, and a library built
    with any goes to its own object folder."""
    build_dir = BUILD if not defines else os.path.join(BUILD, "d_" + "_".join(
        "".join(c if c.isalnum() else "-" for c in d) for d in defines))
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, save_temps, defines, build_dir), sources()))
    for obj, msg in results:
        if verbose and msg.strip():
            print(msg)
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--save-temps", action="store_true")
    ap.add_argument("-D", dest="defines", action="append", default=[], metavar="NAME[=VALUE]")
    ap.add_argument("--out", default=LIB, help="library path (default: the package's libmoeq.so)")
    a = ap.parse_args()
    print(build(a.j, a.save_temps, verbose=True, defines=a.defines, out=os.path.abspath(a.out)))
    sys.exit(0)
