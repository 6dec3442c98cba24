"""Builds libflashcart.so (gfx950) in-tree with hipcc.

Steps: regenerate the coupling tables, compile every ``csrc/*.hip`` to an
object in parallel, link a shared library next to this file.  Always
recompiles (the caller decides when to build).
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libflashcart.so")
ROOT = os.path.dirname(PKG)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + CSRC, "-I" + os.path.join(ROOT, "include"),
    "-Wno-unused-command-line-argument",
]


def sources():
    gen = os.path.join(CSRC, "generated")
    out = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip")]
    out += [os.path.join(gen, f) for f in os.listdir(gen) if f.endswith(".hip")]
    return sorted(out)


def _obj(src: str) -> str:
    return os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")


def _compile(src: str) -> str:
    obj = _obj(src)
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    t = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-8000:]}")
    return f"{os.path.basename(src)} {time.time() - t:.1f}s"


# relative cost of the separately compiled VJP-of-VJP passes at the highest
# ranks (the sender pass with a feature cotangent is the longest unit)
_PART_WEIGHT = {"vx": 400, "vs": 160, "vr": 40, "vg": 40}


def _weight(src: str) -> int:
    """Rough compile cost, so that the largest units start first: the ranks
    of a convolution unit conv_inst_<l_in><l_edge><l_out key>[w | m | vr |
    vg | vs | vx]."""
    name = os.path.basename(src)
    if name.startswith("conv_inst_"):
        stem = name[len("conv_inst_"):-len(".hip")]
        if stem[-2:] in _PART_WEIGHT:
            return _PART_WEIGHT[stem[-2:]]
        xw = stem.endswith("w")   # explicit-weight VJP-of-VJP unit
        if stem.endswith("m"):    # fused radial network: forward and VJP
            return 5 * (int(stem[0]) + int(stem[1]) + int(stem[2:-1]))
        digits = stem.rstrip("w")
        a, b, key = int(digits[0]), int(digits[1]), int(digits[2:])
        return (a + b + key % 8 + (4 if (key // 8) % 2 else 0)) * (8 if xw else 10)
    return 1


def build(verbose: bool = True, jobs: int | None = None) -> str:
    sys.path.insert(0, os.path.join(PKG, "gen"))
    from cartesian_tensor_product_amd.gen import generate
    generate.emit_all()
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 4)))
    # largest units first so the long compiles start early
    srcs.sort(key=lambda p: -_weight(p))
    with cf.ThreadPoolExecutor(jobs) as ex:
        for msg in ex.map(_compile, srcs):
            if verbose:
                print("  compiled", msg, flush=True)
    objs = [_obj(s) for s in srcs]
    tmp = LIB + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr[-8000:])
    os.replace(tmp, LIB)
    if verbose:
        print("  linked", LIB, flush=True)
    return LIB


if __name__ == "__main__":
    build()
