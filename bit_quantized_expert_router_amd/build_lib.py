"""Builds libmoe_q2.so (the HIP library behind the C ABI in include/moe_q2.h)
and the moe_ceilings microbenchmark program for gfx950 with hipcc.  Run as a
module or call build()."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe_q2.so")
CEILINGS = os.path.join(PKG, "moe_ceilings")        # standalone device-ceiling microbenchmarks
SOURCES = ["route.hip", "decode.hip", "prefill.hip", "residency.hip", "api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: never emit packed fp32 VALU ops (v_pk_{add,mul,fma}_f32).
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950", "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include")]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if verbose and out.strip():
        print(out, flush=True)
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=4) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    # VGPR-form MFMA operands: otherwise the probe's loop-carried accumulators
    # are shuffled through AGPR copies every iteration and the probe measures those
    cmd = [HIPCC, *[f for f in COMMON if f != "-fPIC"], "-mllvm", "-amdgpu-mfma-vgpr-form",
           os.path.join(CSRC, "ceilings.hip"), "-o", CEILINGS + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on ceilings.hip:\n{r.stdout}{r.stderr}")
    os.replace(CEILINGS + ".tmp", CEILINGS)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
