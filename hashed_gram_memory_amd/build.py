"""Build libengram.so (HIP kernels + C ABI) and libengram_measure.so (synthetic fill, probes) for gfx950 with hipcc.

Usage: python hashed_gram_memory_amd/build.py   (run by path: importing the package needs the library)
Cross-compiles without a GPU.  Object files go to _build/ next to this file.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libengram.so")
DEMO_SRC = os.path.join(CSRC, "examples", "c_abi_demo.c")
DEMO = os.path.join(HERE, "c_abi_demo")
# the lookup library (the product) and the measurement library (synthetic table fill, memory-ceiling probes)
SOURCES = ["engram_api.cpp", "hash.hip", "gather_reduce.hip", "dedup.hip", "lookup.hip", "gate_io.hip",
           "gather_batched.hip", "dedup_noalloc.hip", "check.hip"]
MEASURE_SOURCES = ["synth_fill.hip", "probe.hip"]
MEASURE_LIB = os.path.join(HERE, "libengram_measure.so")
ARCH = "gfx950"

# -packed-fp32-ops: keep the compiler from forming v_pk_{add,mul,fma}_f32.
COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result",
    f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out) -> None:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(out)} failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + MEASURE_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[f] for f in SOURCES], LIB)
    _link([objs[f] for f in MEASURE_SOURCES], MEASURE_LIB)
    # A plain C consumer of the ABI (host code only), linked against the libraries just built.
    cmd = ["gcc", "-O2", "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE, "-I", "/opt/rocm/include", DEMO_SRC,
           "-o", DEMO + ".tmp", "-L", HERE, "-lengram", "-lengram_measure", "-L", "/opt/rocm/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN", "-Wl,-rpath,/opt/rocm/lib"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"c_abi_demo build failed:\n{r.stdout}\n{r.stderr}")
    os.replace(DEMO + ".tmp", DEMO)
    if verbose:
        print("built", LIB, MEASURE_LIB, "and", DEMO)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
