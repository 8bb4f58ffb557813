"""Build librope_attn.so (HIP, gfx950) in-tree with hipcc.

    python -m bwd_rope_apply_amd.build        # compile + link

Every HIP source is compiled for gfx950 only, with packed fp32 VALU
instructions disabled, then linked into one shared library next to this file.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "librope_attn.so")
EXAMPLE = os.path.join(HERE, "rope_attn_example")
CLOCK_LIB = os.path.join(HERE, "libra_clock.so")
SOURCES = ["api.hip", "prep.hip", "simt.hip", "f32mfma.hip", "mfma.hip", "gram.hip", "noalloc.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument", f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    # the plain C++ caller of the C ABI (examples/), linked against the library
    ex_src = os.path.join(HERE, "examples", "rope_attn_example.cpp")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-O2", "-std=c++17", f"-I{INCLUDE}", ex_src, f"-L{HERE}",
           "-lrope_attn", "-Wl,-rpath,$ORIGIN", "-o", EXAMPLE + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"example build failed:\n{r.stderr}")
    os.replace(EXAMPLE + ".tmp", EXAMPLE)
    # the benchmark's shader-clock probe, a library of its own
    obj = _compile("clockprobe.hip")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", obj, "-o", CLOCK_LIB + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"clock probe link failed:\n{r.stderr}")
    os.replace(CLOCK_LIB + ".tmp", CLOCK_LIB)
    if verbose:
        print(f"built {LIB} and {EXAMPLE}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
