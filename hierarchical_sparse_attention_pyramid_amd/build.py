"""Build the Lighthouse HIP library in-tree: liblighthouse.so next to this file,
and the standalone C-ABI program tests/c_abi/lh_step that the tests run.

Every source is compiled for gfx950 only.  Packed-fp32 instructions are
disabled (`-Xclang -target-feature -Xclang -packed-fp32-ops`): the compiler
would otherwise form v_pk_* float32 ops from ordinary float code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblighthouse.so")
STEP_SRC = os.path.join(ROOT, "tests", "c_abi", "lh_step.cpp")
STEP_BIN = os.path.join(ROOT, "tests", "c_abi", "lh_step")

SOURCES = ["lighthouse.hip", "pyramid.hip", "topk.hip", "gather.hip", "scatter.hip",
           "attention_bf16.hip", "attention_f32.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", INCLUDE, "-I", CSRC]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    if os.path.exists(STEP_SRC):
        # host program linked against the library; found at run time relative to itself
        rpath = "-Wl,-rpath,$ORIGIN/../../" + os.path.basename(HERE)
        cmd = [HIPCC, "--offload-arch=gfx950", "-O2", "-std=c++17", "-I", INCLUDE, STEP_SRC,
               "-o", STEP_BIN, "-L", HERE, "-llighthouse", rpath]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"building {STEP_SRC} failed:\n{r.stderr}")
        if verbose:
            print(f"built {STEP_BIN}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
