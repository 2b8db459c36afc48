"""Builds libgla.so for gfx950 in-tree with hipcc.

    python -m linear_attention_sequence_simple_amd.build [--verbose]

Every HIP source is compiled with the packed-fp32 feature switched off
(hipcc otherwise forms packed fp32 instructions from plain float code).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgla.so")
ARCH = "gfx950"
SOURCES = ["gla_walk.hip", "gla_step.hip", "gla_state16.hip", "gla_bwd.hip", "gla_conv.hip", "gla_debug.hip",
           "gla_api.cpp"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def flags(src: str) -> list[str]:
    f = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
         "-Wall", "-Wno-unused-variable", "-Wno-unused-but-set-variable"]
    f += ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
    if src.endswith(".cpp"):
        f += ["-x", "hip"]
    return f


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".", "_") + ".o")
        objs.append(obj)
        cmds.append([hipcc()] + flags(src) + ["-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 4)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB + ".tmp"
    _run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs, verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
