"""Compile libpagedattn.so for gfx950 with hipcc, in place (next to this file).

    python -m paged_kv_cache_86_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpagedattn.so")
SOURCES = ["pagedattn.hip", "store_gather.hip", "decode.hip", "decode_mfma.hip", "prefill.hip",
           "graph.hip", "probe.hip", "block_manager.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")
ARCH = "gfx950"
# Packed fp32 VALU ops are switched off for the device code (the host pass
# prints a harmless "not a recognized feature" warning for it).
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in p.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link ``libpagedattn.so``; returns its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    objs = [os.path.join(OBJDIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]

    def compile_one(src_obj):
        src, obj = src_obj
        if src.endswith(".cpp"):  # host-only C++
            return _run([CXX, "-O2", "-std=c++17", "-fPIC", "-Wall", "-c", os.path.join(CSRC, src),
                         "-o", obj])
        return _run([HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        logs = list(ex.map(compile_one, zip(SOURCES, objs)))
    tmp = LIB + ".tmp"
    logs.append(_run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]))
    os.replace(tmp, LIB)
    if verbose:
        for log in logs:
            if log.strip():
                print(log)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
