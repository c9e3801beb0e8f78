"""Compile the HIP library (and the synthetic-input fill library) for gfx950, in tree.

    python -m attention_page_table_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")

SOURCES = ["abi.cpp", "plan.cpp", "write.hip", "indexer.hip", "topk.hip", "candidates.hip", "attention.hip"]
LIB = os.path.join(HERE, "libtf.so")
SYNTH_SRC = os.path.join(ROOT, "synth", "synth.hip")
SYNTH_LIB = os.path.join(ROOT, "synth", "libtf_synth.so")

ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall", "-Wno-unused-function",
         # keep packed fp32 instructions out of the device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found (ROCm is required to build)")
    return h


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the packed-fp32 feature: drop that notice
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> None:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    objs = []
    jobs = []
    for s in SOURCES:
        src = os.path.join(CSRC, s)
        obj = os.path.join(BUILD, s + ".o")
        lang = ["-x", "hip"] if s.endswith(".hip") else []
        jobs.append([hipcc] + FLAGS + lang + ["-c", src, "-o", obj])
        objs.append(obj)
    synth_obj = os.path.join(BUILD, "synth.hip.o")
    jobs.append([hipcc] + FLAGS + ["-x", "hip", "-c", SYNTH_SRC, "-o", synth_obj])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    tmp = SYNTH_LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", synth_obj, "-o", tmp])
    os.replace(tmp, SYNTH_LIB)


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print("built", LIB, SYNTH_LIB)
