"""Builds libskinny_gemm.so (gfx950) in-tree with hipcc.

    python -m latency_decode_gemm_amd.build

Each translation unit is compiled in parallel into ``_build/`` and the
objects are linked into ``latency_decode_gemm_amd/libskinny_gemm.so``.
"""
from __future__ import annotations

import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libskinny_gemm.so")

SOURCES = ["skg_valu_lo.hip", "skg_valu_hi.hip", "skg_valu_ga.hip", "skg_f32w_lo.hip",
           "skg_f32w_hi.hip", "skg_f32w_ga.hip", "skg_mfma_mt2.hip", "skg_mfma_mt3.hip",
           "skg_mfma_mt4.hip", "skg_mfma_sync.hip", "skg_launch.hip", "skg_scratch.hip",
           "skg_api.cpp"]
HEADERS = ["skg_device.h", "skg_mfma_mid.h", "skg_internal.h", "tuned_table.inc", "tuned_table_f32w.inc",
           "crossover_table.inc",
           os.path.join("..", "..", "include", "skinny_gemm.h")]
ARCH = "gfx950"
# Packed fp32 VALU instructions are switched off for all device code.
FLAGS = ["-O3", f"--offload-arch={ARCH}", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), "hipcc"):
        if os.path.sep not in c or os.path.exists(c):
            return c
    return "hipcc"


def build(verbose: bool = False) -> str:
    """Compiles every source (always) and links the shared library."""
    os.makedirs(BUILD, exist_ok=True)
    t0 = time.time()
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmd = [hipcc()] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                 stderr=subprocess.STDOUT, text=True)))
    failed = []
    for src, cmd, p in procs:
        out, _ = p.communicate()
        msgs = [ln for ln in (out or "").splitlines() if "packed-fp32-ops" not in ln]
        if p.returncode != 0:
            failed.append((src, "\n".join(msgs)))
        elif verbose and msgs:
            print("\n".join(msgs), file=sys.stderr)
    if failed:
        raise RuntimeError("hipcc failed:\n" + "\n\n".join(f"[{s}]\n{m}" for s, m in failed))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s", file=sys.stderr)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
