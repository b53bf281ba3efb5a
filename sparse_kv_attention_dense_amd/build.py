"""Builds libsfi.so in-tree with hipcc for gfx950 (MI355X).

    python -m sparse_kv_attention_dense_amd.build

Each source is compiled to an object in parallel, then linked into
``sparse_kv_attention_dense_amd/libsfi.so``.  Only the C ABI of include/sfi.h is exported.
Packed fp32 instructions are disabled for the device code (the compiler still emits plain
fp32 VALU and MFMA); the host pass prints a harmless note about that feature.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsfi.so")
SOURCES = ["sfi_attention.hip", "sfi_select.hip", "sfi_reorg.hip", "sfi_stream.hip", "sfi_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wall"]


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(OBJ, src + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [HIPCC] + COMMON + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                                            text=True)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        noise = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln]
        if p.returncode != 0:
            failed.append((src, "\n".join(noise)))
        elif verbose and noise:
            print("\n".join(noise))
    if failed:
        msg = "\n".join(f"--- {s}\n{o}" for s, o in failed)
        raise RuntimeError(f"hipcc failed:\n{msg}")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
