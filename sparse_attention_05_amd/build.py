"""Build libdsa.so in-tree with hipcc for gfx950.

    python -m sparse_attention_05_amd.build        # compile + link
    python -m sparse_attention_05_amd.build --asm  # also write gfx950 assembly to _build/

Each .hip source is compiled to an object in ``_build/`` (in parallel), then
linked into ``sparse_attention_05_amd/libdsa.so`` next to this file.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdsa.so")
SOURCES = ["index_scores.hip", "topk.hip", "sparse_mla.hip", "dsa_api.hip", "check.hip", "cp.hip", "read_probe.hip"]
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # CDNA4 packed-fp32 forms are kept out of generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
# Per-source additions. The attention kernels keep MFMA results in vector
# registers: the compiler otherwise puts them beside the query fragments in
# the accumulation registers, and the 8-wave prefill kernel (256 registers
# per wave) then spills inside its chunk loop.
EXTRA = {"sparse_mla.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found: the HIP toolchain (ROCm) is required to build libdsa.so")
    return h


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(asm: bool = False, verbose: bool = False) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    objs, jobs = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        flags = FLAGS + EXTRA.get(src, [])
        jobs.append([hipcc, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
        if asm:
            jobs.append([hipcc, *flags, "--cuda-device-only", "-S", os.path.join(CSRC, src),
                         "-o", os.path.join(BUILD, src.replace(".hip", f"-{ARCH}.s"))])
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", action="store_true")
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args()
    print(build(asm=args.asm, verbose=args.verbose))
    sys.exit(0)
