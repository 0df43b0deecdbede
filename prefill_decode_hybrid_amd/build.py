"""Build the HIP library in-tree: prefill_decode_hybrid_amd/libpodattn.so (gfx950).

    python -m prefill_decode_hybrid_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libpodattn.so")
SOURCES = ["pod_kernels.hip", "pod_attn.cpp", "pod_plan.cpp"]
ARCH = os.environ.get("POD_ATTN_ARCH", "gfx950")

# Packed fp32 VALU forms are kept out of the generated code on purpose.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]


def build(verbose: bool = True) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objs = []
    procs = []
    t0 = time.time()
    for src in SOURCES:
        obj = os.path.join(CSRC, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, *HIP_FLAGS, "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
        objs.append(obj)
    failed = False
    for src, pr in procs:
        out, _ = pr.communicate()
        if pr.returncode != 0:
            failed = True
            sys.stderr.write(f"[build] {src} failed:\n{out}\n")
        elif verbose and out.strip():
            sys.stderr.write(f"[build] {src}:\n{out}\n")
    if failed:
        raise RuntimeError("HIP library build failed")
    tmp = LIB + ".tmp"
    subprocess.run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp], check=True)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    if verbose:
        sys.stderr.write(f"[build] {LIB} in {time.time() - t0:.1f}s\n")
    return LIB


if __name__ == "__main__":
    build()
