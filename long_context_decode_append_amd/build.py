"""Build libk8v4.so (the HIP kernels and the C ABI) for gfx950, in-tree.

Every source is compiled by hipcc for --offload-arch=gfx950 into
``_build/`` at the repository root and linked into
``long_context_decode_append_amd/lib/libk8v4.so``.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB_DIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIB_DIR, "libk8v4.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Wall",
          # packed fp32 VALU ops are kept out of the generated code
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include")]

# per-source extra flags: the quantizers must not fuse multiply and add; the
# attention kernels keep their MFMA accumulators in VGPRs (the prefill
# kernel's conditional rescale of O otherwise copies all of O between AGPRs
# and VGPRs every tile)
SOURCES = {
    "append_gather.hip": ["-ffp-contract=off"],
    "attn_splitk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "attn_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "page_copy.hip": [],
    "api.cpp": ["-x", "hip"],
    "validate.cpp": ["-x", "hip"],
}


def build(verbose: bool = False, jobs: int = 4) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    objs, procs = [], []
    for src, extra in SOURCES.items():
        obj = os.path.join(BUILD, src + ".o")
        cmd = [HIPCC, *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
        while len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[[i for i, (_, p) in enumerate(procs) if p.poll() is None][0]][1].wait()
    failed = False
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        lines = [l for l in text.splitlines() if "packed-fp32-ops" not in l]
        if p.returncode != 0 or (verbose and lines):
            sys.stderr.write(f"--- {src}\n" + "\n".join(lines) + "\n")
        failed |= p.returncode != 0
    if failed:
        raise RuntimeError("hipcc failed")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
