"""Build libpkv.so in-tree with hipcc for gfx950.

    python -m paged_kv_cache_09_amd.build              # libpkv.so
    python -m paged_kv_cache_09_amd.build --timeline   # libpkv_timeline.so (diagnostics)

Every object is rebuilt on each call (the build check compiles every time).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libpkv.so")
OUT_TIMELINE = os.path.join(HERE, "libpkv_timeline.so")
BUILD = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 instructions are kept out of generated code on purpose. MFMA
# results live in ordinary VGPRs (not AGPRs): the decode kernels feed them to
# VALU work every tile, and the AGPR form added a copy each way and, for
# q4_0, a register count that halved occupancy.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form=1",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wall"]
SOURCES = ["pkv_host.cpp", "pkv_kernels.hip", "pkv_probes.hip"]
EXTRA = os.environ.get("PKV_EXTRA_FLAGS", "").split()


def build(verbose: bool = False, timeline: bool = False) -> str:
    """Build libpkv.so; timeline=True builds libpkv_timeline.so instead, with
    the per-wave timestamps of the decode kernel (PKV_TIMELINE) compiled in."""
    out = OUT_TIMELINE if timeline else OUT
    build_dir = BUILD + ("_timeline" if timeline else "")
    flags = ["-DPKV_TIMELINE"] if timeline else []
    os.makedirs(build_dir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC, *COMMON, *EXTRA, *flags, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc failed on {src}")
        objs.append(obj)
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", f"--offload-arch={ARCH}", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("link of libpkv.so failed")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True, timeline="--timeline" in sys.argv[1:]))
