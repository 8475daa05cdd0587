"""Build libattn_scores.so (the C-ABI library) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn_scores.so")
SOURCES = ["api.cpp", "gemm.hip", "splitk.hip", "attn.hip", "tilecast.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops.
# -falign-loops=64: loop heads on 64-byte boundaries.  Where the hot loop
# of the 256x256 GEMM kernel starts inside a 64-byte block, 8192^3 runs
# 4 % slower, and without the flag that placement shifts with unrelated
# code changes.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-falign-loops=64",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-command-line-argument", "-fvisibility=hidden"]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    fd, tmp = tempfile.mkstemp(suffix=".so", dir=PKG, prefix=".libattn_scores.")
    os.close(fd)
    cmd = [HIPCC] + FLAGS + ["-I", INCLUDE, "-I", CSRC] + srcs + ["-o", tmp]
    try:
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("hipcc failed:\n" + r.stdout + r.stderr)
        if verbose:
            msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
            if msg.strip():
                print(msg)
        os.replace(tmp, LIB)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
