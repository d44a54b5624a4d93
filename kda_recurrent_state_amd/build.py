"""Build libkda.so (HIP, gfx950) in-tree with hipcc.

Usage: ``python -m kda_recurrent_state_amd.build`` (or ``__graft_entry__.build()``).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libkda.so")
SOURCES = ["kda_api.cpp", "state_copy.hip", "chunk_prefill.hip", "decode.hip", "int8_ckpt.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the KDA library needs ROCm's hipcc to build")


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link libkda.so next to this file."""
    cc = hipcc()
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [cc, "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
           # no packed-fp32 instructions in device code
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I" + INCLUDE, "-I" + CSRC, "-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in res.stdout.splitlines() if "packed-fp32-ops" not in line)
    if res.returncode != 0:
        raise RuntimeError("libkda build failed:\n" + out)
    if verbose and out.strip():
        print(out)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
