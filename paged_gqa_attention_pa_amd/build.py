"""Build libpa.so (HIP, gfx950) in-tree with hipcc.

    python -m paged_gqa_attention_pa_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpa.so")
SOURCES = ["pa_decode.hip", "pa_reduce.hip", "pa_prefill.hip", "pa_verify.hip", "pa_append.hip",
           "pa_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def command(out: str):
    return ([hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
             # packed fp32 VALU ops stay off on this target
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include"), "-o", out]
            + [os.path.join(CSRC, s) for s in SOURCES])


def build(verbose: bool = False) -> str:
    """Compile every source into libpa.so (always recompiles)."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    noise = "packed-fp32-ops"  # the host pass warns that it does not know the feature
    msg = "\n".join(l for l in res.stdout.splitlines() if noise not in l)
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed:\n" + msg)
    if verbose and msg.strip():
        print(msg)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
