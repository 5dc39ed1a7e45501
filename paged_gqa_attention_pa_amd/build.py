"""Build libpa.so (HIP, gfx950) in-tree with hipcc.

    python -m paged_gqa_attention_pa_amd.build
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpa.so")
SOURCES = ["pa_decode.hip", "pa_reduce.hip", "pa_prefill.hip", "pa_verify.hip",
           "pa_verify_d64.hip", "pa_verify_d128.hip", "pa_verify_d256.hip", "pa_append.hip",
           "pa_check.hip", "pa_noalloc.hip",
           "pa_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"),
                 shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


FLAGS = ["-O3", "-std=c++17", "-fPIC",
         # packed fp32 VALU ops stay off on this target
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
NOISE = "packed-fp32-ops"  # the host pass warns that it does not know the feature


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer for the C-ABI
# argument checks (pa_api.cpp), device code untouched; the build loads only
# with clang's ASan runtime preloaded (a test-only build).
HOST_SANITIZE = ["-O1", "-g", "-fno-omit-frame-pointer",
                 "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all"]


def compile_command(src: str, obj: str, extra=()):
    return ([hipcc(), f"--offload-arch={ARCH}"] + FLAGS + list(extra) +
            ["-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src), "-o", obj])


def link_command(objs, out: str):
    return [hipcc(), f"--offload-arch={ARCH}", "-fPIC", "-shared", "-o", out] + list(objs)


def _run(cmd):
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    msg = "\n".join(l for l in res.stdout.splitlines() if NOISE not in l)
    return res.returncode, msg


def build(verbose: bool = False, out: str = LIB, sanitize_host_api: bool = False) -> str:
    """Compile every source (in parallel, one object each) and link libpa.so
    (always recompiles); sanitize_host_api builds pa_api.cpp with the host
    sanitizers (for tests; such a build needs clang's ASan runtime preloaded)."""
    tmpdir = tempfile.mkdtemp(prefix="pa_build_")
    try:
        objs = [os.path.join(tmpdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [compile_command(s, o, HOST_SANITIZE if sanitize_host_api and s == "pa_api.cpp"
                                else ()) for s, o in zip(SOURCES, objs)]
        if verbose:
            for c in cmds:
                print(" ".join(c), flush=True)
        workers = max(1, min(len(cmds), os.cpu_count() or 1))
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            results = list(ex.map(_run, cmds))
        for (rc, msg), src in zip(results, SOURCES):
            if rc != 0:
                raise RuntimeError(f"hipcc failed on {src}:\n" + msg)
            if verbose and msg.strip():
                print(msg)
        tmp = out + ".tmp%d" % os.getpid()
        rc, msg = _run(link_command(objs, tmp))
        if rc != 0:
            if os.path.exists(tmp):
                os.remove(tmp)
            raise RuntimeError("link failed:\n" + msg)
        os.replace(tmp, out)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
