"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The fp64 oracle, built with gcc's ASan + UBSan, runs every pin in a child
  process with gcc's ASan runtime preloaded; a copy with a planted
  one-row-past-the-end read of q must be reported.
* libpa.so with its C-ABI argument checks (pa_api.cpp) built with clang's
  host ASan + UBSan (device code unchanged) runs the ABI and tile-table tests
  in a child process with clang's ASan runtime preloaded.  No compute call is
  made: every call there is rejected or answered on the host.
"""
import glob
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)

import oracle  # noqa: E402

GCC_FLAGS = ("-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all")
ENV = {"ASAN_OPTIONS": "detect_leaks=0:alloc_dealloc_mismatch=0",
       "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}


def _gcc_asan():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    path = subprocess.run(["gcc", "-print-file-name=libasan.so"], stdout=subprocess.PIPE,
                          text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip("gcc's ASan runtime not found")
    return path


def _child(code, preload, timeout=600):
    env = dict(os.environ, LD_PRELOAD=preload, **ENV)
    return subprocess.run([sys.executable, "-c", code], stdout=subprocess.PIPE,
                          stderr=subprocess.STDOUT, text=True, timeout=timeout, env=env,
                          cwd=ROOT)


PINS = """
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import oracle, oracle_pins
orc = oracle.Oracle({lib!r})
for pin in oracle_pins.ALL_PINS:
    pin(orc)
print("PINS OK", len(oracle_pins.ALL_PINS))
"""


def test_oracle_pins_under_asan_ubsan(tmp_path):
    preload = _gcc_asan()
    lib = oracle.build(force=True, out=str(tmp_path / "liboracle_san.so"), flags=GCC_FLAGS)
    res = _child(PINS.format(root=ROOT, tests=HERE, lib=lib), preload)
    assert res.returncode == 0 and "PINS OK" in res.stdout, res.stdout[-3000:]


def test_asan_reports_a_planted_overread(tmp_path):
    """The sanitizer set-up itself: the last query row read one row further
    on runs past the end of q, which ASan must report."""
    preload = _gcc_asan()
    src = open(os.path.join(ROOT, "oracle", "pa_oracle.c")).read()
    site = "j->q + (t * Hq + h) * (int64_t)D"
    assert src.count(site) == 1
    bad = tmp_path / "bad.c"
    bad.write_text(src.replace(site, "j->q + (t * Hq + h + 1) * (int64_t)D"))
    lib = oracle.build(force=True, src=str(bad), out=str(tmp_path / "libbad.so"),
                       flags=GCC_FLAGS)
    res = _child(PINS.format(root=ROOT, tests=HERE, lib=lib), preload)
    assert res.returncode != 0 and "AddressSanitizer" in res.stdout, res.stdout[-3000:]


ABI = """
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
from paged_gqa_attention_pa_amd import pa
pa._LIB_PATH = {lib!r}
import pytest
sys.exit(pytest.main(["-q", "-s", "-p", "no:cacheprovider", {abi!r}, {table!r}]))
"""


def test_host_argument_checks_under_asan_ubsan(tmp_path):
    runtimes = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not runtimes:
        pytest.skip("clang's ASan runtime not found")
    from paged_gqa_attention_pa_amd import build
    try:
        build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    lib = build.build(out=str(tmp_path / "libpa_san.so"), sanitize_host_api=True)
    res = _child(ABI.format(root=ROOT, tests=HERE, lib=lib,
                            abi=os.path.join(HERE, "test_abi.py"),
                            table=os.path.join(HERE, "test_tile_table.py")), runtimes[0])
    assert res.returncode == 0, res.stdout[-4000:]
    assert "runtime error" not in res.stdout and "AddressSanitizer" not in res.stdout
