"""The even-work grid's partition on the CPU: tests/even_plan_replay.cpp
replays every workgroup's walk with the arithmetic the kernels include
(csrc/pa_even_plan.h) over seeded random length mixes, built with
AddressSanitizer and UndefinedBehaviorSanitizer, and checks that every tile is
taken exactly once, partial slots stay below num_splits + 1 and piece counts
are exact.  A second build with one slot fewer must be caught."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "even_plan_replay.cpp")
FLAGS = ["-std=c++17", "-O1", "-g", "-Wall", "-Werror", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _build(tmp_path, extra=(), src=SRC):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "even_plan_replay")
    subprocess.check_call(["g++"] + FLAGS + list(extra) + [src, "-o", exe])
    return exe


def _run(exe, cases, seed):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return subprocess.run([exe, str(cases), str(seed)], stdout=subprocess.PIPE,
                          stderr=subprocess.STDOUT, text=True, timeout=300, env=env)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_even_partition_replay(tmp_path, seed):
    res = _run(_build(tmp_path), 120, seed)
    assert res.returncode == 0 and res.stdout.startswith("OK"), res.stdout[-2000:]


def test_replay_catches_a_short_slot_count(tmp_path):
    """The checker itself: with slots = num_splits instead of num_splits + 1,
    the replay must report a slot out of range."""
    src = open(SRC).read()
    assert "const int slots = S + 1;" in src
    bad = tmp_path / "bad.cpp"
    bad.write_text(src.replace("const int slots = S + 1;", "const int slots = S;").replace(
        '"../paged_gqa_attention_pa_amd', '"' + os.path.dirname(HERE) +
        '/paged_gqa_attention_pa_amd'))
    res = _run(_build(tmp_path, src=str(bad)), 120, 1)
    assert res.returncode != 0 and "slot past num_splits + 1" in res.stdout
