"""bench.py's host-side figures on the CPU: the algorithmic FLOP and byte
counts that its roofline fractions divide by, checked against brute-force
counts over the mask, and the one-GPU guard (no GPU needed)."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from paged_gqa_attention_pa_amd import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _allowed_pairs(L, q, causal):
    """Count (query, key) pairs the mask lets through by enumerating them:
    query i of a run of q sits at position L - q + i and sees key j when
    j < L and, if causal, j <= L - q + i."""
    keys = np.arange(L)
    n = 0
    for i in range(q):
        ok = keys < L
        if causal:
            ok &= keys <= L - q + i
        n += int(ok.sum())
    return n


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_prefill_flops_brute_force(causal):
    spec = workloads.small_spec("flops", seed=5, contexts=[300, 77, 1, 0, 64, 40],
                                queries=[140, 77, 1, 0, 3, 1], causal=causal)
    b = workloads.generate(spec)
    pairs = sum(_allowed_pairs(L, q, causal)
                for L, q in zip(b.context_lens.tolist(), b.query_lens))
    assert bench.prefill_flops(b) == 4 * spec.head_dim * spec.num_q_heads * pairs


def test_decode_bytes_per_token():
    """K and V rows of every KV head, bf16: 2 * Hkv * D * 2 bytes per token."""
    for name in ("decode_ctx512", "decode_ctx32k", "decode_b64", "decode_b256_ctx8k"):
        spec = workloads.WORKLOADS[name]
        assert bench.DECODE_BYTES_PER_TOKEN == 2 * spec.num_kv_heads * spec.head_dim * 2


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def test_roofline_bound_follows_the_larger_ideal_time():
    """A line is priced against the bound whose ideal time is larger, and its
    fraction is that ideal time over the measured one."""
    ms = 0.1
    # HBM-heavy: 600 MB and 75 GFLOP (the mixed batch's proportions)
    r = bench.roofline(600e6, 75e9, ms, None)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    ideal = max(600e6 / (bench.HBM_PEAK_GBS * 1e9), 75e9 / (bench.MFMA_BF16_PEAK_TFS * 1e12))
    assert abs(r["frac"] - round(ideal / (ms * 1e-3), 4)) < 1e-9
    # MFMA-heavy: 185 MB and 275 GFLOP (the chunked prefill's)
    r = bench.roofline(185e6, 275e9, ms, 123)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["traffic"] == 123
    ideal = 275e9 / (bench.MFMA_BF16_PEAK_TFS * 1e12)
    assert abs(r["frac"] - round(ideal / (ms * 1e-3), 4)) < 1e-9


PROFILES = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles")


def _profile_numbers(name):
    """(algorithmic bytes, traffic bytes) a counter summary states for a line."""
    import re
    text = open(os.path.join(PROFILES, f"{name}_hbm_counters.md")).read()
    m = re.search(r"`bench.py` reports ([0-9,]+) as", text)
    a = re.search(r"\): ([0-9,]+) → traffic / algorithmic", text)
    assert m and a, name
    return int(a.group(1).replace(",", "")), int(m.group(1).replace(",", ""))


@pytest.mark.parametrize("table,name", [
    ("TRAFFIC", "decode_ctx32k"), ("TRAFFIC", "decode_ctx512"), ("TRAFFIC", "decode_b64"),
    ("TRAFFIC", "decode_b256_ctx8k"), ("PREFILL_TRAFFIC", "prefill_chunk2048"),
    ("PREFILL_TRAFFIC", "mixed_unified"), ("PREFILL_TRAFFIC", "spec_verify_b64")])
def test_traffic_constants_match_their_profiles(table, name):
    """Each roofline.traffic constant is the number its committed counter
    summary says the bench reports, and lies between the algorithmic bytes
    and 1.35 times them (more would mean re-reads worth fixing, less a
    mistyped constant)."""
    alg, reported = _profile_numbers(name)
    value = getattr(bench, table)[name]
    assert value == reported
    assert alg <= value <= 1.35 * alg


def test_append_traffic_constant_matches_its_profile():
    import re
    text = open(os.path.join(PROFILES, "append_prefill_chunk2048_hbm_counters.md")).read()
    reported = int(re.search(r"`bench.py` reports ([0-9,]+) as", text).group(1).replace(",", ""))
    assert bench.APPEND_TRAFFIC["prefill_chunk2048"] == reported
    alg = 8192 * 8 * 2 * 128 * 2 * 2  # tokens x kv heads x (K, V) x D x bf16, read + written
    assert alg <= reported <= 1.05 * alg


def test_step_spread_quantiles():
    """p10 / median / p90 over per-step times (ms in, us out), by rank."""
    per = [0.001 * (i + 1) for i in range(11)]  # 1..11 us, shuffled below
    got = bench.spread(per[5:] + per[:5])
    assert got == {"p10_us": 2.0, "p50_us": 6.0, "p90_us": 10.0, "steps": 11}
    assert bench.spread([0.0357] * 60)["p50_us"] == 35.7
    assert bench.spread([]) is None


def test_bench_layout_default_and_choices(monkeypatch):
    """The benchmark stores the pools' pages head-major unless told
    otherwise, and accepts only the layouts the workloads know."""
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    assert bench.parse().layout == "head_major"
    monkeypatch.setattr(sys, "argv", ["bench.py", "--layout", "token_major"])
    assert bench.parse().layout == "token_major"
    assert set(workloads.KV_LAYOUTS) == {"head_major", "token_major"}


def test_prefill_shape_options(monkeypatch):
    """--prefill-shape re-shapes the prefill workload for profiling runs (same
    lengths and seed, another head dim or grouping); --prefill-tile-splits
    forces the query-tile split count."""
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = bench.parse()
    assert a.prefill_shape == "" and a.prefill_tile_splits == -1
    assert bench.shaped_workload(workloads, "mixed_unified", "") == "mixed_unified"
    monkeypatch.setattr(sys, "argv", ["bench.py", "--prefill-only", "--prefill-workload",
                                      "mixed_unified", "--prefill-shape", "g16",
                                      "--prefill-tile-splits", "1"])
    a = bench.parse()
    assert a.prefill_shape == "g16" and a.prefill_tile_splits == 1
    base = workloads.WORKLOADS["mixed_unified"]
    for shape, want in (("d64", (32, 8, 64)), ("d256", (32, 8, 256)), ("g16", (64, 4, 128))):
        name = bench.shaped_workload(workloads, "mixed_unified", shape)
        spec = workloads.WORKLOADS[name]
        assert (spec.num_q_heads, spec.num_kv_heads, spec.head_dim) == want
        assert (spec.seed, spec.fixed, spec.ctx_range, spec.num_draw) == \
            (base.seed, base.fixed, base.ctx_range, base.num_draw)
    assert workloads.WORKLOADS["mixed_unified"] is base
