"""Calls on several streams, and from several host threads, at once.

The compute calls only enqueue kernels on the caller's stream and share no
mutable state besides the per-device occupancy figures, so independent
problems run on separate streams, enqueued interleaved from one thread or
from separate host threads (ctypes releases the GIL for each call), must give
the bits they give when run alone, which match the oracle.
"""
import threading

import pytest
import torch

from paged_gqa_attention_pa_amd import pa, workloads
from test_gpu_parity import compare, dev, log  # noqa: F401

pytestmark = pytest.mark.gpu


def _batches(dev):
    dec = workloads.generate(workloads.small_spec(
        "st_dec", seed=501, contexts=[9000, 17, 0, 3000, 640], queries=[1] * 5), dev)
    mix = workloads.generate(workloads.small_spec(
        "st_mix", seed=502, contexts=[2000, 700, 1, 4100], queries=[1, 300, 1, 120],
        decode_layout=False), dev)
    short = workloads.generate(workloads.small_spec(
        "st_short", seed=503, contexts=[5000, 64, 900], queries=[4, 3, 5],
        decode_layout=False), dev)
    return {"decode": dec, "mixed": mix, "short": short}


def _run(kind, b):
    """One call on the current stream; returns (out, lse)."""
    lse = torch.empty(b.q.shape[:2], dtype=torch.float32, device=b.q.device)
    if kind == "decode":
        out = pa.decode(b.q, b.k_pool, b.v_pool, b.block_tables, b.context_lens, b.spec.scale,
                        b.max_context_len, out_dtype=torch.float32, lse=lse)
    else:
        out = pa.prefill(b.q, b.query_start_loc, b.k_pool, b.v_pool, b.block_tables,
                         b.context_lens, b.spec.scale, b.max_context_len, b.max_query_len,
                         causal=True, out_dtype=torch.float32, lse=lse)
    return out, lse


@pytest.fixture(scope="module")
def alone(dev):
    """Each problem run by itself on the default stream, checked against the
    oracle."""
    bs = _batches(dev)
    ref = {}
    for kind, b in bs.items():
        out, lse = _run(kind, b)
        torch.cuda.synchronize()
        compare(b, out, lse, label=f"streams: {kind} alone")
        ref[kind] = (out.clone(), lse.clone())
    return bs, ref


def test_interleaved_streams(dev, alone):
    """Three streams, calls enqueued round-robin, four rounds."""
    log("[three streams, interleaved]")
    bs, ref = alone
    streams = {k: torch.cuda.Stream(device=dev) for k in bs}
    torch.cuda.synchronize()
    results = {k: [] for k in bs}
    for _ in range(4):
        for kind, b in bs.items():
            with torch.cuda.stream(streams[kind]):
                results[kind].append(_run(kind, b))
    torch.cuda.synchronize()
    for kind, outs in results.items():
        for out, lse in outs:
            assert torch.equal(out, ref[kind][0]) and torch.equal(lse, ref[kind][1]), kind


def test_host_threads(dev, alone):
    """Three host threads, one stream each, eight calls each."""
    log("[three host threads, one stream each]")
    bs, ref = alone
    results, errors = {}, []

    def worker(kind):
        try:
            s = torch.cuda.Stream(device=dev)
            outs = []
            with torch.cuda.stream(s):
                for _ in range(8):
                    outs.append(_run(kind, bs[kind]))
            s.synchronize()
            results[kind] = outs
        except Exception as e:  # reported below, in the main thread
            errors.append(f"{kind}: {e!r}")

    torch.cuda.synchronize()
    threads = [threading.Thread(target=worker, args=(k,)) for k in bs]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for kind, outs in results.items():
        assert len(outs) == 8
        for out, lse in outs:
            assert torch.equal(out, ref[kind][0]) and torch.equal(lse, ref[kind][1]), kind
