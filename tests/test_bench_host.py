"""Host logic of bench.py (no GPU): the one-GPU refusal, the algorithmic FLOP and
byte counts its lines are priced on, and that the committed traffic records match
the kernel sources they describe."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from mla_latent_kv_41_amd import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_deepseek_step_units():
    """37.59 GFLOP and 151.03 MB of cache per DeepSeek-shaped step: scores
    2·h·4097·576, values 2·h·4097·512, the two per-head projections."""
    w = synth.make_workload(2)
    flops, cache_bytes, alg_bytes = bench.algorithmic(w)
    assert flops == pytest.approx(2 * 128 * 4097 * (576 + 512) * 32 + 2 * 2 * 128 * 32 * 128 * 512)
    assert flops / 1e9 == pytest.approx(37.59, abs=0.01)
    assert cache_bytes == 32 * 4097 * 1152
    assert alg_bytes == pytest.approx(cache_bytes + 2 * 512 * 128 * 256 + 32 * 128 * 192 * 2 + 32 * 128 * 128 * 4)
    assert bench.attention_flops(w) == pytest.approx(2 * 128 * 32 * 4097 * 1088)


def test_ragged_two_query_units_count_the_causal_tokens():
    w = synth.make_workload(4, batch=3, ctx_range=(10, 20))
    vis = sum(int(n) - 2 + j + 1 for n in w.kv_lens for j in range(2))
    assert bench.attention_flops(w) == pytest.approx(2 * 128 * vis * 1088)


def test_fused_append_units():
    w = synth.make_projection("deepseek")
    assert bench.append_bytes(w) == 4096 * 576 * 2 + 32 * 4096 * 2 + 512 * 4 + 32 * 4 + 32 * 576 * 2
    assert bench.append_bytes(w) == 5019776


def test_committed_traffic_records_match_the_sources():
    """The counter records in profiles/ carry the hash of the kernel sources they
    were measured on; while it matches, the bench reports their traffic."""
    assert bench.traffic_from_profile("deepseek_b32_ctx4096") is not None, "attention counters are stale"
    assert bench.append_traffic_from_profile() is not None, "fused-append counters are stale"
