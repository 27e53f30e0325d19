"""Host logic of bench.py, on the CPU: the one-GPU contract, the algorithmic counts of a
hand-worked batch, the roofline arithmetic and the staleness check of the committed
counter summaries."""

import importlib.util
import json
import os
import subprocess
import sys

import numpy as np
import pytest

from workloads import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_counts_hand_worked():
    """B=2, q_len=2, H=16, FP8 pages of 64, lengths 3 and 70: the queries see 2 + 3 and
    69 + 70 tokens (144 pairs); bytes = 73 tokens x 576 + 64 rows x (1152 query + 1024 O +
    4 LSE) + 3 table entries x 4."""
    b = _bench()
    w = gen.make_paged(B=2, H=16, q_len=2, lo=1, hi=1, page_size=64, fmt=gen.FMT_FP8, seed=1, seq_lens=[3, 70])
    flops, nbytes, kv = b.algorithmic_counts(w)
    assert flops == 2.0 * (576 + 512) * 16 * 144
    assert kv == 73 * 576
    assert nbytes == 73 * 576 + 64 * (1152 + 1024 + 4) + 3 * 4


def test_roofline_picks_the_binding_roof():
    b = _bench()
    # 8e9 bytes at 8 TB/s take 1 ms; 1e12 flops at 5 PF/s take 0.2 ms: HBM binds
    r = b.roofline(1e12, 8e9, 2.0, "fp8", {"hbm_stream_read_GBps": 5000.0}, None)
    assert r["bound"] == "hbm" and r["achieved"] == 4000.0 and r["frac"] == 0.5 and r["roof_us"] == 1000.0
    assert r["frac_of_measured"] == 0.8
    # bf16: 5e12 flops at 2.5 PF/s take 2 ms, 1e9 bytes 0.125 ms: the matrix cores bind
    r = b.roofline(5e12, 1e9, 4.0, "bf16", {}, 123)
    assert r["bound"] == "mfma" and r["achieved"] == 1250.0 and r["frac"] == 0.5 and r["traffic"] == 123


def test_traffic_only_for_the_profiled_sources():
    b = _bench()
    sha = b.kernel_source_hash()
    path = os.path.join(ROOT, "profiles", "decode_paged.paged_fp8_b64_h128_s1k_32k.counters.json")
    d = json.load(open(path))
    t = b.traffic_from_profiles("paged_fp8_b64_h128_s1k_32k", sha)
    if d.get("kernel_source_sha") == sha:
        assert t == d["hbm_bytes_per_launch"] and t > 0
    else:
        assert t is None
    assert b.traffic_from_profiles("paged_fp8_b64_h128_s1k_32k", "0" * 16) is None
    assert b.traffic_from_profiles("no_such_workload", sha) is None


def test_variant_traffic_from_the_same_profile():
    """The benchmark's variants (FP8-query decode) take their traffic from the same
    profiled runs, by kernel name, under the same source check."""
    b = _bench()
    path = os.path.join(ROOT, "profiles", "decode_paged.paged_fp8_b64_h128_s1k_32k.counters.json")
    d = json.load(open(path))
    sha = d["kernel_source_sha"]
    t = b.traffic_from_profiles("paged_fp8_b64_h128_s1k_32k", sha, "decode_paged", "decode_paged_kernel<3>")
    assert t == d["variant_hbm_bytes_per_launch"]["decode_paged_kernel<3>"] and t > 0
    assert b.traffic_from_profiles("paged_fp8_b64_h128_s1k_32k", sha, "decode_paged", "no_such_kernel") is None
    assert b.traffic_from_profiles("paged_fp8_b64_h128_s1k_32k", "0" * 16, "decode_paged",
                                   "decode_paged_kernel<3>") is None
