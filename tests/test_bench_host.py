"""Host-side pieces of bench.py (no GPU): the algorithmic byte counts against
the figures worked out by hand for the workloads, the percentile helpers, and
the committed rocprofv3 summaries it reads: keyed to the current forward
kernel sources, so a kernel change without new profiles shows here."""
import os

import pytest

import bench
from delta_rule_sequence_efla_amd import workloads as W


def test_forward_algorithmic_bytes():
    # per head-token q, k, v read and o written (bf16, d = 128) plus beta:
    # 4 * 128 * 2 + 2 = 1026 B; 4 * 16 * 4096 head-tokens; fp32 states
    # [4, 16, 128, 128] read (s0) and written (S_L)
    w = W.get("shape_1p3b")
    n_ht = 4 * 16 * 4096
    state = 4 * 16 * 128 * 128 * 4
    assert bench.fwd_bytes(w, 2, True) == n_ht * 1026 + 2 * state == 277_348_352
    assert bench.fwd_bytes(w, 2, False) == n_ht * 1026 + state
    # small_bf16: B=4, H=8, L=2048, d=64, no initial state
    ws = W.get("small_bf16")
    assert bench.fwd_bytes(ws, 2, False) == 4 * 8 * 2048 * (4 * 64 * 2 + 2) + 4 * 8 * 64 * 64 * 4 == 34_209_792


def test_percentiles():
    xs = [5.0, 1.0, 3.0, 2.0, 4.0]
    assert bench.pct(xs, 50) == 3.0 and bench.pct(xs, 0) == 1.0 and bench.pct(xs, 100) == 5.0
    s = bench.stats_us([0.001, 0.002, 0.003])
    assert s == {"median_us": 2.0, "p10_us": 1.0, "p90_us": 3.0, "samples": 3}


def test_committed_profiles_match_the_forward_sources():
    """The traffic and trace summaries the bench line quotes were taken on the
    current forward kernel sources (else the bench reports them as null)."""
    if not os.path.exists(bench.TRAFFIC_FILE):
        pytest.skip("no committed traffic summary")
    assert bench.read_traffic("recurrence_split_kernel") is not None
    assert bench.read_traffic("ut_wave_kernel") is not None
    assert bench.read_traffic("step_kernel") is not None
    rec_us = bench.read_trace_avg_us("recurrence_split_kernel")
    ut_us = bench.read_trace_avg_us("ut_wave_kernel")
    assert rec_us is not None and ut_us is not None
    # the counted traffic is at least the algorithmic bytes of the launch
    rec_alg = 4 * 16 * 4096 * (2 * 128 + 2 * 128) * 2 + 2 * 4 * 16 * 128 * 128 * 4
    assert bench.read_traffic("recurrence_split_kernel") >= rec_alg
