"""Host-side parts of bench.py (no GPU): the one-GPU rule, the median's
confidence interval, the algorithmic bytes a step reads, the traffic table
lookup and the per-step figures."""
import json
import math
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workloads as W  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def _below(j, n):
    """P(Binomial(n, 1/2) <= j), exactly."""
    return sum(math.comb(n, i) for i in range(j + 1)) / 2 ** n


def test_median_ci_is_the_order_statistic_interval():
    # n = 20: P(B <= 5) = 0.0207 <= 0.025 < P(B <= 6) = 0.0577, so the
    # interval is the 6th to the 15th smallest value (coverage 0.959)
    med, lo, hi = bench.median_ci(list(range(20))[::-1])
    assert (med, lo, hi) == (9.5, 5, 14)
    # any n: the interval [X_(j), X_(n+1-j)] covers the median with
    # probability 1 - 2 P(B <= j - 1) >= 0.95, and one rank further in would not
    for n in (10, 20, 30, 50, 101):
        _, lo, hi = bench.median_ci(list(range(n)))
        j = lo + 1
        assert hi == n - j
        assert 1 - 2 * _below(j - 1, n) >= 0.95
        assert 1 - 2 * _below(j, n) < 0.95
    # too few samples for a 95% interval: the whole range
    assert bench.median_ci([3.0, 1.0, 2.0]) == (2.0, 1.0, 3.0)


def test_algorithmic_bytes_of_the_workloads():
    w = W.sweep(64)
    assert int(w.seq_lens.sum()) == 1_194_599
    # 8 kv heads x (128 K + 128 V) codes per context token
    assert bench.kv_bytes(w, 1) == 1_194_599 * 2048 == 2_446_538_752
    assert bench.kv_bytes(w, 2) == 2 * 2_446_538_752
    read = np.zeros(w.batch, dtype=bool)
    read[:3] = True
    assert bench.kv_bytes(w, 1, read) == int(w.seq_lens[:3].sum()) * 2048
    m = W.mla()
    # one latent head: 576 codes per token
    assert bench.kv_bytes(m, 1) == int(m.seq_lens.sum()) * 576


def test_traffic_table_matches_only_its_kernel_source(monkeypatch):
    w = W.sweep(64)
    digest = bench.kernel_digest("decode_gqa_mfma.hip")
    assert digest == bench.kernel_digest("decode_gqa_mfma.hip") and len(digest) == 16
    monkeypatch.setattr(bench, "TRAFFIC_KIB",
                        {("sweep_b64", 2048, "decode_gqa_mfma.hip", digest): (1000.0, 24.0)})
    assert bench.measured_traffic(w, 2048) == (1000 * 2 + 24) * 1024
    assert bench.measured_traffic(w, 1024) is None
    monkeypatch.setattr(bench, "TRAFFIC_KIB",
                        {("sweep_b64", 2048, "decode_gqa_mfma.hip", "0" * 16): (1000.0, 24.0)})
    assert bench.measured_traffic(w, 2048) is None  # counters of another build


def test_step_record_figures():
    t = {"flushed": [0.5] * 9 + [0.4] * 11, "flushed_graph": [0.6] * 20, "warm": [0.25] * 20,
         "decode": [0.3] * 20, "wall_ms_per_flushed_step": 1.0}
    r = bench.step_record(t, nbytes=2_000_000_000, batch=64)
    assert r["ms_per_step"] == 0.4
    assert r["kv_gbs"] == pytest.approx(5000.0)
    assert r["hbm_frac"] == pytest.approx(0.625)
    assert r["seq_steps_per_s"] == pytest.approx(160000.0)
    assert r["warm_kv_gbs"] == pytest.approx(8000.0)
    assert r["decode_ms"] == 0.3
