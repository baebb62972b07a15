"""Host-side parts of bench.py that need no GPU: the one-GPU refusal, the
algorithmic byte counts behind `value` and the roofline, workload lookup,
and the rule that a stored counter record counts only for the kernel source
it was taken on."""

import importlib.util
import json
import os
import subprocess
import sys

import pytest

import synthetic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_workload_lookup(bench):
    for i, w in synthetic.WORKLOADS.items():
        assert bench.workload_by_name(w.name) is w
        assert bench.workload_by_name(str(i)) is w
    with pytest.raises(SystemExit):
        bench.workload_by_name("no_such_workload")


def test_algorithmic_bytes_fine_grained(bench):
    """Every array read once and written once, kept rows only (the sizes in
    the benchmark's docstring), at the largest workload: N = T*k kept rows,
    every token read, a shared expert and a residual."""
    w = synthetic.WORKLOADS[5]
    T, H, E, k, R = w.T, w.H, w.E, w.k, w.R
    N = T * k
    nb = bench.algorithmic_bytes(w, N, T, has_bias=False)
    assert nb["route"] == 32768 * 512 * 4 + 2 * 32768 * 10 * 4 == 69_730_304
    assert nb["layout"] == 2 * T * k * 4 + N * 4 + (3 * E + 2 * R + 2) * 4
    assert nb["permute"] == T * k * 4 + T * H * 2 + N * H * 2 == 1_477_705_728
    # send rows + shared + residual + out, and pos + weights
    assert nb["combine"] == 2 * T * k * 4 + N * H * 2 + 3 * T * H * 2 == 1_747_451_904
    assert sum(nb.values()) == 3_298_826_760


def test_algorithmic_bytes_capacity_and_bias(bench):
    w = synthetic.WORKLOADS[3]            # capacity-limited, residual, no shared expert
    nb = bench.algorithmic_bytes(w, 8887, 7169, has_bias=True)
    assert nb["route"] == w.T * w.E * 4 + w.E * 4 + 2 * w.T * w.k * 4
    assert nb["permute"] == w.T * w.k * 4 + 7169 * w.H * 2 + 8887 * w.H * 2
    assert nb["combine"] == 2 * w.T * w.k * 4 + 8887 * w.H * 2 + 2 * w.T * w.H * 2


def test_stored_traffic_needs_matching_source(bench, tmp_path, monkeypatch):
    kernel = "combine_kernel"
    src = bench.KERNEL_SOURCES[kernel]
    rec = {"source_sha256_16": bench.source_hash(src), "hbm_bytes_per_launch": 123}
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    path = tmp_path / f"traffic_{kernel}_some_workload.json"
    path.write_text(json.dumps(rec))
    assert bench.stored_traffic(kernel, "some_workload") == 123
    rec["source_sha256_16"] = "0" * 16
    path.write_text(json.dumps(rec))
    assert bench.stored_traffic(kernel, "some_workload") is None
    assert bench.stored_traffic(kernel, "absent_workload") is None


def test_committed_traffic_records_match_sources(bench):
    """The records under profiles/ were taken on the kernel sources as they
    stand; a stale one would make the benchmark report no traffic."""
    for kernel in bench.KERNEL_SOURCES:
        assert bench.stored_traffic(kernel, "fine_grained") is not None, kernel


def test_load_balance_hand_case(bench):
    import numpy as np
    # 4 experts on 2 destinations: demand 6, 2, 0, 0 with capacity 3 keeps 3, 2, 0, 0
    demand = np.array([6, 2, 0, 0], np.int32)
    kept = np.array([3, 2, 0, 0], np.int32)
    dest = np.array([5, 0], np.int32)
    got = bench.load_balance(demand, kept, dest)
    assert got == {"expert_demand_max_over_mean": 3.0, "expert_kept_max_over_mean": 2.4,
                   "dest_rows_max_over_mean": 2.0, "hot_dest_rows": 5, "dropped": 3}
    assert bench.load_balance(np.zeros(4, np.int32), np.zeros(4, np.int32), np.zeros(2, np.int32))[
        "expert_demand_max_over_mean"] is None


def test_token_ready_profile_hand_case(bench):
    """Two sources, two local experts, one-row bands: the work order is
    source 1 (expert 0: row 2; expert 1: rows 3-5), then source 0 (rows 0-1),
    so the tokens' last bands are 4, 1 and 3 of 6."""
    import numpy as np
    cnt = np.array([[2, 0], [1, 3]])
    pos = np.array([[0, 2], [3, -1], [4, 5], [-1, -1]])
    got = bench.token_ready_profile(cnt, pos, band_rows=1, marks=(0.5, 0.7, 1.0))
    assert got == {"bands": 6, "tokens": 3,
                   "share_ready_by_band_share": {"0.5": round(1 / 3, 4), "0.7": round(2 / 3, 4), "1.0": 1.0}}
