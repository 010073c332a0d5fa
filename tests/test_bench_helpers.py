"""The benchmark's accounting, checked on the CPU: the visible (row, key) pair
count behind every TFLOP/s figure against the oracle's own mask, the flop and
byte formulas, and the reading of committed HBM-counter summaries."""
import hashlib
import os

import numpy as np
import pytest

import bench
import oracle
import workloads as W


def _pairs_from_oracle(w):
    """Visible pairs per q head, summed over requests, from the oracle's mask
    (the custom topology bits when the workload has them)."""
    total = 0
    for b in range(w.batch_size):
        Q, L = int(w.qo_lens[b]), int(w.kv_lens[b])
        if w.custom_mask is not None:
            rows = oracle.custom_mask_rows(w.custom_mask, w.mask_indptr, b, Q, L)
            i = np.arange(Q)[:, None]
            j = np.arange(L)[None, :]
            ok = rows.astype(bool)
            if w.window_left >= 0:
                ok &= j + Q + w.window_left >= L + i
            total += int(ok.sum())
        else:
            total += int(oracle.allowed_mask(Q, L, w.causal, w.window_left).sum())
    return total


@pytest.mark.parametrize("case", [
    "c1", "c1w", "c2", "c2w", "c3w0", "c3w31", "c3w8192", "c3p1024", "c4", "c5q64w", "tree"])
def test_visible_pairs_match_the_oracle_mask(case):
    w = {"c1": lambda: W.config1(values=False),
         "c1w": lambda: W.config1(window_left=31, values=False),
         "c2": lambda: W.config2(values=False),
         "c2w": lambda: W.config2(window_left=127, values=False),
         "c3w0": lambda: W.config3(window_left=0, page_size=16, values=False),
         "c3w31": lambda: W.config3(window_left=31, page_size=16, values=False),
         "c3w8192": lambda: W.config3(window_left=8192, page_size=16, values=False),
         "c3p1024": lambda: W.config3(window_left=127, page_size=1024, values=False),
         "c4": lambda: W.config4(batch=4, num_kv_heads=4, values=False),
         "c5q64w": lambda: W.config5(qo_len=64, window_left=4095, values=False),
         "tree": lambda: W.tree_verify(batch=4, values=False)}[case]()
    assert bench.visible_pairs(w) == _pairs_from_oracle(w)


def test_flops_and_bytes_formulas():
    w = W.config4(batch=4, num_kv_heads=8, values=False)
    pairs = bench.visible_pairs(w)
    assert bench.attention_flops(w) == 4.0 * w.head_dim * w.num_qo_heads * pairs
    # causal verify without a window: every key of every request is visible
    keys = int(np.sum(w.kv_lens))
    kv = keys * w.num_kv_heads * 2 * w.head_dim * 2
    qo = 2 * w.total_q * w.num_qo_heads * w.head_dim * 2 + w.total_q * w.num_qo_heads * 4
    assert bench.kv_bytes(w) == kv + qo
    assert bench.kv_bytes(w, kv_elem=1) == kv // 2 + qo


def _write_summary(path, lines):
    with open(path, "w") as f:
        f.write("# a header line: ignored\n")
        for k, v in lines:
            f.write(f"{k}: {v}\n")


def test_measured_traffic_reads_both_summary_forms(tmp_path):
    sha = bench.kernel_source_sha()
    a = tmp_path / "a.txt"
    _write_summary(a, [("traffic_bytes_per_launch", "1234"), ("kernel_source_sha256", sha)])
    assert bench.measured_traffic(str(a)) == 1234.0
    b = tmp_path / "b.txt"
    _write_summary(b, [("fetch_bytes_per_launch", "1000"), ("write_bytes_per_launch", "24"),
                       ("kernel_source_sha256", sha)])
    assert bench.measured_traffic(str(b)) == 1024.0
    # counters taken on another kernel source are not reported
    c = tmp_path / "c.txt"
    _write_summary(c, [("traffic_bytes_per_launch", "1234"), ("kernel_source_sha256", "0" * 64)])
    assert bench.measured_traffic(str(c)) is None
    assert bench.measured_traffic(str(tmp_path / "missing.txt")) is None


def test_kernel_source_hash_covers_the_kernel_files():
    h = hashlib.sha256()
    for path in bench.KERNEL_SOURCES:
        assert os.path.exists(path)
        with open(path, "rb") as f:
            h.update(f.read())
    assert h.hexdigest() == bench.kernel_source_sha()


def test_cpu_baseline_times_whole_passes():
    """The host baseline runs the oracle over every request of the workload in
    whole passes until its minimum time, and says how much it ran."""
    w = W.build("cpu", [3, 5], [20, 9], 4, 2, 64, 4, True, -1, W.BF16, seed=3)
    r = bench.cpu_baseline(w, min_s=0.2, budget_s=5.0)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["value"] > 0
    assert "whole pass" in r["sample"] and "over all 2 requests" in r["sample"]
    passes = int(r["sample"].split("oracle, ")[1].split(" whole")[0])
    assert passes >= 1
