"""bench.py's rocprofv3 record handling, on hand-made counter files (CPU only):
the HBM-traffic record a FETCH_SIZE and a WRITE_SIZE run produce, its scaling by
the calibration copy, and the rule that roofline.traffic is reported only while
the record names the kernel and the sources it was taken on."""
import csv
import importlib.util
import json
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _counter_csv(path, counter, rows):
    """rows: (kernel name, dispatch id, value per instance...)"""
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for name, disp, *vals in rows:
            for v in vals:  # one line per counter instance, summed by the reader
                w.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": counter,
                            "Counter_Value": v})


def _record(bench, tmp_path, kernel):
    copy = "__amd_rocclr_copyBuffer"
    kname = f"void ssa::{kernel}<true>(ssa::AttnArgs)" if kernel == bench.ATTN_KERNEL \
        else f"ssa::{kernel}(int const*)"
    mib = 8
    # the copy of 8 MiB reads as 4 MiB on FETCH_SIZE (x2) and 8 MiB on WRITE_SIZE (x1)
    f = tmp_path / "fetch.csv"
    w = tmp_path / "write.csv"
    _counter_csv(f, "FETCH_SIZE", [(copy, 1, 1024, 1024, 1024, 1024), (kname, 2, 300, 200),
                                   (kname, 3, 500, 0), ("ssa::other", 4, 7)])
    _counter_csv(w, "WRITE_SIZE", [(copy, 1, 4096, 4096), (kname, 2, 50), (kname, 3, 150)])
    return bench.pmc_summary(str(f), str(w), mib, "wl_test", ["cmd-fetch", "cmd-write"], kernel)


@pytest.mark.parametrize("kernel", ["sagesla_attn_kernel", "w8a8_gemm_kernel"])
def test_traffic_record_round_trip(bench, tmp_path, monkeypatch, kernel):
    text = _record(bench, tmp_path, kernel)
    rec = json.loads(re.search(r"```json\n(.*?)\n```", text, re.S).group(1))
    assert rec["kernel"] == kernel and rec["sources_sha256"] == bench.sources_sha256(kernel)
    assert rec["fetch_scale"] == pytest.approx(2.0) and rec["write_scale"] == pytest.approx(1.0)
    k = rec["kernels"][kernel]
    # mean per dispatch: fetch (500 + 500) / 2 KiB x2, write (50 + 150) / 2 KiB x1
    assert k["fetch_bytes"] == pytest.approx(500 * 2 * 1024)
    assert k["write_bytes"] == pytest.approx(100 * 1024)
    assert "cmd-fetch" in text and "cmd-write" in text
    # read back through the same path bench.py uses for roofline.traffic
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    path = bench.traffic_record_path("wl_test", kernel)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as fh:
        fh.write(text)
    monkeypatch.setattr(bench, "sources_sha256", lambda kk: rec["sources_sha256"])
    assert bench.traffic_from_record("wl_test", kernel) == pytest.approx(1100 * 1024)


def test_stale_or_foreign_record_gives_no_traffic(bench, tmp_path, monkeypatch):
    text = _record(bench, tmp_path, bench.ATTN_KERNEL)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles", exist_ok=True)
    with open(bench.traffic_record_path("wl_test", bench.ATTN_KERNEL), "w") as fh:
        fh.write(text)
    sha = json.loads(re.search(r"```json\n(.*?)\n```", text, re.S).group(1))["sources_sha256"]
    monkeypatch.setattr(bench, "sources_sha256", lambda kk: sha)
    assert bench.traffic_from_record("wl_test", bench.ATTN_KERNEL) is not None
    # the kernel's sources changed since the counters were taken
    monkeypatch.setattr(bench, "sources_sha256", lambda kk: "0" * 64)
    assert bench.traffic_from_record("wl_test", bench.ATTN_KERNEL) is None
    # a record of another kernel under this kernel's name, or no record at all
    monkeypatch.setattr(bench, "sources_sha256", lambda kk: sha)
    with open(bench.traffic_record_path("wl_test", bench.ATTN_KERNEL), "w") as fh:
        fh.write(text.replace('"kernel": "sagesla_attn_kernel"', '"kernel": "w8a8_gemm_kernel"'))
    assert bench.traffic_from_record("wl_test", bench.ATTN_KERNEL) is None
    assert bench.traffic_from_record("no_such_workload", bench.ATTN_KERNEL) is None


def test_committed_records_name_their_kernel(bench):
    """Every committed traffic record carries the kernel and source hash fields
    the bench reads (whether or not the sources still match)."""
    prof = os.path.join(ROOT, "profiles")
    found = 0
    for name in os.listdir(prof):
        if "_hbm_traffic_" not in name:
            continue
        rec = json.loads(re.search(r"```json\n(.*?)\n```", open(os.path.join(prof, name)).read(),
                                   re.S).group(1))
        assert rec["kernel"] in (bench.ATTN_KERNEL, bench.W8_KERNEL), name
        assert len(rec["sources_sha256"]) == 64 and rec["kernels"][rec["kernel"]]["fetch_bytes"] > 0
        found += 1
    assert found >= 2


def test_effective_ops_counts_every_head(bench):
    """Dense: 4*D*N^2 per head, over all heads; a sparse selection that keeps
    every block counts the same; ragged tails count only valid tokens."""
    import numpy as np
    B, H, N = 2, 3, 1000  # 8 query blocks (last 104 tokens), 16 key blocks (last 40)
    nqb, nkb = 8, 16
    dense, _ = bench.effective_ops(None, N, nqb, nkb, True, B * H)
    assert dense == 4 * 128 * N * N * B * H
    every = np.broadcast_to(np.arange(nkb, dtype=np.int32), (B, H, nqb, nkb)).copy()
    full, _ = bench.effective_ops(every, N, nqb, nkb, False, B * H)
    assert full == dense
    # keep only the ragged last key block: 40 keys for every query of every head
    last = np.full((B, H, nqb, 1), nkb - 1, dtype=np.int32)
    one, _ = bench.effective_ops(last, N, nqb, nkb, False, B * H)
    assert one == 4 * 128 * N * 40 * B * H
