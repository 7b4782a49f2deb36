"""Host logic of bench.py (CPU): the per-kernel algorithmic byte counts and
the rocprofv3 summariser, on synthetic profiler output written to a temporary
directory (the committed summaries are not touched)."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench
from decode_kv_cache_beacon_amd import synth

KIB = 1024
COPY_KIB = (1 << 32) // KIB  # the 4 GiB calibration copy, in KiB


def test_algorithmic_bytes_by_hand():
    # serving shape, one request at the batch point: N = 2112, P = 1024,
    # T = 64 steps x G = 4 query heads, K = 128 beacons, B = 2048, 8 heads
    wl = synth.WORKLOADS["serving_r128"]
    b = bench.algorithmic_bytes(wl, [2112], [1024], moved_rows=100, hc_per_req=8)
    x = bench.extra_bytes(wl, [2112], [1024], hc_per_req=8)
    # maintenance: 64*4 bf16 queries (65536) + beacons in and out (131072)
    # + counts in and out (1024), per head-cache
    assert b["beacon_update"] == 8 * 197632 and x["beacon_update"] == 0
    # scoring: 2112 keys read once (540672) + fp32 beacons (65536)
    assert b["beacon_score"] == 8 * 606208
    # ... and beside it counts (512) + 132 block-table entries (528) + 1088
    # scores written (4352)
    assert x["beacon_score"] == 8 * 5392
    # selection: 1088 scores read (4352) + 2048 keep entries (8192)
    assert b["topk_select"] == 8 * 12544
    # compaction: 100 moved rows, K and V each read and written (102400);
    # the keep lists it reads (8 x 8192) are extra
    assert b["kv_compact"] == 102400 and x["kv_compact"] == 65536
    # the fused kernel: keys once, beacons, moved rows
    # (N*d*2 + K*d*4 + 4*M*d*2 per head-cache)
    assert b["beacon_evict"] == 8 * (2112 * 128 * 2 + 128 * 128 * 4) + 4 * 100 * 128 * 2
    assert x["beacon_evict"] == 8 * 5392 + 65536


def test_algorithmic_bytes_scale_with_the_cache():
    wl = synth.WORKLOADS["serving_r128"]
    a = bench.algorithmic_bytes(wl, [2112], [1024], 0, 1)
    b = bench.algorithmic_bytes(wl, [2112 + 16], [1024], 0, 1)
    xa = bench.extra_bytes(wl, [2112], [1024], 1)
    xb = bench.extra_bytes(wl, [2112 + 16], [1024], 1)
    # maintenance does not see the cache
    assert a["beacon_update"] == b["beacon_update"]
    # sixteen more slots: 16 keys; one more page and 16 more scores are extra
    assert b["beacon_score"] - a["beacon_score"] == 16 * 256
    assert xb["beacon_score"] - xa["beacon_score"] == 4 + 16 * 4
    assert b["topk_select"] - a["topk_select"] == 16 * 4
    # two requests cost twice one
    two = bench.algorithmic_bytes(wl, [2112, 2112], [1024, 1024], 0, 1)
    for k in ("beacon_update", "beacon_score", "topk_select", "kv_compact", "beacon_evict"):
        assert two[k] == 2 * a[k]


def _write_csv(path, fields, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(fields, r)))


SCORE = "void bkv::(anonymous namespace)::beacon_score_kernel<4>(bkv::CacheView, int)"
COMPACT = "void bkv::(anonymous namespace)::kv_compact_kernel(bkv::CacheView)"
EVICT = "void bkv::(anonymous namespace)::beacon_evict_kernel<2, 2, 2, 2>(bkv::CacheView, int)"
COPY = "__amd_rocclr_copyBuffer.kd"
OTHER = "void at::native::elementwise_kernel<128, 4>(int)"


@pytest.fixture
def fake_profiles(tmp_path):
    prof, pmc = tmp_path / "prof", tmp_path / "pmc"
    ms = 1_000_000  # ns
    _write_csv(str(prof / "bench_kernel_trace.csv"),
               ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
               [(SCORE, 0, 1 * ms), (SCORE, 10 * ms, 13 * ms), (COMPACT, 20 * ms, 25 * ms),
                (OTHER, 30 * ms, 90 * ms), (EVICT, 100 * ms, 107 * ms)])
    cc = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    # the counters over-read the copy by 25 % and under-read its writes by half:
    # read factor 0.8, write factor 2.0; two small copies do not calibrate
    _write_csv(str(pmc / "FETCH_SIZE" / "FETCH_SIZE_counter_collection.csv"), cc,
               [(1, COPY, "FETCH_SIZE", 100.0), (2, COPY, "FETCH_SIZE", 1.25 * COPY_KIB),
                (3, COPY, "FETCH_SIZE", 1.25 * COPY_KIB), (4, COPY, "FETCH_SIZE", 50.0),
                (5, SCORE, "FETCH_SIZE", 1000.0), (6, SCORE, "FETCH_SIZE", 3000.0),
                (7, COMPACT, "FETCH_SIZE", 4000.0), (8, OTHER, "FETCH_SIZE", 9e9)])
    _write_csv(str(pmc / "WRITE_SIZE" / "WRITE_SIZE_counter_collection.csv"), cc,
               [(1, COPY, "WRITE_SIZE", 10.0), (2, COPY, "WRITE_SIZE", 0.5 * COPY_KIB),
                (3, COPY, "WRITE_SIZE", 0.5 * COPY_KIB), (4, COPY, "WRITE_SIZE", 20.0),
                (5, SCORE, "WRITE_SIZE", 10.0), (6, SCORE, "WRITE_SIZE", 30.0),
                (7, COMPACT, "WRITE_SIZE", 2000.0), (8, OTHER, "WRITE_SIZE", 9e9)])
    # MFMA run: per-dispatch rows summed (one row per XCD), then averaged
    _write_csv(str(pmc / "MFMA" / "MFMA_counter_collection.csv"), cc,
               [(5, SCORE, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 100.0),
                (5, SCORE, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 300.0),
                (6, SCORE, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 400.0),
                (5, SCORE, "MfmaUtil", 30.0), (6, SCORE, "MfmaUtil", 40.0)])
    # issue counters: two runs, per-dispatch rows summed, then averaged over dispatches
    _write_csv(str(pmc / "SQ1" / "SQ1_counter_collection.csv"), cc,
               [(5, SCORE, "SQ_WAVES", 40.0), (5, SCORE, "SQ_WAVES", 60.0),
                (6, SCORE, "SQ_WAVES", 100.0),
                (5, SCORE, "SQ_WAVE_CYCLES", 1000.0), (6, SCORE, "SQ_WAVE_CYCLES", 3000.0),
                (5, SCORE, "SQ_INSTS_VALU", 5000.0), (6, SCORE, "SQ_INSTS_VALU", 7000.0),
                (5, SCORE, "SQ_INSTS_SALU", 2000.0), (6, SCORE, "SQ_INSTS_SALU", 2000.0),
                (5, SCORE, "SQ_INSTS_LDS", 300.0), (6, SCORE, "SQ_INSTS_LDS", 100.0),
                (5, SCORE, "SQ_ACTIVE_INST_VALU", 600.0), (6, SCORE, "SQ_ACTIVE_INST_VALU", 600.0),
                (5, SCORE, "SQ_WAIT_INST_ANY", 1.0), (6, SCORE, "SQ_WAIT_INST_ANY", 1.0)])
    _write_csv(str(pmc / "SQ2" / "SQ2_counter_collection.csv"), cc,
               [(5, SCORE, "SQ_INSTS_VMEM", 100.0), (6, SCORE, "SQ_INSTS_VMEM", 300.0),
                (5, SCORE, "SQ_INSTS_BRANCH", 50.0), (6, SCORE, "SQ_INSTS_BRANCH", 150.0),
                (5, SCORE, "SQ_ACTIVE_INST_ANY", 1000.0), (6, SCORE, "SQ_ACTIVE_INST_ANY", 1000.0),
                (5, SCORE, "SQ_ACTIVE_INST_SCA", 200.0), (6, SCORE, "SQ_ACTIVE_INST_SCA", 200.0),
                (5, SCORE, "SQ_WAIT_ANY", 500.0), (6, SCORE, "SQ_WAIT_ANY", 300.0)])
    out = tmp_path / "out"
    bench.summarize_profiles(str(prof), str(pmc), "fake", out=str(out))
    return out


def test_summary_durations(fake_profiles):
    text = (fake_profiles / "fake_kernel_trace.md").read_text()
    rows = {r.split("|")[1].strip(): [c.strip() for c in r.split("|")[2:6]]
            for r in text.splitlines() if r.startswith("| ") and "kernel" not in r}
    assert rows["beacon_score"] == ["2", "2.000", "1.000", "3.000"]
    assert rows["kv_compact"] == ["1", "5.000", "5.000", "5.000"]
    # the fused kernel is told apart from the scoring kernel it shares a source with
    assert rows["beacon_evict"] == ["1", "7.000", "7.000", "7.000"]
    assert set(rows) == {"beacon_score", "kv_compact", "beacon_evict"}  # others not listed
    assert bench.profile_cmd("trace", "fake") in text
    assert "bench.py --workload fake --steps" in text


def test_summary_traffic_calibration(fake_profiles):
    t = json.loads((fake_profiles / "fake_traffic.json").read_text())
    cal = t["_calibration"]
    assert cal["read_factor"] == pytest.approx(0.8)
    assert cal["write_factor"] == pytest.approx(2.0)
    s = t["beacon_score"]
    assert s["fetch_kib"] == 2000.0 and s["write_kib"] == 20.0
    assert s["bytes_read"] == pytest.approx(2000 * KIB * 0.8)
    assert s["bytes_written"] == pytest.approx(20 * KIB * 2.0)
    assert s["bytes_per_launch"] == pytest.approx(s["bytes_read"] + s["bytes_written"])
    assert s["source_sha"] == bench.kernel_source_hash("beacon_score")
    c = t["kv_compact"]
    assert c["bytes_per_launch"] == pytest.approx(4000 * KIB * 0.8 + 2000 * KIB * 2.0)
    assert set(t) == {"_workload", "_calibration", "beacon_score", "kv_compact"}
    assert t["_workload"] == "fake"
    # the MFMA and issue runs add their per-launch figures to the same entries
    assert s["mfma_flop_per_launch"] == pytest.approx(400 * 512)
    assert s["issue_share"] == pytest.approx(0.5) and s["wait_share"] == pytest.approx(0.2)
    md = (fake_profiles / "fake_hbm_counters.md").read_text()
    assert "read factor 0.8000, write factor 2.0000" in md


def test_summary_mfma(fake_profiles):
    text = (fake_profiles / "fake_mfma_counters.md").read_text()
    row = next(r for r in text.splitlines() if r.startswith("| beacon_score"))
    cells = [c.strip() for c in row.split("|")[2:6]]
    # utilisation 35 %, 400 bf16 MFMA ops x 512 flop per launch over 2 ms
    assert cells[0] == "35.0"
    assert float(cells[1]) == pytest.approx(400 * 512)
    assert float(cells[2]) == pytest.approx(round(400 * 512 / 2e-3 / 1e12, 1))


def test_summary_issue(fake_profiles):
    text = (fake_profiles / "fake_issue_counters.md").read_text()
    row = next(r for r in text.splitlines() if r.startswith("| beacon_score"))
    cells = [c.strip() for c in row.split("|")[2:12]]
    # 100 waves, 2000 wave-cycles per dispatch on average; instructions per wave
    assert cells[:6] == ["100", "60", "20", "2", "2", "1"]
    # shares of the wave lifetime: any 1000/2000, VALU 600/2000, scalar 200/2000, wait 400/2000
    assert cells[6:] == ["0.50", "0.30", "0.10", "0.20"]
    assert bench.profile_cmd("pmc_sq1", "fake") in text
    assert bench.profile_cmd("pmc_sq2", "fake") in text


def test_stored_traffic_belongs_to_its_workload(tmp_path, monkeypatch):
    path = tmp_path / "t.json"
    monkeypatch.setattr(bench, "traffic_file", lambda workload, out=None: str(path))
    sha = bench.kernel_source_hash("beacon_evict")
    path.write_text(json.dumps({"_calibration": {"workload": "a"},
                                "beacon_evict": {"bytes_per_launch": 5.0, "source_sha": sha}}))
    assert bench.stored_traffic("beacon_evict", "a") == 5.0
    assert bench.stored_traffic("beacon_evict", "b") is None      # another workload's bytes
    path.write_text(json.dumps({"_calibration": {"workload": "a"},
                                "beacon_evict": {"bytes_per_launch": 5.0, "source_sha": "x"}}))
    assert bench.stored_traffic("beacon_evict", "a") is None      # taken on other source
    path.write_text(json.dumps({"_workload": "a", "beacon_evict": {
        "bytes_per_launch": 5.0, "mfma_flop_per_launch": 7.0, "source_sha": sha}}))
    assert bench.stored_counters("beacon_evict", "a")["mfma_flop_per_launch"] == 7.0
    assert bench.stored_counters("beacon_evict", "b") == {}


def test_traffic_file_names():
    assert bench.traffic_file(bench.DEFAULT_WORKLOAD).endswith("profiles/traffic.json")
    assert bench.traffic_file("a").endswith("profiles/a_traffic.json")


def test_profile_commands_run_committed_files_only():
    for cmd in bench.PROFILE_CMDS.values():
        assert "_work" not in cmd and "/root/reference" not in cmd
    for name in bench.KERNEL_SOURCES.values():
        assert os.path.exists(os.path.join(bench.ROOT, "decode_kv_cache_beacon_amd", "csrc",
                                           name))
    assert set(bench.KERNEL_SYMBOLS.values()) == set(bench.KERNEL_SOURCES)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("workload", ["serving_r128", "qwen3_32b_r32", "qwen3_4b_r16"])
def test_committed_counters_match_the_current_kernel_sources(workload):
    """The bench reports counter traffic only from profiles taken on the
    current kernel sources; the committed summaries of every profiled
    workload must therefore be refreshed with any kernel change, or the
    line's `traffic` field goes null."""
    path = bench.traffic_file(workload)
    with open(path) as f:
        t = json.load(f)
    kernels = [k for k in t if not k.startswith("_")]
    assert {"beacon_update", "beacon_evict"} <= set(kernels), kernels
    for k in kernels:
        assert t[k]["source_sha"] == bench.kernel_source_hash(k), (workload, k)
        assert bench.stored_counters(k, workload), (workload, k)
