"""Host logic of bench.py (no GPU): the one-GPU refusal, the scaling of memory counters by the
calibration copy, the source check of the stored traffic, and the roofline arithmetic."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _counter_csv(d, counter, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        wr = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for i, (name, kib) in enumerate(rows):
            wr.writerow({"Dispatch_Id": i, "Kernel_Name": name, "Counter_Name": counter, "Counter_Value": kib})


def test_counters_are_scaled_by_the_calibration_copy(tmp_path):
    # the copy of 1 GiB reads 2^19 KiB of FETCH_SIZE (so fetch bytes scale by 2) and writes
    # 2^20 KiB of WRITE_SIZE (scale 1); k_chunk reads 1000 KiB and writes 300 KiB per launch over two
    # fit calls, and k_merge_levels runs 3 times per call
    copy = "void at::native::elementwise_kernel<copy>(int)"
    chunk = "void iso::k_chunk<float, true, false, false>(float const*)"
    exact = "void iso::k_chunk<float, true, false, true>(float const*)"
    merge = "void iso::k_merge_levels<float, true, false>(iso::VertexStore<float, true, false>, int, int, long)"
    _counter_csv(str(tmp_path / "f"), "FETCH_SIZE", [(copy, 524288), (chunk, 1000), (exact, 7), (chunk, 1000), (exact, 7)] +
                 [(merge, 10)] * 6)
    _counter_csv(str(tmp_path / "w"), "WRITE_SIZE", [(copy, 1048576), (chunk, 300), (exact, 5), (chunk, 300), (exact, 5)] +
                 [(merge, 4)] * 6)
    sf, sw, lines = bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"))
    assert sf == pytest.approx(2.0) and sw == pytest.approx(1.0)
    got = {k: (fb, wb, lpc) for k, fb, wb, lpc in lines}
    assert got["k_chunk"] == (pytest.approx(1000 * 1024 * 2.0), pytest.approx(300 * 1024 * 1.0), 1.0)
    assert got["k_chunk_exact"] == (pytest.approx(7 * 1024 * 2.0), pytest.approx(5 * 1024 * 1.0), 1.0)
    assert got["k_merge_levels"] == (pytest.approx(10 * 1024 * 2.0), pytest.approx(4 * 1024 * 1.0), 3.0)


def test_stored_traffic_of_other_sources_is_ignored(tmp_path, monkeypatch):
    p = tmp_path / "traffic.txt"
    p.write_text("# comment\nsource_sha256 = %s\nmixed_1e8_f32 k_chunk 100 50 1\n" % ("0" * 64))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(p))
    assert bench.read_traffic() == {}
    p.write_text("source_sha256 = %s\nmixed_1e8_f32 k_chunk 100 50 1\n" % bench.source_hash())
    assert bench.read_traffic() == {"mixed_1e8_f32": {"k_chunk": (100.0, 50.0)}}


def test_roofline_arithmetic():
    # one fit call of a 10^8 fp32 weighted row: the chunk pass (dominant stage) takes 1 ms for the
    # 10^8 elements, whose fit must move 12 bytes each (read y and w, write z); the pass itself reads 8
    st_ms = {"increasing": 0.02, "chunk": 1.0, "exact": 0.01, "scan": 0.01, "merge": 0.2, "ends": 0.01,
             "fit": 0.07}
    st_la = {k: 1 for k in st_ms}
    st_la["merge"] = 13
    traffic = {"w": {"k_chunk": (1.3e9, 0.3e9)}}
    r = bench.roofline_of("w", st_ms, st_la, 1, 10**8, 4, True, False, traffic)
    assert r["kernel"] == "k_chunk" and r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["alg_bytes_per_launch"] == 12 * 10**8
    assert r["kernel_alg_bytes_per_launch"] == 8 * 10**8
    assert r["achieved"] == pytest.approx(1200.0)
    assert r["frac"] == pytest.approx(1200.0 / 8000.0, abs=1e-4)
    assert r["traffic"] == int(1.6e9)
