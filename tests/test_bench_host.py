"""Host-side arithmetic of bench.py: the decode and byte counts behind the reported rooflines, and
the HBM traffic read from rocprofv3 counters.  No GPU: these functions take host arrays and files."""
import csv
import json
import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import pytest

import bench


def test_schedule_figures_count_one_decode_per_unit_of_each_pass():
    # counts per expert; the gate+up pass shares a decode over 64 pairs, the down pass over 32
    counts = np.array([0, 1, 31, 32, 33, 64, 65, 0])
    shape = SimpleNamespace(num_experts=8, hidden=256, inter=128)
    sched = {"gate_up": {"pairs_per_decode": 64}, "down": {"pairs_per_decode": 32}}
    fig = bench.schedule_figures(counts, shape, "grouped", sched)
    assert fig["woken"] == 6
    assert fig["decodes"] == {"gate_up": 1 + 1 + 1 + 1 + 1 + 2, "down": 1 + 1 + 1 + 2 + 2 + 3}
    assert fig["max_count"] == 65
    # packed bytes of the woken experts, counted once: two 128 x 256 matrices of 2-bit codes plus
    # their fp16 row scales for gate+up; one 256 x 128 matrix plus its scales for down
    assert fig["bytes"] == {"gate_up": 6 * (2 * 128 * 256 // 4 + 2 * 128 * 2),
                            "down": 6 * (256 * 128 // 4 + 256 * 2)}
    assert fig["symbols_min"] == {"gate_up": 6 * 2 * 128 * 256, "down": 6 * 256 * 128}
    assert fig["symbols_sched"] == {"gate_up": 7 * 2 * 128 * 256, "down": 10 * 256 * 128}


def test_schedule_figures_with_one_pair_per_decode_decode_every_pair():
    counts = np.array([3, 0, 5])
    shape = SimpleNamespace(num_experts=3, hidden=128, inter=128)
    sched = {"gate_up": {"pairs_per_decode": 1}, "down": {"pairs_per_decode": 1}}
    fig = bench.schedule_figures(counts, shape, "gemv", sched)
    assert fig["decodes"] == {"gate_up": 8, "down": 8}
    assert fig["woken"] == 2


def _write_counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, counter, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


GATE_UP = "void qtip::(anonymous namespace)::expert_kernel<0, 1, qtip::(anonymous namespace)::ExpertCfg<16, 1, 2, 2>, false, false>(qtip::ExpertParams)"
DOWN = "void qtip::(anonymous namespace)::expert_kernel<1, 1, qtip::(anonymous namespace)::ExpertCfg<16, 2, 2, 2>, false, false>(qtip::ExpertParams)"
GEMV_GATE_UP = "void qtip::(anonymous namespace)::expert_kernel<0, 0, qtip::(anonymous namespace)::ExpertCfg<8, 1, 4, 4>, false, true>(qtip::ExpertParams)"
COPY = "__amd_rocclr_copyBuffer"


def test_decode_roofline_counts_one_read_per_weight_pair_on_the_lut_rung():
    # 2 T decoded weights/s: the bitshift rung gathers once per weight, the LUT rung reads its
    # codebook once per pair of weights
    bs = bench.decode_roofline("bitshift", 2e12, 1e12, 5e12)
    assert bs["bound"] == "lds_gather" and bs["gate_up_achieved"] == 2e12
    assert bs["gate_up_frac_measured"] == pytest.approx(0.4)
    assert bs["gate_up_frac_model"] == pytest.approx(2e12 / bench.LDS_GATHER_PEAK)
    lut = bench.decode_roofline("lut", 2e12, 1e12, 5e12)
    assert lut["bound"] == "lds_codebook" and lut["gate_up_achieved"] == 1e12
    assert lut["expert_passes_achieved"] == 0.5e12
    # 32 four-byte reads per clock per CU (128 bytes), 256 CUs at 2.4 GHz
    assert bench.LDS_CODEBOOK_PEAK == pytest.approx(19.6608e12)
    assert lut["gate_up_frac_model"] == pytest.approx(1e12 / 19.6608e12)
    assert "peak_measured" not in lut       # the random-gather probe does not apply to this rung


def test_traffic_is_scaled_by_what_the_counter_reads_for_a_known_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    # the 1 GiB copy reads as 512 MiB of FETCH_SIZE (factor 2) and 1 GiB of WRITE_SIZE (factor 1)
    _write_counter_csv(fetch, [(COPY, "FETCH_SIZE", 524288.0), (GATE_UP, "FETCH_SIZE", 1000.0),
                               (GATE_UP, "FETCH_SIZE", 3000.0), (DOWN, "FETCH_SIZE", 99999.0),
                               (GEMV_GATE_UP, "FETCH_SIZE", 77777.0)])
    _write_counter_csv(write, [(COPY, "WRITE_SIZE", 1048576.0), (GATE_UP, "WRITE_SIZE", 10.0),
                               (DOWN, "WRITE_SIZE", 55555.0)])
    bench.summarize_traffic(str(fetch), str(write), "wl", "grouped", "cmd")
    ent = json.load(open(bench.TRAFFIC_FILE))["wl/grouped/gate_up"]
    assert ent["dispatches"] == [2, 1]
    assert ent["fetch_factor"] == pytest.approx(2.0)
    assert ent["write_factor"] == pytest.approx(1.0)
    assert ent["hbm_bytes_per_launch"] == pytest.approx(2000.0 * 1024 * 2.0 + 10.0 * 1024 * 1.0)
    assert ent["kernel_source_sha"] == bench.kernel_source_sha()


def test_gemv_traffic_counts_the_gemv_arm_dispatches_only(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _write_counter_csv(fetch, [(COPY, "FETCH_SIZE", 524288.0), (GATE_UP, "FETCH_SIZE", 1000.0),
                               (GEMV_GATE_UP, "FETCH_SIZE", 400.0)])
    _write_counter_csv(write, [(COPY, "WRITE_SIZE", 1048576.0), (GEMV_GATE_UP, "WRITE_SIZE", 4.0)])
    bench.summarize_traffic(str(fetch), str(write), "wl", "gemv", "cmd")
    ent = json.load(open(bench.TRAFFIC_FILE))["wl/gemv/gate_up"]
    assert ent["dispatches"] == [1, 1]
    assert ent["hbm_bytes_per_launch"] == pytest.approx(400.0 * 1024 * 2.0 + 4.0 * 1024)


def test_traffic_without_a_calibration_copy_is_refused(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "traffic.json"))
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _write_counter_csv(fetch, [(GATE_UP, "FETCH_SIZE", 1000.0)])
    _write_counter_csv(write, [(COPY, "WRITE_SIZE", 1048576.0), (GATE_UP, "WRITE_SIZE", 10.0)])
    with pytest.raises(SystemExit):
        bench.summarize_traffic(str(fetch), str(write), "wl", "grouped", "cmd")


def test_traffic_is_reported_only_for_the_kernel_source_it_was_taken_on(tmp_path, monkeypatch):
    path = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(path))
    assert bench.read_traffic("wl", "grouped") is None          # no file
    path.write_text("{not json")
    assert bench.read_traffic("wl", "grouped") is None          # unreadable file
    rec = {"wl/grouped/gate_up": {"kernel_source_sha": bench.kernel_source_sha(), "hbm_bytes_per_launch": 123.0}}
    path.write_text(json.dumps(rec))
    assert bench.read_traffic("wl", "grouped") == 123.0
    assert bench.read_traffic("wl", "gemv") is None             # another arm
    rec["wl/grouped/gate_up"]["kernel_source_sha"] = "0" * 16
    path.write_text(json.dumps(rec))
    assert bench.read_traffic("wl", "grouped") is None          # counters of another kernel version


def test_committed_traffic_entries_name_their_kernel_source():
    rec = json.load(open(bench.TRAFFIC_FILE))
    assert rec, "profiles/traffic.json holds no entry"
    for key, ent in rec.items():
        assert key.endswith("/gate_up")
        assert len(ent["kernel_source_sha"]) == 16
        assert ent["hbm_bytes_per_launch"] > 0
        assert ent["fetch_factor"] > 0 and ent["write_factor"] > 0


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)
