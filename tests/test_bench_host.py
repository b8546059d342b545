"""Host logic of bench.py, on the CPU: the refusal of more than one GPU, the
decode step's byte count against an independent count of the layer's bytes,
the steps-per-graph divisor, the batch medians behind `value`, and the HBM
traffic record written from rocprofv3 counter files (synthetic files, written
to a temporary path).
"""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_step_bytes_match_an_independent_count():
    # the 8B layer at group size 64: every weight's codes once, its scales
    # and biases (two BF16 per 64 codes) once, every output written once;
    # x read once by each of the three launches that take it, the gated down
    # projection reading gate, up (14336 BF16 each) and the residual
    shapes = [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096), (14336, 4096), (14336, 4096), (4096, 14336)]
    weights = sum(n * k + n * (k // 64) * 2 * 2 for n, k in shapes)
    outputs = sum(2 * n for n, _ in shapes)
    acts = 3 * 2 * 4096 + 2 * 2 * 14336 + 2 * 4096
    assert bench.plan_bytes(bench.FUSED) == weights + outputs + acts
    # the seven-launch form reads x six times
    assert bench.plan_bytes(bench.UNFUSED) == weights + outputs + 6 * 2 * 4096 + 2 * 2 * 14336 + 2 * 4096


@pytest.mark.parametrize("steps,per", [(300, 12), (24, 12), (7, 7), (13, 1), (10, 10), (120, 12)])
def test_steps_per_graph_divides_the_steps(steps, per):
    assert bench.steps_per_graph(steps) == per
    assert steps % per == 0


class _Event:
    def __init__(self, t_ms):
        self.t = t_ms

    def elapsed_time(self, other):
        return other.t - self.t


def test_batch_medians():
    # six intervals between seven events, two steps each: batches of two
    # intervals (2, 11, 2 ms) give 0.5, 2.75 and 0.5 ms per step
    t = [0.0]
    for dt in (1, 1, 1, 10, 1, 1):
        t.append(t[-1] + dt)
    med, mean, nb = bench.batch_medians([_Event(x) for x in t], 2, 3)
    assert nb == 3
    assert med == pytest.approx(0.5e-3)
    assert mean == pytest.approx(15e-3 / 12)


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Value"])
        w.writeheader()
        for name, grid, v in rows:
            w.writerow({"Kernel_Name": name, "Grid_Size": grid, "Counter_Value": v})


def test_traffic_record_from_counter_files(tmp_path, monkeypatch):
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "traffic_file", lambda name: str(out))
    kern = "void int8w::(anonymous namespace)::k_quantize<4, 8>(unsigned short const*)"
    copy = "__amd_rocclr_copyBuffer"
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    # the calibration copy of 256 MiB reads half its bytes in FETCH_SIZE
    # (factor 2) and all of them in WRITE_SIZE (factor 1); a small copy of
    # the same name is ignored
    _counter_csv(fetch, [(kern, 131072, 1000.0), (kern, 131072, 1200.0), (kern, 131072, 1000.0),
                         (copy, 4096, 131072.0), (copy, 64, 3.0)])
    _counter_csv(write, [(kern, 131072, 500.0), (kern, 131072, 500.0), (kern, 131072, 500.0),
                         (copy, 4096, 262144.0), (copy, 64, 3.0)])
    bench.write_traffic_record("quantize", str(fetch), str(write))
    rec = json.loads(out.read_text())
    t = bench.TARGETS["quantize"]
    assert rec["fetch_factor"] == pytest.approx(2.0)
    assert rec["write_factor"] == pytest.approx(1.0)
    assert rec["fetch_size_kib_median"] == 1000.0
    assert rec["hbm_bytes_per_launch"] == 1000 * 1024 * 2 + 500 * 1024
    assert rec["ratio_to_algorithmic"] == pytest.approx((1000 * 1024 * 2 + 500 * 1024) / t.bytes)
    assert rec["kernel_source_sha256"] == bench.source_sha(t.sources)
    assert rec["kernel"].startswith("k_quantize<4, 8>")
    # current while the kernel's sources are unchanged; null once they change
    assert bench.traffic_record("quantize")["hbm_bytes_per_launch"] == rec["hbm_bytes_per_launch"]
    rec["kernel_source_sha256"] = "0" * 64
    out.write_text(json.dumps(rec))
    assert bench.traffic_record("quantize") is None


def test_traffic_record_needs_one_kernel_and_one_calibration_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "traffic_file", lambda name: str(tmp_path / "traffic.json"))
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    _counter_csv(fetch, [("k_other", 1, 5.0)])
    _counter_csv(write, [("k_other", 1, 5.0)])
    with pytest.raises(SystemExit):
        bench.write_traffic_record("quantize", str(fetch), str(write))


def test_traffic_record_skips_other_copies_with_the_calibration_grid(tmp_path, monkeypatch):
    # a target whose rotated buffers are cloned by the same copy kernel, with
    # the same grid size as the 256 MiB calibration copy: only the calibration
    # dispatches (about 128 MiB read and 256 MiB written in the counters'
    # units) set the factors, however many smaller copies share the key
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "traffic_file", lambda name: str(out))
    kern = "void int8w::(anonymous namespace)::k_fp8_gemv<1, 8, 1, 4, false>(unsigned char const*)"
    copy = "__amd_rocclr_copyBuffer"
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    clones_f = [(copy, 4096, 28672.0)] * 20   # 56 MiB clones: half read ...
    clones_w = [(copy, 4096, 57344.0)] * 20   # ... all written
    _counter_csv(fetch, [(kern, 9, 28941.0)] * 3 + clones_f + [(copy, 4096, 131072.0)] * 5)
    _counter_csv(write, [(kern, 9, 16.0)] * 3 + clones_w + [(copy, 4096, 262144.0)] * 5)
    bench.write_traffic_record("fp8_block_4096x14336", str(fetch), str(write))
    rec = json.loads(out.read_text())
    assert rec["fetch_factor"] == pytest.approx(2.0)
    assert rec["write_factor"] == pytest.approx(1.0)
    assert rec["calibration_fetch_size_kib"] == 131072.0
    assert rec["calibration_write_size_kib"] == 262144.0
    assert rec["hbm_bytes_per_launch"] == round(28941 * 1024 * 2 + 16 * 1024)
