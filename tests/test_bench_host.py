"""Host logic of bench.py that needs no GPU: the counter record built from
rocprofv3 --pmc CSV output, and the refusal of more than one GPU."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
WALK = "void dsw::walk_kernel<1, 10, 10, 1, 0, 0, 0>(dsw::WalkParams)"
COPY = "__amd_rocclr_copyBuffer"


def _csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(FIELDS, r)))


def test_counter_record_scales_each_direction_by_the_copy(tmp_path):
    # the copy: 2 Mi requests of 128 B read as BUBBLE, 4 Mi 64-byte writes
    # (256 MiB each way); the walk: two dispatches of 500 x 32 B + 1,500 x
    # 128 B + 3,000 x 64 B reads, one of 100 x 64 B + 50 x 32 B writes
    reads = [("1", WALK, "TCC_EA0_RDREQ_sum", 5000), ("1", WALK, "TCC_EA0_RDREQ_32B_sum", 500),
             ("1", WALK, "TCC_BUBBLE_sum", 1500), ("2", WALK, "TCC_EA0_RDREQ_sum", 5000),
             ("2", WALK, "TCC_EA0_RDREQ_32B_sum", 500), ("2", WALK, "TCC_BUBBLE_sum", 1500),
             ("3", COPY, "TCC_EA0_RDREQ_sum", 2 << 20), ("3", COPY, "TCC_EA0_RDREQ_32B_sum", 0),
             ("3", COPY, "TCC_BUBBLE_sum", 2 << 20)]
    # per-instance rows of one dispatch are summed: the walk's writes come in two halves
    writes = [("1", WALK, "TCC_EA0_WRREQ_sum", 75), ("1", WALK, "TCC_EA0_WRREQ_sum", 75),
              ("1", WALK, "TCC_EA0_WRREQ_64B_sum", 100), ("3", COPY, "TCC_EA0_WRREQ_sum", 4 << 20),
              ("3", COPY, "TCC_EA0_WRREQ_64B_sum", 4 << 20)]
    _csv(str(tmp_path / "rd" / "host" / "1_counter_collection.csv"), reads)
    _csv(str(tmp_path / "wr" / "host" / "2_counter_collection.csv"), writes)
    rec = bench.summarize_counters(str(tmp_path), "qwen3_vocab_v151936_g7", 151_936, 1, 7, False, dest_dir=str(tmp_path))
    assert rec["read_scale"] == 1.0 and rec["write_scale"] == 1.0
    # per dispatch: 500 x 32 + 1,500 x 128 + 3,000 x 64
    assert rec["read_bytes_per_launch"] == 500 * 32 + 1500 * 128 + 3000 * 64
    assert rec["write_bytes_per_launch"] == 100 * 64 + 50 * 32
    assert rec["hbm_bytes_per_launch"] == rec["read_bytes_per_launch"] + rec["write_bytes_per_launch"]
    assert rec["algorithmic_bytes_per_launch"] == bench.algorithmic_bytes(151_936, 1, 7)
    with open(tmp_path / "counters_qwen3_vocab_v151936_g7_b1_g7.json") as f:
        assert json.load(f)["hbm_bytes_per_launch"] == rec["hbm_bytes_per_launch"]


def test_counter_record_with_an_undercounting_copy(tmp_path):
    # the copy's 128-byte reads show up as 64-byte requests: reads scale x2
    rows = [("1", WALK, "TCC_EA0_RDREQ_sum", 1000), ("1", WALK, "TCC_EA0_RDREQ_32B_sum", 0),
            ("1", WALK, "TCC_BUBBLE_sum", 0),
            ("3", COPY, "TCC_EA0_RDREQ_sum", 2 << 20), ("3", COPY, "TCC_EA0_RDREQ_32B_sum", 0),
            ("3", COPY, "TCC_BUBBLE_sum", 0)]
    _csv(str(tmp_path / "rd" / "1_counter_collection.csv"), rows)
    rec = bench.summarize_counters(str(tmp_path), "qwen3_vocab_v151936_g7", 151_936, 1, 7, True, dest_dir=str(tmp_path))
    assert rec["read_scale"] == 2.0 and rec["read_bytes_per_launch"] == 128_000
    assert rec["write_bytes_per_launch"] is None and "hbm_bytes_per_launch" not in rec
    assert os.path.exists(tmp_path / "counters_qwen3_vocab_v151936_g7_b1_g7_cold.json")


def test_counter_record_takes_the_last_large_copy(tmp_path):
    # input uploads before the walk and a status read-back after the
    # calibration copy are copies too
    rows = [("1", COPY, "TCC_EA0_WRREQ_sum", 9 << 20), ("1", COPY, "TCC_EA0_WRREQ_64B_sum", 9 << 20),
            ("2", WALK, "TCC_EA0_WRREQ_sum", 10), ("2", WALK, "TCC_EA0_WRREQ_64B_sum", 10),
            ("3", COPY, "TCC_EA0_WRREQ_sum", 4 << 20), ("3", COPY, "TCC_EA0_WRREQ_64B_sum", 4 << 20),
            ("4", COPY, "TCC_EA0_WRREQ_sum", 1), ("4", COPY, "TCC_EA0_WRREQ_64B_sum", 0)]
    _csv(str(tmp_path / "wr" / "1_counter_collection.csv"), rows)
    rec = bench.summarize_counters(str(tmp_path), "qwen3_vocab_v151936_g7", 151_936, 1, 7, False,
                                   dest_dir=str(tmp_path))
    assert rec["write_scale"] == 1.0 and rec["write_bytes_per_launch"] == 640


def test_counter_record_needs_the_walk_and_the_copy(tmp_path):
    _csv(str(tmp_path / "x" / "1_counter_collection.csv"), [("1", WALK, "TCC_EA0_RDREQ_sum", 1)])
    with pytest.raises(SystemExit):
        bench.summarize_counters(str(tmp_path), "qwen3_vocab_v151936_g7", 151_936, 1, 7, False, dest_dir=str(tmp_path))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]
