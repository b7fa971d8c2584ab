"""Host logic of bench.py: reading HBM traffic out of rocprofv3 counter CSVs."""

import csv
import os

import bench

K = "void pkv::(anonymous namespace)::paged_decode_kernel<pkv::BF16, 128, 1, 16, {}>(pkv::AttnArgs)"
PASS = K.format("true, false, false, 1")
FUSED = K.format("true, false, true, 1")
STEP = K.format("true, true, true, 1")
RUNS = K.format("true, false, true, 16")  # runs of 16 queries: listed and fused, no token write
COPY = "void pkv::(anonymous namespace)::copy_probe_kernel(uint4 const*, uint4*, long)"


def write_csv(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value", "Grid_Size"])
        w.writeheader()
        for name, ctr, val in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": ctr, "Counter_Value": val, "Grid_Size": 512})


def test_step_kernel_name():
    assert bench.is_step_kernel(STEP)
    assert not bench.is_step_kernel(PASS) and not bench.is_step_kernel(FUSED) and not bench.is_step_kernel(RUNS)
    assert bench.decode_kernel_flags(PASS) == (True, False, False)
    assert bench.decode_kernel_flags(RUNS) == (True, False, True)
    assert bench.decode_kernel_flags(PASS.replace("true, false, false", "false, false, false")) == (False, False, False)
    assert bench.decode_kernel_flags("void pkv::(anonymous namespace)::lse_reduce_kernel<128>(pkv::AttnArgs)") is None


def test_traffic_summary_scales_by_the_copy_and_takes_the_step_kernel(tmp_path):
    gib = 1 << 30
    # the copy reads 1 GiB but its counter reads half of that: a scale of 2; writes read true
    fetch = [(COPY, "FETCH_SIZE", gib / 2 / 1024)] * 3 + [(STEP, "FETCH_SIZE", 1000.0)] * 5 + \
            [(PASS, "FETCH_SIZE", 9999.0)] * 9 + [(FUSED, "FETCH_SIZE", 7777.0)] * 4
    write = [(COPY, "WRITE_SIZE", gib / 1024)] * 3 + [(STEP, "WRITE_SIZE", 10.0)] * 5 + \
            [(PASS, "WRITE_SIZE", 9999.0)] * 9 + [(FUSED, "WRITE_SIZE", 7777.0)] * 4
    write_csv(str(tmp_path / "f" / "p_counter_collection.csv"), fetch)
    write_csv(str(tmp_path / "w" / "p_counter_collection.csv"), write)
    out = bench.traffic_summary([str(tmp_path / "f"), str(tmp_path / "w")], "llama7b_bf16")
    assert out["read_scale"] == 2.0 and out["write_scale"] == 1.0
    assert out["read_dispatches"] == 5 and out["write_dispatches"] == 5
    assert out["read_bytes_per_launch"] == 1000.0 * 1024 * 2
    assert out["write_bytes_per_launch"] == 10.0 * 1024
    assert out["hbm_bytes_per_launch"] == 1000.0 * 1024 * 2 + 10.0 * 1024
