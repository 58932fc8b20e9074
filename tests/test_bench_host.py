"""Host-side logic of bench.py (no GPU): the rocprofv3 counter files turned into
the committed traffic figure and the FETCH_SIZE factor of the kernel's own loads,
and the one-GPU guard."""

import csv
import json
import subprocess
import sys

import bench

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
ATTN = "void sa::(anonymous namespace)::attn_block_kernel<128, 128, 128, true, 1, false>(sa::AttnParams)"
NEG = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda(at::TensorIteratorBase&)>"


def _csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for d, (kernel, counter, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": d + 1, "Kernel_Name": kernel, "Counter_Name": counter,
                        "Counter_Value": value})
    return str(path)


def test_counter_means_per_kernel(tmp_path):
    p = _csv(tmp_path / "c.csv", [(ATTN, "FETCH_SIZE", 10.0), (ATTN, "FETCH_SIZE", 20.0),
                                  ("other", "FETCH_SIZE", 7.0), (ATTN, "WRITE_SIZE", 99.0)])
    m = bench._counter_means(p, "FETCH_SIZE")
    assert m[ATTN] == (15.0, 2)
    assert m["other"] == (7.0, 1)
    assert bench._counter_means(p, "WRITE_SIZE") == {ATTN: (99.0, 1)}


def test_traffic_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    calib_mib = 256
    # the copy moves 256 MiB; FETCH_SIZE reads half of it, WRITE_SIZE all of it
    fetch = _csv(tmp_path / "f.csv", [(NEG, "FETCH_SIZE", 131072.0), (ATTN, "FETCH_SIZE", 1000.0),
                                      (ATTN, "FETCH_SIZE", 1200.0)])
    write = _csv(tmp_path / "w.csv", [(NEG, "WRITE_SIZE", 262144.0), (ATTN, "WRITE_SIZE", 500.0)])
    assert bench._write_traffic(fetch, write, calib_mib) == 0
    t = json.loads(out.read_text())
    assert t["calibration"]["fetch_factor"] == 2.0 and t["calibration"]["write_factor"] == 1.0
    assert t["fetch_kib_per_dispatch"] == 1100.0 and t["dispatches"] == [2, 1]
    assert t["hbm_bytes_per_launch"] == round((1100.0 * 2.0 + 500.0 * 1.0) * 1024.0)
    assert t["kernel_source_sha256_16"] == bench.src_hash()


def test_dma_factor_from_block_diagonal_run(tmp_path, capsys):
    need = 3 * 32 * 8192 * 128 * 2  # Q, K and V of the headline shape, each read once
    kib = need / 1024.0 / 1.993
    p = _csv(tmp_path / "d.csv", [(ATTN, "FETCH_SIZE", kib), (ATTN, "FETCH_SIZE", kib),
                                  ("sa::(anonymous namespace)::count_kernel(...)", "FETCH_SIZE", 5.0)])
    assert bench._dma_factor(p) == 0
    r = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    assert r["dispatches"] == 2 and r["bytes_read_once"] == need
    assert r["factor_per_dispatch"] == [1.993, 1.993]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr
