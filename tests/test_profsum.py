"""Host logic of the rocprofv3 summaries: synthetic counter files with known
values go in, the per-launch figures that bench.py and the profiles quote come
out."""
import csv
import os

from lora_bypass_linear_amd import profsum


def _counter_csv(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], r)))


def test_traffic_scales_by_the_copy_and_sums_instances(tmp_path):
    fd, wd = str(tmp_path / "f"), str(tmp_path / "w")
    # copy of 1 MiB reads as 512 KiB on FETCH_SIZE (factor 2) and 1024 KiB on WRITE_SIZE
    _counter_csv(fd, [(1, "copyBuffer", "FETCH_SIZE", 512.0),
                      (2, "gemm_kernel<A>", "FETCH_SIZE", 100.0), (2, "gemm_kernel<A>", "FETCH_SIZE", 50.0),
                      (3, "gemm_kernel<A>", "FETCH_SIZE", 150.0), (4, "gemm_kernel<A>", "FETCH_SIZE", 170.0)])
    _counter_csv(wd, [(1, "copyBuffer", "WRITE_SIZE", 1024.0),
                      (2, "gemm_kernel<A>", "WRITE_SIZE", 10.0), (3, "gemm_kernel<A>", "WRITE_SIZE", 10.0)])
    out = tmp_path / "t.txt"
    profsum.main(["traffic", "--fetch", fd, "--write", wd, "--kernel", "gemm_kernel", "--sources", "gemm",
                  "--calib-kernel", "copyBuffer", "--calib-bytes", str(1 << 20), "--cmd", "c", "--out", str(out)])
    kv = dict(line.split(": ", 1) for line in out.read_text().splitlines() if ": " in line)
    assert float(kv["fetch_factor"]) == 2.0 and float(kv["write_factor"]) == 1.0
    assert float(kv["fetch_bytes_per_launch"]) == 150.0 * 1024 * 2      # median of 150, 150, 170
    assert float(kv["write_bytes_per_launch"]) == 10.0 * 1024
    assert profsum.read_traffic(str(out), "gemm") == 150.0 * 1024 * 2 + 10.0 * 1024
    assert profsum.read_traffic(str(out), "hpass") is None                # another kernel's sources


def test_mfma_busy_fraction_and_flops(tmp_path):
    d = str(tmp_path / "m")
    rows = []
    for disp in (1, 2, 3):
        rows += [(disp, "gemm_kernel<A>", "SQ_VALU_MFMA_BUSY_CYCLES", 512_000.0),
                 (disp, "gemm_kernel<A>", "SQ_INSTS_VALU_MFMA_MOPS_F16", 1000.0),
                 (disp, "gemm_kernel<A>", "SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0),
                 (disp, "gemm_kernel<A>", "GRBM_GUI_ACTIVE", 8000.0)]     # 1000 cycles on each of 8 XCDs
    _counter_csv(d, rows)
    out = tmp_path / "m.txt"
    profsum.main(["mfma", d, "--kernel", "gemm_kernel", "--cmd", "c", "--out", str(out)])
    kv = dict(line.split(": ", 1) for line in out.read_text().splitlines() if ": " in line)
    assert float(kv["mfma_busy_fraction"]) == 0.5          # 512000 / (1000 cycles x 1024 SIMDs)
    assert float(kv["mfma_flops_per_launch"]) == 512000.0
