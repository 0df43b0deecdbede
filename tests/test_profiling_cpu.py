"""The rocprofv3 summary tool on synthetic CSV files (no GPU): counter
calibration against the device copy, per-kernel HBM bytes, and the counter
ratios of the counters mode."""
import csv
import json
import os

from prefill_decode_hybrid_amd import profiling

HYB = "void pod::pod_hybrid_kernel<pod::Bf16, 128, 4>(pod::PodParams)"
COPY = "__amd_rocclr_copyBuffer"


def _write(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=list(rows[0]))
        w.writeheader()
        w.writerows(rows)


def _counter_rows(counter, hyb_value, copy_value):
    return [{"Kernel_Name": HYB, "Grid_Size": "262144", "Counter_Name": counter, "Counter_Value": str(hyb_value)},
            {"Kernel_Name": HYB, "Grid_Size": "262144", "Counter_Name": counter, "Counter_Value": str(hyb_value)},
            {"Kernel_Name": COPY, "Grid_Size": "1048576", "Counter_Name": counter, "Counter_Value": str(copy_value)},
            {"Kernel_Name": COPY, "Grid_Size": "64", "Counter_Name": counter, "Counter_Value": "1"}]


def test_traffic_calibrates_against_the_copy(tmp_path):
    # the copy reads and writes 512 MiB; FETCH counts 2 KiB units, WRITE 1 KiB units
    _write(str(tmp_path / "f" / "f_counter_collection.csv"),
           _counter_rows("FETCH_SIZE", 1000.0, (512 << 20) / 2048))
    _write(str(tmp_path / "w" / "w_counter_collection.csv"),
           _counter_rows("WRITE_SIZE", 10.0, (512 << 20) / 1024))
    t = profiling.traffic(str(tmp_path / "f"), str(tmp_path / "w"))
    k = t["kernels"]["pod_hybrid_kernel<Bf16, 128, 4>"]
    assert t["fetch_bytes_per_kib"] == 2048 and t["write_bytes_per_kib"] == 1024
    assert k["hbm_read_bytes"] == 1000 * 2048 and k["hbm_write_bytes"] == 10 * 1024


def test_kernel_durations(tmp_path):
    rows = [{"Kernel_Name": HYB, "Start_Timestamp": str(s), "End_Timestamp": str(s + d)}
            for s, d in ((0, 800_000), (10**7, 900_000), (2 * 10**7, 1_000_000))]
    _write(str(tmp_path / "t" / "t_kernel_trace.csv"), rows)
    d = profiling.kernel_durations(str(tmp_path / "t"))["pod_hybrid_kernel<Bf16, 128, 4>"]
    assert d["calls"] == 3 and d["median_us"] == 900.0 and d["min_us"] == 800.0 and abs(d["mean_us"] - 900.0) < 1e-9


def test_counters_mode(tmp_path, capsys):
    rows = []
    for name, val in (("SQ_INSTS_MFMA", 100.0), ("SQ_INSTS_VALU", 650.0), ("SQ_VALU_MFMA_BUSY_CYCLES", 3200.0),
                      ("SQ_LDS_BANK_CONFLICT", 0.0), ("SQ_LDS_IDX_ACTIVE", 500.0)):
        rows.append({"Kernel_Name": HYB, "Grid_Size": "262144", "Counter_Name": name, "Counter_Value": str(val)})
    _write(str(tmp_path / "p1" / "p1_counter_collection.csv"), rows)
    # one dispatch of 1 us: busy share = 3200 / (1024 SIMDs * 1e-6 s * 2.4e9 Hz)
    _write(str(tmp_path / "p1" / "p1_kernel_trace.csv"),
           [{"Kernel_Name": HYB, "Start_Timestamp": "0", "End_Timestamp": "1000"}])
    profiling.counters_main(["--workload", "w", "--pmc", str(tmp_path / "p1"), "--out", str(tmp_path / "out")])
    json.loads(capsys.readouterr().out.strip())
    md = open(tmp_path / "out" / "counters_w.md").read()
    assert "| vector instructions per MFMA | 6.5 |" in md
    assert "| MFMA busy cycles per MFMA instruction | 32 |" in md
    assert "| LDS bank-conflict cycles per LDS-active cycle | 0 |" in md
    assert f"| {3200 / (1024 * 1e-6 * 2.4e9):.3f} |" in md


def test_kernel_code_hash(tmp_path):
    h = profiling.kernel_code_hash()
    assert h is not None and len(h) == 16 and int(h, 16) >= 0
    assert profiling.kernel_code_hash(str(tmp_path / "missing.so")) is None
    junk = tmp_path / "junk.so"
    junk.write_bytes(b"not an ELF file")
    assert profiling.kernel_code_hash(str(junk)) is None
