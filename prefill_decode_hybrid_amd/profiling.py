"""Summaries of rocprofv3 output for the hybrid-batch attention kernels.

Turns a kernel-trace CSV and two counter-collection CSVs (one pass with
FETCH_SIZE, one with WRITE_SIZE, both in KiB per dispatch) into a short text
summary and a JSON record of the HBM bytes each kernel moves per launch.

The counters are calibrated against a plain device-to-device copy of known
size that the counter workload (``bench.py --counters-driver``) runs beside
the kernels: true bytes = counter * (copy bytes / counter value of the copy).

    python -m prefill_decode_hybrid_amd.profiling --workload NAME \
        --trace DIR --fetch DIR --write DIR --out profiles/

A second mode summarises SQ counter passes (instruction mix, MFMA busy
cycles, LDS bank conflicts, waits) per kernel:

    python -m prefill_decode_hybrid_amd.profiling counters --workload NAME \
        --pmc DIR [DIR ...] --out profiles/
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import struct
from collections import defaultdict

HERE = os.path.dirname(os.path.abspath(__file__))
CALIB_BYTES = 512 << 20          # the counter workload's device copy (read and written once)
CALIB_KERNEL = "__amd_rocclr_copyBuffer"


def _elf_section(path: str, name: str):
    """Bytes of section `name` of a 64-bit little-endian ELF file, or None."""
    b = open(path, "rb").read()
    if b[:4] != b"\x7fELF" or b[4] != 2:
        return None
    shoff, = struct.unpack_from("<Q", b, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", b, 0x3A)

    def header(i):
        return struct.unpack_from("<IIQQQQ", b, shoff + i * shentsize)

    names = header(shstrndx)[4]
    for i in range(shnum):
        nm, _, _, _, off, size = header(i)
        if b[names + nm: b.index(b"\0", names + nm)].decode() == name:
            return b[off: off + size]
    return None


def kernel_code_hash(lib: str = os.path.join(HERE, "libpodattn.so")):
    """Hash of the library's GPU code objects (its .hip_fatbin section): counter
    data is tied to the machine code it measured, and edits that leave the
    code unchanged (comments) keep it."""
    if not os.path.exists(lib):
        return None
    code = _elf_section(lib, ".hip_fatbin")
    return None if code is None else hashlib.sha256(code).hexdigest()[:16]


def kernel_resources(lib: str = os.path.join(HERE, "libpodattn.so")) -> dict:
    """Per-kernel resources of the library's gfx950 code object, read from its
    AMDGPU metadata note: {kernel name: {"vgpr", "agpr", "sgpr", "lds",
    "scratch"}} (registers per lane, bytes of static LDS and of private
    memory per work-item)."""
    import msgpack
    fat = _elf_section(lib, ".hip_fatbin")
    if fat is None or not fat.startswith(b"__CLANG_OFFLOAD_BUNDLE__"):
        raise ValueError(f"{lib}: no uncompressed offload bundle")
    n, = struct.unpack_from("<Q", fat, 24)
    pos, code = 32, None
    for _ in range(n):
        off, size, tlen = struct.unpack_from("<QQQ", fat, pos)
        triple = fat[pos + 24: pos + 24 + tlen].decode()
        pos += 24 + tlen
        if triple.endswith("gfx950"):
            code = fat[off: off + size]
    if code is None:
        raise ValueError(f"{lib}: no gfx950 code object")
    shoff, = struct.unpack_from("<Q", code, 0x28)
    shentsize, shnum = struct.unpack_from("<HH", code, 0x3A)
    out = {}
    for k in range(shnum):
        _, typ, _, _, off, size = struct.unpack_from("<IIQQQQ", code, shoff + k * shentsize)
        if typ != 7:  # SHT_NOTE
            continue
        p = off
        while p < off + size:
            namesz, descsz, ntype = struct.unpack_from("<III", code, p)
            p += 12 + ((namesz + 3) & ~3)
            desc = code[p: p + descsz]
            p += (descsz + 3) & ~3
            if ntype != 32:  # NT_AMDGPU_METADATA
                continue
            for kern in msgpack.unpackb(desc, raw=False)["amdhsa.kernels"]:
                out[kern[".name"]] = dict(vgpr=kern[".vgpr_count"], agpr=kern.get(".agpr_count", 0),
                                          sgpr=kern[".sgpr_count"], lds=kern[".group_segment_fixed_size"],
                                          scratch=kern[".private_segment_fixed_size"])
    return out


def short_name(name: str) -> str:
    n = name.replace("void ", "").split("(")[0]
    return n.replace("pod::", "")


def _rows(path_or_dir: str, suffix: str):
    files = [path_or_dir] if path_or_dir.endswith(".csv") else glob.glob(
        os.path.join(path_or_dir, "**", f"*{suffix}"), recursive=True)
    for f in files:
        yield from csv.DictReader(open(f))


def kernel_durations(trace: str) -> dict:
    """Per kernel: number of dispatches and mean / median / min duration in us."""
    d = defaultdict(list)
    for r in _rows(trace, "kernel_trace.csv"):
        d[short_name(r["Kernel_Name"])].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return {k: {"calls": len(v), "mean_us": statistics.mean(v), "median_us": statistics.median(v),
                "min_us": min(v)} for k, v in d.items()}


def counter_values(path: str, counter: str) -> dict:
    """Per kernel: mean counter value per dispatch (copies: only the calibration size)."""
    d = defaultdict(list)
    for r in _rows(path, "counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        name = r["Kernel_Name"]
        if name.startswith(CALIB_KERNEL):
            if int(r["Grid_Size"]) < 65536:  # small helper copies, not the calibration copy
                continue
        d[short_name(name)].append(float(r["Counter_Value"]))
    return {k: statistics.mean(v) for k, v in d.items()}


def traffic(fetch_dir: str, write_dir: str) -> dict:
    fetch = counter_values(fetch_dir, "FETCH_SIZE")
    write = counter_values(write_dir, "WRITE_SIZE")
    f_cal = CALIB_BYTES / fetch[CALIB_KERNEL]
    w_cal = CALIB_BYTES / write[CALIB_KERNEL]
    out = {"fetch_bytes_per_kib": f_cal, "write_bytes_per_kib": w_cal, "kernels": {}}
    for k in fetch:
        if k == CALIB_KERNEL or k not in write:
            continue
        out["kernels"][k] = {"fetch_kib": fetch[k], "write_kib": write[k],
                             "hbm_read_bytes": fetch[k] * f_cal, "hbm_write_bytes": write[k] * w_cal,
                             "hbm_bytes": fetch[k] * f_cal + write[k] * w_cal}
    return out


SIMDS = 256 * 4       # MI355X: 256 compute units of 4 SIMDs
CLOCK_HZ = 2.4e9      # peak engine clock
# Achieved occupancy: SQ_WAVE_CYCLES / SQ_BUSY_CYCLES is proportional to the
# waves resident per compute unit; the factor is read off a dispatch of known
# occupancy (a decode launch of exactly one 4-wave workgroup on each of the
# 256 CUs reads 7.3, i.e. ~2 per resident wave, so per SIMD divide by 2 * 4).
OCC_NORM = 8.0
RATIOS = [  # (label, numerator, denominator): definitions that need no per-chip normalisation
    ("vector instructions per MFMA", "SQ_INSTS_VALU", "SQ_INSTS_MFMA"),
    ("exp/transcendental instructions per MFMA", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_MFMA"),
    ("LDS instructions per MFMA", "SQ_INSTS_LDS", "SQ_INSTS_MFMA"),
    ("scalar instructions per MFMA", "SQ_INSTS_SALU", "SQ_INSTS_MFMA"),
    ("MFMA busy cycles per MFMA instruction", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA"),
    ("LDS bank-conflict cycles per LDS-active cycle", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"),
    ("share of wave time waiting on s_waitcnt", "SQ_WAIT_ANY", "SQ_WAVE_CYCLES"),
]


def counters_main(argv):
    """Summary of SQ counter passes: mean value per dispatch for every pod kernel."""
    ap = argparse.ArgumentParser(prog="profiling counters")
    ap.add_argument("--workload", required=True)
    ap.add_argument("--pmc", nargs="+", required=True, help="rocprofv3 --pmc output directories")
    ap.add_argument("--out", default="profiles")
    ap.add_argument("--command", default="")
    a = ap.parse_args(argv)
    vals = defaultdict(lambda: defaultdict(list))
    for d in a.pmc:
        for r in _rows(d, "counter_collection.csv"):
            k = short_name(r["Kernel_Name"])
            if k.startswith("pod_"):
                vals[k][r["Counter_Name"]].append(float(r["Counter_Value"]))
    names = sorted({c for v in vals.values() for c in v})
    kernels = sorted(vals)
    lines = [f"# rocprofv3 counters: {a.workload}", "", f"kernel code objects: `{kernel_code_hash()}`", ""]
    if a.command:
        lines += ["Commands:", "", "```", a.command, "```", ""]
    lines += ["Mean value per dispatch (counters summed over the chip by rocprofv3).", "",
              "| counter | " + " | ".join(f"`{k}`" for k in kernels) + " |",
              "|---|" + "---|" * len(kernels)]
    mean = {k: {c: statistics.mean(v) for c, v in vals[k].items()} for k in kernels}
    for c in names:
        lines.append(f"| {c} | " + " | ".join(f"{mean[k][c]:.4g}" if c in mean[k] else "" for k in kernels) + " |")
    lines += ["", "| ratio | " + " | ".join(f"`{k}`" for k in kernels) + " |", "|---|" + "---|" * len(kernels)]
    for label, num, den in RATIOS:
        cells = []
        for k in kernels:
            m = mean[k]
            cells.append(f"{m[num] / m[den]:.3g}" if num in m and den in m and m[den] else "")
        lines.append(f"| {label} | " + " | ".join(cells) + " |")
    # durations of the same dispatches, when the passes also ran --kernel-trace
    dur = defaultdict(list)
    for d in a.pmc:
        for r in _rows(d, "kernel_trace.csv"):
            k = short_name(r["Kernel_Name"])
            if k in mean:
                dur[k].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    cells = []
    for k in kernels:
        m = mean[k]
        ok = "SQ_WAVE_CYCLES" in m and m.get("SQ_BUSY_CYCLES")
        cells.append(f"{m['SQ_WAVE_CYCLES'] / m['SQ_BUSY_CYCLES'] / OCC_NORM:.2f}" if ok else "")
    if any(cells):
        lines.append("| resident waves per SIMD (achieved occupancy) | " + " | ".join(cells) + " |")
    if dur:
        lines.append("| mean duration in these runs (us) | " +
                     " | ".join(f"{statistics.mean(dur[k]):.1f}" if dur[k] else "" for k in kernels) + " |")
        cells = []
        for k in kernels:
            m = mean[k]
            ok = dur[k] and "SQ_VALU_MFMA_BUSY_CYCLES" in m
            cells.append(f"{m['SQ_VALU_MFMA_BUSY_CYCLES'] / (SIMDS * statistics.mean(dur[k]) * 1e-6 * CLOCK_HZ):.3f}"
                         if ok else "")
        lines.append(f"| MFMA busy share ({SIMDS} SIMDs at {CLOCK_HZ / 1e9:.1f} GHz) | " + " | ".join(cells) + " |")
    os.makedirs(a.out, exist_ok=True)
    open(os.path.join(a.out, f"counters_{a.workload}.md"), "w").write("\n".join(lines) + "\n")
    print(json.dumps({"workload": a.workload, "kernels": kernels, "counters": names}))


def main():
    import sys
    if len(sys.argv) > 1 and sys.argv[1] == "counters":
        return counters_main(sys.argv[2:])
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch", required=True)
    ap.add_argument("--write", required=True)
    ap.add_argument("--out", default="profiles")
    ap.add_argument("--command", default="", help="the command lines that produced the inputs")
    a = ap.parse_args()
    dur = kernel_durations(a.trace)
    tr = traffic(a.fetch, a.write)
    src = kernel_code_hash()
    hybrid = next((k for k in tr["kernels"] if k.startswith("pod_hybrid")), None)
    rec = {"workload": a.workload, "kernel_code": src, "kernel": hybrid,
           "hbm_bytes_per_launch": tr["kernels"][hybrid]["hbm_bytes"] if hybrid else None,
           "calibration": {"copy_bytes": CALIB_BYTES, "fetch_bytes_per_kib": tr["fetch_bytes_per_kib"],
                           "write_bytes_per_kib": tr["write_bytes_per_kib"]},
           "kernels": tr["kernels"]}
    os.makedirs(a.out, exist_ok=True)
    json.dump(rec, open(os.path.join(a.out, f"traffic_{a.workload}.json"), "w"), indent=1)
    lines = [f"# rocprofv3 summary: {a.workload}", "", f"kernel code objects: `{src}`", ""]
    if a.command:
        lines += ["Commands:", "", "```", a.command, "```", ""]
    lines += ["| kernel | calls | mean us | median us | min us | HBM read MB | HBM write MB | HBM GB/s (mean) |",
              "|---|---|---|---|---|---|---|---|"]
    for k, v in sorted(dur.items(), key=lambda kv: -kv[1]["mean_us"]):
        if not k.startswith("pod_"):
            continue
        t = tr["kernels"].get(k, {})
        rd = f"{t['hbm_read_bytes'] / 1e6:.1f}" if t else ""
        wr = f"{t['hbm_write_bytes'] / 1e6:.1f}" if t else ""
        bw = f"{t['hbm_bytes'] / (v['mean_us'] * 1e-6) / 1e9:.0f}" if t else ""
        lines.append(f"| `{k}` | {v['calls']} | {v['mean_us']:.1f} | {v['median_us']:.1f} | {v['min_us']:.1f} | {rd} | {wr} | {bw} |")
    lines += ["", f"Counter calibration: a {CALIB_BYTES >> 20} MiB device copy reads "
              f"{CALIB_BYTES / tr['fetch_bytes_per_kib'] :.0f} KiB of FETCH_SIZE and writes "
              f"{CALIB_BYTES / tr['write_bytes_per_kib']:.0f} KiB of WRITE_SIZE, so one FETCH_SIZE KiB is "
              f"{tr['fetch_bytes_per_kib']:.0f} bytes and one WRITE_SIZE KiB {tr['write_bytes_per_kib']:.0f} bytes."]
    open(os.path.join(a.out, f"{a.workload}.md"), "w").write("\n".join(lines) + "\n")
    print(json.dumps({"workload": a.workload, "hbm_bytes_per_launch": rec["hbm_bytes_per_launch"]}))


if __name__ == "__main__":
    main()
