"""Measured peaks against the number of workgroups: the library's plain HBM
read and MFMA loop (pod_attn_peak_read, pod_attn_peak_mfma), each launched
with W workgroups of four waves.  Up to one workgroup per CU the dispatcher
places a launch's workgroups one per CU, so the read's rate per workgroup
there is what one CU streams by itself; past 256 CUs hold two.  The read
covers 4 GiB at every W (more than the 256 MB Infinity Cache, so the bytes
come from HBM), in W x 4 contiguous slices.

    python -m prefill_decode_hybrid_amd.peaks [--workgroups 16,32,64,128,256,512] [--out profiles]
"""
from __future__ import annotations

import argparse
import os
import statistics
import sys

READ_BYTES = 4 << 30
MFMA_ITERS = 4096


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workgroups", default="16,32,64,128,256,512")
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--out", default="", help="write peaks_by_workgroups.md here")
    a = ap.parse_args(argv)

    import torch
    import prefill_decode_hybrid_amd as pod

    if not torch.cuda.is_available():
        sys.exit("the peaks need a GPU")
    pod.load()
    buf = torch.zeros(READ_BYTES, dtype=torch.uint8, device="cuda:0")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")

    def timed(fn):
        fn()
        ts = []
        for _ in range(a.steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            ts.append((e0, e1))
        torch.cuda.synchronize()
        return statistics.median(x.elapsed_time(y) for x, y in ts) * 1e3  # us

    rows = []
    for w in (int(x) for x in a.workgroups.split(",")):
        t_r = timed(lambda: pod.pod_attn_peak_read(buf, READ_BYTES, w, sink))
        t_m = timed(lambda: pod.pod_attn_peak_mfma(w, MFMA_ITERS, sink))
        flops = w * 4 * MFMA_ITERS * pod.PEAK_MFMA_FLOPS_PER_ITER_WAVE
        rows.append((w, t_r, READ_BYTES / t_r / 1e6, READ_BYTES / t_r / 1e3 / w, t_m, flops / t_m / 1e6,
                     flops / t_m / 1e6 / w))
        print(f"workgroups {w:4d}  read {t_r:8.1f} us {rows[-1][2]:6.2f} TB/s {rows[-1][3]:6.1f} GB/s per wg   "
              f"mfma {t_m:8.1f} us {rows[-1][5]:7.1f} TFLOP/s {rows[-1][6]:6.2f} per wg", flush=True)
    if int(sink.item()) != 0:
        sys.exit("sink written: the read saw data it should not have")
    if a.out:
        os.makedirs(a.out, exist_ok=True)
        cmd = "python -m prefill_decode_hybrid_amd.peaks " + " ".join(argv if argv is not None else sys.argv[1:])
        lines = ["# Measured peaks against workgroups (HBM read, bf16 MFMA loop)", "",
                 f"pod_attn_peak_read over {READ_BYTES >> 30} GiB (nontemporal 16-byte buffer loads, two 16 KB "
                 "register buffers per wave) and pod_attn_peak_mfma (four independent 32x32x16 bf16 chains per "
                 f"wave, {MFMA_ITERS} iterations of 16 MFMAs), W workgroups of four waves each; median of the "
                 "timed calls after one warm-up.", "", "Command:", "", "```", cmd, "```", "",
                 "| workgroups | read us | TB/s | GB/s per workgroup | MFMA us | TFLOP/s | TFLOP/s per workgroup |",
                 "|---|---|---|---|---|---|---|"]
        for w, t_r, tbs, gbw, t_m, tf, tfw in rows:
            lines.append(f"| {w} | {t_r:.1f} | {tbs:.2f} | {gbw:.1f} | {t_m:.1f} | {tf:.1f} | {tfw:.2f} |")
        open(os.path.join(a.out, "peaks_by_workgroups.md"), "w").write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
