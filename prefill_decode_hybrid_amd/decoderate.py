"""Decode stream rate against the number of decode workgroups: decode-only
launches of N requests of the same context (Llama-3-8B heads: 32 q / 8 kv,
d 128, bf16), one split length, so that N fixes how many workgroups stream
at once.  Shows how many workgroups it takes to reach the HBM plateau and
what one workgroup streams on its own, the yardstick for a decode
workgroup that shares its CU with a prefill workgroup in a fused launch.

    python -m prefill_decode_hybrid_amd.decoderate [--requests 4,8,16,32,64] [--context 16384]
        [--split 4096] [--wg-per-cu 2] [--contiguous] [--out profiles]
"""
from __future__ import annotations

import argparse
import os
import sys


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--requests", default="4,8,16,32,64", help="decode batch sizes")
    ap.add_argument("--context", type=int, default=16384)
    ap.add_argument("--split", type=int, default=4096, help="decode tokens per wave task")
    ap.add_argument("--wg-per-cu", type=int, default=2)
    ap.add_argument("--contiguous", action="store_true", help="identity page tables")
    ap.add_argument("--steps", type=int, default=15)
    ap.add_argument("--out", default="", help="write decode_rate_<...>.md here")
    a = ap.parse_args(argv)

    import torch
    import prefill_decode_hybrid_amd as pod
    from prefill_decode_hybrid_amd import inputs
    from prefill_decode_hybrid_amd.timing import interleaved_us

    if not torch.cuda.is_available():
        sys.exit("the decode rate needs a GPU")
    pod.load()
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    rows = []
    for n in (int(x) for x in a.requests.split(",")):
        sp = dict(name=f"decode{n}", dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128, chunk_len=16,
                  chunk_offset=0, decode_lens=[a.context] * n, contiguous=a.contiguous)
        b = inputs.make_batch(sp, seed=0)
        dev = b.to("cuda:0")
        ctx = b.context_lens.clone().contiguous()
        att = pod.PodAttention(pod.config_for_batch(b, wg_per_cu=a.wg_per_cu, decode_split_tokens=a.split))
        od = torch.empty_like(dev.q_decode)
        (us,) = interleaved_us([lambda: att.decode_only(dev, od, ctx)], a.steps, 3, flush)
        st = att.stats()
        att.close()
        kv_bytes = n * a.context * b.num_kv_heads * b.head_dim * 2 * 2
        wgs = st["decode_wg_tasks"]
        rows.append((n, wgs, st["wg_per_cu"], us, kv_bytes / us / 1e6, kv_bytes / us / 1e3 / wgs))
        print(f"requests {n:4d}  workgroups {wgs:5d}  {us:8.1f} us  {rows[-1][4]:6.2f} TB/s  "
              f"{rows[-1][5]:6.1f} GB/s per workgroup", flush=True)
        del dev, b
        torch.cuda.empty_cache()
    if a.out:
        os.makedirs(a.out, exist_ok=True)
        cmd = "python -m prefill_decode_hybrid_amd.decoderate " + " ".join(argv if argv is not None else sys.argv[1:])
        name = f"decode_rate_c{a.context}_T{a.split}_wg{a.wg_per_cu}" + ("_contiguous" if a.contiguous else "")
        lines = [f"# Decode stream rate against decode workgroups ({a.context}-token contexts, "
                 f"{a.split}-token splits, envelope {a.wg_per_cu} per CU"
                 + (", contiguous pages)" if a.contiguous else ", permuted pages)"), "",
                 "Decode-only launches of N requests, Llama-3-8B heads (32 q / 8 kv, d 128, bf16); each call "
                 "after a 1 GiB cache flush, median of the timed calls.  Bytes are the visible K and V rows.",
                 "", "Command:", "", "```", cmd, "```", "",
                 "| requests | decode workgroups | envelope | us | TB/s | GB/s per workgroup |",
                 "|---|---|---|---|---|---|"]
        for n, wgs, env, us, tbs, gbw in rows:
            lines.append(f"| {n} | {wgs} | {env} | {us:.1f} | {tbs:.2f} | {gbw:.1f} |")
        open(os.path.join(a.out, name + ".md"), "w").write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
