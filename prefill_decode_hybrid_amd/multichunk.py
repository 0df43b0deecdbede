"""Several prefill chunks beside a decode batch, timed three ways on one GPU.

A serving step may carry chunks of several prompts at once; the pages'
hybrid batch commonly holds one ([Paper] §2.1).  The batch here packs
`--chunks` (length@offset, one prompt each) with `--num-decode` decodes of
`--decode-context` tokens and times one fused varlen launch
(pod_attn_hybrid_varlen), the split launches on one stream
(pod_attn_prefill_only_varlen then pod_attn_decode_only) and the split
launches on two streams, interleaved with a cache flush before each call.
The fused result is also compared bit for bit with the split launches.

    python -m prefill_decode_hybrid_amd.multichunk \\
        --chunks 512@0,512@4096,512@8192,512@12288 --num-decode 64 --decode-context 16384

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import sys

PEAK_BF16_FLOPS = 2.5166e15  # MI355X dense bf16 MFMA
PEAK_F32_FLOPS = 157.3e12
PEAK_HBM = 8.0e12


def parse_chunks(text):
    out = []
    for item in text.split(","):
        c, _, p = item.partition("@")
        out.append((int(c), int(p or 0)))
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--chunks", default="512@0,512@4096,512@8192,512@12288",
                    help="comma-separated length@offset, one prompt each")
    ap.add_argument("--num-decode", type=int, default=64)
    ap.add_argument("--decode-context", type=int, default=16384)
    ap.add_argument("--num-q-heads", type=int, default=32)
    ap.add_argument("--num-kv-heads", type=int, default=8)
    ap.add_argument("--head-dim", type=int, default=128)
    ap.add_argument("--policy", type=int, default=0)
    ap.add_argument("--slots-x256", type=int, default=0,
                    help="CU-balanced policy: prefill workgroups per CU in 1/256 (0: the planner's choice)")
    ap.add_argument("--wg-per-cu", type=int, default=2,
                    help="resource envelope: 2 or 4 workgroups per CU, 0 chosen per call")
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    a = ap.parse_args(argv)
    chunks = parse_chunks(a.chunks)

    import torch
    import prefill_decode_hybrid_amd as pod
    from prefill_decode_hybrid_amd import inputs
    from prefill_decode_hybrid_amd.timing import interleaved_us, on_two_streams

    if not torch.cuda.is_available():
        sys.exit("the multi-chunk timing needs a GPU")
    pod.load()
    spec = dict(name=f"multichunk_{len(chunks)}", dtype="bf16", num_q_heads=a.num_q_heads,
                num_kv_heads=a.num_kv_heads, head_dim=a.head_dim, chunk_len=0, chunk_offset=0, chunks=chunks,
                decode_lens=[a.decode_context] * a.num_decode, contiguous=False)
    b = inputs.make_batch(spec, seed=a.seed)
    dev = b.to("cuda:0")
    ctx = b.context_lens.clone().contiguous()
    att = pod.PodAttention(pod.config_for_batch(b, policy=a.policy, prefill_slots_x256=a.slots_x256,
                                                wg_per_cu=a.wg_per_cu))
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    op, od = torch.empty_like(dev.q_prefill), torch.empty_like(dev.q_decode)
    op2, od2 = torch.empty_like(op), torch.empty_like(od)

    def fused():
        att.hybrid_varlen(dev, op, od, ctx)

    def serial():
        att.prefill_only_varlen(dev, op2)
        att.decode_only(dev, od2, ctx)

    def streams():
        on_two_streams(lambda s: att.prefill_only_varlen(dev, op2, stream=s),
                       lambda s: att.decode_only(dev, od2, ctx, stream=s), s1, s2)

    fused()
    plan = att.stats()
    serial()
    torch.cuda.synchronize()
    same = bool(torch.equal(op, op2) and torch.equal(od, od2))
    t_f, t_s, t_2 = interleaved_us((fused, serial, streams), a.steps, a.warmup, flush)

    hq, hkv, d = a.num_q_heads, a.num_kv_heads, a.head_dim
    flops = 4.0 * d * hq * (b.visible_keys_prefill() + sum(int(x) for x in b.context_lens))
    nbytes = 2.0 * hkv * d * 2 * b.kv_tokens() + 2.0 * (b.chunk_len + a.num_decode) * hq * d * 2
    t_roof = max(flops / PEAK_BF16_FLOPS, nbytes / PEAK_HBM) * 1e6
    out = {"batch": "several prefill chunks beside a decode batch", "chunks": chunks,
           "num_decode": a.num_decode, "decode_context": a.decode_context, "heads": [hq, hkv], "head_dim": d,
           "policy": a.policy, "slots_x256": a.slots_x256, "steps": a.steps, "fused_us": round(t_f, 1), "serial_us": round(t_s, 1),
           "two_stream_us": round(t_2, 1), "speedup_vs_serial": round(t_s / t_f, 4),
           "speedup_vs_two_stream": round(t_2 / t_f, 4),
           "overlap_roofline": {"t_roof_us": round(t_roof, 1), "frac": round(t_roof / t_f, 4),
                                "flops": flops, "bytes": nbytes},
           "fused_equals_split": same,
           "plan": {k: plan[k] for k in ("prefill_chunks", "prefill_tiles", "prefill_tasks", "decode_split_tokens",
                                         "decode_wg_tasks", "cu_prefill_x256", "grid")}}
    print(json.dumps(out), flush=True)
    att.close()


if __name__ == "__main__":
    main()
