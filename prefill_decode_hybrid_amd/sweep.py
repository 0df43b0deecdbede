"""Chunk-sequence sweep: one long prompt prefilled chunk by chunk while a
fixed decode batch runs beside every chunk (the kernel-level view of the
paper's chunked-prefill experiments, [Paper] §5.4 Table 8 / Figure 15).

For every chunk i of a `--prompt`-token prompt (chunk length C, offset i*C)
the same hybrid batch shape is timed three ways on one GPU: the fused
launch, the two split launches on one stream, and the split launches on two
streams, interleaved round-robin with an L2/Infinity-Cache flush before each
call.  The prompt's K/V and the decodes' K/V live in one paged pool, so chunk
i reads the first i*C + C keys of the prompt exactly as a serving engine
would.  Each chunk's fused result is also compared bit for bit with the split
launches.

    python -m prefill_decode_hybrid_amd.sweep --prompt 16384 --chunk 512 \\
        --num-decode 64 --decode-context 16384 [--last 4] [--split-cap 0] \\
        [--prefill-splits 0] [--wg-per-cu 2]

Prints one JSON line per run: per-chunk medians and the totals over the
prompt.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import sys
import time


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--prompt", type=int, default=16384, help="prompt tokens prefilled chunk by chunk")
    ap.add_argument("--chunk", type=int, default=512, help="chunk length C")
    ap.add_argument("--num-decode", type=int, default=64)
    ap.add_argument("--decode-context", type=int, default=16384)
    ap.add_argument("--num-q-heads", type=int, default=32)
    ap.add_argument("--num-kv-heads", type=int, default=8)
    ap.add_argument("--head-dim", type=int, default=128)
    ap.add_argument("--last", type=int, default=0, help="time only the last N chunks (0: all)")
    ap.add_argument("--split-cap", type=int, default=0,
                    help="prefill split cap in waves of resident workgroups (0: the default, 2; -1: no cap)")
    ap.add_argument("--prefill-splits", type=int, default=0,
                    help="KV splits per prefill tile (0: the planner's choice)")
    ap.add_argument("--wg-per-cu", type=int, default=2,
                    help="resource envelope: 2 or 4 workgroups per CU, 0 chosen per call (the fused and "
                         "split calls may then pick different envelopes and differ in rounding)")
    ap.add_argument("--policy", type=int, default=0)
    ap.add_argument("--slots-x256", type=int, default=0,
                    help="CU-balanced policy: prefill workgroups per CU in 1/256 (0: the planner's choice)")
    ap.add_argument("--split-tokens", type=int, default=0,
                    help="decode tokens per wave task (0: the planner's choice)")
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--seed", type=int, default=0)
    a = ap.parse_args(argv)
    if a.prompt % a.chunk:
        sys.exit("--prompt must be a multiple of --chunk")

    import torch
    import prefill_decode_hybrid_amd as pod
    from prefill_decode_hybrid_amd import inputs
    from prefill_decode_hybrid_amd.timing import interleaved_us, on_two_streams

    if not torch.cuda.is_available():
        sys.exit("the sweep needs a GPU")
    pod.load()
    spec = dict(name=f"sweep_p{a.prompt}_c{a.chunk}", dtype="bf16", num_q_heads=a.num_q_heads,
                num_kv_heads=a.num_kv_heads, head_dim=a.head_dim, chunk_len=a.prompt, chunk_offset=0,
                decode_lens=[a.decode_context] * a.num_decode, contiguous=False)
    t0 = time.time()
    full = inputs.make_batch(spec, seed=a.seed)
    print(f"[sweep] generated {inputs.describe(full)} in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    dev = full.to("cuda:0")
    ctx_host = full.context_lens.clone().contiguous()
    cfg = pod.config_for_batch(full, policy=a.policy, prefill_split_cap_waves=a.split_cap,
                               prefill_slots_x256=a.slots_x256, decode_split_tokens=a.split_tokens,
                               prefill_splits=a.prefill_splits, wg_per_cu=a.wg_per_cu)
    att = pod.PodAttention(cfg)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    od, od2 = torch.empty_like(dev.q_decode), torch.empty_like(dev.q_decode)

    n_chunks = a.prompt // a.chunk
    first = n_chunks - a.last if a.last else 0
    rows = []
    all_same = True
    for i in range(first, n_chunks):
        p0 = i * a.chunk
        b = dataclasses.replace(dev, q_prefill=dev.q_prefill[p0:p0 + a.chunk], chunk_len=a.chunk, chunk_offset=p0)
        op, op2 = torch.empty_like(b.q_prefill), torch.empty_like(b.q_prefill)

        def fused():
            att.hybrid(b, op, od, ctx_host)

        def serial():
            att.prefill_only(b, op2)
            att.decode_only(b, od2, ctx_host)

        def streams():
            on_two_streams(lambda s: att.prefill_only(b, op2, stream=s),
                           lambda s: att.decode_only(b, od2, ctx_host, stream=s), s1, s2)

        fused()
        plan = att.stats()
        serial()
        torch.cuda.synchronize()
        same = bool(torch.equal(op, op2) and torch.equal(od, od2))
        all_same &= same
        med = interleaved_us((fused, serial, streams), a.steps, a.warmup, flush)
        rows.append({"chunk": i, "offset": p0, "fused_us": round(med[0], 1), "serial_us": round(med[1], 1),
                     "two_stream_us": round(med[2], 1), "prefill_tasks": plan["prefill_tasks"],
                     "prefill_splits": plan["prefill_splits"], "cu_prefill_x256": plan["cu_prefill_x256"],
                     "decode_split_tokens": plan["decode_split_tokens"], "wg_per_cu": plan["wg_per_cu"],
                     "fused_equals_split": same})
        print(f"[sweep] chunk {i} @ {p0}: fused {med[0]:.1f} serial {med[1]:.1f} streams {med[2]:.1f} us "
              f"(splits {plan['prefill_splits']}, x256 {plan['cu_prefill_x256']})", file=sys.stderr, flush=True)
    tot = {k: round(sum(r[k] for r in rows), 1) for k in ("fused_us", "serial_us", "two_stream_us")}
    out = {"sweep": "chunked prefill beside a fixed decode batch", "prompt": a.prompt, "chunk": a.chunk,
           "num_decode": a.num_decode, "decode_context": a.decode_context, "heads": [a.num_q_heads, a.num_kv_heads],
           "head_dim": a.head_dim, "chunks_timed": len(rows), "split_cap_waves": a.split_cap or 2, "prefill_splits": a.prefill_splits,
           "wg_per_cu": a.wg_per_cu,
           "policy": a.policy, "slots_x256": a.slots_x256, "split_tokens": a.split_tokens, "steps": a.steps, "totals": tot,
           "speedup_vs_serial": round(tot["serial_us"] / tot["fused_us"], 4),
           "speedup_vs_two_stream": round(tot["two_stream_us"] / tot["fused_us"], 4),
           "fused_equals_split": all_same, "chunks": rows}
    print(json.dumps(out), flush=True)
    att.close()


if __name__ == "__main__":
    main()
