"""The realised role mix of a fused launch, from its task records
(pod_attn_role_trace): which compute unit ran each prefill and decode task,
and when.

The method's claim is about placement: every compute unit should run
prefill and decode work side by side (paper §4.1, SM-aware CTA scheduling;
the Silicon & Systems digest asks the runtime to report the virtual-CTA mix
it achieved).  From the records this module reports, per role, the tasks and
the CUs they ran on, per XCD the task counts, the mean number of prefill and
decode workgroups resident per CU over the launch (to set beside the plan's
prefill slots per CU), the share of CU-busy time during which a CU ran
both roles at once, and a timeline of running workgroups with the decode's
approximate stream rate (each decode task's K/V bytes spread evenly over
its own start-to-end time).

    python -m prefill_decode_hybrid_amd.roletrace --config 3 [--wg-per-cu 2] [--buckets 20] [--out profiles]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
from collections import defaultdict

TICK_US = 0.01  # the real-time counter runs at 100 MHz


def xcd_of(key: int) -> int:
    return (key >> 8) & 7


def unit_tokens(lens, T: int, T2: int = 0, k: int = 0) -> list:
    """Keys of every decode unit in the order a fused launch numbers them:
    each request's long splits of T keys (request by request), then its
    tail: with k = 0 the remainder as one unit, with k = 1 the last full
    split and the remainder in units of T2 keys (request by request)."""
    longs, tails = [], []
    for L in (int(x) for x in lens):
        F = L // T
        a = F - k if F > k else 0
        longs += [T] * a
        tail = L - a * T
        if k == 0:
            if tail > 0:
                tails.append(tail)
        else:
            while tail > 0:
                tails.append(min(T2, tail))
                tail -= T2
    return longs + tails


def decode_task_bytes(lens, T: int, T2: int, hkv: int, head_dim: int, elem_bytes: int,
                      waves_per_wg: int = 4) -> list:
    """K and V bytes each decode workgroup task of a fused launch streams:
    wave task w is (unit w // hkv, kv head w % hkv), a workgroup task runs
    waves_per_wg consecutive wave tasks."""
    units = unit_tokens(lens, T, T2, 1 if T2 else 0)
    row = 2 * head_dim * elem_bytes  # one key's K and V row of one kv head
    n_wave = len(units) * hkv
    out = []
    for t in range((n_wave + waves_per_wg - 1) // waves_per_wg):
        out.append(sum(units[w // hkv] * row for w in range(t * waves_per_wg, min(n_wave, (t + 1) * waves_per_wg))))
    return out


def summarize(records, num_cus: int = 256, buckets: int = 10, decode_bytes=None) -> dict:
    """records: iterable of (cu_key, role, task, start, end); decode_bytes:
    K/V bytes of each decode workgroup task, for the timeline's stream rate."""
    recs = [tuple(int(x) for x in r) for r in records]
    if not recs:
        return {"tasks": 0}
    t_lo = min(r[3] for r in recs)
    t_hi = max(r[4] for r in recs)
    span = max(1, t_hi - t_lo)
    by_cu = defaultdict(list)
    per_role = {0: 0, 1: 0}
    cus_role = {0: set(), 1: set()}
    per_xcd = defaultdict(lambda: [0, 0])
    busy_role = {0: 0, 1: 0}
    for key, role, task, t0, t1 in recs:
        by_cu[key].append((t0, t1, role))
        per_role[role] += 1
        cus_role[role].add(key)
        per_xcd[xcd_of(key)][role] += 1
        busy_role[role] += max(0, t1 - t0)
    both_time = any_time = 0
    for key, iv in by_cu.items():
        events = []
        for t0, t1, role in iv:
            events.append((t0, 1, role))
            events.append((t1, -1, role))
        events.sort(key=lambda e: (e[0], e[1]))  # ends before starts at equal times
        n = [0, 0]
        last = events[0][0]
        for t, d, role in events:
            if t > last:
                if n[0] > 0 and n[1] > 0:
                    both_time += t - last
                if n[0] + n[1] > 0:
                    any_time += t - last
                last = t
            n[role] += d
    # mean running workgroups per CU of each role in equal time buckets, and
    # the decode's bytes per bucket (each task's spread over its own time)
    nb = max(1, int(buckets))
    tl = [[0, 0] for _ in range(nb)]
    db = [0.0] * nb
    width = span / nb
    for key, role, task, t0, t1 in recs:
        for k in range(nb):
            lo, hi = t_lo + k * width, t_lo + (k + 1) * width
            ov = min(t1, hi) - max(t0, lo)
            if ov > 0:
                tl[k][role] += ov
                if role == 1 and decode_bytes is not None and t1 > t0:
                    db[k] += decode_bytes[task] * ov / (t1 - t0)
    timeline = []
    for k, (a, b) in enumerate(tl):
        e = {"prefill": round(a / (num_cus * width), 3), "decode": round(b / (num_cus * width), 3)}
        if decode_bytes is not None:
            e["decode_tb_s"] = round(db[k] / (width * TICK_US * 1e-6) / 1e12, 2)
        timeline.append(e)
    return {
        "tasks": len(recs),
        "span_us": round(span * TICK_US, 1),
        "prefill_tasks": per_role[0], "decode_tasks": per_role[1],
        "cus_running_prefill": len(cus_role[0]), "cus_running_decode": len(cus_role[1]),
        "cus_running_both": len(cus_role[0] & cus_role[1]), "cus_seen": len(by_cu),
        "mean_prefill_wgs_per_cu": round(busy_role[0] / (num_cus * span), 3),
        "mean_decode_wgs_per_cu": round(busy_role[1] / (num_cus * span), 3),
        "share_of_cu_busy_time_with_both_roles": round(both_time / any_time, 4) if any_time else 0.0,
        "tasks_per_xcd": {str(x): {"prefill": v[0], "decode": v[1]} for x, v in sorted(per_xcd.items())},
        "timeline_wgs_per_cu": timeline,
    }


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--wg-per-cu", type=int, default=2)
    ap.add_argument("--policy", type=int, default=0)
    ap.add_argument("--slots-x256", type=int, default=0)
    ap.add_argument("--decode-split-tokens", type=int, default=0)
    ap.add_argument("--prefill-splits", type=int, default=0)
    ap.add_argument("--decode-tail-split-tokens", type=int, default=0)
    ap.add_argument("--buckets", type=int, default=10, help="time buckets of the timeline")
    ap.add_argument("--tag", default="", help="suffix of the output file name")
    ap.add_argument("--out", default="", help="write role_mix_<workload>[_<tag>].md here")
    a = ap.parse_args(argv)

    import torch
    import prefill_decode_hybrid_amd as pod
    from prefill_decode_hybrid_amd import inputs

    if not torch.cuda.is_available():
        sys.exit("the role trace needs a GPU")
    pod.load()
    b = inputs.make_batch(a.config, seed=a.seed)
    dev = b.to("cuda:0")
    ctx = b.context_lens.clone().contiguous()
    att = pod.PodAttention(pod.config_for_batch(b, wg_per_cu=a.wg_per_cu, policy=a.policy,
                                                prefill_slots_x256=a.slots_x256, record_roles=1,
                                                decode_split_tokens=a.decode_split_tokens,
                                                decode_tail_split_tokens=a.decode_tail_split_tokens,
                                                prefill_splits=a.prefill_splits))
    op, od = torch.empty_like(dev.q_prefill), torch.empty_like(dev.q_decode)
    # as in the benchmark: the L2s and the Infinity Cache are flushed (1 GiB
    # written) before every call, so the recorded call reads its K/V from HBM
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    for _ in range(3):
        flush.zero_()
        att.hybrid(dev, op, od, ctx)
    torch.cuda.synchronize()
    plan = att.stats()
    dbytes = decode_task_bytes(b.context_lens.tolist(), plan["decode_split_tokens"],
                               plan["decode_tail_split_tokens"], b.num_kv_heads, b.head_dim,
                               2 if b.spec["dtype"] == "bf16" else 4)
    assert len(dbytes) == plan["decode_wg_tasks"], "decode task numbering differs from the plan"
    s = summarize(att.role_trace(), plan["num_cus"], a.buckets, dbytes)
    att.close()
    workload = f"config{a.config}_{b.spec['name']}"
    # the role rule the launch ran (the planner may take another rule than the
    # configured CU-balanced one; the stats report it)
    pol = plan["policy"]
    pol_text = f"policy {pol}" + (f" (configured {a.policy})" if pol != a.policy else "")
    out = {"workload": workload, "wg_per_cu": plan["wg_per_cu"], "policy": pol, "configured_policy": a.policy,
           "planned_prefill_slots_per_cu": plan["cu_prefill_x256"] / 256, "fixed_order": plan["fixed_order"],
           "grid": plan["grid"], "summary": s}
    print(json.dumps(out), flush=True)
    if a.out:
        os.makedirs(a.out, exist_ok=True)
        cmd = "python -m prefill_decode_hybrid_amd.roletrace " + " ".join(argv if argv is not None else sys.argv[1:])
        lines = [f"# Realised role mix: {workload}", "", "Command:", "", "```", cmd, "```", "",
                 f"Plan: {plan['wg_per_cu']} workgroups per CU, {plan['grid']} workgroups, "
                 f"{plan['prefill_tasks']} prefill tasks, {plan['decode_wg_tasks']} decode workgroup tasks, "
                 f"planned prefill slots per CU {plan['cu_prefill_x256'] / 256:.3f}, {pol_text}, "
                 f"roles {'by workgroup id' if plan['fixed_order'] else 'claimed after dispatch'}.", "",
                 "| quantity | value |", "|---|---|"]
        for k, v in s.items():
            if k not in ("tasks_per_xcd", "timeline_wgs_per_cu"):
                lines.append(f"| {k} | {v} |")
        lines += ["", "| XCD | prefill tasks | decode tasks |", "|---|---|---|"]
        for x, v in s["tasks_per_xcd"].items():
            lines.append(f"| {x} | {v['prefill']} | {v['decode']} |")
        width = s["span_us"] / a.buckets
        lines += ["", f"Running workgroups per CU over the launch in {a.buckets} equal parts of its span "
                  f"({width:.1f} us each), and the decode's stream rate (each decode task's K/V bytes "
                  "spread evenly over its own start-to-end time, so an approximation):", "",
                  "| part | from us | prefill | decode | idle slots | decode TB/s |", "|---|---|---|---|---|---|"]
        for k, v in enumerate(s["timeline_wgs_per_cu"]):
            lines.append(f"| {k + 1} | {k * width:.0f} | {v['prefill']} | {v['decode']} | "
                         f"{round(plan['wg_per_cu'] - v['prefill'] - v['decode'], 3)} | {v.get('decode_tb_s', '')} |")
        name = f"role_mix_{workload}" + (f"_{a.tag}" if a.tag else "")
        open(os.path.join(a.out, name + ".md"), "w").write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
