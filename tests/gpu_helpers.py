"""Shared helpers for the GPU tests: run the three entry points through the C
ABI on a seeded batch and compare with the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import prefill_decode_hybrid_amd as pod
from prefill_decode_hybrid_amd import inputs

TOL = {"bf16": dict(max=2e-2, mean=2e-3), "f32": dict(max=1e-4, mean=1e-5)}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class Run:
    """A batch on cuda:0 plus a handle sized for it."""

    def __init__(self, batch, **cfg_kw):
        # one resource envelope for every entry point unless a test asks
        # otherwise, so that fused and split launches run the same tiles
        cfg_kw.setdefault("wg_per_cu", 2)
        self.cpu = batch
        self.dev = batch.to("cuda:0")
        self.cfg = pod.config_for_batch(batch, **cfg_kw)
        self.att = pod.PodAttention(self.cfg)
        self.ctx_host = None if batch.context_lens is None else batch.context_lens.clone().contiguous()

    def outputs(self):
        b = self.dev
        op = None if b.q_prefill is None else torch.full_like(b.q_prefill, float("nan"))
        od = None if b.q_decode is None else torch.full_like(b.q_decode, float("nan"))
        return op, od

    def hybrid(self):
        op, od = self.outputs()
        self.att.hybrid(self.dev, op, od, self.ctx_host)
        torch.cuda.synchronize()
        return op, od

    def separate(self):
        op, od = self.outputs()
        if op is not None:
            self.att.prefill_only(self.dev, op)
        if od is not None:
            self.att.decode_only(self.dev, od, self.ctx_host)
        torch.cuda.synchronize()
        return op, od

    def close(self):
        self.att.close()


def errors(got, ref):
    g = got.detach().float().cpu().numpy().astype(np.float64)
    d = np.abs(g - ref)
    return float(np.max(d)) if d.size else 0.0, float(np.mean(d)) if d.size else 0.0, bool(np.isfinite(g).all())


def _oracle_errors(got, ref_fn, idx, step, label, what):
    """Max and mean |got - oracle| over the rows idx (all rows if None),
    computing the oracle `step` rows at a time with a progress line each."""
    n = got.shape[0] if idx is None else len(idx)
    picks = list(range(got.shape[0])) if idx is None else list(idx)
    mx, tot, cnt, fin = 0.0, 0.0, 0, True
    for a in range(0, n, step):
        part = picks[a:a + step]
        ref = ref_fn(part)
        g = got[torch.as_tensor(part, device=got.device)]
        m, mean, f = errors(g, ref)
        mx, tot, cnt, fin = max(mx, m), tot + mean * ref.size, cnt + ref.size, fin and f
        if n > step:
            say(f"    {label} {what}: rows {a + len(part)}/{n} max so far {mx:.2e}")
    return mx, (tot / cnt if cnt else 0.0), fin


def check_against_oracle(run: Run, op, od, rows=None, reqs=None, label="", step=None):
    """Compare the outputs with the fp64 oracle on rows / reqs (all if None).
    step: compute the oracle that many rows (requests) at a time, printing
    progress (for batches whose oracle takes minutes)."""
    b = run.cpu
    tol = TOL[b.spec["dtype"]]
    report = {}
    if op is not None:
        ref_fn = lambda part: oracle.prefill(b.q_prefill, b.k_pool, b.v_pool, b.page_table_prefill,
                                             b.chunk_offset, b.sm_scale, rows=part)
        mx, mn, fin = _oracle_errors(op, ref_fn, rows, step or op.shape[0], label, "prefill")
        report["prefill"] = (mx, mn)
        assert fin, f"{label}: non-finite prefill output"
        assert mx <= tol["max"] and mn <= tol["mean"], f"{label}: prefill max {mx:.3e} mean {mn:.3e}"
    if od is not None:
        ref_fn = lambda part: oracle.decode(b.q_decode, b.k_pool, b.v_pool, b.page_table_decode,
                                            b.context_lens, b.sm_scale, reqs=part)
        mx, mn, fin = _oracle_errors(od, ref_fn, reqs, step or od.shape[0], label, "decode")
        report["decode"] = (mx, mn)
        assert fin, f"{label}: non-finite decode output"
        assert mx <= tol["max"] and mn <= tol["mean"], f"{label}: decode max {mx:.3e} mean {mn:.3e}"
    say(f"  {label}: " + ", ".join(f"{k} max {v[0]:.2e} mean {v[1]:.2e}" for k, v in report.items()))
    return report


def sample_rows(C, rows_per_tile=32, n_random=16, seed=0):
    """Rows at tile edges, the first and last rows, and a few random ones."""
    rng = np.random.default_rng(seed)
    edge = {0, 1, C - 1, C - 2}
    for t in range(0, C, rows_per_tile):
        edge |= {t, min(C - 1, t + rows_per_tile - 1)}
    picks = set(rng.choice(C, size=min(C, n_random), replace=False).tolist())
    return sorted(r for r in edge | picks if 0 <= r < C)


def sample_reqs(lens, n_random=6, seed=0):
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens)
    pick = {int(np.argmin(lens)), int(np.argmax(lens)), 0, len(lens) - 1}
    pick |= set(rng.choice(len(lens), size=min(len(lens), n_random), replace=False).tolist())
    return sorted(pick)
