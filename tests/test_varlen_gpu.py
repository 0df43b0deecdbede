"""Several prefill chunks in one call (pod_attn_hybrid_varlen and
pod_attn_prefill_only_varlen) against the fp64 oracle, chunk by chunk.

Each chunk is its own request: the oracle's prefill definition applied to
that chunk's rows, its own page-table row and its own offset.  Bars as for
one chunk (bf16: max |err| <= 2e-2, mean <= 2e-3; fp32: max <= 1e-4).  The
fused call must equal the split calls bit for bit, and a one-chunk varlen
call must equal the single-chunk entry point bit for bit."""
import dataclasses
import io
import json
from contextlib import redirect_stdout

import numpy as np
import pytest
import torch

import oracle
import prefill_decode_hybrid_amd as pod
from prefill_decode_hybrid_amd import inputs, multichunk
from gpu_helpers import TOL, errors, sample_reqs, sample_rows, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pod.load()


def vspec(dtype, hq, hkv, d, chunks, lens):
    tag = "_".join(f"{c}@{p}" for c, p in chunks[:4]) + ("_..." if len(chunks) > 4 else "")
    return dict(name=f"{dtype}_h{hq}x{hkv}_d{d}_n{len(chunks)}_{tag}", dtype=dtype, num_q_heads=hq,
                num_kv_heads=hkv, head_dim=d, chunk_len=0, chunk_offset=0, chunks=list(chunks),
                decode_lens=list(lens), contiguous=False)


CASES = [
    vspec("bf16", 8, 2, 128, [(77, 300), (5, 0), (130, 2000), (33, 33)], [17, 1500, 300]),
    vspec("bf16", 32, 8, 128, [(64, 15000), (200, 4000), (96, 0)], [16384, 3000, 100]),
    vspec("bf16", 8, 4, 64, [(1, 0), (1, 9), (1, 4000), (40, 7)], [33]),
    vspec("bf16", 16, 2, 128, [(16 + i, 97 * i) for i in range(16)], [900, 2]),
    vspec("bf16", 8, 8, 128, [(300, 20000), (31, 0)], [5, 40000]),
    vspec("f32", 8, 2, 64, [(100, 29), (3, 3000), (64, 0)], [3, 999]),
    # the chunk limit: 64 single-row chunks
    vspec("bf16", 8, 2, 128, [(1, 100 * i) for i in range(64)], [77]),
    # multi-token decode queries (3 new tokens each, contexts 1-16K) passed as chunks
    # of 3 rows at offset L - 3, beside one prompt chunk and single-token decodes
    vspec("bf16", 32, 8, 128, [(256, 0)] + [(3, 1000 + (997 * i) % 15000 - 3) for i in range(47)],
          [16384, 4096, 9]),
]


def oracle_chunks(b, rows_per_chunk=None):
    """The oracle's prefill per chunk; rows_per_chunk: chunk-local rows to compute (None: all)."""
    outs, r = [], 0
    for i, (c, p) in enumerate(b.chunk_list()):
        n = -(-(c + p) // 16)
        rows = None if rows_per_chunk is None else rows_per_chunk[i]
        outs.append(oracle.prefill(b.q_prefill[r:r + c], b.k_pool, b.v_pool, b.page_table_prefill[i, :n], p,
                                   b.sm_scale, rows=rows))
        r += c
    return np.concatenate(outs)


def check(b, op, od, label, rows_per_chunk=None, reqs=None):
    tol = TOL[b.spec["dtype"]]
    ref = oracle_chunks(b, rows_per_chunk)
    if rows_per_chunk is None:
        got = op
    else:
        starts = np.cumsum([0] + [c for c, _ in b.chunk_list()])[:-1]
        idx = np.concatenate([s + np.asarray(r, dtype=np.int64) for s, r in zip(starts, rows_per_chunk)])
        got = op[torch.as_tensor(idx, device=op.device)]
    mx, mn, fin = errors(got, ref)
    assert fin and mx <= tol["max"] and mn <= tol["mean"], f"{label}: prefill max {mx:.3e} mean {mn:.3e}"
    refd = oracle.decode(b.q_decode, b.k_pool, b.v_pool, b.page_table_decode, b.context_lens, b.sm_scale, reqs=reqs)
    gotd = od if reqs is None else od[torch.as_tensor(reqs, device=od.device)]
    mxd, mnd, find = errors(gotd, refd)
    assert find and mxd <= tol["max"] and mnd <= tol["mean"], f"{label}: decode max {mxd:.3e} mean {mnd:.3e}"
    say(f"  {label}: prefill max {mx:.2e} mean {mn:.2e}, decode max {mxd:.2e} mean {mnd:.2e}")


@pytest.mark.parametrize("sp", CASES, ids=lambda s: s["name"])
def test_varlen_matches_oracle(sp):
    say(f"case {sp['name']}")
    b = inputs.make_batch(sp, seed=2)
    dev = b.to("cuda:0")
    ctx = b.context_lens.clone().contiguous()
    att = pod.PodAttention(pod.config_for_batch(b, wg_per_cu=2))
    try:
        op = torch.full_like(dev.q_prefill, float("nan"))
        od = torch.full_like(dev.q_decode, float("nan"))
        att.hybrid_varlen(dev, op, od, ctx)
        torch.cuda.synchronize()
        st = att.stats()
        assert st["prefill_chunks"] == len(sp["chunks"]) and st["mode"] == 0
        check(b, op, od, "hybrid_varlen")
        op2, od2 = torch.full_like(op, float("nan")), torch.full_like(od, float("nan"))
        att.prefill_only_varlen(dev, op2)
        att.decode_only(dev, od2, ctx)
        torch.cuda.synchronize()
        assert torch.equal(op, op2) and torch.equal(od, od2), "fused result differs from split launches"
    finally:
        att.close()


@pytest.mark.parametrize("policy", [pod.POD_POLICY_PROPORTIONAL, pod.POD_POLICY_HALF, pod.POD_POLICY_STATIC])
def test_varlen_policies_bitwise(policy):
    sp = CASES[1]
    b = inputs.make_batch(sp, seed=4)
    dev = b.to("cuda:0")
    ctx = b.context_lens.clone().contiguous()
    outs = []
    for pol in (pod.POD_POLICY_CU_BALANCED, policy):
        att = pod.PodAttention(pod.config_for_batch(b, policy=pol, wg_per_cu=2))
        try:
            op, od = torch.empty_like(dev.q_prefill), torch.empty_like(dev.q_decode)
            att.hybrid_varlen(dev, op, od, ctx)
            torch.cuda.synchronize()
            outs.append((op, od))
        finally:
            att.close()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


def test_one_chunk_varlen_equals_single_chunk_call():
    sp = dict(name="one", dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128, chunk_len=300,
              chunk_offset=5000, decode_lens=[4000, 17, 9000], contiguous=False)
    b = inputs.make_batch(sp, seed=6)
    dev = b.to("cuda:0")
    ctx = b.context_lens.clone().contiguous()
    att = pod.PodAttention(pod.config_for_batch(b, wg_per_cu=2))
    try:
        op, od = torch.empty_like(dev.q_prefill), torch.empty_like(dev.q_decode)
        att.hybrid(dev, op, od, ctx)
        v = dataclasses.replace(dev, page_table_prefill=dev.page_table_prefill[None, :].contiguous(),
                                chunks=[(300, 5000)])
        op2, od2 = torch.empty_like(op), torch.empty_like(od)
        att.hybrid_varlen(v, op2, od2, ctx)
        torch.cuda.synchronize()
        assert torch.equal(op, op2) and torch.equal(od, od2)
    finally:
        att.close()


def test_four_prompts_beside_long_decodes():
    # four 512-token chunks of four prompts (offsets 0..12K) beside 32 decodes of 8K,
    # Llama-3-8B heads; sampled rows of every chunk and sampled requests
    chunks = [(512, 0), (512, 4096), (512, 8192), (512, 12288)]
    sp = vspec("bf16", 32, 8, 128, chunks, [8192] * 32)
    b = inputs.make_batch(sp, seed=7)
    dev = b.to("cuda:0")
    ctx = b.context_lens.clone().contiguous()
    att = pod.PodAttention(pod.config_for_batch(b, wg_per_cu=2))
    try:
        op, od = torch.full_like(dev.q_prefill, float("nan")), torch.full_like(dev.q_decode, float("nan"))
        say("four prompts: hybrid_varlen")
        att.hybrid_varlen(dev, op, od, ctx)
        torch.cuda.synchronize()
        assert torch.isfinite(op.float()).all() and torch.isfinite(od.float()).all()
        rows = [sample_rows(c, n_random=8, seed=i) for i, (c, _) in enumerate(chunks)]
        check(b, op, od, "four prompts", rows_per_chunk=rows, reqs=sample_reqs(b.context_lens.tolist()))
    finally:
        att.close()


def test_multichunk_cli_small():
    buf = io.StringIO()
    with redirect_stdout(buf):
        multichunk.main(["--chunks", "100@0,64@900,7@3", "--num-decode", "4", "--decode-context", "2048",
                         "--steps", "2", "--warmup", "1"])
    out = json.loads(buf.getvalue().strip().splitlines()[-1])
    assert out["fused_equals_split"] and out["plan"]["prefill_chunks"] == 3
    assert out["fused_us"] > 0 and out["serial_us"] > 0 and out["two_stream_us"] > 0
