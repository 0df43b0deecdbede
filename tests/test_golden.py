"""The golden hybrid batch (tests/golden/hybrid_closed_forms.json): a
hand-built batch whose attention has closed forms ([Paper] §2.1: causal
chunked prefill at an offset and decodes over a paged KV cache, with GQA).
Its stored outputs were written by tests/golden/make_golden.py from the fp64
oracle.  The CPU tests pin those values to the closed forms and check that
the oracle still reproduces them; the GPU test runs the fused and the split
launches through the C ABI on the same batch."""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
G = json.load(open(os.path.join(HERE, "golden", "hybrid_closed_forms.json")))


def arrays():
    hq, hkv, d, B = G["num_q_heads"], G["num_kv_heads"], G["head_dim"], G["page_size"]
    x = dict(q_prefill=np.zeros((G["chunk_len"], hq, d), np.float32),
             q_decode=np.zeros((G["num_decode"], hq, d), np.float32),
             k_pool=np.zeros((G["num_pages"], B, hkv, d), np.float32),
             v_pool=np.zeros((G["num_pages"], B, hkv, d), np.float32))
    for name, entries in G["nonzero"].items():
        for *idx, val in entries:
            x[name][tuple(idx)] = val
    return x


def closed_forms():
    """Expected outputs and lse from the batch's construction (see make_golden.py)."""
    hq, d = G["num_q_heads"], G["head_dim"]
    op = np.zeros((G["chunk_len"], hq, d))
    lp = np.zeros((G["chunk_len"], hq))
    for i in range(G["chunk_len"]):
        n = G["chunk_offset"] + i + 1          # visible keys of row i
        op[i, :, 0] = (n + 1) / 2              # mean of 1..n
        op[i, :, 1] = (n + 1) * (2 * n + 1) / 6  # mean of 1..n squared
        lp[i, :] = math.log(n)
    od = np.zeros((G["num_decode"], hq, d))
    ld = np.zeros((G["num_decode"], hq))
    e = math.e
    od[0, :, 0], od[0, :, 1], ld[0, :] = 1 / (1 + e), e / (1 + e), math.log(1 + e)
    od[1, :, 0], od[1, :, 1] = 2.0, 20.0
    ld[1, 0], ld[1, 1] = math.log(3), 800.0
    return op, lp, od, ld


def test_stored_values_are_the_closed_forms():
    op, lp, od, ld = closed_forms()
    np.testing.assert_allclose(np.array(G["out_prefill"]), op, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.array(G["lse_prefill"]), lp, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.array(G["out_decode"]), od, rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.array(G["lse_decode"]), ld, rtol=0, atol=1e-12)


def test_oracle_reproduces_stored_values():
    x = arrays()
    op, lp = oracle.prefill(x["q_prefill"], x["k_pool"], x["v_pool"], np.array(G["page_table_prefill"], np.int32),
                            G["chunk_offset"], G["sm_scale"], with_lse=True)
    od, ld = oracle.decode(x["q_decode"], x["k_pool"], x["v_pool"], np.array(G["page_table_decode"], np.int32),
                           np.array(G["context_lens"], np.int32), G["sm_scale"], with_lse=True)
    for got, key in ((op, "out_prefill"), (lp, "lse_prefill"), (od, "out_decode"), (ld, "lse_decode")):
        np.testing.assert_allclose(got, np.array(G[key]), rtol=0, atol=1e-14)


@pytest.mark.gpu
def test_hip_path_on_golden_batch():
    from gpu_helpers import Run, say
    from prefill_decode_hybrid_amd import inputs
    x = arrays()
    guard = G["num_pages"]
    nan_page = np.full((1,) + x["k_pool"].shape[1:], np.nan, np.float32)  # padding slots must stay unread
    spec = dict(name="golden", dtype="f32", num_q_heads=G["num_q_heads"], num_kv_heads=G["num_kv_heads"],
                head_dim=G["head_dim"])
    batch = inputs.HybridBatch(
        spec=spec, dtype=torch.float32,
        q_prefill=torch.from_numpy(x["q_prefill"]), q_decode=torch.from_numpy(x["q_decode"]),
        k_pool=torch.from_numpy(np.concatenate([x["k_pool"], nan_page])),
        v_pool=torch.from_numpy(np.concatenate([x["v_pool"], nan_page])),
        page_table_prefill=torch.tensor(G["page_table_prefill"], dtype=torch.int32),
        page_table_decode=torch.tensor(G["page_table_decode"], dtype=torch.int32),
        context_lens=torch.tensor(G["context_lens"], dtype=torch.int32),
        chunk_len=G["chunk_len"], chunk_offset=G["chunk_offset"], sm_scale=G["sm_scale"], guard_page=guard)
    say("golden batch: fp32, 2 query heads / 1 kv head, d=64, chunk 3 @ 2, decodes of 2 and 3 keys")
    run = Run(batch)
    try:
        for mode in ("hybrid", "separate"):
            op, od = getattr(run, mode)()
            for got, key in ((op, "out_prefill"), (od, "out_decode")):
                err = np.abs(got.cpu().numpy().astype(np.float64) - np.array(G[key]))
                assert np.isfinite(err).all() and err.max() <= 1e-5, (mode, key, float(np.nanmax(err)))
    finally:
        run.close()
