"""Write tests/golden/hybrid_closed_forms.json: a hand-built hybrid batch whose
attention has closed forms, with the fp64 oracle's outputs stored beside the
inputs.  Only the oracle computes the stored values; tests/test_golden.py
checks them against the closed forms and the HIP path against them.

    python tests/golden/make_golden.py

The batch (fp32, 2 query heads sharing 1 kv head, d = 64, pages of 16
tokens, scale 1/8), following the definition of causal chunked-prefill and
decode attention over a paged KV cache ([Paper] §2.1, hybrid batches of one
prefill chunk and several decodes):
  * prefill: 3 rows at offset 2 with q = 0, keys in physical page 1.  Row i
    sees keys 0 .. 2+i, all logits are 0, so it is the mean of n = 3+i value
    rows; value row j is (j+1, (j+1)^2, 0, ...), so the mean is
    ((n+1)/2, (n+1)(2n+1)/6, 0, ...) and lse = ln n;
  * decode 0 (page 0, 2 keys): q = 8 e0, k0 = 0, k1 = e0 -> logits 0 and 1,
    v0 = e0, v1 = e1 -> out = (1/(1+e), e/(1+e), 0, ...), lse = ln(1+e),
    for both heads;
  * decode 1 (page 2, 3 keys, k_j[0] = 0, 1, 0; v_j = (j+1, 10(j+1), 0, ...)):
    head 0 has q = 0 -> mean (2, 20, 0, ...), lse = ln 3; head 1 has
    q = 6400 e0 -> logits 0, 800, 0 -> exactly v1 = (2, 20, 0, ...) (e^-800
    is below the smallest double), lse = 800.
"""
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402

HQ, HKV, D, B, SCALE = 2, 1, 64, 16, 0.125


def inputs():
    k = np.zeros((3, B, HKV, D), np.float32)
    v = np.zeros((3, B, HKV, D), np.float32)
    # page 0: decode 0
    k[0, 1, 0, 0] = 1.0
    v[0, 0, 0, 0] = 1.0
    v[0, 1, 0, 1] = 1.0
    # page 1: the prefill prefix and chunk (keys 0..4); keys are arbitrary, q = 0
    for j in range(5):
        k[1, j, 0, :4] = (j - 2.0, 0.5 * j, 3.0 - j, 1.0)
        v[1, j, 0, 0] = j + 1.0
        v[1, j, 0, 1] = (j + 1.0) ** 2
    # page 2: decode 1
    k[2, 1, 0, 0] = 1.0
    for j in range(3):
        v[2, j, 0, 0] = j + 1.0
        v[2, j, 0, 1] = 10.0 * (j + 1)
    qp = np.zeros((3, HQ, D), np.float32)
    qd = np.zeros((2, HQ, D), np.float32)
    qd[0, :, 0] = 8.0
    qd[1, 1, 0] = 6400.0
    return dict(q_prefill=qp, q_decode=qd, k_pool=k, v_pool=v,
                page_table_prefill=np.array([1], np.int32), chunk_offset=2,
                page_table_decode=np.array([[0], [2]], np.int32),
                context_lens=np.array([2, 3], np.int32))


def main():
    x = inputs()
    op, lp = oracle.prefill(x["q_prefill"], x["k_pool"], x["v_pool"], x["page_table_prefill"],
                            x["chunk_offset"], SCALE, with_lse=True)
    od, ld = oracle.decode(x["q_decode"], x["k_pool"], x["v_pool"], x["page_table_decode"],
                           x["context_lens"], SCALE, with_lse=True)
    nz = lambda a: [[*map(int, idx), float(a[idx])] for idx in zip(*np.nonzero(a))]
    doc = {
        "what": "hybrid batch with closed-form attention; expected values written by make_golden.py from the fp64 oracle",
        "cite": "[Paper] §2.1: causal chunked prefill (row i of a chunk at offset P0 sees keys 0..P0+i) and decode over a paged KV cache in one hybrid batch",
        "num_q_heads": HQ, "num_kv_heads": HKV, "head_dim": D, "page_size": B, "sm_scale": SCALE,
        "num_pages": int(x["k_pool"].shape[0]), "chunk_len": int(x["q_prefill"].shape[0]),
        "chunk_offset": x["chunk_offset"], "num_decode": int(x["q_decode"].shape[0]),
        "page_table_prefill": x["page_table_prefill"].tolist(),
        "page_table_decode": x["page_table_decode"].tolist(),
        "context_lens": x["context_lens"].tolist(),
        "nonzero": {n: nz(x[n]) for n in ("q_prefill", "q_decode", "k_pool", "v_pool")},
        "out_prefill": op.tolist(), "lse_prefill": lp.tolist(),
        "out_decode": od.tolist(), "lse_decode": ld.tolist(),
    }
    with open(os.path.join(HERE, "hybrid_closed_forms.json"), "w") as f:
        json.dump(doc, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
