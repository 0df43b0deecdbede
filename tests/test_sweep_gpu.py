"""The chunk-sequence sweep: one prompt prefilled chunk by chunk beside a
fixed decode batch, every chunk a view into one paged pool.  Each chunk's
fused result is compared with the fp64 oracle (the oracle reads the same
prompt pages with the chunk's offset) and with the split launches."""
import dataclasses
import io
import json
from contextlib import redirect_stdout

import numpy as np
import pytest
import torch

import oracle
import prefill_decode_hybrid_amd as pod
from prefill_decode_hybrid_amd import inputs, sweep
from gpu_helpers import TOL, errors, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pod.load()


def test_chunks_of_one_prompt_match_oracle():
    prompt, C = 1000, 256  # ragged last chunk handled by the caller: 3 full chunks + 232 rows
    spec = dict(name="sweep_small", dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=128, chunk_len=prompt,
                chunk_offset=0, decode_lens=[700, 1500, 33], contiguous=False)
    full = inputs.make_batch(spec, seed=5)
    dev = full.to("cuda:0")
    ctx = full.context_lens.clone().contiguous()
    att = pod.PodAttention(pod.config_for_batch(full, wg_per_cu=2))
    try:
        for p0 in range(0, prompt, C):
            n = min(C, prompt - p0)
            say(f"chunk @ {p0} x {n}")
            b = dataclasses.replace(dev, q_prefill=dev.q_prefill[p0:p0 + n], chunk_len=n, chunk_offset=p0)
            op, od = torch.empty_like(b.q_prefill), torch.empty_like(b.q_decode)
            att.hybrid(b, op, od, ctx)
            op2, od2 = torch.empty_like(op), torch.empty_like(od)
            att.prefill_only(b, op2)
            att.decode_only(b, od2, ctx)
            torch.cuda.synchronize()
            assert torch.equal(op, op2) and torch.equal(od, od2)
            ref = oracle.prefill(full.q_prefill[p0:p0 + n], full.k_pool, full.v_pool, full.page_table_prefill, p0,
                                 full.sm_scale)
            mx, mn, fin = errors(op, ref)
            assert fin and mx <= TOL["bf16"]["max"] and mn <= TOL["bf16"]["mean"], (p0, mx, mn)
        refd = oracle.decode(full.q_decode, full.k_pool, full.v_pool, full.page_table_decode, full.context_lens,
                             full.sm_scale)
        mx, mn, fin = errors(od, refd)
        assert fin and mx <= TOL["bf16"]["max"] and mn <= TOL["bf16"]["mean"]
    finally:
        att.close()


def test_sweep_cli_small():
    buf = io.StringIO()
    with redirect_stdout(buf):
        sweep.main(["--prompt", "1024", "--chunk", "512", "--num-decode", "4", "--decode-context", "2048",
                    "--steps", "2", "--warmup", "1"])
    out = json.loads(buf.getvalue().strip().splitlines()[-1])
    assert out["chunks_timed"] == 2 and out["fused_equals_split"]
    assert all(r["fused_us"] > 0 and r["serial_us"] > 0 for r in out["chunks"])
