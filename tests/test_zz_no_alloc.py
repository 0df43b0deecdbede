"""pod_attn_hybrid_noalloc: the handle-free variant of pod_attn_hybrid whose
workspace is the library's fixed device scratch.  Through the C ABI, its
outputs must equal pod_attn_hybrid's bit for bit (same kernels, same plan)
and match the fp64 oracle, on two calls in a row where the second batch is
smaller than the first (the scratch keeps what the first call left); a
batch whose workspace exceeds the scratch is refused before anything runs."""
import ctypes

import pytest
import torch

import prefill_decode_hybrid_amd as pod
from prefill_decode_hybrid_amd import inputs
from gpu_helpers import Run, check_against_oracle, say
from parity_cases import spec

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pod.load()


def noalloc(run):
    b = run.dev
    op, od = run.outputs()
    pa, da = run.att.args(b, op, od, run.ctx_host)
    pod.pod_attn_hybrid_noalloc(run.cfg, b.k_pool, b.v_pool, pa, da)
    torch.cuda.synchronize()
    return op, od


@pytest.mark.timeout(600)
def test_noalloc_equals_hybrid_on_two_calls():
    # first the long-context workload (its prefill and decode splits fill
    # tens of MB of the scratch), then a smaller batch with splits of its own
    for label, sp, seed in (("long-context batch", 3, 0),
                            ("small batch", spec("bf16", 8, 2, 128, 64, 12000, [20000, 300, 1]), 5)):
        say(f"noalloc: {label}")
        run = Run(inputs.make_batch(sp, seed=seed))
        try:
            ref_p, ref_d = run.hybrid()
            st = run.att.stats()
            say(f"  plan {st}")
            assert st["prefill_splits"] > 1 or st["decode_wave_tasks"] > 4 * st["decode_wg_tasks"] - 4
            for rep in range(2):
                op, od = noalloc(run)
                assert torch.equal(op, ref_p) and torch.equal(od, ref_d), f"{label} call {rep} differs from pod_attn_hybrid"
            check_against_oracle(run, op, od, label=f"noalloc {label}", step=256)
        finally:
            run.close()


def test_noalloc_refuses_a_batch_beyond_the_scratch():
    # 1024 decodes of 4096 tokens in 256-token splits with 8 query heads per
    # kv head: ~545 MB of decode partials.  Every page id is 0 (a valid page
    # of a two-page pool), so the inputs are small and in bounds.
    N, L, hq, hkv, d = 1024, 4096, 64, 8, 128
    dev = "cuda:0"
    pool = torch.zeros((2, 16, hkv, d), dtype=torch.bfloat16, device=dev)
    q = torch.zeros((N, hq, d), dtype=torch.bfloat16, device=dev)
    o = torch.zeros_like(q)
    pt = torch.zeros((N, L // 16), dtype=torch.int32, device=dev)
    ctx_host = torch.full((N,), L, dtype=torch.int32)
    ctx = ctx_host.to(dev)
    cfg = pod.make_config(num_q_heads=hq, num_kv_heads=hkv, head_dim=d, max_chunk_len=1, max_num_decode=N,
                          max_context=L, decode_split_tokens=256)
    da = pod.decode_args(q, o, pt, ctx, ctx_host)
    rc = pod.load().pod_attn_hybrid_noalloc(ctypes.byref(cfg), pool.data_ptr(), pool.data_ptr(), 2, None,
                                            ctypes.byref(da), None)
    assert rc == pod.POD_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert int(o.abs().sum()) == 0  # nothing ran
