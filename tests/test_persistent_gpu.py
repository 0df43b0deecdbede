"""The persistent fused launch (config persistent = 1): a resident grid of
workgroups that loops over the task queues.  It runs the same tasks and
merges as the one-workgroup-per-task launch, so its outputs must be bitwise
equal to that launch's (and within the oracle tolerance), under every role
policy, with one or several prefill chunks."""
import pytest
import torch

import prefill_decode_hybrid_amd as pod
from prefill_decode_hybrid_amd import inputs
from gpu_helpers import Run, check_against_oracle, sample_reqs, sample_rows, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pod.load()


def spec(dtype, hq, hkv, d, C, P0, lens):
    return dict(name=f"{dtype}_h{hq}x{hkv}_d{d}_C{C}_P{P0}", dtype=dtype, num_q_heads=hq, num_kv_heads=hkv,
                head_dim=d, chunk_len=C, chunk_offset=P0, decode_lens=list(lens), contiguous=False)


CASES = [
    spec("bf16", 8, 2, 128, 77, 300, [1, 15, 300, 1025, 2100]),
    spec("bf16", 8, 2, 128, 64, 12000, [20000, 33]),
    spec("bf16", 16, 2, 64, 130, 17, [33, 700]),
    spec("bf16", 64, 8, 128, 200, 9000, [5000, 17, 9000]),
    spec("f32", 8, 2, 64, 100, 29, [3, 999]),
]


def _hybrid(run, att):
    op, od = run.outputs()
    att.hybrid(run.dev, op, od, run.ctx_host)
    torch.cuda.synchronize()
    return op, od


@pytest.mark.parametrize("sp", CASES, ids=lambda s: s["name"])
def test_persistent_equals_per_task_launch(sp):
    say(f"case {sp['name']}")
    run = Run(inputs.make_batch(sp, seed=3))
    pers = pod.PodAttention(pod.config_for_batch(run.cpu, persistent=1))
    try:
        ref = run.hybrid()
        for pol in (pod.POD_POLICY_CU_BALANCED, pod.POD_POLICY_PROPORTIONAL, pod.POD_POLICY_HALF,
                    pod.POD_POLICY_STATIC):
            att = pod.PodAttention(pod.config_for_batch(run.cpu, persistent=1, policy=pol))
            try:
                op, od = _hybrid(run, att)
                st = att.stats()
                assert st["persistent"] == 1 and st["grid"] <= 256 * 2 and st["policy"] == pol
                assert torch.equal(op, ref[0]) and torch.equal(od, ref[1]), f"policy {pol}"
            finally:
                att.close()
        op, od = _hybrid(run, pers)
        check_against_oracle(run, op, od, label="persistent")
        op2, od2 = _hybrid(run, pers)  # the next launch runs on the other control block
        assert torch.equal(op, op2) and torch.equal(od, od2)
    finally:
        pers.close()
        run.close()


def test_persistent_long_context_batch():
    b = inputs.make_batch(3, seed=0)
    run = Run(b)
    pers = pod.PodAttention(pod.config_for_batch(b, persistent=1))
    try:
        say("config 3 persistent")
        ref = run.hybrid()
        op, od = _hybrid(run, pers)
        assert torch.equal(op, ref[0]) and torch.equal(od, ref[1])
        check_against_oracle(run, op, od, rows=sample_rows(b.chunk_len, seed=1),
                             reqs=sample_reqs(b.context_lens.tolist(), seed=1), label="persistent config 3")
    finally:
        pers.close()
        run.close()


def test_persistent_several_chunks():
    sp = dict(name="pv", dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128, chunk_len=0, chunk_offset=0,
              chunks=[(300, 0), (64, 7000), (9, 100)], decode_lens=[3000, 12000, 5], contiguous=False)
    b = inputs.make_batch(sp, seed=5)
    dev = b.to("cuda:0")
    ctx = b.context_lens.clone().contiguous()
    outs = []
    for persistent in (0, 1):
        att = pod.PodAttention(pod.config_for_batch(b, persistent=persistent, wg_per_cu=2))
        try:
            op, od = torch.empty_like(dev.q_prefill), torch.empty_like(dev.q_decode)
            att.hybrid_varlen(dev, op, od, ctx)
            torch.cuda.synchronize()
            outs.append((op, od))
        finally:
            att.close()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
