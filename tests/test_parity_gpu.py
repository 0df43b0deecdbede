"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Every entry point (pod_attn_hybrid, pod_attn_prefill_only,
pod_attn_decode_only) is compared element by element with the oracle on the
same seeded inputs.  Bars: bf16 inputs with fp32 accumulation, max abs error
<= 2e-2 and mean abs error <= 2e-3; fp32 inputs, max abs error <= 1e-4.
Small cases span several tiles and ragged tails and together reach every
kernel instantiation; the five workload configs are compared on every row
and request, at two seeds, in the launch configuration the benchmark times.  Fusion must not change the result: the fused call is
bitwise equal to the two split calls, and repeated calls are bitwise equal.
"""
import numpy as np
import pytest
import torch

import prefill_decode_hybrid_amd as pod
from prefill_decode_hybrid_amd import inputs
from gpu_helpers import Run, check_against_oracle, say
from parity_cases import SMALL, spec

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pod.load()


@pytest.mark.parametrize("sp", SMALL, ids=lambda s: s["name"])
def test_small_cases(sp):
    say(f"case {sp['name']}")
    run = Run(inputs.make_batch(sp, seed=1))
    try:
        op, od = run.hybrid()
        check_against_oracle(run, op, od, label="hybrid")
        sp_, sd_ = run.separate()
        check_against_oracle(run, sp_, sd_, label="separate")
        assert torch.equal(op, sp_) and torch.equal(od, sd_), "fused result differs from split launches"
        op2, od2 = run.hybrid()
        assert torch.equal(op, op2) and torch.equal(od, od2), "hybrid not run-to-run deterministic"
    finally:
        run.close()


@pytest.mark.parametrize("policy", [pod.POD_POLICY_PROPORTIONAL, pod.POD_POLICY_HALF, pod.POD_POLICY_STATIC])
def test_policies_give_identical_results(policy):
    sp = SMALL[0]
    base = Run(inputs.make_batch(sp, seed=2))
    alt = Run(inputs.make_batch(sp, seed=2), policy=policy)
    try:
        a = base.hybrid()
        b = alt.hybrid()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    finally:
        base.close()
        alt.close()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_single_key_is_exact(dtype):
    # decode over one key and prefill row 0 at offset 0 return that V row bit for bit
    sp = spec(dtype, 8, 2, 64 if dtype == "f32" else 128, 33, 0, [1, 1, 2])
    run = Run(inputs.make_batch(sp, seed=3))
    try:
        op, od = run.hybrid()
        b = run.cpu
        G = b.num_q_heads // b.num_kv_heads
        for r in (0, 1):
            page = int(b.page_table_decode[r, 0])
            v0 = b.v_pool[page, 0].repeat_interleave(G, dim=0)
            assert torch.equal(od[r].cpu(), v0)
        page = int(b.page_table_prefill[0])
        assert torch.equal(op[0].cpu(), b.v_pool[page, 0].repeat_interleave(G, dim=0))
    finally:
        run.close()


def test_hybrid_with_one_half_missing():
    run = Run(inputs.make_batch(SMALL[0], seed=4))
    try:
        b = run.dev
        op, od = run.outputs()
        pa, da = run.att.args(b, op, od, run.ctx_host)
        pod.pod_attn_hybrid(run.att.h, b.k_pool, b.v_pool, pa, None)
        assert run.att.stats()["fallback"] == 1
        pod.pod_attn_hybrid(run.att.h, b.k_pool, b.v_pool, None, da)
        assert run.att.stats()["fallback"] == 2
        torch.cuda.synchronize()
        check_against_oracle(run, op, od, label="single-role hybrid")
    finally:
        run.close()


_CACHE = {}


def config_run(cid, seed):
    if (cid, seed) not in _CACHE:
        for r in _CACHE.values():
            r.close()
        _CACHE.clear()
        torch.cuda.empty_cache()
        say(f"generating config {cid} seed {seed}")
        _CACHE[(cid, seed)] = Run(inputs.make_batch(cid, seed=seed))
    return _CACHE[(cid, seed)]


@pytest.mark.timeout(1200)
@pytest.mark.parametrize("seed", [0, 1])
@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_config_full(cid, seed):
    # every output row and request of the workload against the oracle, in
    # the launch configuration the benchmark times; the split launches must
    # give the same bits
    run = config_run(cid, seed)
    op, od = run.hybrid()
    say(f"config {cid} seed {seed} plan {run.att.stats()}")
    check_against_oracle(run, op, od, label=f"config {cid} seed {seed} hybrid", step=256)
    sp_, sd_ = run.separate()
    assert torch.equal(op, sp_) and torch.equal(od, sd_), "fused result differs from split launches"
    op2, od2 = run.hybrid()
    assert torch.equal(op, op2) and torch.equal(od, od2), "hybrid not run-to-run deterministic"


def test_decode_first_by_workgroup_id():
    # a short chunk beside longer decodes: decode first, all decode workgroups in one round
    sp = spec("bf16", 8, 2, 128, 32, 0, [8192] * 16 + [3, 700])
    run = Run(inputs.make_batch(sp, seed=11))
    try:
        op, od = run.hybrid()
        st = run.att.stats()
        say(f"decode first plan {st}")
        assert st["fixed_order"] == 2 and st["cu_prefill_x256"] == 0
        check_against_oracle(run, op, od, label="decode first")
        sp_, sd_ = run.separate()
        assert torch.equal(op, sp_) and torch.equal(od, sd_)
    finally:
        run.close()


@pytest.mark.parametrize("persistent", [0, 1])
def test_fused_launch_in_a_captured_graph(persistent):
    # the control words are restored by the launch itself, so replays of a
    # captured launch (with eager work in between) give the eager result every time
    # 256-token decode splits make the grid longer than one round, so roles are claimed
    sp = spec("bf16", 8, 2, 128, 64, 12000, [8192] * 40)
    run = Run(inputs.make_batch(sp, seed=12), persistent=persistent, decode_split_tokens=256)
    try:
        ref = run.hybrid()
        st = run.att.stats()
        assert st["fixed_order"] == 0 and st["policy"] == pod.POD_POLICY_CU_BALANCED  # roles are claimed
        assert st["persistent"] == persistent
        op, od = run.outputs()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run.att.hybrid(run.dev, op, od, run.ctx_host)  # warm-up on the capture stream
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run.att.hybrid(run.dev, op, od, run.ctx_host)
        scratch = torch.zeros(1 << 20, device="cuda:0")
        for i in range(4):
            op.fill_(float("nan"))
            od.fill_(float("nan"))
            scratch.add_(1.0)  # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            say(f"replay {i}")
            assert torch.equal(op, ref[0]) and torch.equal(od, ref[1]), f"replay {i} differs from the eager launch"
        # and an eager launch after the replays still matches
        op2, od2 = run.hybrid()
        assert torch.equal(op2, ref[0]) and torch.equal(od2, ref[1])
        # the split launches (their merge counters are restored by the last arriver)
        g2 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g2):
            run.att.prefill_only(run.dev, op)
            run.att.decode_only(run.dev, od, run.ctx_host)
        for i in range(3):
            op.fill_(float("nan"))
            od.fill_(float("nan"))
            g2.replay()
            torch.cuda.synchronize()
            assert torch.equal(op, ref[0]) and torch.equal(od, ref[1]), f"split replay {i} differs"
    finally:
        run.close()
