"""The four-workgroups-per-CU envelope (wg_per_cu = 4: 16-row prefill
tiles and page-by-page decode waves within 128 registers and 40 KB of LDS
per workgroup) and the runtime choice between the envelopes, through the C
ABI against the fp64 oracle.

Bars as everywhere: bf16 max |err| <= 2e-2, mean <= 2e-3.  With the
envelope fixed, the fused call equals the split calls bit for bit and
repeats bit for bit; with the runtime choice (wg_per_cu = 0) each call picks
its own envelope, so only the oracle bar applies across calls."""
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


BF16 = [sp for sp in SMALL if sp["dtype"] == "bf16"]


@pytest.mark.parametrize("sp", BF16, ids=lambda s: s["name"])
def test_small_cases_wg4(sp):
    say(f"case {sp['name']} (4 workgroups per CU)")
    run = Run(inputs.make_batch(sp, seed=1), wg_per_cu=4)
    try:
        op, od = run.hybrid()
        assert run.att.stats()["wg_per_cu"] == 4
        check_against_oracle(run, op, od, label="hybrid")
        sp_, sd_ = run.separate()
        check_against_oracle(run, sp_, sd_, label="separate")
        assert torch.equal(op, sp_) and torch.equal(od, sd_), "fused result differs from split launches"
        op2, od2 = run.hybrid()
        assert torch.equal(op, op2) and torch.equal(od, od2), "hybrid not run-to-run deterministic"
    finally:
        run.close()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_configs_wg4(cid):
    say(f"config {cid} (4 workgroups per CU): generating")
    run = Run(inputs.make_batch(cid, seed=0), wg_per_cu=4)
    try:
        op, od = run.hybrid()
        st = run.att.stats()
        say(f"config {cid} plan {st}")
        assert st["wg_per_cu"] == 4
        check_against_oracle(run, op, od, label=f"config {cid} wg4 hybrid", step=256)
        sp_, sd_ = run.separate()
        assert torch.equal(op, sp_) and torch.equal(od, sd_), "fused result differs from split launches"
    finally:
        run.close()


@pytest.mark.parametrize("cid,decode_alone", [(2, 4), (4, 2)])
def test_runtime_envelope_choice(cid, decode_alone):
    # the fused call keeps two workgroups per CU; the decode-only call picks
    # four when its workgroups fit one round of four per CU; every call
    # matches the oracle
    run = Run(inputs.make_batch(cid, seed=0), wg_per_cu=0)
    try:
        op, od = run.hybrid()
        assert run.att.stats()["wg_per_cu"] == 2
        check_against_oracle(run, op, od, label=f"config {cid} runtime choice", step=256)
        sp_, sd_ = run.separate()
        assert run.att.stats()["wg_per_cu"] == decode_alone  # the decode-only call ran last
        check_against_oracle(run, sp_, sd_, label=f"config {cid} runtime choice, split calls", step=256)
    finally:
        run.close()


@pytest.mark.parametrize("policy", [pod.POD_POLICY_PROPORTIONAL, pod.POD_POLICY_HALF, pod.POD_POLICY_STATIC])
def test_policies_wg4(policy):
    sp = SMALL[0]
    base = Run(inputs.make_batch(sp, seed=2), wg_per_cu=4)
    alt = Run(inputs.make_batch(sp, seed=2), wg_per_cu=4, policy=policy)
    try:
        a = base.hybrid()
        b = alt.hybrid()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    finally:
        base.close()
        alt.close()


def test_several_chunks_wg4():
    from test_varlen_gpu import CASES, check
    for sp in (CASES[1], CASES[6]):
        say(f"case {sp['name']} (4 workgroups per CU)")
        b = inputs.make_batch(sp, seed=2)
        dev = b.to("cuda:0")
        ctx = b.context_lens.clone().contiguous()
        att = pod.PodAttention(pod.config_for_batch(b, wg_per_cu=4))
        try:
            op = torch.full_like(dev.q_prefill, float("nan"))
            od = torch.full_like(dev.q_decode, float("nan"))
            att.hybrid_varlen(dev, op, od, ctx)
            torch.cuda.synchronize()
            check(b, op, od, "hybrid_varlen wg4")
            op2, od2 = torch.full_like(op, float("nan")), torch.full_like(od, float("nan"))
            att.prefill_only_varlen(dev, op2)
            att.decode_only(dev, od2, ctx)
            torch.cuda.synchronize()
            assert torch.equal(op, op2) and torch.equal(od, od2)
        finally:
            att.close()


def test_fused_launch_in_a_captured_graph_wg4():
    # 80 decodes in 256-token splits: more workgroups than one round of four
    # per CU, so roles are claimed and the control words counted out
    sp = spec("bf16", 8, 2, 128, 64, 12000, [8192] * 80)
    run = Run(inputs.make_batch(sp, seed=12), wg_per_cu=4, decode_split_tokens=256)
    try:
        ref = run.hybrid()
        st = run.att.stats()
        assert st["fixed_order"] == 0 and st["wg_per_cu"] == 4  # roles are claimed
        op, od = run.outputs()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            run.att.hybrid(run.dev, op, od, run.ctx_host)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run.att.hybrid(run.dev, op, od, run.ctx_host)
        scratch = torch.zeros(1 << 20, device="cuda:0")
        for i in range(3):
            op.fill_(float("nan"))
            od.fill_(float("nan"))
            scratch.add_(1.0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(op, ref[0]) and torch.equal(od, ref[1]), f"replay {i} differs from the eager launch"
    finally:
        run.close()


def test_decode_unit_scan_extreme_wg4():
    # 32768 splits in the first 64-request group, with a split chunk beside
    sp = dict(name="group32768_wg4", dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=64, chunk_len=64,
              chunk_offset=16384 + 37, decode_lens=[131072] * 64 + [16] * 136, contiguous=False)
    say("group32768 (4 workgroups per CU): generating")
    run = Run(inputs.make_batch(sp, seed=13), wg_per_cu=4)
    try:
        op, od = run.hybrid()
        st = run.att.stats()
        assert st["decode_split_tokens"] == 256 and st["wg_per_cu"] == 4
        check_against_oracle(run, op, od, rows=[0, 1, 15, 16, 63], reqs=[0, 31, 62, 63, 64, 199], label="group32768 wg4")
        sp_, sd_ = run.separate()
        assert torch.equal(op, sp_) and torch.equal(od, sd_)
    finally:
        run.close()
