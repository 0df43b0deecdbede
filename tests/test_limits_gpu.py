"""The largest sizes the library accepts, on the GPU against the oracle.

* a decode at the maximum context (261888 tokens, at most 1023 splits;
  here several hundred splits that one last-arriver merge combines) beside
  a prefill chunk ending at that same position (its rows see up to 261888
  keys in over a hundred KV splits), checked on sampled rows;
* a batch of 512 single-token decodes (context 1) beside a one-row chunk:
  the degenerate shapes, checked in full.
"""
import pytest
import torch

import prefill_decode_hybrid_amd as pod
from prefill_decode_hybrid_amd import inputs
from gpu_helpers import Run, check_against_oracle, say

pytestmark = pytest.mark.gpu

MAX_CONTEXT = 1023 * 256


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pod.load()


def test_maximum_context():
    C = 64
    sp = dict(name="max_ctx", dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=128, chunk_len=C,
              chunk_offset=MAX_CONTEXT - C, decode_lens=[MAX_CONTEXT, 3], contiguous=False)
    say("maximum context: generating")
    b = inputs.make_batch(sp, seed=9)
    run = Run(b)
    try:
        op, od = run.hybrid()
        st = run.att.stats()
        say(f"maximum context plan {st}")
        assert st["prefill_split_keys"] <= 16384 and st["prefill_splits"] * st["prefill_split_keys"] >= MAX_CONTEXT
        assert torch.isfinite(op.float()).all() and torch.isfinite(od.float()).all()
        check_against_oracle(run, op, od, rows=[0, 1, 31, 32, C - 1], label="maximum context")
        sp_, sd_ = run.separate()
        assert torch.equal(op, sp_) and torch.equal(od, sd_)
    finally:
        run.close()


def test_one_token_everything():
    sp = dict(name="ones", dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128, chunk_len=1,
              chunk_offset=0, decode_lens=[1] * 512, contiguous=False)
    b = inputs.make_batch(sp, seed=10)
    run = Run(b)
    try:
        op, od = run.hybrid()
        check_against_oracle(run, op, od, label="one token")
        # one visible key: the output is that key's V row, exactly
        g = torch.arange(32) // 4
        page = int(b.page_table_prefill[0])
        assert torch.equal(op[0].cpu(), b.v_pool[page, 0, g])
        sp_, sd_ = run.separate()
        assert torch.equal(op, sp_) and torch.equal(od, sd_)
    finally:
        run.close()


@pytest.mark.parametrize("case", ["group32768", "group65472"])
def test_decode_unit_scan_extremes(case):
    # The decode-unit lookup scans packed split counts of 64 requests at a
    # time.  These batches fill one 64-request group with 32768 splits (64 x
    # 131072 tokens at 256-token splits, default planning) and with the most
    # a group can hold (64 x 1023 splits), beside short decodes and a chunk
    # whose KV splits share the workspace; a lookup that lost a bit would
    # put partial records in the wrong place.
    if case == "group32768":
        sp = dict(name=case, dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=64, chunk_len=64,
                  chunk_offset=16384 + 37, decode_lens=[131072] * 64 + [16] * 136, contiguous=False)
        want_T, groups, kw = 256, [0, 31, 62, 63, 64, 65, 199], {}
    else:
        sp = dict(name=case, dtype="bf16", num_q_heads=4, num_kv_heads=1, head_dim=64, chunk_len=64,
                  chunk_offset=20000, decode_lens=[MAX_CONTEXT] * 64 + [40] * 3, contiguous=False)
        # the planner would pick long splits here; fix the shortest allowed
        want_T, groups, kw = 256, [0, 1, 62, 63, 64, 66], dict(decode_split_tokens=256)
    say(f"{case}: generating")
    b = inputs.make_batch(sp, seed=13)
    run = Run(b, **kw)
    try:
        op, od = run.hybrid()
        st = run.att.stats()
        say(f"{case} plan {st}")
        assert st["decode_split_tokens"] == want_T
        assert st["prefill_splits"] > 1, "the chunk's KV splits should share the workspace"
        check_against_oracle(run, op, od, rows=[0, 1, 31, 32, 63], reqs=groups, label=case)
        assert torch.isfinite(op.float()).all() and torch.isfinite(od.float()).all()
        sp_, sd_ = run.separate()
        assert torch.equal(op, sp_) and torch.equal(od, sd_), "fused result differs from split launches"
    finally:
        run.close()
