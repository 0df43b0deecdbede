"""Decode tail splits (decode_tail_split_tokens): the last full split and the
remainder of every decode request are cut into short splits numbered after
all long ones.  Only where a unit's keys begin and end changes, so every
output must still match the fp64 oracle, the fused call must equal the split
calls bit for bit, and odd and even split counts, one-page tails and
requests shorter than two long splits must all be covered."""
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


CASES = [
    # (case, long split, tail split)
    (spec("bf16", 8, 2, 128, 77, 300, [1, 15, 16, 17, 300, 1023, 1025, 2100, 4096, 5000, 9001]), 1024, 256),
    (spec("bf16", 16, 2, 64, 40, 0, [5, 64, 2000, 3333, 8191, 8192, 8193], outliers=0.02), 2048, 512),
    (spec("bf16", 8, 2, 128, 64, 12000, [20000, 16384, 4111]), 4096, 1040),
    (spec("f32", 4, 2, 64, 67, 500, [2, 64, 65, 1300, 2600]), 512, 128),
]


@pytest.mark.parametrize("case,wg", [(c, 2) for c in range(len(CASES))] + [(0, 4), (2, 4)])
def test_tail_splits_match_the_oracle(case, wg):
    sp, T, T2 = CASES[case]
    run = Run(inputs.make_batch(sp, seed=21), decode_split_tokens=T, decode_tail_split_tokens=T2, wg_per_cu=wg)
    try:
        op, od = run.hybrid()
        st = run.att.stats()
        say(f"{sp['name']} T {T} T2 {T2} wg {wg}: plan {st}")
        assert st["decode_split_tokens"] == T and st["decode_tail_split_tokens"] == T2
        check_against_oracle(run, op, od, label=f"{sp['name']} tail splits")
        sp_, sd_ = run.separate()
        assert torch.equal(op, sp_) and torch.equal(od, sd_), "fused result differs from split launches"
    finally:
        run.close()


def test_tail_splits_on_the_prefill_heavy_batch():
    # the one measured batch where tail splits pay: 16 decodes of 32K in the
    # prefill's tail; every decode request against the oracle
    b = inputs.make_batch(5, seed=0)
    run = Run(b, decode_tail_split_tokens=832)
    try:
        op, od = run.hybrid()
        st = run.att.stats()
        say(f"config 5 tail splits: plan {st}")
        assert st["decode_tail_split_tokens"] == 832
        check_against_oracle(run, None, od, label="config 5 tail splits")
        _, sd_ = run.separate()
        assert torch.equal(od, sd_), "fused decode differs from the decode-only launch"
    finally:
        run.close()
