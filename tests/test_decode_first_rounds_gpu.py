"""Decode-first fused launches of several rounds: the decode tasks go to the
first workgroup ids in length-class order (remainders longest first) and the
short prefill's to the last.  One case per built (dtype, head dim, group
size) instantiation, each a batch of 1100 decodes of 1-1200 tokens beside a
16-row chunk: the plan must take that path, every output must match the
fp64 oracle, and the fused result must equal the split launches bit for
bit."""
import numpy as np
import pytest
import torch

import prefill_decode_hybrid_amd as pod
from prefill_decode_hybrid_amd import inputs
from gpu_helpers import Run, check_against_oracle, say
from parity_cases import spec

pytestmark = pytest.mark.gpu

INSTANTIATIONS = [("bf16", d, G) for d in (128, 64) for G in (1, 2, 4, 8)] + [("f32", 64, G) for G in (1, 2, 4, 8)]


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pod.load()


@pytest.mark.parametrize("inst", INSTANTIATIONS, ids=lambda t: f"{t[0]}_d{t[1]}_G{t[2]}")
def test_decode_first_over_several_rounds(inst):
    dtype, d, G = inst
    lens = np.random.default_rng(7).integers(1, 1201, size=1100).tolist()
    sp = spec(dtype, 2 * G, 2, d, 16, 100, lens)
    say(f"case {sp['name']} ({len(lens)} decodes)")
    run = Run(inputs.make_batch(sp, seed=3))
    try:
        op, od = run.hybrid()
        st = run.att.stats()
        assert st["cu_prefill_x256"] == 0 and st["decode_wg_tasks"] > st["num_cus"] * 2, st
        assert st["fixed_order"] == 2 and st["decode_unit_classes"] == 8, st
        check_against_oracle(run, op, od, label="hybrid")
        sp_, sd_ = run.separate()
        assert torch.equal(op, sp_) and torch.equal(od, sd_), "fused result differs from split launches"
        op2, od2 = run.hybrid()
        assert torch.equal(op, op2) and torch.equal(od, od2), "hybrid not run-to-run deterministic"
    finally:
        run.close()
