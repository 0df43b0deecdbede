"""Role trace of fused launches (pod_attn_role_trace): one record per task,
each task exactly once with its role, a valid CU key and a start before its
end; recording changes no output bit."""
import pytest
import torch

import prefill_decode_hybrid_amd as pod
from prefill_decode_hybrid_amd import inputs
from prefill_decode_hybrid_amd.roletrace import summarize
from gpu_helpers import Run, say
from parity_cases import spec

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    pod.load()


@pytest.mark.parametrize("kw", [dict(), dict(persistent=1), dict(wg_per_cu=4), dict(policy=pod.POD_POLICY_PROPORTIONAL)],
                         ids=["claimed", "persistent", "four_per_cu", "proportional"])
def test_role_trace_records_every_task_once(kw):
    sp = spec("bf16", 8, 2, 128, 64, 12000, [8192] * 80)
    batch = inputs.make_batch(sp, seed=12)
    plain = Run(batch, decode_split_tokens=256, **kw)
    rec = Run(batch, decode_split_tokens=256, record_roles=1, **kw)
    try:
        ref = plain.hybrid()
        out = rec.hybrid()
        assert torch.equal(ref[0], out[0]) and torch.equal(ref[1], out[1]), "recording changed the result"
        st = rec.att.stats()
        recs = rec.att.role_trace()
        say(f"{kw}: {len(recs)} records, plan {st}")
        assert len(recs) == st["prefill_tasks"] + st["decode_wg_tasks"]
        seen = {(r[1], r[2]) for r in recs}
        assert seen == {(0, t) for t in range(st["prefill_tasks"])} | {(1, t) for t in range(st["decode_wg_tasks"])}
        for key, role, task, t0, t1 in recs:
            assert (key >> 8) < 8 and t0 <= t1
        s = summarize(recs, st["num_cus"])
        say(f"  summary {s}")
        assert s["prefill_tasks"] == st["prefill_tasks"]
        assert s["cus_seen"] <= st["num_cus"]
    finally:
        plain.close()
        rec.close()


def test_role_trace_needs_a_recording_handle():
    run = Run(inputs.make_batch(spec("bf16", 8, 2, 128, 40, 100, [300]), seed=1))
    try:
        run.hybrid()
        with pytest.raises(pod.PodAttnError) as e:
            run.att.role_trace()
        assert e.value.status == pod.POD_ERR_INVALID_ARG
    finally:
        run.close()
