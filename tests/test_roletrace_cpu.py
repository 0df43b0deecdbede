"""The role-mix summary of task records, on hand-built records (CPU)."""
from prefill_decode_hybrid_amd.roletrace import summarize


def test_overlap_and_means():
    # CU 5 (XCD 0): prefill [0, 100), decode [50, 150); CU 0x105 (XCD 1):
    # decode only [0, 100).  Span 150 ticks.
    recs = [(5, 0, 0, 0, 100), (5, 1, 0, 50, 150), (0x105, 1, 1, 0, 100)]
    s = summarize(recs, num_cus=2)
    assert s["tasks"] == 3 and s["prefill_tasks"] == 1 and s["decode_tasks"] == 2
    assert s["cus_running_both"] == 1 and s["cus_seen"] == 2
    # both roles on CU 5 during [50, 100); busy time: CU 5 150, CU 0x105 100
    assert abs(s["share_of_cu_busy_time_with_both_roles"] - 50 / 250) < 1e-9
    assert abs(s["mean_prefill_wgs_per_cu"] - 100 / (2 * 150)) < 1e-3
    assert abs(s["mean_decode_wgs_per_cu"] - 200 / (2 * 150)) < 1e-3
    assert s["tasks_per_xcd"] == {"0": {"prefill": 1, "decode": 1}, "1": {"prefill": 0, "decode": 1}}


def test_back_to_back_tasks_do_not_overlap():
    # a prefill task ending exactly when a decode task starts on the same CU
    recs = [(1, 0, 0, 0, 10), (1, 1, 0, 10, 20)]
    s = summarize(recs, num_cus=1)
    assert s["share_of_cu_busy_time_with_both_roles"] == 0.0
    assert s["span_us"] == 0.2
