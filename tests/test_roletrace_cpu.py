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


def test_decode_task_bytes_follow_the_fused_numbering():
    # contexts 5000 and 300 at T = 1024: long splits 4 x 1024 of request 0,
    # then the remainders 904 and 300; two kv heads, four waves per task
    from prefill_decode_hybrid_amd.roletrace import decode_task_bytes, unit_tokens
    assert unit_tokens([5000, 300], 1024) == [1024] * 4 + [904, 300]
    # the tail of each request (last full split and remainder) in 512-key splits
    assert unit_tokens([5000, 300], 1024, 512, 1) == [1024] * 3 + [512, 512, 512, 392, 300]
    row = 2 * 128 * 2
    b = decode_task_bytes([5000, 300], 1024, 0, 2, 128, 2)
    # wave tasks: units 0..5 x 2 heads = 12 -> 3 workgroup tasks
    assert b == [2 * 1024 * row * 2, 2 * 1024 * row * 2, (904 + 300) * row * 2]
    assert sum(b) == 2 * (5000 + 300) * row


def test_stream_rate_timeline_integrates_to_the_bytes():
    # one decode task of 1e9 bytes over 100 us (10000 ticks) -> 10 TB/s in
    # each of its buckets; a prefill task alongside changes nothing
    recs = [(1, 1, 0, 0, 10000), (2, 0, 0, 0, 5000)]
    s = summarize(recs, num_cus=2, buckets=4, decode_bytes=[1e9])
    rates = [e["decode_tb_s"] for e in s["timeline_wgs_per_cu"]]
    assert rates == [10.0, 10.0, 10.0, 10.0]
    assert [e["prefill"] for e in s["timeline_wgs_per_cu"]] == [0.5, 0.5, 0.0, 0.0]
