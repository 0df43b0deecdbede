"""Several prefill chunks in one call, on the CPU: the planner's view of a
varlen batch through pod_attn_plan_varlen (no kernel is launched), argument
validation, and the generator's several-chunk layout."""
import math

import numpy as np
import pytest
import torch

import prefill_decode_hybrid_amd as pod
from prefill_decode_hybrid_amd import inputs

FAKE = 0x1000


def _cfg(**kw):
    base = dict(dtype=pod.POD_BF16, num_q_heads=32, num_kv_heads=8, head_dim=128, max_chunk_len=8192,
                max_num_decode=512, max_context=65536, max_total_context=4 << 20)
    base.update(kw)
    return pod.make_config(**base)


def _batch(chunks, stride=None):
    lens = np.ascontiguousarray([c for c, _ in chunks], dtype=np.int32)
    offs = np.ascontiguousarray([p for _, p in chunks], dtype=np.int32)
    if stride is None:
        stride = max(-(-(c + p) // 16) for c, p in chunks)
    a = pod.PodPrefillBatch(FAKE, FAKE, FAKE, stride, lens.ctypes.data, offs.ctypes.data, len(chunks))
    a._keep = (lens, offs)
    return a


def _decode(lens):
    lens = np.ascontiguousarray(np.asarray(lens, dtype=np.int32))
    a = pod.PodDecodeArgs(FAKE, FAKE, FAKE, max(1, -(-int(lens.max()) // 16)), FAKE, lens.ctypes.data, len(lens))
    a._keep = lens
    return a


def test_one_chunk_plans_like_the_single_chunk_call():
    rng = np.random.default_rng(3)
    for _ in range(200):
        C, P0 = int(rng.integers(1, 4096)), int(rng.choice([0, rng.integers(0, 60000)]))
        lens = rng.integers(1, 20000, size=int(rng.integers(1, 64)))
        cfg = _cfg(prefill_split_cap_waves=int(rng.choice([0, 1, 2])))
        for mode in (pod.MODE_HYBRID, pod.MODE_PREFILL):
            da = _decode(lens) if mode == pod.MODE_HYBRID else None
            a = pod.pod_attn_plan(cfg, 256, mode, pod.PodPrefillArgs(FAKE, FAKE, FAKE, C, P0), da)
            b = pod.pod_attn_plan_varlen(cfg, 256, mode, _batch([(C, P0)]), da)
            assert a == b


@pytest.mark.parametrize("seed", range(10))
def test_varlen_plan_counts(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, pod.POD_MAX_CHUNKS + 1))
    rows = max(2, min(600, 8000 // n))  # all chunks within max_chunk_len
    chunks = [(int(rng.integers(1, rows)), int(rng.choice([0, rng.integers(0, 40000)]))) for _ in range(n)]
    st = pod.pod_attn_plan_varlen(_cfg(), 256, pod.MODE_HYBRID, _batch(chunks), _decode([5000] * 8))
    rpt = st["prefill_rows_per_tile"]
    assert st["prefill_chunks"] == n
    assert st["prefill_tiles"] == sum(-(-c // rpt) for c, _ in chunks) * 8
    assert st["prefill_tasks"] >= st["prefill_tiles"]
    # the first chunk in task order has the longest key range; its splits cover it
    lp = max(c + p for c, p in chunks)
    assert st["prefill_splits"] * st["prefill_split_keys"] >= lp
    assert (st["prefill_splits"] - 1) * st["prefill_split_keys"] < lp
    assert st["prefill_split_keys"] <= 16384
    # splits added for parallelism stay within the cap (two waves) plus one task per tile
    assert st["prefill_tasks"] <= 2 * 256 * st["wg_per_cu"] + st["prefill_tiles"] or \
        st["prefill_tasks"] <= st["prefill_tiles"] * math.ceil(lp / 16384)
    assert st["grid"] == st["prefill_tasks"] + st["decode_wg_tasks"]


def test_long_chunks_split_more_than_short_ones():
    # equal rows, very different key ranges: the long one takes the splits
    a = pod.pod_attn_plan_varlen(_cfg(), 256, pod.MODE_PREFILL, _batch([(128, 30000), (128, 0)]), None)
    solo = pod.pod_attn_plan_varlen(_cfg(), 256, pod.MODE_PREFILL, _batch([(128, 0)]), None)
    long_tasks = (128 // a["prefill_rows_per_tile"]) * 8 * a["prefill_splits"]
    assert a["prefill_splits"] > 1 and a["prefill_tasks"] - long_tasks < long_tasks
    assert solo["prefill_tasks"] >= a["prefill_tasks"] - long_tasks


@pytest.mark.parametrize("chunks,stride,max_rows", [
    ([], None, 8192),                                  # no chunk
    ([(8, 0)] * (pod.POD_MAX_CHUNKS + 1), None, 8192),  # too many chunks
    ([(8, 0), (0, 4)], None, 8192),                    # empty chunk
    ([(8, 0), (8, -1)], None, 8192),                   # negative offset
    ([(100, 100), (100, 0)], 5, 8192),                 # table row shorter than a chunk's pages
    ([(600, 0), (600, 0)], None, 1000),                # rows above max_chunk_len
    ([(8, 65530)], None, 8192),                        # offset + chunk above max_context
])
def test_varlen_validation(chunks, stride, max_rows):
    cfg = _cfg(max_chunk_len=max_rows)
    if chunks:
        b = _batch(chunks, stride)
    else:
        b = pod.PodPrefillBatch(FAKE, FAKE, FAKE, 1, FAKE, FAKE, 0)
    with pytest.raises(pod.PodAttnError) as e:
        pod.pod_attn_plan_varlen(cfg, 256, pod.MODE_PREFILL, b, None)
    assert e.value.status == pod.POD_ERR_INVALID_ARG


def test_varlen_null_host_arrays():
    b = _batch([(8, 0), (9, 3)])
    b.chunk_offsets_host = None
    with pytest.raises(pod.PodAttnError) as e:
        pod.pod_attn_plan_varlen(_cfg(), 256, pod.MODE_PREFILL, b, None)
    assert e.value.status == pod.POD_ERR_INVALID_ARG


def test_generator_several_chunks():
    spec = dict(name="v", dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=64, chunk_len=0, chunk_offset=0,
                chunks=[(40, 0), (7, 300), (100, 33)], decode_lens=[50, 700], contiguous=False)
    b = inputs.make_batch(spec, seed=1)
    assert b.chunk_list() == [(40, 0), (7, 300), (100, 33)]
    assert b.q_prefill.shape == (147, 8, 64) and b.chunk_len == 147
    pt = b.page_table_prefill
    assert pt.shape == (3, -(-307 // 16))
    used = []
    for i, (c, p) in enumerate(b.chunk_list()):
        n = -(-(c + p) // 16)
        assert (pt[i, n:] == b.guard_page).all()
        used += pt[i, :n].tolist()
    used += b.page_table_decode[0, :4].tolist() + b.page_table_decode[1, :44].tolist()
    assert len(set(used)) == len(used) == b.num_pages - 1  # every request owns its pages
    assert b.visible_keys_prefill() == sum(c * p + c * (c + 1) // 2 for c, p in b.chunk_list())
    # the single-chunk layout is unchanged by the several-chunk path
    one = inputs.make_batch(dict(spec, chunks=None, chunk_len=40, chunk_offset=0), seed=1)
    assert one.chunks is None and one.page_table_prefill.dim() == 1
    cfg = pod.config_for_batch(b)
    assert cfg.max_chunk_len == 147 and cfg.max_context == 700
