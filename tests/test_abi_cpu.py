"""The C-ABI library on the CPU: symbols, argument validation and the host
planner (no kernel is launched here)."""
import ctypes
import math
import os
import random
import re

import numpy as np
import pytest

import prefill_decode_hybrid_amd as pod
from prefill_decode_hybrid_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x1000  # a non-null device pointer; planning never dereferences it


@pytest.fixture(scope="module")
def lib():
    return pod.load()


def header_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            txt = open(os.path.join(ROOT, "include", fn)).read()
            names |= set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(pod_\w+)\s*\(", txt, re.M))
    return sorted(names)


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert len(names) >= 9, names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"
    assert set(names) == set(pod.EXPORTED)


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4):
        assert pod.status_string(code) not in ("", "unknown status")


def _prefill(C, P0):
    return pod.PodPrefillArgs(FAKE, FAKE, FAKE, C, P0)


def _decode(lens, stride=None):
    lens = np.ascontiguousarray(np.asarray(lens, dtype=np.int32))
    stride = stride or max(1, -(-int(lens.max()) // 16))
    a = pod.PodDecodeArgs(FAKE, FAKE, FAKE, stride, FAKE, lens.ctypes.data, len(lens))
    a._keep = lens
    return a


def _cfg(spec, **kw):
    spec = dict(inputs.CONFIGS[spec]) if isinstance(spec, int) else spec
    base = dict(dtype=pod.POD_BF16 if spec["dtype"] == "bf16" else pod.POD_F32,
                num_q_heads=spec["num_q_heads"], num_kv_heads=spec["num_kv_heads"],
                head_dim=spec["head_dim"], max_chunk_len=4096, max_num_decode=512,
                max_context=32768, max_total_context=4 << 20, wg_per_cu=2)
    base.update(kw)
    return pod.make_config(**base)


def plan(cfg, mode, pa, da, cus=256):
    return pod.pod_attn_plan(cfg, cus, mode, pa, da)


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_plan_invariants_on_configs(cid):
    spec = inputs.CONFIGS[cid]
    lens = inputs.draw_context_lens(cid, 0)
    cfg = _cfg(cid)
    C, P0 = spec["chunk_len"], spec["chunk_offset"]
    st = plan(cfg, pod.MODE_HYBRID, _prefill(C, P0), _decode(lens))
    hq, hkv = spec["num_q_heads"], spec["num_kv_heads"]
    G = hq // hkv
    # prefill tiles cover every (row, head) once
    assert st["prefill_heads_per_tile"] == min(G, 4)
    assert st["prefill_rows_per_tile"] * st["prefill_heads_per_tile"] == (32 if spec["dtype"] == "bf16" else 64) * 4
    row_blocks = -(-C // st["prefill_rows_per_tile"])
    assert st["prefill_tiles"] == row_blocks * hkv * (G // st["prefill_heads_per_tile"])
    Lp = C + P0
    bn = 64 if spec["dtype"] == "bf16" else 32
    assert st["prefill_split_keys"] % bn == 0
    assert st["prefill_splits"] * st["prefill_split_keys"] >= Lp
    assert (st["prefill_splits"] - 1) * st["prefill_split_keys"] < Lp
    assert st["prefill_tasks"] == st["prefill_tiles"] * st["prefill_splits"]
    slots = 256 * st["wg_per_cu"]
    assert st["prefill_split_keys"] <= 16384  # a split's page ids fit the LDS table
    if st["prefill_splits"] > -(-Lp // 16384):  # splits for parallelism: at most two waves of workgroups
        assert st["prefill_tasks"] <= 2 * slots
    # decode: every (request, kv head) split into ceil(L / T) one-wave units
    T = st["decode_split_tokens"]
    assert T % 16 == 0 and (256 if spec["dtype"] == "bf16" else 64) <= T <= 4096
    assert st["decode_tail_split_tokens"] == 0  # no tail splits unless asked for
    assert st["decode_wave_tasks"] == hkv * sum(-(-int(L) // T) for L in lens)
    assert st["decode_wg_tasks"] == -(-st["decode_wave_tasks"] // 4)
    assert st["grid"] == st["prefill_tasks"] + st["decode_wg_tasks"]
    assert 0 < st["share_num"] < st["share_den"]
    assert st["fallback"] == 0


def test_plan_single_role_fallbacks():
    cfg = _cfg(2)
    st = plan(cfg, pod.MODE_HYBRID, _prefill(100, 7), None)
    assert st["fallback"] == 1 and st["decode_wg_tasks"] == 0 and st["grid"] == st["prefill_tasks"]
    st = plan(cfg, pod.MODE_HYBRID, None, _decode([5, 9]))
    assert st["fallback"] == 2 and st["prefill_tasks"] == 0 and st["grid"] == st["decode_wg_tasks"]


def test_split_cap_limits_prefill_tasks():
    # few tiles over a long prefix: splits fill the machine but never exceed the cap
    cfg = _cfg(2, prefill_split_cap_waves=1)
    st = plan(cfg, pod.MODE_PREFILL, _prefill(32, 30000), None)
    assert st["prefill_splits"] > 1
    assert st["prefill_tasks"] <= 1 * 256 * st["wg_per_cu"]


def test_forced_decode_split_tokens():
    lens = [5000, 300, 16384]
    for T in (256, 1024, 4096):
        st = plan(_cfg(3, decode_split_tokens=T), pod.MODE_HYBRID, _prefill(512, 1024), _decode(lens))
        assert st["decode_split_tokens"] == T and st["decode_tail_split_tokens"] == 0
        assert st["decode_wave_tasks"] == 8 * sum(-(-L // T) for L in lens)
    for bad in (100, 255, 4112, 1000, -16):  # bf16: multiples of 16 in 256 .. 4096
        with pytest.raises(pod.PodAttnError) as e:
            plan(_cfg(3, decode_split_tokens=bad), pod.MODE_DECODE, None, _decode(lens))
        assert e.value.status == pod.POD_ERR_INVALID_ARG


def test_forced_tail_split_tokens():
    # 5000 = one long split of 4096 is not kept (the last full split joins the
    # tail): 5000 in 512-token pieces -> 10; 300 -> 1; 16384 = 3 long + 8
    lens = [5000, 300, 16384]
    st = plan(_cfg(3, decode_split_tokens=4096, decode_tail_split_tokens=512), pod.MODE_DECODE, None,
              _decode(lens))
    assert st["decode_tail_split_tokens"] == 512
    assert st["decode_wave_tasks"] == 8 * (10 + 1 + 11)
    # a tail split not below the split itself means no tail splits
    st = plan(_cfg(3, decode_split_tokens=1024, decode_tail_split_tokens=1024), pod.MODE_DECODE, None,
              _decode(lens))
    assert st["decode_tail_split_tokens"] == 0
    assert st["decode_wave_tasks"] == 8 * sum(-(-L // 1024) for L in lens)
    for bad in (100, 255, 4112, 1000, -1):
        with pytest.raises(pod.PodAttnError) as e:
            plan(_cfg(3, decode_tail_split_tokens=bad), pod.MODE_DECODE, None, _decode(lens))
        assert e.value.status == pod.POD_ERR_INVALID_ARG


def test_decode_split_is_the_same_in_every_mode():
    # the split depends on the decode batch alone, so decode results match bit for bit
    lens = inputs.draw_context_lens(4, 0)
    cfg = _cfg(4)
    a = plan(cfg, pod.MODE_HYBRID, _prefill(256, 2048), _decode(lens))
    b = plan(cfg, pod.MODE_DECODE, None, _decode(lens))
    assert a["decode_split_tokens"] == b["decode_split_tokens"]
    assert a["decode_tail_split_tokens"] == b["decode_tail_split_tokens"]
    assert a["decode_wave_tasks"] == b["decode_wave_tasks"]


@pytest.mark.parametrize("P0,x", [(0, 0), (4096, 0), (15872, 0), (15360, 352)])
def test_role_mix_by_work_ratio(P0, x):
    # 64 decodes of 16K beside one chunk of a 16K prompt: a short chunk runs
    # after the decodes, a long one overlaps them on every CU
    C = 1024 if P0 == 15360 else 512
    st = plan(_cfg(3), pod.MODE_HYBRID, _prefill(C, P0), _decode([16384] * 64))
    assert st["cu_prefill_x256"] == x
    # decode first in one round of resident workgroups: roles by workgroup id
    assert st["fixed_order"] == (2 if x == 0 else 0)
    assert st["decode_wg_tasks"] <= 256 * st["wg_per_cu"]


def test_fixed_order_rule():
    # the decode-heavy batch runs decode first over several rounds: decode
    # tasks to the first workgroup ids, in length classes (as decode alone)
    spec = inputs.CONFIGS[4]
    st = plan(_cfg(4), pod.MODE_HYBRID, _prefill(spec["chunk_len"], spec["chunk_offset"]),
              _decode(inputs.draw_context_lens(4, 0)))
    assert st["cu_prefill_x256"] == 0 and st["decode_wg_tasks"] > 512 and st["fixed_order"] == 2
    assert st["decode_unit_classes"] == 8 and st["prefill_priority"] == 1
    for kw in (dict(persistent=1), dict(policy=pod.POD_POLICY_PROPORTIONAL)):
        st = plan(_cfg(3, **kw), pod.MODE_HYBRID, _prefill(512, 0), _decode([16384] * 64))
        assert st["fixed_order"] == 0
    # small batches resident in one round: roles to workgroup ids, decode
    # first when the prefill is under 4/11 of the decode, else prefill first
    spec = inputs.CONFIGS[2]
    st = plan(_cfg(2), pod.MODE_HYBRID, _prefill(spec["chunk_len"], spec["chunk_offset"]),
              _decode(inputs.draw_context_lens(2, 0)))
    assert st["grid"] <= 512 and st["cu_prefill_x256"] == 0 and st["fixed_order"] == 2
    spec = inputs.CONFIGS[1]
    st = plan(_cfg(1), pod.MODE_HYBRID, _prefill(spec["chunk_len"], spec["chunk_offset"]),
              _decode(inputs.draw_context_lens(1, 0)))
    assert st["grid"] <= 512 and st["cu_prefill_x256"] > 0 and st["fixed_order"] == 1
    st = plan(_cfg(3), pod.MODE_HYBRID, _prefill(256, 2048), _decode([4000] * 16))
    assert st["grid"] <= 512 and 0 < st["cu_prefill_x256"] < 512 and st["fixed_order"] == 1
    # the long-context batch takes several rounds: claims
    spec = inputs.CONFIGS[3]
    st = plan(_cfg(3), pod.MODE_HYBRID, _prefill(spec["chunk_len"], spec["chunk_offset"]),
              _decode(inputs.draw_context_lens(3, 0)))
    assert st["grid"] > 512 and st["fixed_order"] == 0


def test_prefill_first_rounds_take_proportional_tickets():
    # the prefill-heavy batch: prefill takes every slot over several rounds,
    # so the CU-balanced policy hands the roles out by proportional tickets
    spec = inputs.CONFIGS[5]
    pa, da = _prefill(spec["chunk_len"], spec["chunk_offset"]), _decode(inputs.draw_context_lens(5, 0))
    st = plan(_cfg(5), pod.MODE_HYBRID, pa, da)
    assert st["cu_prefill_x256"] == 512 and st["grid"] > 512 and st["policy"] == pod.POD_POLICY_PROPORTIONAL
    assert st["share_num"] * (st["prefill_tasks"] + st["decode_wg_tasks"]) == pytest.approx(
        st["share_den"] * st["prefill_tasks"], rel=0.02)
    # not where the config fixes another policy or the grid, nor for the other batches
    assert plan(_cfg(5, policy=pod.POD_POLICY_HALF), pod.MODE_HYBRID, pa, da)["policy"] == pod.POD_POLICY_HALF
    assert plan(_cfg(5, persistent=1), pod.MODE_HYBRID, pa, da)["policy"] == pod.POD_POLICY_CU_BALANCED
    for slots in (448, 512):
        st = plan(_cfg(5, prefill_slots_x256=slots), pod.MODE_HYBRID, pa, da)
        assert st["policy"] == pod.POD_POLICY_CU_BALANCED and st["cu_prefill_x256"] == slots
    for cid in (2, 3, 4):
        sp = inputs.CONFIGS[cid]
        st = plan(_cfg(cid), pod.MODE_HYBRID, _prefill(sp["chunk_len"], sp["chunk_offset"]),
                  _decode(inputs.draw_context_lens(cid, 0)))
        assert st["policy"] == pod.POD_POLICY_CU_BALANCED, cid


def test_decode_unit_classes_rule():
    # length classes (remainders longest first) where the decode's end is not
    # filled by a prefill: decode-only calls and decode-first fused launches
    # of several rounds; request order in other fused launches
    spec4 = inputs.CONFIGS[4]
    ctx4 = inputs.draw_context_lens(4, 0)
    pa4 = _prefill(spec4["chunk_len"], spec4["chunk_offset"])
    assert plan(_cfg(4), pod.MODE_DECODE, None, _decode(ctx4))["decode_unit_classes"] == 8
    # the same batch with the role order or the grid changed: request order, claims
    for kw in (dict(persistent=1), dict(policy=pod.POD_POLICY_PROPORTIONAL), dict(prefill_slots_x256=256),
               dict(wg_per_cu=4)):
        st = plan(_cfg(4, **kw), pod.MODE_HYBRID, pa4, _decode(ctx4))
        assert st["decode_unit_classes"] == 1 and st["fixed_order"] == 0, kw
    # decode first in one round (Llama batch) and the overlapped long-context batch: request order
    spec2 = inputs.CONFIGS[2]
    st = plan(_cfg(2), pod.MODE_HYBRID, _prefill(spec2["chunk_len"], spec2["chunk_offset"]),
              _decode(inputs.draw_context_lens(2, 0)))
    assert st["cu_prefill_x256"] == 0 and st["decode_unit_classes"] == 1
    spec3 = inputs.CONFIGS[3]
    st = plan(_cfg(3), pod.MODE_HYBRID, _prefill(spec3["chunk_len"], spec3["chunk_offset"]),
              _decode(inputs.draw_context_lens(3, 0)))
    assert st["cu_prefill_x256"] > 0 and st["decode_unit_classes"] == 1
    # the units are the same set in every numbering
    assert (plan(_cfg(4), pod.MODE_HYBRID, pa4, _decode(ctx4))["decode_wave_tasks"]
            == plan(_cfg(4, persistent=1), pod.MODE_HYBRID, pa4, _decode(ctx4))["decode_wave_tasks"])
    assert plan(_cfg(4), pod.MODE_PREFILL, _prefill(256, 0), None)["decode_unit_classes"] == 0


def test_prefill_priority_rule():
    # equal issue priority only for a decode-first launch whose workgroups all
    # start in the first round (the decode is the critical path from the start)
    spec = inputs.CONFIGS[2]
    st = plan(_cfg(2), pod.MODE_HYBRID, _prefill(spec["chunk_len"], spec["chunk_offset"]),
              _decode(inputs.draw_context_lens(2, 0)))
    assert st["fixed_order"] == 2 and st["grid"] <= 512 and st["prefill_priority"] == 0
    # decode first, prefill in the decode's tail (grid above one round)
    st = plan(_cfg(3), pod.MODE_HYBRID, _prefill(512, 8192), _decode([16384] * 64))
    assert st["fixed_order"] == 2 and st["grid"] > 512 and st["prefill_priority"] == 1
    for cid in (1, 3, 4, 5):
        spec = inputs.CONFIGS[cid]
        st = plan(_cfg(cid), pod.MODE_HYBRID, _prefill(spec["chunk_len"], spec["chunk_offset"]),
                  _decode(inputs.draw_context_lens(cid, 0)))
        assert st["prefill_priority"] == 1, cid
    st = plan(_cfg(2), pod.MODE_PREFILL, _prefill(512, 0), None)
    assert st["prefill_priority"] == 1


@pytest.mark.parametrize("bad,code", [
    (dict(prefill=(0, 0)), pod.POD_ERR_INVALID_ARG),       # empty chunk
    (dict(prefill=(8, -1)), pod.POD_ERR_INVALID_ARG),      # negative offset
    (dict(prefill=(5000, 0)), pod.POD_ERR_INVALID_ARG),    # chunk above max_chunk_len
    (dict(prefill=(100, 32700)), pod.POD_ERR_INVALID_ARG), # offset + chunk above max_context
    (dict(decode=[0, 4]), pod.POD_ERR_INVALID_ARG),        # context 0
    (dict(decode=[40000]), pod.POD_ERR_INVALID_ARG),       # above max_context
    (dict(decode=[33], stride=2), pod.POD_ERR_INVALID_ARG),  # context beyond the table
])
def test_validation_codes(bad, code):
    cfg = _cfg(2)
    pa = _prefill(*bad["prefill"]) if "prefill" in bad else None
    da = _decode(bad["decode"], bad.get("stride")) if "decode" in bad else None
    mode = pod.MODE_PREFILL if pa is not None else pod.MODE_DECODE
    with pytest.raises(pod.PodAttnError) as e:
        plan(cfg, mode, pa, da)
    assert e.value.status == code


def test_validation_null_pointers():
    cfg = _cfg(2)
    pa = pod.PodPrefillArgs(None, FAKE, FAKE, 8, 0)
    with pytest.raises(pod.PodAttnError) as e:
        plan(cfg, pod.MODE_PREFILL, pa, None)
    assert e.value.status == pod.POD_ERR_INVALID_ARG
    da = _decode([5])
    da.context_lens_host = None
    with pytest.raises(pod.PodAttnError) as e:
        plan(cfg, pod.MODE_DECODE, None, da)
    assert e.value.status == pod.POD_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(head_dim=96), dict(num_q_heads=24, num_kv_heads=8),
                                dict(page_size=8), dict(dtype=pod.POD_F32, head_dim=128),
                                dict(num_q_heads=32, num_kv_heads=2), dict(dtype=pod.POD_F32, head_dim=64, wg_per_cu=4),
                                dict(max_context=261889)])
def test_unsupported_shapes(kw):
    cfg = _cfg(2, **kw)
    with pytest.raises(pod.PodAttnError) as e:
        plan(cfg, pod.MODE_DECODE, None, _decode([5]))
    assert e.value.status == pod.POD_ERR_UNSUPPORTED


def test_workspace_limit():
    cfg = _cfg(2, max_total_context=1000)
    with pytest.raises(pod.PodAttnError) as e:
        plan(cfg, pod.MODE_DECODE, None, _decode([800, 800]))
    assert e.value.status == pod.POD_ERR_INVALID_ARG


def test_create_without_gpu_fails_cleanly(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    h = ctypes.c_void_p()
    rc = lib.pod_attn_create(ctypes.byref(_cfg(2)), ctypes.byref(h))
    assert rc == pod.POD_ERR_HIP and not h.value


def simulate_fused_claims(n_p, n_d, num, den, n_cus, seed, balanced=False, slots=1):
    """Host model of the fused kernel's role pick and queue claims: per-CU
    tickets or running counts, per-XCD prefill and decode queues (own queue
    with one atomic, then the others), random arrival order and CU placement
    (running workgroups finish at random).  Returns the claimed (role, task)
    list."""
    rng = random.Random(seed)
    tickets = [0] * n_cus
    running = [[] for _ in range(n_cus)]
    heads = {0: [0] * 8, 1: [0] * 8}
    ntask = {0: n_p, 1: n_d}
    claims = []

    def qlen(n, x):
        return (n - x + 7) // 8 if n > x else 0

    def claim(role, xcc):
        h, n = heads[role], ntask[role]
        i = h[xcc]  # own queue: one atomic, a head past the end is harmless
        h[xcc] += 1
        if i < qlen(n, xcc):
            return xcc + 8 * i
        for k in range(1, 8):
            x = (xcc + k) % 8
            if h[x] >= qlen(n, x):
                continue
            i = h[x]
            h[x] += 1
            if i < qlen(n, x):
                return x + 8 * i
        return None

    for _ in range(n_p + n_d):
        cu = rng.randrange(n_cus)
        if running[cu] and rng.random() < 0.5:
            running[cu].pop(rng.randrange(len(running[cu])))
        if balanced:
            role = 0 if sum(1 for r in running[cu] if r == 0) < slots else 1
        else:
            t = tickets[cu] % den
            tickets[cu] += 1
            role = 0 if ((t + 1) * num + den - 1) // den > (t * num + den - 1) // den else 1
        task = claim(role, cu % 8)
        if task is None:
            role ^= 1
            task = claim(role, cu % 8)
        assert task is not None, "a workgroup found no task"
        running[cu].append(role)
        claims.append((role, task))
    return claims


@pytest.mark.parametrize("balanced", [False, True])
@pytest.mark.parametrize("n_p,n_d,num,den", [(256, 2048, 7, 64), (1, 5, 1, 2), (40, 3, 63, 64),
                                             (100, 100, 32, 64), (5, 1000, 1, 64), (9, 9, 1, 2)])
def test_fused_claims_cover_every_task_once(n_p, n_d, num, den, balanced):
    for seed in range(20):
        claims = simulate_fused_claims(n_p, n_d, num, den, n_cus=16, seed=seed, balanced=balanced)
        p = sorted(x for r, x in claims if r == 0)
        d = sorted(x for r, x in claims if r == 1)
        assert p == list(range(n_p)) and d == list(range(n_d))


def test_role_rule_is_proportional_and_prefill_first():
    for num, den in [(1, 9), (7, 64), (1, 2), (63, 64)]:
        roles = [((t + 1) * num + den - 1) // den > (t * num + den - 1) // den for t in range(den)]
        assert sum(roles) == num and roles[0]


def test_persistent_plan():
    spec = inputs.CONFIGS[3]
    lens = inputs.draw_context_lens(3, 0)
    a = plan(_cfg(3), pod.MODE_HYBRID, _prefill(spec["chunk_len"], spec["chunk_offset"]), _decode(lens))
    b = plan(_cfg(3, persistent=1), pod.MODE_HYBRID, _prefill(spec["chunk_len"], spec["chunk_offset"]),
             _decode(lens))
    assert a["persistent"] == 0 and b["persistent"] == 1
    assert b["grid"] == min(a["grid"], 256 * b["wg_per_cu"])
    assert {k: v for k, v in a.items() if k not in ("grid", "persistent")} == \
        {k: v for k, v in b.items() if k not in ("grid", "persistent")}
    # split launches and one-sided calls keep one workgroup per task
    for mode, pa, da in ((pod.MODE_PREFILL, _prefill(100, 0), None), (pod.MODE_DECODE, None, _decode([5, 9])),
                         (pod.MODE_HYBRID, None, _decode([5, 9]))):
        st = plan(_cfg(3, persistent=1), mode, pa, da)
        assert st["persistent"] == 0
    with pytest.raises(pod.PodAttnError) as e:
        plan(_cfg(3, persistent=2), pod.MODE_DECODE, None, _decode([5]))
    assert e.value.status == pod.POD_ERR_INVALID_ARG


def test_fp32_decode_splits_and_the_split_limit():
    # fp32 decode waves take splits down to 64 tokens, but never more than 1023 splits a request
    cfg = _cfg(1, max_context=32768)
    st = plan(cfg, pod.MODE_DECODE, None, _decode([37, 100, 256, 511]))
    assert st["decode_split_tokens"] == 64
    big = _cfg(1, max_context=200000, max_total_context=1 << 20)
    st = plan(big, pod.MODE_DECODE, None, _decode([37, 511]))
    assert st["decode_split_tokens"] >= -(-200000 // 1023)
    with pytest.raises(pod.PodAttnError):
        plan(_cfg(1, max_context=200000, decode_split_tokens=64), pod.MODE_DECODE, None, _decode([37]))
    assert plan(_cfg(1, decode_split_tokens=64), pod.MODE_DECODE, None, _decode([37]))["decode_split_tokens"] == 64


def test_envelope_validation(lib):
    # workgroups per CU: 0 (chosen per call), 2 or 4; the four-workgroup
    # envelope is bf16 only and has no persistent grid
    for wg, dtype, persistent, want in [(3, pod.POD_BF16, 0, pod.POD_ERR_INVALID_ARG),
                                        (8, pod.POD_BF16, 0, pod.POD_ERR_INVALID_ARG),
                                        (4, pod.POD_F32, 0, pod.POD_ERR_UNSUPPORTED),
                                        (4, pod.POD_BF16, 1, pod.POD_ERR_UNSUPPORTED)]:
        cfg = pod.make_config(dtype=dtype, num_q_heads=8, num_kv_heads=2, head_dim=64, wg_per_cu=wg,
                              persistent=persistent)
        with pytest.raises(pod.PodAttnError) as e:
            pod.pod_attn_plan(cfg, 256, pod.MODE_DECODE, None, _decode([100]))
        assert e.value.status == want, (wg, dtype, persistent)


@pytest.mark.parametrize("cid", [2, 3, 4, 5])
def test_four_workgroup_plan(cid):
    # 16-row prefill tiles (four heads of a kv head per tile, or more rows
    # for smaller groups), splits and slots counted in waves of 4 per CU
    spec = inputs.CONFIGS[cid]
    lens = inputs.draw_context_lens(cid, 0)
    C, P0 = spec["chunk_len"], spec["chunk_offset"]
    hq, hkv = spec["num_q_heads"], spec["num_kv_heads"]
    G = hq // hkv
    st = plan(_cfg(cid, wg_per_cu=4), pod.MODE_HYBRID, _prefill(C, P0), _decode(lens))
    assert st["wg_per_cu"] == 4
    assert st["prefill_rows_per_tile"] * st["prefill_heads_per_tile"] == 16 * 4
    assert st["prefill_tiles"] == -(-C // st["prefill_rows_per_tile"]) * hkv * (G // st["prefill_heads_per_tile"])
    assert st["prefill_tasks"] == st["prefill_tiles"] * st["prefill_splits"]
    if st["prefill_splits"] > -(-(C + P0) // 16384):
        assert st["prefill_tasks"] <= 2 * 4 * 256
    T = st["decode_split_tokens"]
    assert st["decode_wave_tasks"] == hkv * sum(-(-int(L) // T) for L in lens)
    assert st["grid"] == st["prefill_tasks"] + st["decode_wg_tasks"]
    assert 0 <= st["cu_prefill_x256"] <= 4 * 256
    # the decode split is the same as in the two-workgroup envelope
    st2 = plan(_cfg(cid), pod.MODE_HYBRID, _prefill(C, P0), _decode(lens))
    assert st2["wg_per_cu"] == 2 and st2["decode_split_tokens"] == T


@pytest.mark.parametrize("cid,decode_alone", [(1, 2), (2, 4), (3, 4), (4, 2), (5, 4)])
def test_runtime_envelope_choice(cid, decode_alone):
    # hybrid and prefill calls keep two workgroups per CU; a decode-only call
    # takes four when its workgroups all start in one round of four per CU
    # (the Llama, long-context and prefill-heavy batches' decodes), two when
    # they take several (the decode-heavy batch) and for fp32
    spec = inputs.CONFIGS[cid]
    lens = inputs.draw_context_lens(cid, 0)
    pa = _prefill(spec["chunk_len"], spec["chunk_offset"])
    assert plan(_cfg(cid, wg_per_cu=0), pod.MODE_HYBRID, pa, _decode(lens))["wg_per_cu"] == 2
    assert plan(_cfg(cid, wg_per_cu=0), pod.MODE_PREFILL, pa, None)["wg_per_cu"] == 2
    st = plan(_cfg(cid, wg_per_cu=0), pod.MODE_DECODE, None, _decode(lens))
    assert st["wg_per_cu"] == decode_alone
    if decode_alone == 4:
        assert st["decode_wg_tasks"] <= 4 * 256
    # a hybrid call without its prefill half runs the decode alone, and chooses as such
    assert plan(_cfg(cid, wg_per_cu=0), pod.MODE_HYBRID, None, _decode(lens))["wg_per_cu"] == decode_alone


def test_prefill_split_knobs():
    # the last 512-token chunk of a 16K prompt beside 64 decodes of 16K
    # (the split-limiting study's shape): one wave of tasks by default,
    # finest splits without the cap, or a fixed count
    pa, da = _prefill(512, 15872), _decode([16384] * 64)
    st = plan(_cfg(3), pod.MODE_HYBRID, pa, da)
    assert st["prefill_tasks"] <= 512
    st = plan(_cfg(3, prefill_split_cap_waves=-1), pod.MODE_HYBRID, pa, da)
    assert st["prefill_splits"] == 16 and st["prefill_split_keys"] == 1024
    for n in (1, 3, 8):
        st = plan(_cfg(3, prefill_splits=n), pod.MODE_HYBRID, pa, da)
        assert st["prefill_splits"] == n
        assert st["prefill_tasks"] == st["prefill_tiles"] * n
    for bad in (dict(prefill_split_cap_waves=-2), dict(prefill_splits=-1)):
        with pytest.raises(pod.PodAttnError) as e:
            plan(_cfg(3, **bad), pod.MODE_HYBRID, pa, da)
        assert e.value.status == pod.POD_ERR_INVALID_ARG


def test_peak_kernels_validate_before_launch(lib):
    # measured-peak entry points reject bad arguments without touching a device
    inv = pod.POD_ERR_INVALID_ARG
    assert lib.pod_attn_peak_read(None, 1 << 20, 4, FAKE, None) == inv
    assert lib.pod_attn_peak_read(FAKE, 1 << 20, 4, None, None) == inv
    assert lib.pod_attn_peak_read(FAKE, 0, 4, FAKE, None) == inv
    assert lib.pod_attn_peak_read(FAKE, 1 << 20, 0, FAKE, None) == inv
    # each wave's slice must be whole 16 KB buffers ...
    assert lib.pod_attn_peak_read(FAKE, 4 * 16384 + 4096, 1, FAKE, None) == inv
    # ... and at most 1 GiB
    assert lib.pod_attn_peak_read(FAKE, 4 * ((1 << 30) + 16384), 1, FAKE, None) == inv
    assert lib.pod_attn_peak_mfma(0, 8, FAKE, None) == inv
    assert lib.pod_attn_peak_mfma(4, 0, FAKE, None) == inv
    assert lib.pod_attn_peak_mfma(4, 8, None, None) == inv


def test_peak_wrappers_check_tensor_sizes():
    # a host or undersized tensor never reaches the kernel
    import torch
    small = torch.zeros(1024, dtype=torch.uint8)
    with pytest.raises(ValueError):
        pod.pod_attn_peak_read(small, 1 << 20, 4, torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError):
        pod.pod_attn_peak_mfma(4, 8, torch.zeros(1, dtype=torch.int32))
