"""Resource budget of the built kernels, read from the library's code-object
metadata on the CPU: the launch configuration assumes two 4-wave workgroups
per CU (at most 256 registers per lane and 80 KB of static LDS each), and a
kernel that spills to scratch memory runs several times slower."""
import os
import re

import pytest

import prefill_decode_hybrid_amd as pod
from prefill_decode_hybrid_amd import profiling

pytest.importorskip("msgpack")


@pytest.fixture(scope="module")
def res():
    pod.load()
    return profiling.kernel_resources(pod.LIB_PATH)


def _short(name):
    m = re.match(r"_ZN3pod\d+(pod_\w+_kernel)INS_\d+(\w+?)ELi(\d+)ELi(\d+)E", name)
    return m.groups() if m else None


def _short4(name):
    m = re.match(r"_ZN3pod\d+(pod_\w+4_kernel)ILi(\d+)ELi(\d+)E", name)
    return m.groups() if m else None


def test_every_instantiation_is_present(res):
    got = {_short(n) for n in res}
    for kind in ("pod_hybrid_kernel", "pod_prefill_kernel", "pod_decode_kernel", "pod_persistent_kernel"):
        for G in ("1", "2", "4", "8"):
            for D in ("64", "128"):
                assert (kind, "Bf16", D, G) in got
            assert (kind, "F32", "64", G) in got


def test_workgroups_fit_one_cu(res):
    # the two-workgroup envelope: <= 256 registers, <= 80 KB LDS per
    # workgroup; the four-workgroup kernels (pod_*4_kernel): <= 128, <= 40 KB
    for name, r in res.items():
        four = re.search(r"pod_\w+4_kernel", name) is not None
        assert r["vgpr"] + r["agpr"] <= (128 if four else 256), (name, r)
        assert r["lds"] <= (40 if four else 80) * 1024, (name, r)


def test_four_workgroup_kernels_are_built(res):
    got = {_short4(n) for n in res}
    for kind in ("pod_hybrid4_kernel", "pod_prefill4_kernel", "pod_decode4_kernel"):
        for D in ("64", "128"):
            for G in ("1", "2", "4", "8"):
                assert (kind, D, G) in got


def test_launched_kernels_use_no_scratch(res):
    # the optional persistent grid (bf16 d=128, G=8; fp32) keeps a few bytes
    for name, r in res.items():
        short, short4 = _short(name), _short4(name)
        if short is None and short4 is None:
            # the fill kernel of the allocation-free entry point and the two
            # measured-peak kernels
            assert re.search(r"pod_(zero|peak_read|peak_mfma)_kernel", name), name
        if short4 is not None and short4[0] == "pod_hybrid4_kernel" and short4[1] == "128":
            # a few values are kept in scratch across the decode loop (stored
            # once before it, reloaded once after it; the fused 128-register
            # kernel holds both roles)
            assert r["scratch"] <= 16, (name, r)
        elif short is None or short[0] != "pod_persistent_kernel":
            assert r["scratch"] == 0, (name, r)


def test_gpu_parity_cases_reach_every_instantiation(res):
    # every (dtype, head dim, group size) the library builds appears in a
    # small GPU parity case checked against the oracle
    from parity_cases import SMALL, instantiation
    built = {(t[1], int(t[2]), int(t[3])) for t in (_short(n) for n in res) if t}
    covered = {({"bf16": "Bf16", "f32": "F32"}[dt], d, G) for dt, d, G in map(instantiation, SMALL)}
    assert built == covered, f"built but not covered: {sorted(built - covered)}"
