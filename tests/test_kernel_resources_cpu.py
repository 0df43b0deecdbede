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


def test_every_instantiation_is_present(res):
    got = {_short(n) for n in res}
    for kind in ("pod_hybrid_kernel", "pod_prefill_kernel", "pod_decode_kernel", "pod_persistent_kernel"):
        for G in ("1", "2", "4", "8"):
            for D in ("64", "128"):
                assert (kind, "Bf16", D, G) in got
            assert (kind, "F32", "64", G) in got


def test_two_workgroups_fit_one_cu(res):
    for name, r in res.items():
        assert r["vgpr"] + r["agpr"] <= 256, (name, r)
        assert r["lds"] <= 80 * 1024, (name, r)


def test_launched_kernels_use_no_scratch(res):
    # the optional persistent grid (bf16 d=128, G=8; fp32) keeps a few bytes
    for name, r in res.items():
        short = _short(name)
        if short is None:  # the fill kernel of the allocation-free entry point
            assert "pod_zero_kernel" in name, name
        if short is None or short[0] != "pod_persistent_kernel":
            assert r["scratch"] == 0, (name, r)


def test_gpu_parity_cases_reach_every_instantiation(res):
    # every (dtype, head dim, group size) the library builds appears in a
    # small GPU parity case checked against the oracle
    from parity_cases import SMALL, instantiation
    built = {(t[1], int(t[2]), int(t[3])) for t in (_short(n) for n in res) if t}
    covered = {({"bf16": "Bf16", "f32": "F32"}[dt], d, G) for dt, d, G in map(instantiation, SMALL)}
    assert built == covered, f"built but not covered: {sorted(built - covered)}"
