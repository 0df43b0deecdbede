"""Decode-unit numbering: the lookup that maps a decode wave's unit index to
(request, split, splits of the request, record base) must agree with a plain
enumeration of the units for every batch the planner accepts.

Units are numbered longest first (every request's full splits, request by
request, then the remainders); the record of (r, s) is base(r) + s with
base(r) = the splits of the requests before r.  The lookup scans packed
per-request counts 64 requests at a time (prefill_decode_hybrid_amd/csrc/
pod_units.h); the cases here include the largest counts one 64-request
group can hold (1023 splits each, 65472 in the group) and 32768 splits in a
group, where a signed 16/16 packing would overflow.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "native", "unit_scan_mirror.cpp")


@pytest.fixture(scope="module")
def mirror(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path_factory.mktemp("scan") / "unit_scan_mirror")
    subprocess.run([gxx, "-O2", "-std=c++17", "-Wall", "-Werror", SRC, "-o", exe], check=True)

    def run(lens, T):
        inp = f"{len(lens)} {T}\n" + " ".join(str(int(x)) for x in lens) + "\n"
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout.split("\n")
        return [ln for ln in out if ln]
    return run


def enumerate_units(lens, T):
    """The numbering written out: full splits request by request, then remainders."""
    lens = [int(x) for x in lens]
    S = [(L + T - 1) // T for L in lens]
    base = np.concatenate([[0], np.cumsum(S)[:-1]]).astype(int).tolist()
    units = []
    for r, L in enumerate(lens):
        for s in range(L // T):
            units.append((r, s, S[r], base[r]))
    for r, L in enumerate(lens):
        if L % T:
            units.append((r, L // T, S[r], base[r]))
    return units


def check(mirror, lens, T):
    got = mirror(lens, T)
    want = enumerate_units(lens, T)
    assert got[-1] == "miss", "a unit past the last must not be found"
    got = [tuple(int(x) for x in ln.split()) for ln in got[:-1]]
    assert len(got) == len(want)
    for u, (g, w) in enumerate(zip(got, want)):
        assert g == w, f"unit {u}: lookup {g}, enumeration {w}"
    # records: base + s covers 0 .. units-1 exactly once
    recs = sorted(b + s for _, s, _, b in got)
    assert recs == list(range(len(got)))


def test_group_of_32768_splits(mirror):
    # 64 decodes of 131072 tokens at T = 256 (512 splits each: 32768 in the
    # first scan group) plus 136 decodes of 16 tokens
    lens = [131072] * 64 + [16] * 136
    check(mirror, lens, 256)


def test_group_of_65472_splits(mirror):
    # the most one group can hold: 64 requests of 1023 splits, twice over,
    # with remainders in the second group
    lens = [1023 * 256] * 64 + [1023 * 256 - 5] * 64 + [3] * 7
    check(mirror, lens, 256)


def test_remainders_only(mirror):
    check(mirror, [100, 7, 255, 1], 256)


@pytest.mark.parametrize("seed", range(12))
def test_random_batches(mirror, seed):
    rng = np.random.default_rng(seed)
    T = int(rng.choice([256, 512, 1024, 2048, 4096]))
    N = int(rng.integers(1, 300))
    hi = min(261888, 1023 * T)
    kind = seed % 3
    if kind == 0:
        lens = rng.integers(1, hi + 1, size=N)
    elif kind == 1:
        lens = np.exp(rng.uniform(np.log(1), np.log(hi), size=N)).astype(int).clip(1, hi)
    else:
        lens = rng.choice([1, T - 1, T, T + 1, 2 * T, hi], size=N)
    check(mirror, lens.tolist(), T)
