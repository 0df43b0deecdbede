"""Decode-unit numbering: the lookup that maps a decode wave's unit index to
(request, split, splits of the request, record base, key range) must agree
with a plain enumeration of the units for every batch the planner accepts.

A request of L keys is cut into long splits of T keys from its start and a
tail cut into short splits of T2 keys: with k = 0 the tail is the remainder
L mod T (one split); with k = 1 it also takes the last full long split.
Units are numbered long splits first (every request's, request by request);
then, with k = 0, the remainders in request order (fused launches) or
longest first in eight length classes ([7T/8, T) first, [0, T/8) last;
request by request within a class; decode-only launches), or, with k = 1,
every request's short splits.  The record of (r, s) is
base(r) + s with base(r) = the splits of the requests before r.  The lookup
scans packed per-request counts 64 requests at a time
(prefill_decode_hybrid_amd/csrc/pod_units.h); the cases here include the
largest counts one 64-request group can hold (1023 splits each, 65472 in
the group) and 32768 splits in a group, where a signed 16/16 packing would
overflow.
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

    def run(lens, T, T2=None, k=0, nb=1):
        inp = f"{len(lens)} {T} {T2 or T} {k} {nb}\n" + " ".join(str(int(x)) for x in lens) + "\n"
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout.split("\n")
        return [ln for ln in out if ln]
    return run


def split_ranges(L, T, T2, k):
    """Key ranges of one request's splits, in split order."""
    F = L // T
    a = F - k if F > k else 0
    out = [(s * T, (s + 1) * T) for s in range(a)]
    t = a * T
    while t < L:
        out.append((t, min(L, t + T2)))
        t += T2
    return out, a


def enumerate_units(lens, T, T2=None, k=0, nb=1):
    """The numbering written out: long splits request by request, then the
    remainders (k = 0: in request order for nb = 1, by length class for
    nb = 8) or every request's short splits (k = 1)."""
    T2 = T2 or T
    lens = [int(x) for x in lens]
    per = [split_ranges(L, T, T2, k) for L in lens]
    S = [len(r) for r, _ in per]
    base = np.concatenate([[0], np.cumsum(S)[:-1]]).astype(int).tolist()
    units = []
    for r, (rng, a) in enumerate(per):
        for s in range(a):
            units.append((r, s, S[r], base[r]) + rng[s])
    if k == 0:
        classes = range(7, -1, -1) if nb == 8 else [None]
        for cls in classes:  # remainder length class floor(8 rem / T), longest first
            for r, (rng, a) in enumerate(per):
                if S[r] > a:
                    rem = rng[a][1] - rng[a][0]
                    if cls is None or (8 * rem) // T == cls:
                        units.append((r, a, S[r], base[r]) + rng[a])
    else:
        for r, (rng, a) in enumerate(per):
            for s in range(a, S[r]):
                units.append((r, s, S[r], base[r]) + rng[s])
    return units


def check(mirror, lens, T, T2=None, k=0, nb=None):
    if nb is None:  # both numberings of the remainders
        for b in (1, 8):
            check(mirror, lens, T, T2, k, b)
        return
    got = mirror(lens, T, T2, k, nb)
    want = enumerate_units(lens, T, T2, k, nb)
    assert got[-1] == "miss", "a unit past the last must not be found"
    got = [tuple(int(x) for x in ln.split()) for ln in got[:-1]]
    assert len(got) == len(want)
    for u, (g, w) in enumerate(zip(got, want)):
        assert g == w, f"unit {u}: lookup {g}, enumeration {w}"
    # records: base + s covers 0 .. units-1 exactly once
    recs = sorted(b + s for _, s, _, b, _, _ in got)
    assert recs == list(range(len(got)))
    # each request's splits tile its keys exactly
    for r, L in enumerate(lens):
        rng = sorted((t0, t1) for rr, _, _, _, t0, t1 in got if rr == r)
        assert rng[0][0] == 0 and rng[-1][1] == L
        assert all(x[1] == y[0] for x, y in zip(rng, rng[1:]))


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


def test_tail_splits_long_context_batch(mirror):
    # 64 decodes of 16K at T = 4096 with the tail in quarters: three long
    # splits and four 1024-token short splits per request
    lens = [16384] * 64
    check(mirror, lens, 4096, 1024, 1)
    want = enumerate_units(lens, 4096, 1024, 1)
    assert sum(1 for u in want if u[5] - u[4] == 4096) == 64 * 3
    assert len(want) == 64 * 7


def test_tail_splits_short_requests(mirror):
    # requests shorter than two long splits are all tail
    check(mirror, [1, 15, 16, 1023, 1024, 2047, 2048, 2049, 4095, 5000], 1024, 256, 1)


@pytest.mark.parametrize("seed", range(12))
def test_random_batches_with_tail_splits(mirror, seed):
    rng = np.random.default_rng(100 + seed)
    T = int(rng.choice([1024, 2048, 3280, 4096]))
    T2 = max(256, -(-T // 4 // 16) * 16) if seed % 2 else int(rng.choice([256, 512, T // 2 // 16 * 16]))
    N = int(rng.integers(1, 300))
    hi = 261888
    if seed % 3 == 0:
        lens = rng.integers(1, hi + 1, size=N)
    elif seed % 3 == 1:
        lens = np.exp(rng.uniform(0, np.log(hi), size=N)).astype(int).clip(1, hi)
    else:
        lens = rng.choice([1, T2 - 1, T2, T - 1, T, T + 1, 2 * T - 1, 2 * T, 2 * T + 1, hi], size=N)
    check(mirror, lens.tolist(), T, T2, 1)
