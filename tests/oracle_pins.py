"""Pins for the fp64 oracle: checks against things other than the oracle itself.

Each pin_* function takes a loaded oracle library (ctypes) and raises
AssertionError if the oracle disagrees with what the mathematics fixes.
They are shared by test_oracle_pins.py (real oracle must pass every pin) and
test_oracle_mutants.py (each planted mistake must fail at least one pin).

The pages print no worked example with numbers, so the pins are:
  P1  brute force from the definition in 50-digit mpmath on tiny inputs
  P2  single visible key: output is that V row, exactly
  P3  two keys with weights 1/4 and 3/4 (hand-computable)
  P4  q = 0: output is the mean of the visible V rows (causal boundary of
      every prefill row, context length of every decode)
  P5  decoding chunk row i over context P0+i+1 equals prefill row i
  P6  invariants: shift of all keys, shift of all values, physical page
      permutation, GQA vs MHA with repeated KV heads
  P7  outputs lie in the convex hull of the visible V rows
  P8  torch's fp64 scaled_dot_product_attention on the gathered, contiguous
      KV (a library routine for the prefill special case)
  P9  one logit above all others by more than 750: output is that V row
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle

B16 = 16


# ----------------------------------------------------------------- builders
def to_bf16_exact(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 and return them as float64 (exact)."""
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def encode(x: np.ndarray, dtype: str):
    """float64 values (already representable) -> raw array for the oracle."""
    if dtype == "f32":
        return np.ascontiguousarray(x.astype(np.float32))
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().copy()


def paged(klog, vlog, page_size, rng, dtype="f32", permute=True):
    """Scatter per-request logical K/V ([L, Hkv, d] each) into a paged pool.

    Pages are handed out request by request; physical ids are a permutation
    drawn from rng.  Tail slots and one extra guard page are NaN.
    Returns (k_pool, v_pool, tables, guard) with pools in raw oracle form."""
    hkv, d = klog[0].shape[1], klog[0].shape[2]
    npg = [-(-k.shape[0] // page_size) for k in klog]
    total = sum(npg)
    phys = rng.permutation(total) if permute else np.arange(total)
    kp = np.full((total + 1, page_size, hkv, d), np.nan)
    vp = np.full((total + 1, page_size, hkv, d), np.nan)
    tables, at = [], 0
    for k, v, n in zip(klog, vlog, npg):
        ids = phys[at:at + n]
        at += n
        for j in range(k.shape[0]):
            kp[ids[j // page_size], j % page_size] = k[j]
            vp[ids[j // page_size], j % page_size] = v[j]
        tables.append(ids.astype(np.int32))
    return encode(kp, dtype), encode(vp, dtype), tables, total


def pad_tables(tables, guard):
    stride = max(len(t) for t in tables)
    out = np.full((len(tables), stride), guard, dtype=np.int32)
    for i, t in enumerate(tables):
        out[i, :len(t)] = t
    return out


def rand_vals(rng, shape, dtype, scale=1.0):
    x = rng.standard_normal(shape) * scale
    return x.astype(np.float32).astype(np.float64) if dtype == "f32" else to_bf16_exact(x)


def run_prefill(lib, q, kp, vp, table, P0, scale, dtype, rows=None):
    return oracle.prefill(encode(q, dtype), kp, vp, table, P0, scale, rows=rows, lib=lib)


def run_decode(lib, q, kp, vp, tables, ctx, scale, dtype, reqs=None):
    return oracle.decode(encode(q, dtype), kp, vp, tables, np.asarray(ctx, np.int32), scale,
                         reqs=reqs, lib=lib)


# ------------------------------------------------------------------ brute
def brute_attention(q, klog, vlog, visible, scale, hq):
    """mpmath, 50 digits, straight from the definition.

    q [Hq, d]; klog/vlog [L, Hkv, d] contiguous logical rows; visible: list of
    booleans per key.  KV heads are expanded to Hq by repetition (head h reads
    kv head h // (Hq/Hkv)).  Exponentials are not shifted."""
    import mpmath as mp
    mp.mp.dps = 50
    L, hkv, d = klog.shape
    G = hq // hkv
    kx = np.repeat(klog, G, axis=1)
    vx = np.repeat(vlog, G, axis=1)
    out = np.zeros((hq, d))
    for h in range(hq):
        num = [mp.mpf(0)] * d
        den = mp.mpf(0)
        for j in range(L):
            if not visible[j]:
                continue
            s = mp.mpf(scale) * mp.fsum(mp.mpf(float(q[h, k])) * mp.mpf(float(kx[j, h, k])) for k in range(d))
            e = mp.exp(s)
            den += e
            for k in range(d):
                num[k] += e * mp.mpf(float(vx[j, h, k]))
        for k in range(d):
            out[h, k] = float(num[k] / den)
    return out


def close(a, b, rel):
    a, b = np.asarray(a), np.asarray(b)
    assert np.all(np.isfinite(a)), "non-finite oracle output"
    err = np.max(np.abs(a - b) / (1.0 + np.abs(b)))
    assert err <= rel, f"max rel err {err:.3e} > {rel:.1e}"


# ------------------------------------------------------------------- pins
def pin_p1_brute(lib):
    rng = np.random.default_rng(1234)
    cases = [  # (d, Hq, Hkv, page_size, P0, C, decode lens, dtype)
        (1, 1, 1, 1, 0, 3, [1, 4], "f32"),
        (2, 2, 1, 2, 2, 3, [3, 5], "f32"),
        (4, 4, 2, 16, 1, 4, [6, 2], "bf16"),
        (4, 4, 2, 2, 3, 2, [5], "f32"),
        (2, 2, 1, 16, 0, 5, [6, 1, 3], "bf16"),
    ]
    for d, hq, hkv, B, P0, C, lens, dt in cases:
        Lp = P0 + C
        klog = [rand_vals(rng, (L, hkv, d), dt) for L in [Lp] + lens]
        vlog = [rand_vals(rng, (L, hkv, d), dt) for L in [Lp] + lens]
        kp, vp, tables, guard = paged(klog, vlog, B, rng, dt)
        scale = 1.0 / math.sqrt(d) if d > 1 else 0.7
        qp = rand_vals(rng, (C, hq, d), dt)
        got = run_prefill(lib, qp, kp, vp, tables[0], P0, scale, dt)
        for i in range(C):
            vis = [j <= P0 + i for j in range(Lp)]
            ref = brute_attention(qp[i], klog[0], vlog[0], vis, scale, hq)
            close(got[i], ref, 1e-13)
        qd = rand_vals(rng, (len(lens), hq, d), dt)
        got = run_decode(lib, qd, kp, vp, pad_tables(tables[1:], guard), lens, scale, dt)
        for r, L in enumerate(lens):
            ref = brute_attention(qd[r], klog[1 + r], vlog[1 + r], [True] * L, scale, hq)
            close(got[r], ref, 1e-13)


def pin_p2_single_key(lib):
    rng = np.random.default_rng(7)
    for dt in ("f32", "bf16"):
        d, hq, hkv = 8, 4, 2
        klog = [rand_vals(rng, (1, hkv, d), dt), rand_vals(rng, (5, hkv, d), dt)]
        vlog = [rand_vals(rng, (1, hkv, d), dt), rand_vals(rng, (5, hkv, d), dt)]
        kp, vp, tables, guard = paged(klog, vlog, 16, rng, dt)
        q = rand_vals(rng, (1, hq, d), dt)
        out = run_decode(lib, q, kp, vp, pad_tables(tables[:1], guard), [1], 0.3, dt)
        expect = np.repeat(vlog[0][0], hq // hkv, axis=0)
        assert np.array_equal(out[0], expect), "decode over one key must return that V row"
        # prefill row 0 at offset 0 sees only key 0 (of the second request)
        qp = rand_vals(rng, (5, hq, d), dt)
        out = run_prefill(lib, qp, kp, vp, tables[1], 0, 0.3, dt, rows=[0])
        expect = np.repeat(vlog[1][0], hq // hkv, axis=0)
        assert np.array_equal(out[0], expect), "prefill row 0 at offset 0 must return V_0"


def pin_p3_two_keys(lib):
    # d = 1, q = 1, keys (0, 1), scale ln 3 -> logits (0, ln 3) -> weights (1/4, 3/4)
    # values (1, 5): O = 1/4 + 15/4 = 4
    rng = np.random.default_rng(0)
    for dt in ("f32", "bf16"):
        klog = [np.array([[[0.0]], [[1.0]]])]
        vlog = [np.array([[[1.0]], [[5.0]]])]
        kp, vp, tables, guard = paged(klog, vlog, 16, rng, dt)
        q = np.ones((1, 1, 1))
        out = run_decode(lib, q, kp, vp, pad_tables(tables, guard), [2], math.log(3.0), dt)
        assert abs(out[0, 0, 0] - 4.0) <= 1e-15 * 4, out
        out = run_prefill(lib, q, kp, vp, tables[0], 1, math.log(3.0), dt)
        assert abs(out[0, 0, 0] - 4.0) <= 1e-15 * 4, out


def pin_p4_uniform(lib):
    rng = np.random.default_rng(11)
    d, hq, hkv, P0, C = 8, 4, 2, 23, 40
    lens = [1, 2, 15, 16, 17, 33, 64]
    for dt in ("f32", "bf16"):
        klog = [rand_vals(rng, (L, hkv, d), dt) for L in [P0 + C] + lens]
        vlog = [rand_vals(rng, (L, hkv, d), dt) for L in [P0 + C] + lens]
        kp, vp, tables, guard = paged(klog, vlog, 16, rng, dt)
        G = hq // hkv
        out = run_prefill(lib, np.zeros((C, hq, d)), kp, vp, tables[0], P0, 0.5, dt)
        for i in range(C):
            mean = vlog[0][:P0 + i + 1].mean(axis=0)  # [hkv, d]
            close(out[i], np.repeat(mean, G, axis=0), 1e-14)
        out = run_decode(lib, np.zeros((len(lens), hq, d)), kp, vp, pad_tables(tables[1:], guard),
                         lens, 0.5, dt)
        for r, L in enumerate(lens):
            close(out[r], np.repeat(vlog[1 + r].mean(axis=0), G, axis=0), 1e-14)


def pin_p5_consistency(lib):
    rng = np.random.default_rng(5)
    d, hq, hkv, P0, C = 16, 8, 2, 37, 29
    for dt in ("f32", "bf16"):
        klog = [rand_vals(rng, (P0 + C, hkv, d), dt)]
        vlog = [rand_vals(rng, (P0 + C, hkv, d), dt)]
        kp, vp, tables, guard = paged(klog, vlog, 16, rng, dt)
        qp = rand_vals(rng, (C, hq, d), dt)
        pre = run_prefill(lib, qp, kp, vp, tables[0], P0, 0.25, dt)
        ctx = [P0 + i + 1 for i in range(C)]
        pt = np.repeat(tables[0][None, :], C, axis=0)
        dec = run_decode(lib, qp, kp, vp, pt, ctx, 0.25, dt)
        close(dec, pre, 1e-14)


def pin_p6_invariants(lib):
    rng = np.random.default_rng(6)
    d, hq, hkv, P0, C = 8, 8, 2, 20, 12
    lens = [5, 31, 48]
    dt = "f32"
    # small integers keep K + b and V + c exact in f32
    klog = [rng.integers(-4, 5, size=(L, hkv, d)).astype(np.float64) for L in [P0 + C] + lens]
    vlog = [rng.integers(-4, 5, size=(L, hkv, d)).astype(np.float64) for L in [P0 + C] + lens]
    qp = rng.integers(-2, 3, size=(C, hq, d)).astype(np.float64)
    qd = rng.integers(-2, 3, size=(len(lens), hq, d)).astype(np.float64)
    scale = 0.3

    def both(kl, vl, perm_rng, permute=True, hkv_=hkv):
        kp, vp, tables, guard = paged(kl, vl, 16, perm_rng, dt, permute)
        a = run_prefill(lib, qp, kp, vp, tables[0], P0, scale, dt)
        b = run_decode(lib, qd, kp, vp, pad_tables(tables[1:], guard), lens, scale, dt)
        return a, b

    base = both(klog, vlog, np.random.default_rng(1))
    # (a) physical page permutation: bitwise identical
    other = both(klog, vlog, np.random.default_rng(99))
    assert np.array_equal(base[0], other[0]) and np.array_equal(base[1], other[1])
    # (b) K_j + b for every key: same output
    bvec = rng.integers(-3, 4, size=(hkv, d)).astype(np.float64)
    sh = both([k + bvec for k in klog], vlog, np.random.default_rng(1))
    close(sh[0], base[0], 1e-13)
    close(sh[1], base[1], 1e-13)
    # (c) V + c: output + c
    cvec = rng.integers(-3, 4, size=(hkv, d)).astype(np.float64)
    sv = both(klog, [v + cvec for v in vlog], np.random.default_rng(1))
    G = hq // hkv
    cexp = np.repeat(cvec, G, axis=0)
    close(sv[0], base[0] + cexp, 1e-13)
    close(sv[1], base[1] + cexp, 1e-13)
    # (d) GQA == MHA over KV heads repeated G times
    mk = [np.repeat(k, G, axis=1) for k in klog]
    mv = [np.repeat(v, G, axis=1) for v in vlog]
    mha = both(mk, mv, np.random.default_rng(1), hkv_=hq)
    assert np.array_equal(mha[0], base[0]) and np.array_equal(mha[1], base[1])


def pin_p7_convex(lib):
    rng = np.random.default_rng(8)
    d, hq, hkv, P0, C = 16, 4, 1, 50, 30
    lens = [3, 70, 129]
    for dt in ("f32", "bf16"):
        klog = [rand_vals(rng, (L, hkv, d), dt, 3.0) for L in [P0 + C] + lens]
        vlog = [rand_vals(rng, (L, hkv, d), dt) for L in [P0 + C] + lens]
        kp, vp, tables, guard = paged(klog, vlog, 16, rng, dt)
        qp = rand_vals(rng, (C, hq, d), dt, 3.0)
        qd = rand_vals(rng, (len(lens), hq, d), dt, 3.0)
        pre = run_prefill(lib, qp, kp, vp, tables[0], P0, 0.5, dt)
        dec = run_decode(lib, qd, kp, vp, pad_tables(tables[1:], guard), lens, 0.5, dt)
        eps = 1e-12
        for i in range(C):
            vis = vlog[0][:P0 + i + 1, 0]
            assert np.all(pre[i] >= vis.min(0) - eps) and np.all(pre[i] <= vis.max(0) + eps)
        for r, L in enumerate(lens):
            vis = vlog[1 + r][:, 0]
            assert np.all(dec[r] >= vis.min(0) - eps) and np.all(dec[r] <= vis.max(0) + eps)
        # weights sum to one: V = 1 everywhere gives O = 1
        ones = [np.ones_like(v) for v in vlog]
        kp, vp, tables, guard = paged(klog, ones, 16, rng, dt)
        pre = run_prefill(lib, qp, kp, vp, tables[0], P0, 0.5, dt)
        dec = run_decode(lib, qd, kp, vp, pad_tables(tables[1:], guard), lens, 0.5, dt)
        assert np.max(np.abs(pre - 1.0)) <= 1e-15 and np.max(np.abs(dec - 1.0)) <= 1e-15


def pin_p8_sdpa(lib):
    rng = np.random.default_rng(9)
    d, hq, hkv = 32, 8, 2
    G = hq // hkv
    for P0, C in ((0, 48), (45, 19)):
        for dt in ("f32", "bf16"):
            Lp = P0 + C
            klog = [rand_vals(rng, (Lp, hkv, d), dt)]
            vlog = [rand_vals(rng, (Lp, hkv, d), dt)]
            kp, vp, tables, guard = paged(klog, vlog, 16, rng, dt)
            qp = rand_vals(rng, (C, hq, d), dt)
            got = run_prefill(lib, qp, kp, vp, tables[0], P0, 1.0 / math.sqrt(d), dt)
            q = torch.from_numpy(qp).permute(1, 0, 2)[None]                       # [1, Hq, C, d]
            k = torch.from_numpy(np.repeat(klog[0], G, axis=1)).permute(1, 0, 2)[None]
            v = torch.from_numpy(np.repeat(vlog[0], G, axis=1)).permute(1, 0, 2)[None]
            F = torch.nn.functional
            if P0 == 0:
                ref = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=1.0 / math.sqrt(d))
            else:
                mask = torch.arange(Lp)[None, :] <= (P0 + torch.arange(C))[:, None]
                ref = F.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=1.0 / math.sqrt(d))
            close(got, ref[0].permute(1, 0, 2).numpy(), 1e-12)


def pin_p9_dominant(lib):
    rng = np.random.default_rng(10)
    for dt in ("f32", "bf16"):
        klog = [np.array([[[0.0]], [[-3.0]], [[800.0]], [[2.0]]])]
        vlog = [np.array([[[1.5]], [[-2.0]], [[0.75]], [[9.0]]])]
        kp, vp, tables, guard = paged(klog, vlog, 16, rng, dt)
        q = np.ones((1, 1, 1))
        out = run_decode(lib, q, kp, vp, pad_tables(tables, guard), [4], 1.0, dt)
        assert out[0, 0, 0] == 0.75, out
        out = run_prefill(lib, q, kp, vp, tables[0], 3, 1.0, dt)
        assert out[0, 0, 0] == 0.75, out


ALL_PINS = [pin_p1_brute, pin_p2_single_key, pin_p3_two_keys, pin_p4_uniform,
            pin_p5_consistency, pin_p6_invariants, pin_p7_convex, pin_p8_sdpa, pin_p9_dominant]
