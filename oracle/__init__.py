"""fp64 CPU oracle for hybrid-batch attention (test infrastructure).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg
import this package; the product path never does.  The arithmetic lives in
pod_oracle.c (plain C, fp64, OpenMP): the textbook definition of exact
softmax attention over a paged grouped-query KV cache, with the visible sets
of chunked prefill (keys j <= P0 + i for chunk row i) and decode (keys
j < L).  This file only marshals arrays into that library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pod_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

BF16, F32 = 0, 1


def build(src: str = _SRC, out: str = _LIB, extra=()) -> str:
    """Compile the oracle with gcc (no fast-math: fp64 semantics are kept)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", *extra, src, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path: Optional[str] = None):
    """Load (building first if missing or stale) and return the ctypes library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    P = ctypes.c_void_p
    i = ctypes.c_int
    lib.pod_oracle_prefill.argtypes = [i, i, i, i, i, P, P, P, P, i, i, ctypes.c_double, P, i, P, P]
    lib.pod_oracle_prefill.restype = i
    lib.pod_oracle_decode.argtypes = [i, i, i, i, i, P, P, P, P, i, P, i, ctypes.c_double, P, i, P, P]
    lib.pod_oracle_decode.restype = i
    return lib


def _raw(x):
    """Return (contiguous numpy array of raw element bits, dtype code)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy(), BF16
            if x.dtype == torch.float32:
                return x.numpy(), F32
            raise TypeError(f"unsupported dtype {x.dtype}")
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.float32:
        return x, F32
    if x.dtype in (np.uint16, np.int16):
        return x, BF16
    raise TypeError(f"unsupported dtype {x.dtype}")


def _i32(x):
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def prefill(q, k_pool, v_pool, page_table, chunk_offset: int, sm_scale: float,
            rows=None, with_lse: bool = False, lib=None):
    """Exact attention of chunk rows.  q [C, Hq, d]; pools [pages, B, Hkv, d].

    Returns out [nrows, Hq, d] float64 (and lse [nrows, Hq] if with_lse)."""
    lib = lib or load()
    qa, dt = _raw(q)
    ka, dtk = _raw(k_pool)
    va, dtv = _raw(v_pool)
    assert dt == dtk == dtv, "q, k and v must share a dtype"
    C, hq, d = qa.shape
    _, B, hkv, dk = ka.shape
    assert dk == d
    pt = _i32(page_table)
    r = _i32(rows)
    n = C if r is None else len(r)
    out = np.zeros((n, hq, d), dtype=np.float64)
    lse = np.zeros((n, hq), dtype=np.float64) if with_lse else None
    rc = lib.pod_oracle_prefill(dt, hq, hkv, d, B, _ptr(qa), _ptr(ka), _ptr(va), _ptr(pt),
                                C, int(chunk_offset), float(sm_scale), _ptr(r), n,
                                _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle prefill rejected its arguments")
    return (out, lse) if with_lse else out


def decode(q, k_pool, v_pool, page_table, context_lens, sm_scale: float,
           reqs=None, with_lse: bool = False, lib=None):
    """Exact attention of decode queries.  q [N, Hq, d]; page_table [N, stride].

    Returns out [nreqs, Hq, d] float64 (and lse [nreqs, Hq] if with_lse)."""
    lib = lib or load()
    qa, dt = _raw(q)
    ka, dtk = _raw(k_pool)
    va, dtv = _raw(v_pool)
    assert dt == dtk == dtv, "q, k and v must share a dtype"
    N, hq, d = qa.shape
    _, B, hkv, dk = ka.shape
    assert dk == d
    pt = _i32(page_table)
    ctx = _i32(context_lens)
    r = _i32(reqs)
    n = N if r is None else len(r)
    out = np.zeros((n, hq, d), dtype=np.float64)
    lse = np.zeros((n, hq), dtype=np.float64) if with_lse else None
    rc = lib.pod_oracle_decode(dt, hq, hkv, d, B, _ptr(qa), _ptr(ka), _ptr(va), _ptr(pt),
                               pt.shape[1], _ptr(ctx), N, float(sm_scale), _ptr(r), n,
                               _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle decode rejected its arguments")
    return (out, lse) if with_lse else out


def hybrid(batch, rows=None, reqs=None):
    """Both halves of a hybrid batch object (attributes as produced by the
    seeded generator).  Returns (out_prefill or None, out_decode or None)."""
    op = od = None
    if batch.q_prefill is not None:
        op = prefill(batch.q_prefill, batch.k_pool, batch.v_pool, batch.page_table_prefill,
                     batch.chunk_offset, batch.sm_scale, rows=rows)
    if batch.q_decode is not None:
        od = decode(batch.q_decode, batch.k_pool, batch.v_pool, batch.page_table_decode,
                    batch.context_lens, batch.sm_scale, reqs=reqs)
    return op, od
