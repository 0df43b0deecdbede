"""Seeded synthetic hybrid batches: one chunked-prefill request (or several,
with a "chunks" list) plus N decodes over a paged GQA KV cache.

This module only draws numbers and lays them out; it holds none of the
attention arithmetic. Both the HIP path and the fp64 oracle consume what it
returns, so the two sides always see bit-identical inputs.

Workload shapes follow the POD-Attention pages: a hybrid batch holds one
prefill chunk plus many decodes (paper §2.1, "Chunked-prefill hybrid
batching"), the KV cache is paged (PagedAttention, listed among the works the
paper builds on) and heads are grouped (GQA, same list). Llama-3-8B shapes
(32 query / 8 KV heads, head dim 128) come from the models named in the
artifact checklist (§A.2) and the split-limiting study (§5.4.3, Table 8).

Readings where the pages are silent:
  * K = 1024 tokens ("16K" = 16384).
  * Softmax scale = 1/sqrt(d).
  * A request's own K/V (including the prefill chunk's and each decode's
    current token) are already in the pool.
  * Pool pages are handed out prefill request(s) first, then decodes in order;
    physical ids are a seeded permutation (identity for "contiguous KV").
  * Slots past a request's length in its last page are NaN, page-table
    padding points at one extra all-NaN guard page, so a kernel that reads
    or weights an invisible key shows up as a NaN.
  * Independent sub-streams come from SeedSequence(seed).spawn(7) in the
    order [q_prefill, q_decode, k_pool, v_pool, lengths, permutation,
    outliers].
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch

PAGE_SIZE = 16
KTOK = 1024  # "K" in 16K, 32K ... is a binary thousand

# The five workloads. Each is a plain dict so tests can build variants.
CONFIGS = {
    1: dict(name="tiny_fp32", dtype="f32", num_q_heads=8, num_kv_heads=2, head_dim=64,
            chunk_len=64, chunk_offset=64, decode_lens=[37, 100, 256, 511],
            contiguous=True, input_scale=1.0, sm_scale=1.0 / 8.0, k_outlier_frac=0.0),
    2: dict(name="llama3_8b_c512", dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
            chunk_len=512, chunk_offset=0, decode_lens=("uniform", 32, 1 * KTOK, 4 * KTOK),
            contiguous=False, input_scale=1.0, sm_scale=None, k_outlier_frac=0.0),
    3: dict(name="long_ctx_16k", dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
            chunk_len=1 * KTOK, chunk_offset=15 * KTOK, decode_lens=[16 * KTOK] * 64,
            contiguous=False, input_scale=1.0, sm_scale=None, k_outlier_frac=0.01),
    4: dict(name="decode_heavy", dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128,
            chunk_len=256, chunk_offset=2 * KTOK, decode_lens=("loguniform", 256, 128, 32 * KTOK),
            contiguous=False, input_scale=1.0, sm_scale=None, k_outlier_frac=0.0),
    5: dict(name="prefill_heavy_gqa8", dtype="bf16", num_q_heads=64, num_kv_heads=8, head_dim=128,
            chunk_len=2 * KTOK, chunk_offset=30 * KTOK, decode_lens=[32 * KTOK] * 16,
            contiguous=False, input_scale=1.0, sm_scale=None, k_outlier_frac=0.0),
}

_STREAMS = ("q_prefill", "q_decode", "k_pool", "v_pool", "lengths", "permutation", "outliers")
_GEN_CHUNK_PAGES = 2048  # fixed so the draw order never depends on memory


@dataclasses.dataclass
class HybridBatch:
    """One hybrid batch, all tensors on the CPU.

    q_prefill   [C, Hq, d]            dtype (several chunks: their rows back to back)
    q_decode    [N, Hq, d]            dtype
    k_pool      [num_pages+1, B, Hkv, d]  (last page = NaN guard)
    v_pool      same as k_pool
    page_table_prefill [ceil((P0+C)/B)] int32 (several chunks: [n, stride],
                                        padding -> guard page)
    page_table_decode  [N, stride]      int32 (padding -> guard page)
    context_lens       [N]              int32
    """
    spec: dict
    dtype: torch.dtype
    q_prefill: Optional[torch.Tensor]
    q_decode: Optional[torch.Tensor]
    k_pool: torch.Tensor
    v_pool: torch.Tensor
    page_table_prefill: Optional[torch.Tensor]
    page_table_decode: Optional[torch.Tensor]
    context_lens: Optional[torch.Tensor]
    chunk_len: int
    chunk_offset: int
    sm_scale: float
    guard_page: int
    outlier_rows: int = 0
    chunks: Optional[list] = None  # several chunks: [(chunk_len, chunk_offset), ...]

    @property
    def num_q_heads(self): return self.spec["num_q_heads"]
    @property
    def num_kv_heads(self): return self.spec["num_kv_heads"]
    @property
    def head_dim(self): return self.spec["head_dim"]
    @property
    def num_decode(self): return 0 if self.context_lens is None else int(self.context_lens.numel())
    @property
    def num_pages(self): return int(self.k_pool.shape[0])

    def to(self, device) -> "HybridBatch":
        def mv(t):
            return None if t is None else t.to(device)
        return dataclasses.replace(
            self, q_prefill=mv(self.q_prefill), q_decode=mv(self.q_decode),
            k_pool=mv(self.k_pool), v_pool=mv(self.v_pool),
            page_table_prefill=mv(self.page_table_prefill),
            page_table_decode=mv(self.page_table_decode),
            context_lens=mv(self.context_lens))

    # ---- work counts (used for reporting; nothing here is attention math) ----
    def chunk_list(self) -> list:
        """[(chunk_len, chunk_offset)] of every prefill chunk ([] without prefill)."""
        if self.q_prefill is None:
            return []
        return list(self.chunks) if self.chunks is not None else [(self.chunk_len, self.chunk_offset)]

    def visible_keys_prefill(self) -> int:
        return sum(c * p0 + c * (c + 1) // 2 for c, p0 in self.chunk_list())

    def kv_tokens(self) -> int:
        lp = sum(c + p0 for c, p0 in self.chunk_list())
        ld = 0 if self.context_lens is None else int(self.context_lens.sum())
        return lp + ld


def _torch_dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def _draw_lengths(rule, rng: np.random.Generator) -> np.ndarray:
    if isinstance(rule, (list, tuple)) and rule and isinstance(rule[0], str):
        kind, n, lo, hi = rule
        if kind == "uniform":  # integers uniform on [lo, hi], both ends included
            return rng.integers(lo, hi + 1, size=n).astype(np.int64)
        if kind == "loguniform":  # floor(exp(U(ln lo, ln hi))), clipped to [lo, hi]
            u = rng.uniform(math.log(lo), math.log(hi), size=n)
            return np.clip(np.floor(np.exp(u)), lo, hi).astype(np.int64)
        raise ValueError(f"unknown length rule {kind}")
    return np.asarray(list(rule), dtype=np.int64)


def _normal(rng: np.random.Generator, shape, scale: float) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


def _fill_pool(rng, num_pages, B, hkv, d, scale, dtype) -> torch.Tensor:
    pool = torch.empty((num_pages + 1, B, hkv, d), dtype=dtype)
    for p0 in range(0, num_pages, _GEN_CHUNK_PAGES):
        p1 = min(num_pages, p0 + _GEN_CHUNK_PAGES)
        x = _normal(rng, (p1 - p0, B, hkv, d), scale)
        pool[p0:p1] = torch.from_numpy(x).to(dtype)
    pool[num_pages] = float("nan")
    return pool


def make_batch(spec, seed: int = 0, with_prefill: bool = True, with_decode: bool = True) -> HybridBatch:
    """Build the hybrid batch for `spec` (a config id 1..5 or a dict)."""
    if isinstance(spec, int):
        spec = dict(CONFIGS[spec])
    else:
        spec = dict(spec)
    B = spec.get("page_size", PAGE_SIZE)
    hq, hkv, d = spec["num_q_heads"], spec["num_kv_heads"], spec["head_dim"]
    dtype = _torch_dtype(spec["dtype"])
    scale = float(spec.get("input_scale", 1.0))
    sm_scale = spec.get("sm_scale")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)

    ss = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    rngs = {name: np.random.Generator(np.random.PCG64(s)) for name, s in zip(_STREAMS, ss)}

    multi = spec.get("chunks") is not None
    if multi:
        chunks = [(int(c), int(p)) for c, p in spec["chunks"]]
        C, P0 = sum(c for c, _ in chunks), 0
    else:
        C, P0 = int(spec["chunk_len"]), int(spec["chunk_offset"])
        chunks = [(C, P0)]
    lens = _draw_lengths(spec["decode_lens"], rngs["lengths"]) if with_decode else np.zeros(0, np.int64)
    N = len(lens)
    n_pre = len(chunks) if with_prefill else 0

    # logical page lists: prefill request(s) first, then decodes in order
    req_lens = ([c + p for c, p in chunks] if with_prefill else []) + [int(x) for x in lens]
    req_pages = [-(-L // B) for L in req_lens]
    num_pages = int(sum(req_pages))
    if spec.get("contiguous", False):
        phys = np.arange(num_pages, dtype=np.int64)
    else:
        phys = rngs["permutation"].permutation(num_pages).astype(np.int64)
    guard = num_pages

    k_pool = _fill_pool(rngs["k_pool"], num_pages, B, hkv, d, scale, dtype)
    v_pool = _fill_pool(rngs["v_pool"], num_pages, B, hkv, d, scale, dtype)

    # per-request physical page ids
    starts = np.concatenate([[0], np.cumsum(req_pages)]).astype(np.int64)
    req_phys = [phys[starts[i]:starts[i + 1]] for i in range(len(req_lens))]

    # NaN tails past each request's length
    for L, pages in zip(req_lens, req_phys):
        tail = L % B
        if tail:
            k_pool[int(pages[-1]), tail:] = float("nan")
            v_pool[int(pages[-1]), tail:] = float("nan")

    # outliers: a fraction of the valid (token, kv-head) K rows scaled by 8
    n_out = 0
    frac = float(spec.get("k_outlier_frac", 0.0))
    if frac > 0:
        rows_per_req = np.asarray(req_lens, dtype=np.int64) * hkv
        n_rows = int(rows_per_req.sum())
        n_out = int(round(frac * n_rows))
        pick = rngs["outliers"].choice(n_rows, size=n_out, replace=False)
        cum = np.concatenate([[0], np.cumsum(rows_per_req)])
        req = np.searchsorted(cum, pick, side="right") - 1
        local = pick - cum[req]
        tok, head = local // hkv, local % hkv
        page_idx = tok // B
        phys_page = np.array([req_phys[r][p] for r, p in zip(req.tolist(), page_idx.tolist())], dtype=np.int64)
        slot = tok % B
        kp = k_pool.view(-1, hkv, d)  # [(page*B+slot), hkv, d]
        flat = torch.from_numpy(phys_page * B + slot)
        hh = torch.from_numpy(head)
        kp[flat, hh] = kp[flat, hh] * 8  # power of two: exact in bf16 and f32

    pt_p = None
    q_p = None
    if with_prefill:
        if multi:
            pt = np.full((n_pre, max(req_pages[:n_pre])), guard, dtype=np.int32)
            for i in range(n_pre):
                pt[i, :len(req_phys[i])] = req_phys[i]
            pt_p = torch.from_numpy(pt)
        else:
            pt_p = torch.from_numpy(req_phys[0].astype(np.int32))
        q_p = torch.from_numpy(_normal(rngs["q_prefill"], (C, hq, d), scale)).to(dtype)

    pt_d = q_d = ctx = None
    if with_decode and N > 0:
        first = n_pre
        stride = max(req_pages[first:])
        pt = np.full((N, stride), guard, dtype=np.int32)
        for i in range(N):
            pg = req_phys[first + i]
            pt[i, :len(pg)] = pg
        pt_d = torch.from_numpy(pt)
        ctx = torch.from_numpy(lens.astype(np.int32))
        q_d = torch.from_numpy(_normal(rngs["q_decode"], (N, hq, d), scale)).to(dtype)

    return HybridBatch(spec=spec, dtype=dtype, q_prefill=q_p, q_decode=q_d,
                       k_pool=k_pool, v_pool=v_pool, page_table_prefill=pt_p,
                       page_table_decode=pt_d, context_lens=ctx,
                       chunk_len=C if with_prefill else 0,
                       chunk_offset=P0 if with_prefill else 0,
                       sm_scale=float(sm_scale), guard_page=guard, outlier_rows=n_out,
                       chunks=chunks if (multi and with_prefill) else None)


def draw_context_lens(spec, seed: int = 0) -> np.ndarray:
    """The decode context lengths make_batch(spec, seed) would draw (no pools)."""
    if isinstance(spec, int):
        spec = dict(CONFIGS[spec])
    ss = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    rng = np.random.Generator(np.random.PCG64(ss[_STREAMS.index("lengths")]))
    return _draw_lengths(spec["decode_lens"], rng)


def describe(b: HybridBatch) -> dict:
    """Small JSON-able summary of a batch (sizes and drawn lengths)."""
    lens = [] if b.context_lens is None else b.context_lens.tolist()
    return dict(name=b.spec.get("name", "custom"), dtype=b.spec["dtype"],
                num_q_heads=b.num_q_heads, num_kv_heads=b.num_kv_heads, head_dim=b.head_dim,
                chunk_len=b.chunk_len, chunk_offset=b.chunk_offset, num_decode=b.num_decode,
                sum_context=int(sum(lens)), min_context=min(lens) if lens else 0,
                max_context=max(lens) if lens else 0, num_pages=b.num_pages,
                sm_scale=b.sm_scale, k_outlier_rows=b.outlier_rows)
