"""Python binding of the hybrid-batch attention library (libpodattn.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/pod_attn.h.  The functions keep
the C names (pod_attn_create, pod_attn_hybrid, pod_attn_prefill_only,
pod_attn_decode_only, ...) and take torch tensors that already live on the
GPU; torch supplies device memory and streams, nothing else.

Importing this module never loads a CPU fallback: if the library is missing
the calls raise, loudly.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpodattn.so")

POD_OK, POD_ERR_INVALID_ARG, POD_ERR_UNSUPPORTED, POD_ERR_WORKSPACE, POD_ERR_HIP = 0, -1, -2, -3, -4
POD_BF16, POD_F32 = 0, 1
POD_POLICY_CU_BALANCED, POD_POLICY_PROPORTIONAL, POD_POLICY_HALF, POD_POLICY_STATIC = 0, 1, 2, 3
MODE_HYBRID, MODE_PREFILL, MODE_DECODE = 0, 1, 2

POD_MAX_CHUNKS = 64

EXPORTED = ("pod_attn_create", "pod_attn_destroy", "pod_attn_hybrid", "pod_attn_prefill_only",
            "pod_attn_decode_only", "pod_attn_hybrid_noalloc", "pod_attn_hybrid_varlen", "pod_attn_prefill_only_varlen",
            "pod_attn_get_stats", "pod_attn_role_trace", "pod_attn_plan", "pod_attn_plan_varlen",
            "pod_attn_status_string", "pod_attn_last_error", "pod_attn_peak_read", "pod_attn_peak_mfma")


class PodAttnConfig(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("sm_scale", ctypes.c_float),
                ("max_chunk_len", ctypes.c_int32), ("max_num_decode", ctypes.c_int32),
                ("max_context", ctypes.c_int32), ("max_total_context", ctypes.c_int64),
                ("wg_per_cu", ctypes.c_int32), ("prefill_split_cap_waves", ctypes.c_int32),
                ("policy", ctypes.c_int32), ("device", ctypes.c_int32),
                ("prefill_slots_x256", ctypes.c_int32), ("decode_split_tokens", ctypes.c_int32),
                ("persistent", ctypes.c_int32), ("prefill_splits", ctypes.c_int32),
                ("record_roles", ctypes.c_int32), ("decode_tail_split_tokens", ctypes.c_int32)]


class PodTaskRecord(ctypes.Structure):
    _fields_ = [("cu_key", ctypes.c_uint32), ("role", ctypes.c_int32), ("task", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("start", ctypes.c_uint64), ("end", ctypes.c_uint64)]


class PodPrefillArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("o", ctypes.c_void_p), ("page_table", ctypes.c_void_p),
                ("chunk_len", ctypes.c_int32), ("chunk_offset", ctypes.c_int32)]


class PodDecodeArgs(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("o", ctypes.c_void_p), ("page_table", ctypes.c_void_p),
                ("page_table_stride", ctypes.c_int32), ("context_lens", ctypes.c_void_p),
                ("context_lens_host", ctypes.c_void_p), ("num_decode", ctypes.c_int32)]


class PodPrefillBatch(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("o", ctypes.c_void_p), ("page_table", ctypes.c_void_p),
                ("page_table_stride", ctypes.c_int32), ("chunk_lens_host", ctypes.c_void_p),
                ("chunk_offsets_host", ctypes.c_void_p), ("num_chunks", ctypes.c_int32)]


class PodAttnStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "mode", "fallback", "num_cus", "wg_per_cu", "grid", "prefill_rows_per_tile",
        "prefill_heads_per_tile", "prefill_tiles", "prefill_splits", "prefill_split_keys",
        "prefill_tasks", "decode_split_tokens", "decode_wave_tasks", "decode_wg_tasks",
        "share_num", "share_den", "cu_prefill_x256", "policy", "prefill_chunks", "persistent",
        "fixed_order", "prefill_priority", "decode_tail_split_tokens", "decode_unit_classes")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class PodAttnError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str = ""):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})" + (f": {detail}" if detail else ""))


_lib = None


def load(path: str = LIB_PATH):
    """Load libpodattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m prefill_decode_hybrid_amd.build`")
    lib = ctypes.CDLL(path)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.pod_attn_create.argtypes = [ctypes.POINTER(PodAttnConfig), ctypes.POINTER(ctypes.c_void_p)]
    lib.pod_attn_destroy.argtypes = [P]
    lib.pod_attn_hybrid.argtypes = [P, P, P, i64, ctypes.POINTER(PodPrefillArgs),
                                    ctypes.POINTER(PodDecodeArgs), P]
    lib.pod_attn_hybrid_noalloc.argtypes = [ctypes.POINTER(PodAttnConfig), P, P, i64, ctypes.POINTER(PodPrefillArgs),
                                            ctypes.POINTER(PodDecodeArgs), P]
    lib.pod_attn_prefill_only.argtypes = [P, P, P, i64, ctypes.POINTER(PodPrefillArgs), P]
    lib.pod_attn_decode_only.argtypes = [P, P, P, i64, ctypes.POINTER(PodDecodeArgs), P]
    lib.pod_attn_hybrid_varlen.argtypes = [P, P, P, i64, ctypes.POINTER(PodPrefillBatch),
                                           ctypes.POINTER(PodDecodeArgs), P]
    lib.pod_attn_prefill_only_varlen.argtypes = [P, P, P, i64, ctypes.POINTER(PodPrefillBatch), P]
    lib.pod_attn_plan_varlen.argtypes = [ctypes.POINTER(PodAttnConfig), i32, i32, ctypes.POINTER(PodPrefillBatch),
                                         ctypes.POINTER(PodDecodeArgs), ctypes.POINTER(PodAttnStats)]
    lib.pod_attn_get_stats.argtypes = [P, ctypes.POINTER(PodAttnStats)]
    lib.pod_attn_role_trace.argtypes = [P, ctypes.POINTER(PodTaskRecord), i32, ctypes.POINTER(i32)]
    lib.pod_attn_plan.argtypes = [ctypes.POINTER(PodAttnConfig), i32, i32, ctypes.POINTER(PodPrefillArgs),
                                  ctypes.POINTER(PodDecodeArgs), ctypes.POINTER(PodAttnStats)]
    lib.pod_attn_status_string.argtypes = [ctypes.c_int]
    lib.pod_attn_status_string.restype = ctypes.c_char_p
    lib.pod_attn_last_error.argtypes = [P]
    lib.pod_attn_last_error.restype = ctypes.c_char_p
    lib.pod_attn_peak_read.argtypes = [P, i64, i32, P, P]
    lib.pod_attn_peak_mfma.argtypes = [i32, i32, P, P]
    for name in ("pod_attn_create", "pod_attn_destroy", "pod_attn_hybrid", "pod_attn_hybrid_noalloc",
                 "pod_attn_prefill_only", "pod_attn_decode_only", "pod_attn_hybrid_varlen",
                 "pod_attn_prefill_only_varlen", "pod_attn_get_stats", "pod_attn_role_trace", "pod_attn_plan",
                 "pod_attn_plan_varlen", "pod_attn_peak_read", "pod_attn_peak_mfma"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    try:
        return load().pod_attn_status_string(status).decode()
    except RuntimeError:
        return str(status)


def make_config(dtype=POD_BF16, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16,
                sm_scale=0.0, max_chunk_len=4096, max_num_decode=256, max_context=32768,
                max_total_context=0, wg_per_cu=0, prefill_split_cap_waves=0,
                policy=POD_POLICY_CU_BALANCED, device=-1, prefill_slots_x256=0,
                decode_split_tokens=0, persistent=0, prefill_splits=0, record_roles=0,
                decode_tail_split_tokens=0) -> PodAttnConfig:
    return PodAttnConfig(dtype, num_q_heads, num_kv_heads, head_dim, page_size, sm_scale,
                         max_chunk_len, max_num_decode, max_context, max_total_context,
                         wg_per_cu, prefill_split_cap_waves, policy, device, prefill_slots_x256,
                         decode_split_tokens, persistent, prefill_splits, record_roles,
                         decode_tail_split_tokens)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def prefill_args(q, o, page_table, chunk_offset: int) -> PodPrefillArgs:
    return PodPrefillArgs(_ptr(q), _ptr(o), _ptr(page_table), int(q.shape[0]), int(chunk_offset))


def prefill_batch(q, o, page_table, chunks) -> PodPrefillBatch:
    """chunks: [(chunk_len, chunk_offset)] in row order; page_table: device int32 [n, stride]."""
    import numpy as np
    lens = np.ascontiguousarray([c for c, _ in chunks], dtype=np.int32)
    offs = np.ascontiguousarray([p for _, p in chunks], dtype=np.int32)
    a = PodPrefillBatch(_ptr(q), _ptr(o), _ptr(page_table), int(page_table.shape[1]), lens.ctypes.data,
                        offs.ctypes.data, len(chunks))
    a._keep = (lens, offs)  # the host arrays live as long as the struct
    return a


def decode_args(q, o, page_table, context_lens, context_lens_host) -> PodDecodeArgs:
    """context_lens: device int32 [N]; context_lens_host: CPU int32 tensor with the same values."""
    assert context_lens_host.device.type == "cpu" and context_lens_host.is_contiguous()
    return PodDecodeArgs(_ptr(q), _ptr(o), _ptr(page_table), int(page_table.shape[1]),
                         _ptr(context_lens), context_lens_host.data_ptr(), int(q.shape[0]))


def _stream_ptr(stream) -> Optional[int]:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def pod_attn_create(cfg: PodAttnConfig) -> ctypes.c_void_p:
    lib = load()
    h = ctypes.c_void_p()
    rc = lib.pod_attn_create(ctypes.byref(cfg), ctypes.byref(h))
    if rc != POD_OK:
        raise PodAttnError(rc, "pod_attn_create")
    return h


def pod_attn_destroy(h) -> None:
    rc = load().pod_attn_destroy(h)
    if rc != POD_OK:
        raise PodAttnError(rc, "pod_attn_destroy")


def _check(h, rc, what):
    if rc != POD_OK:
        detail = load().pod_attn_last_error(h).decode() if h else ""
        raise PodAttnError(rc, what, detail)


def pod_attn_hybrid(h, k_pool, v_pool, prefill: Optional[PodPrefillArgs], decode: Optional[PodDecodeArgs],
                    stream=None) -> None:
    lib = load()
    rc = lib.pod_attn_hybrid(h, _ptr(k_pool), _ptr(v_pool), int(k_pool.shape[0]),
                             ctypes.byref(prefill) if prefill is not None else None,
                             ctypes.byref(decode) if decode is not None else None, _stream_ptr(stream))
    _check(h, rc, "pod_attn_hybrid")


def pod_attn_hybrid_noalloc(cfg: PodAttnConfig, k_pool, v_pool, prefill: Optional[PodPrefillArgs],
                            decode: Optional[PodDecodeArgs], stream=None) -> None:
    """pod_attn_hybrid without a handle: workspace in the library's fixed device scratch."""
    rc = load().pod_attn_hybrid_noalloc(ctypes.byref(cfg), _ptr(k_pool), _ptr(v_pool), int(k_pool.shape[0]),
                                        ctypes.byref(prefill) if prefill is not None else None,
                                        ctypes.byref(decode) if decode is not None else None, _stream_ptr(stream))
    if rc != POD_OK:
        raise PodAttnError(rc, "pod_attn_hybrid_noalloc")


def pod_attn_prefill_only(h, k_pool, v_pool, prefill: PodPrefillArgs, stream=None) -> None:
    rc = load().pod_attn_prefill_only(h, _ptr(k_pool), _ptr(v_pool), int(k_pool.shape[0]),
                                      ctypes.byref(prefill), _stream_ptr(stream))
    _check(h, rc, "pod_attn_prefill_only")


def pod_attn_decode_only(h, k_pool, v_pool, decode: PodDecodeArgs, stream=None) -> None:
    rc = load().pod_attn_decode_only(h, _ptr(k_pool), _ptr(v_pool), int(k_pool.shape[0]),
                                     ctypes.byref(decode), _stream_ptr(stream))
    _check(h, rc, "pod_attn_decode_only")


def pod_attn_hybrid_varlen(h, k_pool, v_pool, prefill: Optional[PodPrefillBatch],
                           decode: Optional[PodDecodeArgs], stream=None) -> None:
    rc = load().pod_attn_hybrid_varlen(h, _ptr(k_pool), _ptr(v_pool), int(k_pool.shape[0]),
                                       ctypes.byref(prefill) if prefill is not None else None,
                                       ctypes.byref(decode) if decode is not None else None, _stream_ptr(stream))
    _check(h, rc, "pod_attn_hybrid_varlen")


def pod_attn_prefill_only_varlen(h, k_pool, v_pool, prefill: PodPrefillBatch, stream=None) -> None:
    rc = load().pod_attn_prefill_only_varlen(h, _ptr(k_pool), _ptr(v_pool), int(k_pool.shape[0]),
                                             ctypes.byref(prefill), _stream_ptr(stream))
    _check(h, rc, "pod_attn_prefill_only_varlen")


def pod_attn_get_stats(h) -> dict:
    st = PodAttnStats()
    _check(h, load().pod_attn_get_stats(h, ctypes.byref(st)), "pod_attn_get_stats")
    return st.as_dict()


def pod_attn_role_trace(h) -> list:
    """Task records of the last fused call of a recording handle:
    [(cu_key, role, task, start, end)], start/end in 100 MHz ticks."""
    lib = load()
    count = ctypes.c_int32(0)
    _check(h, lib.pod_attn_role_trace(h, None, 0, ctypes.byref(count)), "pod_attn_role_trace")
    n = count.value
    recs = (PodTaskRecord * max(1, n))()
    _check(h, lib.pod_attn_role_trace(h, recs, n, ctypes.byref(count)), "pod_attn_role_trace")
    return [(r.cu_key, r.role, r.task, r.start, r.end) for r in recs[:n]]


def pod_attn_plan(cfg: PodAttnConfig, num_cus: int, mode: int, prefill=None, decode=None) -> dict:
    """Host-only plan (no GPU needed).  Raises PodAttnError on invalid arguments."""
    st = PodAttnStats()
    rc = load().pod_attn_plan(ctypes.byref(cfg), int(num_cus), int(mode),
                              ctypes.byref(prefill) if prefill is not None else None,
                              ctypes.byref(decode) if decode is not None else None, ctypes.byref(st))
    if rc != POD_OK:
        raise PodAttnError(rc, "pod_attn_plan")
    return st.as_dict()


def pod_attn_plan_varlen(cfg: PodAttnConfig, num_cus: int, mode: int, prefill=None, decode=None) -> dict:
    """Host-only plan of a several-chunk call (no GPU needed)."""
    st = PodAttnStats()
    rc = load().pod_attn_plan_varlen(ctypes.byref(cfg), int(num_cus), int(mode),
                                     ctypes.byref(prefill) if prefill is not None else None,
                                     ctypes.byref(decode) if decode is not None else None, ctypes.byref(st))
    if rc != POD_OK:
        raise PodAttnError(rc, "pod_attn_plan_varlen")
    return st.as_dict()


def _check_device_bytes(t, nbytes: int, what: str) -> None:
    """A tensor argument must hold at least nbytes of device memory (a raw
    pointer is the caller's responsibility)."""
    if hasattr(t, "data_ptr"):
        if not t.is_cuda or not t.is_contiguous() or t.numel() * t.element_size() < nbytes:
            raise ValueError(f"{what}: needs a contiguous device tensor of at least {nbytes} bytes")


def pod_attn_peak_read(buf, nbytes: int, workgroups: int, sink, stream=None) -> None:
    """Enqueue the HBM-read kernel over `nbytes` of device buffer `buf` (a
    tensor or pointer); `sink` is a device uint32 word (tensor or pointer)."""
    _check_device_bytes(buf, int(nbytes), "pod_attn_peak_read buffer")
    _check_device_bytes(sink, 4, "pod_attn_peak_read sink")
    rc = load().pod_attn_peak_read(_ptr(buf) if hasattr(buf, "data_ptr") else buf, int(nbytes), int(workgroups),
                                   _ptr(sink) if hasattr(sink, "data_ptr") else sink, _stream_ptr(stream))
    if rc != POD_OK:
        raise PodAttnError(rc, "pod_attn_peak_read")


def pod_attn_peak_mfma(workgroups: int, iters: int, sink, stream=None) -> None:
    """Enqueue the MFMA loop: workgroups x 4 waves x iters x 16 bf16 32x32x16 MFMAs."""
    _check_device_bytes(sink, 4, "pod_attn_peak_mfma sink")
    rc = load().pod_attn_peak_mfma(int(workgroups), int(iters), _ptr(sink) if hasattr(sink, "data_ptr") else sink,
                                   _stream_ptr(stream))
    if rc != POD_OK:
        raise PodAttnError(rc, "pod_attn_peak_mfma")


PEAK_MFMA_FLOPS_PER_ITER_WAVE = 16 * 2 * 32 * 32 * 16  # 16 MFMAs of 32x32x16 per loop iteration


class PodAttention:
    """Owns one handle; methods take a HybridBatch-like object already on the GPU."""

    def __init__(self, cfg: PodAttnConfig):
        self.cfg = cfg
        self.h = pod_attn_create(cfg)

    def close(self):
        if self.h:
            pod_attn_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def args(batch, o_prefill, o_decode, ctx_host):
        pa = da = None
        if batch.q_prefill is not None and o_prefill is not None:
            pa = prefill_args(batch.q_prefill, o_prefill, batch.page_table_prefill, batch.chunk_offset)
        if batch.q_decode is not None and o_decode is not None:
            da = decode_args(batch.q_decode, o_decode, batch.page_table_decode, batch.context_lens, ctx_host)
        return pa, da

    def hybrid(self, batch, o_prefill, o_decode, ctx_host, stream=None):
        pa, da = self.args(batch, o_prefill, o_decode, ctx_host)
        pod_attn_hybrid(self.h, batch.k_pool, batch.v_pool, pa, da, stream)

    def prefill_only(self, batch, o_prefill, stream=None):
        pa, _ = self.args(batch, o_prefill, None, None)
        pod_attn_prefill_only(self.h, batch.k_pool, batch.v_pool, pa, stream)

    def decode_only(self, batch, o_decode, ctx_host, stream=None):
        _, da = self.args(batch, None, o_decode, ctx_host)
        pod_attn_decode_only(self.h, batch.k_pool, batch.v_pool, da, stream)

    # several prefill chunks (batch.chunks set, page_table_prefill [n, stride])
    def hybrid_varlen(self, batch, o_prefill, o_decode, ctx_host, stream=None):
        _, da = self.args(batch, None, o_decode, ctx_host)
        pa = None
        if batch.q_prefill is not None and o_prefill is not None:
            pa = prefill_batch(batch.q_prefill, o_prefill, batch.page_table_prefill, batch.chunk_list())
        pod_attn_hybrid_varlen(self.h, batch.k_pool, batch.v_pool, pa, da, stream)

    def prefill_only_varlen(self, batch, o_prefill, stream=None):
        pa = prefill_batch(batch.q_prefill, o_prefill, batch.page_table_prefill, batch.chunk_list())
        pod_attn_prefill_only_varlen(self.h, batch.k_pool, batch.v_pool, pa, stream)

    def stats(self) -> dict:
        return pod_attn_get_stats(self.h)

    def role_trace(self) -> list:
        return pod_attn_role_trace(self.h)


def config_for_batch(batch, **kw) -> PodAttnConfig:
    """A config whose limits fit `batch` (a HybridBatch from .inputs)."""
    lens = [] if batch.context_lens is None else batch.context_lens.tolist()
    lp = max([c + p for c, p in batch.chunk_list()] + [0])
    return make_config(
        dtype=POD_BF16 if batch.spec["dtype"] == "bf16" else POD_F32,
        num_q_heads=batch.num_q_heads, num_kv_heads=batch.num_kv_heads, head_dim=batch.head_dim,
        sm_scale=batch.sm_scale, max_chunk_len=max(1, batch.chunk_len),
        max_num_decode=max(1, len(lens)), max_context=max([lp, 1] + lens),
        max_total_context=max(1, sum(lens)), **kw)
