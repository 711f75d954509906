"""Thin Python binding over libpa_decode.so (ctypes).

The functions carry the C entry points' names and only marshal arguments:
they check dtype, device and contiguity of torch tensors, then pass raw
device pointers and the current HIP stream.  Every step of the computation
runs in the library's kernels; if the library is not built this module
raises on import -- there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpa_decode.so")

PA_OK = 0
STATUS_NAMES = {0: "PA_OK", -1: "PA_ERR_NULL", -2: "PA_ERR_SHAPE", -3: "PA_ERR_UNSUPPORTED",
                -4: "PA_ERR_ALIGN", -5: "PA_ERR_WORKSPACE", -6: "PA_ERR_LAUNCH"}

EXPORTS = ("pa_decode", "pa_decode_splitkv", "pa_merge_lse", "pa_decode_workspace_size",
           "pa_decode_partition_size", "mla_absorbed_decode",
           "mla_absorbed_decode_workspace_size", "pa_kv_insert", "mla_cache_insert",
           "pa_decode_multiquery", "pa_decode_multiquery_workspace_size", "pa_decode_fp8",
           "pa_decode_f32", "mla_cache_insert_fp8", "mla_absorbed_decode_fp8",
           "mla_absorbed_decode_multiquery", "mla_absorbed_decode_multiquery_fp8",
           "pa_decode_noalloc", "pa_profile_next", "pa_last_error")


class PaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class KvLayout(C.Structure):
    _fields_ = [("num_pages", C.c_int32), ("page_size", C.c_int32),
                ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("page_stride", C.c_int64), ("head_stride", C.c_int64),
                ("token_stride", C.c_int64)]


def _load() -> C.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m paged_attention_decode_05_amd.build`"
                          " (or __graft_entry__.build())")
    lib = C.CDLL(LIB_PATH)
    vp, i32, f32p, i32p = C.c_void_p, C.c_int32, C.POINTER(C.c_float), C.c_void_p
    kvp = C.POINTER(KvLayout)
    lib.pa_decode.argtypes = [vp, vp, vp, kvp, i32p, i32, i32p, i32, i32, i32, C.c_float, i32, vp,
                              vp, vp, C.c_size_t, vp]
    lib.pa_decode.restype = C.c_int
    lib.pa_decode_fp8.argtypes = [vp, vp, vp, kvp, i32p, i32, i32p, i32, i32, i32, C.c_float,
                                  C.c_float, C.c_float, i32, vp, vp, vp, C.c_size_t, vp]
    lib.pa_decode_fp8.restype = C.c_int
    lib.pa_decode_noalloc.argtypes = [vp, vp, vp, kvp, i32p, i32, i32p, i32, i32, i32, C.c_float,
                                      i32, vp, vp, vp]
    lib.pa_decode_noalloc.restype = C.c_int
    lib.pa_decode_f32.argtypes = lib.pa_decode.argtypes
    lib.pa_decode_f32.restype = C.c_int
    lib.pa_decode_splitkv.argtypes = [vp, vp, vp, kvp, i32p, i32, i32p, i32, i32, i32, C.c_float,
                                      i32, i32, i32, vp, vp, vp, vp]
    lib.pa_decode_splitkv.restype = C.c_int
    lib.pa_merge_lse.argtypes = [vp, vp, vp, i32p, i32, i32, i32, i32, i32, i32, vp, vp, vp]
    lib.pa_merge_lse.restype = C.c_int
    lib.pa_decode_workspace_size.argtypes = [i32] * 7
    lib.pa_decode_workspace_size.restype = C.c_size_t
    lib.pa_decode_partition_size.argtypes = [i32] * 7
    lib.pa_decode_partition_size.restype = C.c_int32
    lib.mla_absorbed_decode.argtypes = [vp, vp, vp, kvp, vp, vp, i32p, i32, i32p, i32, i32, i32,
                                        C.c_float, i32, vp, vp, C.c_size_t, vp]
    lib.mla_absorbed_decode.restype = C.c_int
    lib.mla_absorbed_decode_fp8.argtypes = list(lib.mla_absorbed_decode.argtypes)
    lib.mla_absorbed_decode_fp8.restype = C.c_int
    for f in (lib.mla_absorbed_decode_multiquery, lib.mla_absorbed_decode_multiquery_fp8):
        f.argtypes = [vp, vp, vp, kvp, vp, vp, i32p, i32, i32p, i32, i32, i32, i32, i32,
                      C.c_float, i32, vp, vp, C.c_size_t, vp]
        f.restype = C.c_int
    lib.mla_absorbed_decode_workspace_size.argtypes = [i32] * 5
    lib.mla_absorbed_decode_workspace_size.restype = C.c_size_t
    lib.pa_decode_multiquery.argtypes = [vp, vp, vp, kvp, i32p, i32, i32p, i32, i32, i32, i32,
                                         i32, C.c_float, i32, vp, vp, vp, C.c_size_t, vp]
    lib.pa_decode_multiquery.restype = C.c_int
    lib.pa_decode_multiquery_workspace_size.argtypes = [i32] * 8
    lib.pa_decode_multiquery_workspace_size.restype = C.c_size_t
    i64, i64p = C.c_int64, C.POINTER(C.c_int64)
    lib.pa_kv_insert.argtypes = [vp, vp, i64, i64, vp, vp, kvp, vp, i32, vp]
    lib.pa_kv_insert.restype = C.c_int
    lib.mla_cache_insert.argtypes = [vp, i64, vp, i64, vp, kvp, vp, i32, vp]
    lib.mla_cache_insert.restype = C.c_int
    lib.mla_cache_insert_fp8.argtypes = [vp, i64, vp, i64, vp, kvp, vp, i32, vp]
    lib.mla_cache_insert_fp8.restype = C.c_int
    lib.pa_profile_next.argtypes = [vp, vp]
    lib.pa_profile_next.restype = None
    lib.pa_last_error.argtypes = []
    lib.pa_last_error.restype = C.c_char_p
    return lib


LIB = _load()


def pa_profile_next(start_event: Optional[int], stop_event: Optional[int]) -> None:
    """Arm the next call on this thread to record two hipEvent_t handles around
    its dominant kernel (see include/pa_decode.h)."""
    LIB.pa_profile_next(start_event, stop_event)


def pa_last_error() -> str:
    return LIB.pa_last_error().decode()


def _check(rc: int) -> None:
    if rc != PA_OK:
        raise PaError(rc, pa_last_error())


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _ptr(t: Optional[torch.Tensor], dtype=None, name: str = "") -> Optional[int]:
    if t is None:
        return None
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    return t.data_ptr()


def _contig(t: torch.Tensor, name: str) -> None:
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def kv_layout(pool: torch.Tensor, layout: str = "PHSD") -> KvLayout:
    """Descriptor of a pool tensor (bf16, or uint8 holding E4M3 bytes; strides
    in elements): "PHSD" = [page][kv head][slot][dim], "PSHD" = [page][slot]
    [kv head][dim], "PSR" = [page][slot][row] (MLA)."""
    s = pool.stride()
    if layout == "PHSD":
        P, H, S, D = pool.shape
        return KvLayout(P, S, H, D, s[0], s[1], s[2])
    if layout == "PSHD":
        P, S, H, D = pool.shape
        return KvLayout(P, S, H, D, s[0], s[2], s[1])
    if layout == "PSR":
        P, S, R = pool.shape
        return KvLayout(P, S, 1, R, s[0], 0, s[1])
    raise ValueError(layout)


def pa_decode_workspace_size(batch, num_q_heads, num_kv_heads, head_dim, max_pages_per_seq,
                             page_size, window=0) -> int:
    return int(LIB.pa_decode_workspace_size(batch, num_q_heads, num_kv_heads, head_dim,
                                            max_pages_per_seq, page_size, window))


def pa_decode_partition_size(batch, num_q_heads, num_kv_heads, head_dim, max_pages_per_seq,
                             page_size, window=0) -> int:
    return int(LIB.pa_decode_partition_size(batch, num_q_heads, num_kv_heads, head_dim,
                                            max_pages_per_seq, page_size, window))


def mla_absorbed_decode_workspace_size(batch, num_heads, max_pages_per_seq, page_size,
                                       partition_size=0) -> int:
    return int(LIB.mla_absorbed_decode_workspace_size(batch, num_heads, max_pages_per_seq,
                                                      page_size, partition_size))


def pa_decode(q, k_pool, v_pool, kv: KvLayout, block_table, context_lens, scale: float,
              window: int, out, lse_out=None, workspace=None, max_pages_per_seq=None,
              stream=None) -> None:
    for t, n in ((q, "q"), (block_table, "block_table"), (context_lens, "context_lens"),
                 (out, "out")):
        _contig(t, n)
    B, H = q.shape[0], q.shape[1]
    maxp = block_table.shape[1] if max_pages_per_seq is None else max_pages_per_seq
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = LIB.pa_decode(_ptr(q, torch.bfloat16, "q"), _ptr(k_pool, torch.bfloat16, "k_pool"),
                       _ptr(v_pool, torch.bfloat16, "v_pool"), C.byref(kv),
                       _ptr(block_table, torch.int32, "block_table"), block_table.stride(0),
                       _ptr(context_lens, torch.int32, "context_lens"), B, H, maxp, float(scale),
                       int(window), _ptr(out, torch.bfloat16, "out"),
                       _ptr(lse_out, torch.float32, "lse_out"), _ptr(workspace), ws_bytes,
                       _stream(stream))
    _check(rc)


def pa_decode_noalloc(q, k_pool, v_pool, kv: KvLayout, block_table, context_lens, scale: float,
                      window: int, out, lse_out=None, max_pages_per_seq=None,
                      stream=None) -> None:
    """pa_decode with the library's own device scratch instead of a workspace."""
    for t, n in ((q, "q"), (block_table, "block_table"), (context_lens, "context_lens"),
                 (out, "out")):
        _contig(t, n)
    B, H = q.shape[0], q.shape[1]
    maxp = block_table.shape[1] if max_pages_per_seq is None else max_pages_per_seq
    rc = LIB.pa_decode_noalloc(_ptr(q, torch.bfloat16, "q"), _ptr(k_pool, torch.bfloat16, "k_pool"),
                               _ptr(v_pool, torch.bfloat16, "v_pool"), C.byref(kv),
                               _ptr(block_table, torch.int32, "block_table"),
                               block_table.stride(0),
                               _ptr(context_lens, torch.int32, "context_lens"), B, H, maxp,
                               float(scale), int(window), _ptr(out, torch.bfloat16, "out"),
                               _ptr(lse_out, torch.float32, "lse_out"), _stream(stream))
    _check(rc)


def pa_decode_fp8(q, k_pool, v_pool, kv: KvLayout, block_table, context_lens, scale: float,
                  k_scale: float, v_scale: float, window: int, out, lse_out=None, workspace=None,
                  max_pages_per_seq=None, stream=None) -> None:
    """pa_decode over E4M3 pools (uint8 tensors of the raw bytes)."""
    for t, n in ((q, "q"), (block_table, "block_table"), (context_lens, "context_lens"),
                 (out, "out")):
        _contig(t, n)
    B, H = q.shape[0], q.shape[1]
    maxp = block_table.shape[1] if max_pages_per_seq is None else max_pages_per_seq
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = LIB.pa_decode_fp8(_ptr(q, torch.bfloat16, "q"), _ptr(k_pool, torch.uint8, "k_pool"),
                           _ptr(v_pool, torch.uint8, "v_pool"), C.byref(kv),
                           _ptr(block_table, torch.int32, "block_table"), block_table.stride(0),
                           _ptr(context_lens, torch.int32, "context_lens"), B, H, maxp,
                           float(scale), float(k_scale), float(v_scale), int(window),
                           _ptr(out, torch.bfloat16, "out"), _ptr(lse_out, torch.float32, "lse_out"),
                           _ptr(workspace), ws_bytes, _stream(stream))
    _check(rc)


def pa_decode_f32(q, k_pool, v_pool, kv: KvLayout, block_table, context_lens, scale: float,
                  window: int, out, lse_out=None, workspace=None, max_pages_per_seq=None,
                  stream=None) -> None:
    """pa_decode over float32 pools."""
    for t, n in ((q, "q"), (block_table, "block_table"), (context_lens, "context_lens"),
                 (out, "out")):
        _contig(t, n)
    B, H = q.shape[0], q.shape[1]
    maxp = block_table.shape[1] if max_pages_per_seq is None else max_pages_per_seq
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = LIB.pa_decode_f32(_ptr(q, torch.bfloat16, "q"), _ptr(k_pool, torch.float32, "k_pool"),
                           _ptr(v_pool, torch.float32, "v_pool"), C.byref(kv),
                           _ptr(block_table, torch.int32, "block_table"), block_table.stride(0),
                           _ptr(context_lens, torch.int32, "context_lens"), B, H, maxp,
                           float(scale), int(window), _ptr(out, torch.bfloat16, "out"),
                           _ptr(lse_out, torch.float32, "lse_out"), _ptr(workspace), ws_bytes,
                           _stream(stream))
    _check(rc)


def pa_decode_splitkv(q, k_pool, v_pool, kv: KvLayout, block_table, context_lens, scale: float,
                      window: int, partition_size: int, max_partitions: int, part_out, part_max,
                      part_sum, max_pages_per_seq=None, stream=None) -> None:
    for t, n in ((q, "q"), (block_table, "block_table"), (context_lens, "context_lens"),
                 (part_out, "part_out"), (part_max, "part_max"), (part_sum, "part_sum")):
        _contig(t, n)
    B, H = q.shape[0], q.shape[1]
    maxp = block_table.shape[1] if max_pages_per_seq is None else max_pages_per_seq
    rc = LIB.pa_decode_splitkv(_ptr(q, torch.bfloat16, "q"), _ptr(k_pool, torch.bfloat16, "k"),
                               _ptr(v_pool, torch.bfloat16, "v"), C.byref(kv),
                               _ptr(block_table, torch.int32, "block_table"),
                               block_table.stride(0),
                               _ptr(context_lens, torch.int32, "context_lens"), B, H, maxp,
                               float(scale), int(window), int(partition_size),
                               int(max_partitions), _ptr(part_out, torch.float32, "part_out"),
                               _ptr(part_max, torch.float32, "part_max"),
                               _ptr(part_sum, torch.float32, "part_sum"), _stream(stream))
    _check(rc)


def pa_merge_lse(part_out, part_max, part_sum, context_lens, partition_size: int, window: int,
                 out, lse_out=None, stream=None) -> None:
    for t, n in ((part_out, "part_out"), (part_max, "part_max"), (part_sum, "part_sum"),
                 (out, "out")):
        _contig(t, n)
    B, H, P, D = part_out.shape
    rc = LIB.pa_merge_lse(_ptr(part_out, torch.float32, "part_out"),
                          _ptr(part_max, torch.float32, "part_max"),
                          _ptr(part_sum, torch.float32, "part_sum"),
                          _ptr(context_lens, torch.int32, "context_lens"), B, H, D,
                          int(partition_size), P, int(window), _ptr(out, torch.bfloat16, "out"),
                          _ptr(lse_out, torch.float32, "lse_out"), _stream(stream))
    _check(rc)


def _mla_decode(fn, cache_dtype, q_nope, q_rope, kv_cache, cache, w_uk, w_uv, block_table,
                context_lens, scale, out, workspace, partition_size, max_pages_per_seq, stream,
                queries=None):
    """queries: None for the one-query entries, else (num_queries, causal)."""
    for t, n in ((q_nope, "q_nope"), (q_rope, "q_rope"), (w_uk, "w_uk"), (w_uv, "w_uv"),
                 (block_table, "block_table"), (context_lens, "context_lens"), (out, "out")):
        _contig(t, n)
    B, H = q_nope.shape[0], q_nope.shape[-2]
    extra = () if queries is None else (int(queries[0]), int(bool(queries[1])))
    maxp = block_table.shape[1] if max_pages_per_seq is None else max_pages_per_seq
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = fn(_ptr(q_nope, torch.bfloat16, "q_nope"), _ptr(q_rope, torch.bfloat16, "q_rope"),
            _ptr(kv_cache, cache_dtype, "kv_cache"), C.byref(cache),
            _ptr(w_uk, torch.bfloat16, "w_uk"), _ptr(w_uv, torch.bfloat16, "w_uv"),
            _ptr(block_table, torch.int32, "block_table"), block_table.stride(0),
            _ptr(context_lens, torch.int32, "context_lens"), B, H, *extra, maxp, float(scale),
            int(partition_size), _ptr(out, torch.bfloat16, "out"), _ptr(workspace), ws_bytes,
            _stream(stream))
    _check(rc)


def mla_absorbed_decode(q_nope, q_rope, kv_cache, cache: KvLayout, w_uk, w_uv, block_table,
                        context_lens, scale: float, out, workspace, partition_size: int = 0,
                        max_pages_per_seq=None, stream=None) -> None:
    _mla_decode(LIB.mla_absorbed_decode, torch.bfloat16, q_nope, q_rope, kv_cache, cache, w_uk,
                w_uv, block_table, context_lens, scale, out, workspace, partition_size,
                max_pages_per_seq, stream)


MLA_FP8_ROW = 656   # bytes per token of the FP8 latent cache


def mla_absorbed_decode_fp8(q_nope, q_rope, kv_cache, cache: KvLayout, w_uk, w_uv, block_table,
                            context_lens, scale: float, out, workspace, partition_size: int = 0,
                            max_pages_per_seq=None, stream=None) -> None:
    """kv_cache: uint8 FP8 latent rows (cache.head_dim 656, strides in bytes)."""
    _mla_decode(LIB.mla_absorbed_decode_fp8, torch.uint8, q_nope, q_rope, kv_cache, cache, w_uk,
                w_uv, block_table, context_lens, scale, out, workspace, partition_size,
                max_pages_per_seq, stream)


def mla_absorbed_decode_multiquery(q_nope, q_rope, kv_cache, cache: KvLayout, w_uk, w_uv,
                                   block_table, context_lens, scale: float, out, workspace,
                                   causal: bool = True, partition_size: int = 0,
                                   max_pages_per_seq=None, stream=None) -> None:
    """q_nope [B, S, H, 128], q_rope [B, S, H, 64], out [B, S, H, 128] bf16
    (3-D tensors mean S = 1); kv_cache bf16 576-wide rows, or uint8 FP8 rows
    of MLA_FP8_ROW bytes, which select the _fp8 entry."""
    S = q_nope.shape[1] if q_nope.dim() == 4 else 1
    fp8 = kv_cache.dtype == torch.uint8
    fn = LIB.mla_absorbed_decode_multiquery_fp8 if fp8 else LIB.mla_absorbed_decode_multiquery
    _mla_decode(fn, torch.uint8 if fp8 else torch.bfloat16, q_nope, q_rope, kv_cache, cache, w_uk,
                w_uv, block_table, context_lens, scale, out, workspace, partition_size,
                max_pages_per_seq, stream, queries=(S, causal))


def _rows(t: torch.Tensor, name: str, ndim: int) -> None:
    if t.dim() != ndim or t.stride(-1) != 1:
        raise ValueError(f"{name}: expected {ndim} dims with a contiguous last axis")


def pa_kv_insert(k_new, v_new, k_pool, v_pool, kv: KvLayout, slots, stream=None) -> None:
    """k_new / v_new [T, Hkv, D] bf16 (any strides with a contiguous last
    axis, the same for both); slots [T] int64 flat slot indices."""
    _rows(k_new, "k_new", 3)
    _rows(v_new, "v_new", 3)
    if k_new.shape != v_new.shape or k_new.stride() != v_new.stride():
        raise ValueError("k_new and v_new must have the same shape and strides")
    _contig(slots, "slots")
    rc = LIB.pa_kv_insert(_ptr(k_new, torch.bfloat16, "k_new"), _ptr(v_new, torch.bfloat16, "v_new"),
                          k_new.stride(0), k_new.stride(1), _ptr(k_pool, torch.bfloat16, "k_pool"),
                          _ptr(v_pool, torch.bfloat16, "v_pool"), C.byref(kv),
                          _ptr(slots, torch.int64, "slots"), k_new.shape[0], _stream(stream))
    _check(rc)


def mla_cache_insert(kv_c, k_pe, kv_cache, cache: KvLayout, slots, stream=None) -> None:
    """kv_c [T, 512] and k_pe [T, 64] bf16 (row strides free, last axis
    contiguous); slots [T] int64."""
    _rows(kv_c, "kv_c", 2)
    _rows(k_pe, "k_pe", 2)
    if kv_c.shape[0] != k_pe.shape[0]:
        raise ValueError("kv_c and k_pe must have the same number of rows")
    _contig(slots, "slots")
    rc = LIB.mla_cache_insert(_ptr(kv_c, torch.bfloat16, "kv_c"), kv_c.stride(0),
                              _ptr(k_pe, torch.bfloat16, "k_pe"), k_pe.stride(0),
                              _ptr(kv_cache, torch.bfloat16, "kv_cache"), C.byref(cache),
                              _ptr(slots, torch.int64, "slots"), kv_c.shape[0], _stream(stream))
    _check(rc)


def mla_cache_insert_fp8(kv_c, k_pe, kv_cache, cache: KvLayout, slots, stream=None) -> None:
    """As mla_cache_insert, into the FP8 latent cache (uint8 rows of 656
    bytes; cache strides in bytes)."""
    _rows(kv_c, "kv_c", 2)
    _rows(k_pe, "k_pe", 2)
    if kv_c.shape[0] != k_pe.shape[0]:
        raise ValueError("kv_c and k_pe must have the same number of rows")
    _contig(slots, "slots")
    rc = LIB.mla_cache_insert_fp8(_ptr(kv_c, torch.bfloat16, "kv_c"), kv_c.stride(0),
                                  _ptr(k_pe, torch.bfloat16, "k_pe"), k_pe.stride(0),
                                  _ptr(kv_cache, torch.uint8, "kv_cache"), C.byref(cache),
                                  _ptr(slots, torch.int64, "slots"), kv_c.shape[0],
                                  _stream(stream))
    _check(rc)


def pa_decode_multiquery_workspace_size(batch, num_q_heads, num_kv_heads, head_dim,
                                        max_pages_per_seq, page_size, window, num_queries) -> int:
    return int(LIB.pa_decode_multiquery_workspace_size(batch, num_q_heads, num_kv_heads, head_dim,
                                                       max_pages_per_seq, page_size, window,
                                                       num_queries))


def pa_decode_multiquery(q, k_pool, v_pool, kv: KvLayout, block_table, context_lens, scale: float,
                         window: int, causal: bool, out, lse_out=None, workspace=None,
                         max_pages_per_seq=None, stream=None) -> None:
    """q and out [B, S, Hq, D] bf16 (contiguous); lse_out [B, S, Hq] fp32 or None."""
    for t, n in ((q, "q"), (block_table, "block_table"), (context_lens, "context_lens"),
                 (out, "out")):
        _contig(t, n)
    B, S, H = q.shape[0], q.shape[1], q.shape[2]
    maxp = block_table.shape[1] if max_pages_per_seq is None else max_pages_per_seq
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = LIB.pa_decode_multiquery(_ptr(q, torch.bfloat16, "q"), _ptr(k_pool, torch.bfloat16, "k_pool"),
                                  _ptr(v_pool, torch.bfloat16, "v_pool"), C.byref(kv),
                                  _ptr(block_table, torch.int32, "block_table"),
                                  block_table.stride(0),
                                  _ptr(context_lens, torch.int32, "context_lens"), B, H, S,
                                  int(bool(causal)), maxp, float(scale), int(window),
                                  _ptr(out, torch.bfloat16, "out"),
                                  _ptr(lse_out, torch.float32, "lse_out"), _ptr(workspace),
                                  ws_bytes, _stream(stream))
    _check(rc)
