"""Python handle on the CPU oracle (libpa_oracle.so).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg.  The product package never imports it.

``Oracle(path)`` wraps one build of the library (the shipped one, or a copy
with a planted mistake).  Every call takes CPU tensors/arrays (bf16 tensors
are passed as their raw 16-bit patterns) and returns float64 numpy arrays.
``precision`` selects the _f64 (gate) or _f32 instantiation.
"""
from __future__ import annotations

import copy
import ctypes as C
import os
from typing import Optional

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_LIB = os.path.join(HERE, "libpa_oracle.so")


class _Pool(C.Structure):
    _fields_ = [("num_pages", C.c_int32), ("page_size", C.c_int32),
                ("num_kv_heads", C.c_int32), ("head_dim", C.c_int32),
                ("page_stride", C.c_int64), ("head_stride", C.c_int64),
                ("token_stride", C.c_int64)]


def _bits(t: torch.Tensor) -> np.ndarray:
    """Raw bf16 bit patterns of a CPU tensor, as a uint16 array (no copy of
    values through any arithmetic).  Non-contiguous views keep their strides
    only through the pool descriptor, so the base storage is passed."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def _i32(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu().numpy()
    return np.ascontiguousarray(t, dtype=np.int32)


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(C.POINTER(ctype))


class OracleError(RuntimeError):
    pass


class Oracle:
    def __init__(self, path: Optional[str] = None):
        path = path or DEFAULT_LIB
        if not os.path.exists(path):
            raise OracleError(f"oracle library {path} is not built (run oracle/build.py)")
        self.path = path
        self.lib = C.CDLL(path)
        u16p, i32p, f64p = C.POINTER(C.c_uint16), C.POINTER(C.c_int32), C.POINTER(C.c_double)
        pool = C.POINTER(_Pool)
        for sfx in ("_f64", "_f32"):
            f = getattr(self.lib, "oracle_pa_decode" + sfx)
            f.argtypes = [u16p, u16p, u16p, pool, i32p, C.c_int32, i32p, C.c_int32, C.c_int32,
                          C.c_double, C.c_int32, f64p, f64p]
            f.restype = C.c_int
            f = getattr(self.lib, "oracle_pa_partials" + sfx)
            f.argtypes = [u16p, u16p, u16p, pool, i32p, C.c_int32, i32p, C.c_int32, C.c_int32,
                          C.c_double, C.c_int32, C.c_int32, C.c_int32, f64p, f64p, f64p]
            f.restype = C.c_int
            f = getattr(self.lib, "oracle_pa_merge" + sfx)
            f.argtypes = [f64p, f64p, f64p, i32p, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                          C.c_int32, C.c_int32, f64p, f64p]
            f.restype = C.c_int
            f = getattr(self.lib, "oracle_pa_decode_multi" + sfx)
            f.argtypes = [u16p, u16p, u16p, pool, i32p, C.c_int32, i32p, C.c_int32, C.c_int32,
                          C.c_int32, C.c_int32, C.c_double, C.c_int32, f64p, f64p]
            f.restype = C.c_int
            f = getattr(self.lib, "oracle_mla_decode" + sfx)
            f.argtypes = [u16p, u16p, u16p, pool, u16p, u16p, i32p, C.c_int32, i32p, C.c_int32,
                          C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_int32, C.c_double,
                          f64p, f64p, f64p]
            f.restype = C.c_int
        i64p = C.POINTER(C.c_int64)
        self.lib.oracle_kv_insert.argtypes = [u16p, u16p, C.c_int64, C.c_int64, u16p, u16p, pool,
                                              i64p, C.c_int32]
        self.lib.oracle_kv_insert.restype = C.c_int
        self.lib.oracle_mla_cache_insert.argtypes = [u16p, C.c_int64, u16p, C.c_int64, u16p, pool,
                                                     i64p, C.c_int32, C.c_int32, C.c_int32]
        self.lib.oracle_mla_cache_insert.restype = C.c_int
        u8p = C.POINTER(C.c_uint8)
        self.lib.oracle_e4m3_value.argtypes = [C.c_uint8]
        self.lib.oracle_e4m3_value.restype = C.c_double
        self.lib.oracle_pa_decode_fp8.argtypes = [u16p, u8p, u8p, pool, i32p, C.c_int32, i32p,
                                                  C.c_int32, C.c_int32, C.c_double, C.c_double,
                                                  C.c_double, C.c_int32, f64p, f64p]
        self.lib.oracle_pa_decode_fp8.restype = C.c_int
        self.lib.oracle_e4m3_encode.argtypes = [C.c_double]
        self.lib.oracle_e4m3_encode.restype = C.c_uint8
        self.lib.oracle_mla_cache_insert_fp8.argtypes = [u16p, C.c_int64, u16p, C.c_int64, u8p,
                                                         pool, i64p, C.c_int32, C.c_int32,
                                                         C.c_int32]
        self.lib.oracle_mla_cache_insert_fp8.restype = C.c_int
        self.lib.oracle_mla_decode_fp8.argtypes = [u16p, u16p, u8p, pool, u16p, u16p, i32p,
                                                   C.c_int32, i32p, C.c_int32, C.c_int32,
                                                   C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                                   C.c_double, f64p, f64p]
        self.lib.oracle_mla_decode_fp8.restype = C.c_int
        f32p = C.POINTER(C.c_float)
        self.lib.oracle_pa_decode_f32pool.argtypes = [u16p, f32p, f32p, pool, i32p, C.c_int32,
                                                      i32p, C.c_int32, C.c_int32, C.c_double,
                                                      C.c_int32, f64p, f64p]
        self.lib.oracle_pa_decode_f32pool.restype = C.c_int
        self.lib.oracle_set_num_threads.argtypes = [C.c_int32]
        self.lib.oracle_max_threads.restype = C.c_int32
        self.lib.oracle_mutation.restype = C.c_int32

    # ---- helpers ---------------------------------------------------------
    def set_threads(self, n: int) -> None:
        self.lib.oracle_set_num_threads(int(n))

    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())

    @property
    def mutation(self) -> int:
        return int(self.lib.oracle_mutation())

    @staticmethod
    def _pool_of(case) -> _Pool:
        ps, hs, ts = case.strides()
        return _Pool(case.num_pages, case.page_size, case.num_kv_heads, case.head_dim, ps, hs, ts)

    def _check(self, rc: int, what: str) -> None:
        if rc != 0:
            raise OracleError(f"{what} returned {rc}")

    # ---- GQA paged decode --------------------------------------------------
    def decode(self, case, precision: str = "f64", window: Optional[int] = None):
        """(out [B,Hq,D] float64, lse [B,Hq] float64) for a GqaCase."""
        B, H, D = case.batch, case.num_q_heads, case.head_dim
        q, k, v = _bits(case.q), _bits(case.k_pool), _bits(case.v_pool)
        bt, ctx = _i32(case.block_table), _i32(case.context_lens)
        out = np.zeros((B, H, D), np.float64)
        lse = np.zeros((B, H), np.float64)
        pool = self._pool_of(case)
        w = case.window if window is None else window
        u16, i32, f64 = C.c_uint16, C.c_int32, C.c_double
        rc = getattr(self.lib, "oracle_pa_decode_" + precision)(
            _ptr(q, u16), _ptr(k, u16), _ptr(v, u16), C.byref(pool), _ptr(bt, i32),
            bt.shape[1], _ptr(ctx, i32), B, H, float(case.scale), int(w),
            _ptr(out, f64), _ptr(lse, f64))
        self._check(rc, "oracle_pa_decode")
        return out, lse

    def e4m3_value(self, byte: int) -> float:
        return float(self.lib.oracle_e4m3_value(int(byte)))

    def e4m3_encode(self, v: float) -> int:
        return int(self.lib.oracle_e4m3_encode(float(v)))

    def decode_fp8(self, case, window: Optional[int] = None):
        """(out [B,Hq,D], lse [B,Hq]) float64 for a GqaCase with FP8 pools."""
        assert case.kv_dtype == "fp8"
        B, H, D = case.batch, case.num_q_heads, case.head_dim
        q = _bits(case.q)
        k = np.ascontiguousarray(case.k_pool.cpu().contiguous().numpy(), dtype=np.uint8)
        v = np.ascontiguousarray(case.v_pool.cpu().contiguous().numpy(), dtype=np.uint8)
        bt, ctx = _i32(case.block_table), _i32(case.context_lens)
        out = np.zeros((B, H, D), np.float64)
        lse = np.zeros((B, H), np.float64)
        pool = self._pool_of(case)
        w = case.window if window is None else window
        u8, u16, i32, f64 = C.c_uint8, C.c_uint16, C.c_int32, C.c_double
        rc = self.lib.oracle_pa_decode_fp8(
            _ptr(q, u16), _ptr(k, u8), _ptr(v, u8), C.byref(pool), _ptr(bt, i32), bt.shape[1],
            _ptr(ctx, i32), B, H, float(case.scale), float(case.k_scale), float(case.v_scale),
            int(w), _ptr(out, f64), _ptr(lse, f64))
        self._check(rc, "oracle_pa_decode_fp8")
        return out, lse

    def decode_f32pool(self, case, window: Optional[int] = None):
        """(out [B,Hq,D], lse [B,Hq]) float64 for a GqaCase with f32 pools."""
        assert case.kv_dtype == "f32"
        B, H, D = case.batch, case.num_q_heads, case.head_dim
        q = _bits(case.q)
        k = np.ascontiguousarray(case.k_pool.cpu().contiguous().numpy(), dtype=np.float32)
        v = np.ascontiguousarray(case.v_pool.cpu().contiguous().numpy(), dtype=np.float32)
        bt, ctx = _i32(case.block_table), _i32(case.context_lens)
        out = np.zeros((B, H, D), np.float64)
        lse = np.zeros((B, H), np.float64)
        pool = self._pool_of(case)
        w = case.window if window is None else window
        u16, f32, i32, f64 = C.c_uint16, C.c_float, C.c_int32, C.c_double
        rc = self.lib.oracle_pa_decode_f32pool(
            _ptr(q, u16), _ptr(k, f32), _ptr(v, f32), C.byref(pool), _ptr(bt, i32), bt.shape[1],
            _ptr(ctx, i32), B, H, float(case.scale), int(w), _ptr(out, f64), _ptr(lse, f64))
        self._check(rc, "oracle_pa_decode_f32pool")
        return out, lse

    def decode_multi(self, case, causal: bool = True, precision: str = "f64"):
        """(out [B,S,Hq,D], lse [B,S,Hq]) for a GqaCase whose q is [B, S, Hq, D]."""
        q4 = case.q if case.q.dim() == 4 else case.q[:, None]
        B, S, H, D = q4.shape
        q, k, v = _bits(q4), _bits(case.k_pool), _bits(case.v_pool)
        bt, ctx = _i32(case.block_table), _i32(case.context_lens)
        out = np.zeros((B, S, H, D), np.float64)
        lse = np.zeros((B, S, H), np.float64)
        pool = self._pool_of(case)
        u16, i32, f64 = C.c_uint16, C.c_int32, C.c_double
        rc = getattr(self.lib, "oracle_pa_decode_multi_" + precision)(
            _ptr(q, u16), _ptr(k, u16), _ptr(v, u16), C.byref(pool), _ptr(bt, i32),
            bt.shape[1], _ptr(ctx, i32), B, H, S, int(bool(causal)), float(case.scale),
            int(case.window), _ptr(out, f64), _ptr(lse, f64))
        self._check(rc, "oracle_pa_decode_multi")
        return out, lse

    def partials(self, case, partition_size: int, max_parts: int, precision: str = "f64"):
        """(part_out [B,Hq,max_parts,D], part_max, part_sum [B,Hq,max_parts])."""
        B, H, D = case.batch, case.num_q_heads, case.head_dim
        q, k, v = _bits(case.q), _bits(case.k_pool), _bits(case.v_pool)
        bt, ctx = _i32(case.block_table), _i32(case.context_lens)
        po = np.zeros((B, H, max_parts, D), np.float64)
        pm = np.zeros((B, H, max_parts), np.float64)
        pl = np.zeros((B, H, max_parts), np.float64)
        pool = self._pool_of(case)
        u16, i32, f64 = C.c_uint16, C.c_int32, C.c_double
        rc = getattr(self.lib, "oracle_pa_partials_" + precision)(
            _ptr(q, u16), _ptr(k, u16), _ptr(v, u16), C.byref(pool), _ptr(bt, i32),
            bt.shape[1], _ptr(ctx, i32), B, H, float(case.scale), int(case.window),
            int(partition_size), int(max_parts), _ptr(po, f64), _ptr(pm, f64), _ptr(pl, f64))
        self._check(rc, "oracle_pa_partials")
        return po, pm, pl

    def merge(self, part_out, part_max, part_sum, context_lens, partition_size: int,
              window: int, precision: str = "f64"):
        po = np.ascontiguousarray(part_out, np.float64)
        pm = np.ascontiguousarray(part_max, np.float64)
        pl = np.ascontiguousarray(part_sum, np.float64)
        B, H, P, D = po.shape
        ctx = _i32(context_lens)
        out = np.zeros((B, H, D), np.float64)
        lse = np.zeros((B, H), np.float64)
        i32, f64 = C.c_int32, C.c_double
        rc = getattr(self.lib, "oracle_pa_merge_" + precision)(
            _ptr(po, f64), _ptr(pm, f64), _ptr(pl, f64), _ptr(ctx, i32), B, H, D,
            int(partition_size), P, int(window), _ptr(out, f64), _ptr(lse, f64))
        self._check(rc, "oracle_pa_merge")
        return out, lse

    # ---- cache writes ----------------------------------------------------------
    def kv_insert(self, k_new: torch.Tensor, v_new: torch.Tensor, k_pool: torch.Tensor,
                  v_pool: torch.Tensor, pool: _Pool, slots) -> tuple:
        """Copies of the two pools after inserting k_new / v_new ([T, Hkv, D]
        bf16, contiguous) at the flat slots (int64); bf16 CPU tensors."""
        kn, vn = _bits(k_new), _bits(v_new)
        kp, vp = _bits(k_pool).copy(), _bits(v_pool).copy()
        sl = np.ascontiguousarray(torch.as_tensor(slots).cpu().numpy(), np.int64)
        T, Hkv, D = k_new.shape
        u16, i64 = C.c_uint16, C.c_int64
        rc = self.lib.oracle_kv_insert(_ptr(kn, u16), _ptr(vn, u16), Hkv * D, D, _ptr(kp, u16),
                                       _ptr(vp, u16), C.byref(pool), _ptr(sl, i64), T)
        self._check(rc, "oracle_kv_insert")
        back = lambda a, like: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).reshape(like.shape)
        return back(kp, k_pool), back(vp, v_pool)

    def mla_cache_insert(self, kv_c: torch.Tensor, k_pe: torch.Tensor, cache: torch.Tensor,
                         slots) -> torch.Tensor:
        """Copy of the latent cache [P, page, d_lat + d_rope] after writing
        kv_c [T, d_lat] ++ k_pe [T, d_rope] (bf16, contiguous) at the slots."""
        c, pe = _bits(kv_c), _bits(k_pe)
        out = _bits(cache).copy()
        sl = np.ascontiguousarray(torch.as_tensor(slots).cpu().numpy(), np.int64)
        T, d_lat = kv_c.shape
        d_rope = k_pe.shape[1]
        P, S, R = cache.shape
        pool = _Pool(P, S, 1, R, S * R, 0, R)
        u16, i64 = C.c_uint16, C.c_int64
        rc = self.lib.oracle_mla_cache_insert(_ptr(c, u16), d_lat, _ptr(pe, u16), d_rope,
                                              _ptr(out, u16), C.byref(pool), _ptr(sl, i64), T,
                                              d_lat, d_rope)
        self._check(rc, "oracle_mla_cache_insert")
        return torch.from_numpy(out.view(np.int16)).view(torch.bfloat16).reshape(cache.shape)

    def mla_cache_insert_fp8(self, kv_c: torch.Tensor, k_pe: torch.Tensor, cache: torch.Tensor,
                             slots) -> torch.Tensor:
        """Copy of the FP8 latent cache [P, page, row bytes] (uint8) after
        quantizing kv_c [T, d_lat] and writing it with k_pe [T, d_rope] (bf16,
        contiguous) at the slots."""
        c, pe = _bits(kv_c), _bits(k_pe)
        out = np.ascontiguousarray(cache.cpu().numpy(), dtype=np.uint8).copy()
        sl = np.ascontiguousarray(torch.as_tensor(slots).cpu().numpy(), np.int64)
        T, d_lat = kv_c.shape
        d_rope = k_pe.shape[1]
        P, S, R = cache.shape
        pool = _Pool(P, S, 1, R, S * R, 0, R)
        u8, u16, i64 = C.c_uint8, C.c_uint16, C.c_int64
        rc = self.lib.oracle_mla_cache_insert_fp8(_ptr(c, u16), d_lat, _ptr(pe, u16), d_rope,
                                                  _ptr(out, u8), C.byref(pool), _ptr(sl, i64), T,
                                                  d_lat, d_rope)
        self._check(rc, "oracle_mla_cache_insert_fp8")
        return torch.from_numpy(out)

    def mla_fp8(self, case):
        """(out [B,H,d_v], lse [B,H]) float64 for an MlaCase with an FP8 cache."""
        assert case.cache_dtype == "fp8"
        B, H = case.batch, case.num_heads
        qn, qr = _bits(case.q_nope), _bits(case.q_rope)
        cache = np.ascontiguousarray(case.cache.cpu().numpy(), dtype=np.uint8)
        wuk, wuv = _bits(case.w_uk), _bits(case.w_uv)
        bt, ctx = _i32(case.block_table), _i32(case.context_lens)
        P, S, R = case.cache.shape
        pool = _Pool(case.num_pages, case.page_size, 1, R, S * R, 0, R)
        out = np.zeros((B, H, case.d_v), np.float64)
        lse = np.zeros((B, H), np.float64)
        u8, u16, i32, f64 = C.c_uint8, C.c_uint16, C.c_int32, C.c_double
        rc = self.lib.oracle_mla_decode_fp8(
            _ptr(qn, u16), _ptr(qr, u16), _ptr(cache, u8), C.byref(pool), _ptr(wuk, u16),
            _ptr(wuv, u16), _ptr(bt, i32), bt.shape[1], _ptr(ctx, i32), B, H, case.d_nope,
            case.d_rope, case.d_lat, case.d_v, float(case.scale), _ptr(out, f64), _ptr(lse, f64))
        self._check(rc, "oracle_mla_decode_fp8")
        return out, lse

    # ---- absorbed MLA --------------------------------------------------------
    def mla(self, case, precision: str = "f64", want_q_abs: bool = False):
        """(out [B,H,d_v], lse [B,H], q_abs [B,H,d_lat] or None) for an MlaCase."""
        B, H = case.batch, case.num_heads
        qn, qr, cache = _bits(case.q_nope), _bits(case.q_rope), _bits(case.cache)
        wuk, wuv = _bits(case.w_uk), _bits(case.w_uv)
        bt, ctx = _i32(case.block_table), _i32(case.context_lens)
        row = case.d_lat + case.d_rope
        s = case.cache.stride()
        pool = _Pool(case.num_pages, case.page_size, 1, row, s[0], 0, s[1])
        out = np.zeros((B, H, case.d_v), np.float64)
        lse = np.zeros((B, H), np.float64)
        qa = np.zeros((B, H, case.d_lat), np.float64) if want_q_abs else None
        u16, i32, f64 = C.c_uint16, C.c_int32, C.c_double
        rc = getattr(self.lib, "oracle_mla_decode_" + precision)(
            _ptr(qn, u16), _ptr(qr, u16), _ptr(cache, u16), C.byref(pool), _ptr(wuk, u16),
            _ptr(wuv, u16), _ptr(bt, i32), bt.shape[1], _ptr(ctx, i32), B, H, case.d_nope,
            case.d_rope, case.d_lat, case.d_v, float(case.scale), _ptr(out, f64),
            _ptr(qa, f64) if qa is not None else None, _ptr(lse, f64))
        self._check(rc, "oracle_mla_decode")
        return out, lse, qa


    # ---- absorbed MLA with S queries per sequence ------------------------------
    def mla_multi(self, case, causal: bool = True):
        """(out [B,S,H,d_v], lse [B,S,H]) float64 for an MlaCase whose q_nope /
        q_rope are [B, S, H, *], bf16 or FP8 cache.

        The S queries of sequence b stand at its last S positions [pegainfer
        PR #938: plain decode and the speculative verify step run through the
        same absorbed-MLA kernel; vllm.cpp kernel matrix, row
        KERNEL-ATTN-DFLASH-PAGED-BLOCK: the (1+k) block queries attend over
        the paged context that holds their own block, under a causal or a
        non-causal in-block mask].  Causal: query s sees keys t <= n - S + s,
        so it is the one-query absorbed decode of its own q over the first
        max(0, n - S + 1 + s) keys; not causal: over all n keys.  A query with
        no key gives out = 0, lse = -inf."""
        S = case.num_queries
        out = np.zeros((case.batch, S, case.num_heads, case.d_v), np.float64)
        lse = np.zeros((case.batch, S, case.num_heads), np.float64)
        n = case.context_lens.to(torch.int64)
        for s in range(S):
            one = copy.copy(case)
            q4n = case.q_nope if case.q_nope.dim() == 4 else case.q_nope[:, None]
            q4r = case.q_rope if case.q_rope.dim() == 4 else case.q_rope[:, None]
            one.q_nope, one.q_rope = q4n[:, s].contiguous(), q4r[:, s].contiguous()
            if causal:
                one.context_lens = (n - S + 1 + s).clamp(min=0).to(torch.int32)
            if case.cache_dtype == "fp8":
                out[:, s], lse[:, s] = self.mla_fp8(one)
            else:
                out[:, s], lse[:, s], _ = self.mla(one)
        return out, lse


_DEFAULT: Optional[Oracle] = None


def default() -> Oracle:
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT
