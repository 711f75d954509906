"""Seeded synthetic inputs for paged decode attention.

This module only draws random numbers and lays them out: context lengths, a
random physical-page permutation, block tables, q / K / V pools (or the MLA
latent cache and weights), and NaN canaries in every pool slot that no
correct reader may touch.  It holds none of the attention arithmetic, so the
CPU oracle and the GPU path can both consume it.

Recipe (one ``torch.Generator`` on the CPU, draws in this fixed order):
context lengths -> page permutation -> q -> K pool -> V pool (MLA: q_nope ->
q_rope -> latent cache -> W_UK -> W_UV).  Values are drawn as float32 normals
and rounded to bf16 (round-to-nearest-even) on the CPU, so every consumer sees
identical bytes.  Sequence b owns the next ceil(ctx_b / page_size) entries of
the permutation; unused block-table entries are -1.

Named workloads (sizes of the pages' serving shapes; scale 1/sqrt(head_dim)
unless stated, pool = ceil(1.1 * pages in use) unless stated):
  tiny   8 seqs, ctx {1,31,32,33,64,100,685,1000}, 8 q / 2 KV heads, D 128,
         page 32, 128-page pool
  llama  64 seqs, 32 q / 8 KV heads, D 128, page 32, ctx ~ U{512..8192}
  d256w  32 seqs, 16 q / 2 KV heads, D 256, page 32, ctx ~ U{1024..16384},
         window 4096, q ~ N(0, 0.5^2)
  long   4 seqs, 32 q / 8 KV heads, D 128, page 32,
         ctx {32768, 65536, 100000, 131072}, 512-token partitions
  llama_fp8  the llama shape with OCP E4M3 K/V pools, k_scale 0.0173,
         v_scale 0.0291 (values N(0, 1) rounded to E4M3 precision)
  llama_f32  the llama shape with float32 K/V pools
  mla    16 seqs, 128 heads, q_nope 128 + q_rope 64, 576-wide latent rows in
         64-token pages, ctx ~ U{1024..8192}, W_UK/W_UV ~ N(0, 0.02^2),
         scale 1/sqrt(192)
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Sequence

import torch

# Pool axis orders.  "PHSD" = [page][kv head][slot][dim]: one (page, head)
# tile is a contiguous page_size x D block.  "PSHD" = [page][slot][kv head]
# [dim], the layout the pages' engines use; the library takes strides, so both
# run through the same kernels.
LAYOUTS = ("PHSD", "PSHD")

SEED_BASE = 1000


@dataclass
class GqaCase:
    q: torch.Tensor                 # [B, Hq, D] bf16
    k_pool: torch.Tensor            # bf16, shape per layout
    v_pool: torch.Tensor
    block_table: torch.Tensor       # [B, max_pages] int32, -1 padded
    context_lens: torch.Tensor      # [B] int32
    num_pages: int
    page_size: int
    num_kv_heads: int
    head_dim: int
    layout: str
    scale: float
    window: int                     # <= 0: no window
    partition_size: Optional[int] = None
    name: str = "custom"
    seed: int = 0
    # "bf16" pools, "f32" pools, or "fp8": one OCP E4M3 byte per element (uint8
    # tensors), the element's value being e4m3(byte) * k_scale (K) or * v_scale (V)
    kv_dtype: str = "bf16"
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def kv_elem_bytes(self) -> int:
        return {"fp8": 1, "bf16": 2, "f32": 4}[self.kv_dtype]

    @property
    def num_q_heads(self) -> int:
        return int(self.q.shape[-2])

    @property
    def num_queries(self) -> int:
        """Query tokens per sequence: q is [B, Hq, D] (1) or [B, S, Hq, D]."""
        return int(self.q.shape[1]) if self.q.dim() == 4 else 1

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    def strides(self) -> tuple[int, int, int]:
        """(page_stride, head_stride, token_stride) in elements."""
        s = self.k_pool.stride()
        if self.layout == "PHSD":
            return s[0], s[1], s[2]
        return s[0], s[2], s[1]

    def kv_read_tokens(self) -> int:
        """Keys each KV head streams per call (window-limited; with several
        queries, the union of their key ranges)."""
        tot = 0
        reach = self.window + self.num_queries - 1
        for n in self.context_lens.tolist():
            lo = max(0, n - reach) if self.window > 0 else 0
            tot += n - lo
        return tot

    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes one decode call must read."""
        return self.kv_read_tokens() * 2 * self.num_kv_heads * self.head_dim * self.kv_elem_bytes

    def to(self, device) -> "GqaCase":
        c = GqaCase(**{f: getattr(self, f) for f in self.__dataclass_fields__})
        c.q = self.q.to(device)
        c.k_pool = self.k_pool.to(device)
        c.v_pool = self.v_pool.to(device)
        c.block_table = self.block_table.to(device)
        c.context_lens = self.context_lens.to(device)
        return c


@dataclass
class MlaCase:
    q_nope: torch.Tensor            # [B, H, d_nope] bf16, or [B, S, H, d_nope] (S queries)
    q_rope: torch.Tensor            # [B, H, d_rope] bf16, or [B, S, H, d_rope]
    cache: torch.Tensor             # [P, page_size, d_lat + d_rope] bf16, or
                                    # [P, page_size, MLA_FP8_ROW] uint8 (FP8 rows)
    w_uk: torch.Tensor              # [H, d_nope, d_lat] bf16
    w_uv: torch.Tensor              # [H, d_v, d_lat] bf16
    block_table: torch.Tensor       # [B, max_pages] int32
    context_lens: torch.Tensor      # [B] int32
    num_pages: int
    page_size: int
    d_nope: int
    d_rope: int
    d_lat: int
    d_v: int
    scale: float
    name: str = "custom"
    seed: int = 0
    cache_dtype: str = "bf16"       # "bf16" or "fp8"

    @property
    def batch(self) -> int:
        return int(self.q_nope.shape[0])

    @property
    def num_heads(self) -> int:
        return int(self.q_nope.shape[-2])

    @property
    def num_queries(self) -> int:
        return int(self.q_nope.shape[1]) if self.q_nope.dim() == 4 else 1

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    def latent_bytes(self) -> int:
        row = MLA_FP8_ROW if self.cache_dtype == "fp8" else (self.d_lat + self.d_rope) * 2
        return int(self.context_lens.sum()) * row

    def algorithmic_bytes(self) -> int:
        """Latent rows + both weight tensors + q in + out, read/written once."""
        w = (self.w_uk.numel() + self.w_uv.numel()) * 2
        q = (self.q_nope.numel() + self.q_rope.numel()) * 2
        out = self.batch * self.num_queries * self.num_heads * self.d_v * 2
        return self.latent_bytes() + w + q + out

    def to(self, device) -> "MlaCase":
        c = MlaCase(**{f: getattr(self, f) for f in self.__dataclass_fields__})
        for f in ("q_nope", "q_rope", "cache", "w_uk", "w_uv", "block_table", "context_lens"):
            setattr(c, f, getattr(self, f).to(device))
        return c


def _normal_bf16(gen: torch.Generator, shape, std: float = 1.0) -> torch.Tensor:
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16)


def _assign_pages(gen, ctx: Sequence[int], page_size: int, max_pages: int,
                  pool_pages: Optional[int]):
    need = [(n + page_size - 1) // page_size for n in ctx]
    used = sum(need)
    if pool_pages is None:
        pool_pages = max(1, math.ceil(1.1 * used))
    if used > pool_pages:
        raise ValueError(f"pool of {pool_pages} pages cannot hold {used}")
    perm = torch.randperm(pool_pages, generator=gen).to(torch.int32)
    bt = torch.full((len(ctx), max_pages), -1, dtype=torch.int32)
    pos = 0
    for b, k in enumerate(need):
        if k > max_pages:
            raise ValueError(f"sequence {b} needs {k} pages > max_pages {max_pages}")
        bt[b, :k] = perm[pos:pos + k]
        pos += k
    return bt, pool_pages


# E4M3 bit pattern of NaN (S.1111.111), the canary of an FP8 pool
FP8_NAN = 0x7F

# FP8 latent-cache row of the MLA path, in bytes: 512 E4M3 latent values
# (8 blocks of 64), 64 bf16 rope values, 8 block-scale bytes, 8 zero bytes.
MLA_FP8_LAT, MLA_FP8_ROPE = 512, 64
MLA_FP8_SCALES = MLA_FP8_LAT + 2 * MLA_FP8_ROPE          # offset of the scale bytes
MLA_FP8_ROW = MLA_FP8_SCALES + 16


def _fp8_mla_rows(gen: torch.Generator, pages: int, page_size: int) -> torch.Tensor:
    """Random FP8 latent-cache rows [pages, page_size, MLA_FP8_ROW] uint8:
    latent bytes are E4M3 codes of N(0, 1) * 112 (torch's conversion, clamped
    to +-448), scale bytes uniform in 118..121 (block scales 2^-9 .. 2^-6, so
    the latent values are about N(0, 1) * 0.2 .. 1.75), the rope part bf16
    normals, the padding zero."""
    rows = torch.zeros(pages, page_size, MLA_FP8_ROW, dtype=torch.uint8)
    rows[..., :MLA_FP8_LAT] = _normal_fp8(gen, (pages, page_size, MLA_FP8_LAT), 1.0 / 112.0)
    rope = _normal_bf16(gen, (pages, page_size, MLA_FP8_ROPE))
    rows[..., MLA_FP8_LAT:MLA_FP8_SCALES] = rope.view(torch.uint8)
    rows[..., MLA_FP8_SCALES:MLA_FP8_SCALES + MLA_FP8_LAT // 64] = torch.randint(
        118, 122, (pages, page_size, MLA_FP8_LAT // 64), generator=gen, dtype=torch.int64).to(torch.uint8)
    return rows


def _poison_fp8_rows(rows: torch.Tensor, sel) -> None:
    """NaN canaries in FP8 latent rows: E4M3 NaN latent bytes and bf16 NaN
    rope values (0x7FC0)."""
    rows[sel + (slice(0, MLA_FP8_LAT),)] = FP8_NAN
    rope = rows[sel + (slice(MLA_FP8_LAT, MLA_FP8_SCALES),)]
    rope[..., 0::2] = 0xC0
    rope[..., 1::2] = 0x7F
    rows[sel + (slice(MLA_FP8_LAT, MLA_FP8_SCALES),)] = rope


def _normal_fp8(gen: torch.Generator, shape, scale: float) -> torch.Tensor:
    """Bytes of N(0, 1) / scale cast to OCP E4M3 (torch's round-to-nearest
    conversion, clamped to the finite range +-448), as a uint8 tensor: the
    element's value is e4m3(byte) * scale."""
    x = torch.randn(*shape, generator=gen, dtype=torch.float32).div_(scale).clamp_(-448.0, 448.0)
    return x.to(torch.float8_e4m3fn).view(torch.uint8)


def _poison_gqa(pool: torch.Tensor, layout: str, bt: torch.Tensor, ctx, page_size: int,
                window: int) -> None:
    """NaN every slot no correct reader touches: unused pages, the tail of each
    sequence's last page, and (with a window) every key older than the window."""
    nan = FP8_NAN if pool.dtype == torch.uint8 else float("nan")
    live = torch.zeros(pool.shape[0], dtype=torch.bool)
    for b, n in enumerate(ctx):
        k = (n + page_size - 1) // page_size
        if k:
            live[bt[b, :k].long()] = True
    pool[~live] = nan

    def poison_slots(page: int, s0: int, s1: int):
        if s1 <= s0:
            return
        if layout == "PHSD":
            pool[page, :, s0:s1, :] = nan
        else:
            pool[page, s0:s1, :, :] = nan

    for b, n in enumerate(ctx):
        k = (n + page_size - 1) // page_size
        if k == 0:
            continue
        poison_slots(int(bt[b, k - 1]), n - (k - 1) * page_size, page_size)
        lo = max(0, n - window) if window > 0 else 0
        for p in range(lo // page_size):
            poison_slots(int(bt[b, p]), 0, page_size)
        if lo % page_size:
            poison_slots(int(bt[b, lo // page_size]), 0, lo % page_size)


def make_gqa_case(*, context_lens: Sequence[int], num_q_heads: int, num_kv_heads: int,
                  head_dim: int, page_size: int, seed: int, max_pages: Optional[int] = None,
                  pool_pages: Optional[int] = None, layout: str = "PHSD", window: int = 0,
                  q_std: float = 1.0, scale: Optional[float] = None, poison: bool = True,
                  partition_size: Optional[int] = None, name: str = "custom",
                  ctx_draw: Optional[tuple] = None, batch: Optional[int] = None,
                  num_queries: int = 1, kv_dtype: str = "bf16", k_scale: float = 1.0,
                  v_scale: float = 1.0) -> GqaCase:
    """Build one GQA decode case.  ``ctx_draw=(lo, hi)`` draws ``batch`` context
    lengths uniformly from the integers lo..hi (inclusive) instead of using
    ``context_lens``.  ``num_queries`` > 1 gives q of shape [B, S, Hq, D] (the
    last S positions of each context), for multi-query decode; the NaN
    canaries then spare the S - 1 keys the earlier queries' windows reach
    further back.  ``kv_dtype="fp8"`` draws E4M3 pools whose values times
    k_scale / v_scale are N(0, 1) samples rounded to E4M3 precision;
    ``kv_dtype="f32"`` draws float32 N(0, 1) pools (full float32 mantissas)."""
    if layout not in LAYOUTS:
        raise ValueError(layout)
    gen = torch.Generator().manual_seed(int(seed))
    if ctx_draw is not None:
        lo, hi = ctx_draw
        ctx = torch.randint(lo, hi + 1, (int(batch),), generator=gen, dtype=torch.int64).tolist()
    else:
        ctx = [int(n) for n in context_lens]
    if max_pages is None:
        top = ctx_draw[1] if ctx_draw is not None else max(ctx + [1])
        max_pages = max(1, (top + page_size - 1) // page_size)
    bt, pool_pages = _assign_pages(gen, ctx, page_size, max_pages, pool_pages)
    B = len(ctx)
    qshape = (B, num_q_heads, head_dim) if num_queries == 1 else (B, num_queries, num_q_heads, head_dim)
    q = _normal_bf16(gen, qshape, q_std)
    if layout == "PHSD":
        shape = (pool_pages, num_kv_heads, page_size, head_dim)
    else:
        shape = (pool_pages, page_size, num_kv_heads, head_dim)
    if kv_dtype == "fp8":
        k_pool = _normal_fp8(gen, shape, k_scale)
        v_pool = _normal_fp8(gen, shape, v_scale)
    elif kv_dtype == "bf16":
        k_pool = _normal_bf16(gen, shape)
        v_pool = _normal_bf16(gen, shape)
    elif kv_dtype == "f32":
        k_pool = torch.randn(*shape, generator=gen, dtype=torch.float32)
        v_pool = torch.randn(*shape, generator=gen, dtype=torch.float32)
    else:
        raise ValueError(kv_dtype)
    if poison:
        reach = window + num_queries - 1 if window > 0 else 0
        _poison_gqa(k_pool, layout, bt, ctx, page_size, reach)
        _poison_gqa(v_pool, layout, bt, ctx, page_size, reach)
    return GqaCase(q=q, k_pool=k_pool, v_pool=v_pool, block_table=bt,
                   context_lens=torch.tensor(ctx, dtype=torch.int32), num_pages=pool_pages,
                   page_size=page_size, num_kv_heads=num_kv_heads, head_dim=head_dim,
                   layout=layout, scale=(1.0 / math.sqrt(head_dim)) if scale is None else scale,
                   window=window, partition_size=partition_size, name=name, seed=seed,
                   kv_dtype=kv_dtype, k_scale=k_scale if kv_dtype == "fp8" else 1.0,
                   v_scale=v_scale if kv_dtype == "fp8" else 1.0)


def make_mla_case(*, context_lens: Sequence[int] = (), num_heads: int, page_size: int, seed: int,
                  d_nope: int = 128, d_rope: int = 64, d_lat: int = 512, d_v: int = 128,
                  max_pages: Optional[int] = None, pool_pages: Optional[int] = None,
                  w_std: float = 0.02, scale: Optional[float] = None, poison: bool = True,
                  name: str = "custom", ctx_draw: Optional[tuple] = None,
                  batch: Optional[int] = None, cache_dtype: str = "bf16",
                  num_queries: int = 1) -> MlaCase:
    """``num_queries`` > 1 gives q_nope / q_rope of shape [B, S, H, *]: the S
    queries of a sequence stand at its last S positions (its context length
    counts them)."""
    gen = torch.Generator().manual_seed(int(seed))
    if ctx_draw is not None:
        lo, hi = ctx_draw
        ctx = torch.randint(lo, hi + 1, (int(batch),), generator=gen, dtype=torch.int64).tolist()
    else:
        ctx = [int(n) for n in context_lens]
    if max_pages is None:
        top = ctx_draw[1] if ctx_draw is not None else max(ctx + [1])
        max_pages = max(1, (top + page_size - 1) // page_size)
    bt, pool_pages = _assign_pages(gen, ctx, page_size, max_pages, pool_pages)
    B = len(ctx)
    qs = (B, num_heads) if num_queries == 1 else (B, num_queries, num_heads)
    q_nope = _normal_bf16(gen, qs + (d_nope,))
    q_rope = _normal_bf16(gen, qs + (d_rope,))
    if cache_dtype == "fp8":
        assert (d_lat, d_rope) == (MLA_FP8_LAT, MLA_FP8_ROPE)
        cache = _fp8_mla_rows(gen, pool_pages, page_size)
    elif cache_dtype == "bf16":
        cache = _normal_bf16(gen, (pool_pages, page_size, d_lat + d_rope))
    else:
        raise ValueError(cache_dtype)
    w_uk = _normal_bf16(gen, (num_heads, d_nope, d_lat), w_std)
    w_uv = _normal_bf16(gen, (num_heads, d_v, d_lat), w_std)
    if poison:
        live = torch.zeros(pool_pages, dtype=torch.bool)
        for b, n in enumerate(ctx):
            k = (n + page_size - 1) // page_size
            if k:
                live[bt[b, :k].long()] = True
                tail = (int(bt[b, k - 1]), slice(n - (k - 1) * page_size, None))
                if cache_dtype == "fp8":
                    _poison_fp8_rows(cache, tail)
                else:
                    cache[tail + (slice(None),)] = float("nan")
        if cache_dtype == "fp8":
            _poison_fp8_rows(cache, (~live,))
        else:
            cache[~live] = float("nan")
    qk_dim = d_nope + d_rope
    return MlaCase(q_nope=q_nope, q_rope=q_rope, cache=cache, w_uk=w_uk, w_uv=w_uv,
                   block_table=bt, context_lens=torch.tensor(ctx, dtype=torch.int32),
                   num_pages=pool_pages, page_size=page_size, d_nope=d_nope, d_rope=d_rope,
                   d_lat=d_lat, d_v=d_v,
                   scale=(1.0 / math.sqrt(qk_dim)) if scale is None else scale,
                   name=name, seed=seed, cache_dtype=cache_dtype)


# ---- the five named workloads ------------------------------------------------

TINY_CTX = (1, 31, 32, 33, 64, 100, 685, 1000)
LONG_CTX = (32768, 65536, 100000, 131072)


def tiny(layout: str = "PHSD", poison: bool = True, seed: int = SEED_BASE + 1) -> GqaCase:
    return make_gqa_case(context_lens=TINY_CTX, num_q_heads=8, num_kv_heads=2, head_dim=128,
                         page_size=32, seed=seed, pool_pages=128, layout=layout, poison=poison,
                         name="tiny")


def llama(layout: str = "PHSD", poison: bool = True, seed: int = SEED_BASE + 2) -> GqaCase:
    return make_gqa_case(context_lens=(), ctx_draw=(512, 8192), batch=64, num_q_heads=32,
                         num_kv_heads=8, head_dim=128, page_size=32, seed=seed, layout=layout,
                         poison=poison, name="llama")


def llama_fp8(layout: str = "PHSD", poison: bool = True, seed: int = SEED_BASE + 5) -> GqaCase:
    """The llama shape over OCP E4M3 pools, one scale per pool."""
    return make_gqa_case(context_lens=(), ctx_draw=(512, 8192), batch=64, num_q_heads=32,
                         num_kv_heads=8, head_dim=128, page_size=32, seed=seed, layout=layout,
                         poison=poison, name="llama_fp8", kv_dtype="fp8", k_scale=0.0173,
                         v_scale=0.0291)


def llama_f32(layout: str = "PHSD", poison: bool = True, seed: int = SEED_BASE + 6) -> GqaCase:
    """The llama shape over float32 pools."""
    return make_gqa_case(context_lens=(), ctx_draw=(512, 8192), batch=64, num_q_heads=32,
                         num_kv_heads=8, head_dim=128, page_size=32, seed=seed, layout=layout,
                         poison=poison, name="llama_f32", kv_dtype="f32")


def d512(layout: str = "PHSD", poison: bool = True, seed: int = SEED_BASE + 7) -> GqaCase:
    """head_dim 512 (a global-attention layer's head size), 16 q / 2 KV heads:
    the same K/V bytes per key as the llama shape."""
    return make_gqa_case(context_lens=(), ctx_draw=(512, 8192), batch=64, num_q_heads=16,
                         num_kv_heads=2, head_dim=512, page_size=32, seed=seed, layout=layout,
                         poison=poison, name="d512")


def d256w(layout: str = "PHSD", poison: bool = True, seed: int = SEED_BASE + 3) -> GqaCase:
    return make_gqa_case(context_lens=(), ctx_draw=(1024, 16384), batch=32, num_q_heads=16,
                         num_kv_heads=2, head_dim=256, page_size=32, seed=seed, layout=layout,
                         window=4096, q_std=0.5, poison=poison, name="d256w")


def long_ctx(layout: str = "PHSD", poison: bool = True, seed: int = SEED_BASE + 4) -> GqaCase:
    return make_gqa_case(context_lens=LONG_CTX, num_q_heads=32, num_kv_heads=8, head_dim=128,
                         page_size=32, seed=seed, layout=layout, poison=poison,
                         partition_size=512, name="long")


def mla(poison: bool = True, seed: int = SEED_BASE + 5) -> MlaCase:
    return make_mla_case(ctx_draw=(1024, 8192), batch=16, num_heads=128, page_size=64,
                         seed=seed, poison=poison, name="mla")


def mla_fp8(poison: bool = True, seed: int = SEED_BASE + 5) -> MlaCase:
    """The mla workload (same seed: the same context lengths, q, weights and
    block tables) over an FP8 latent cache."""
    return make_mla_case(ctx_draw=(1024, 8192), batch=16, num_heads=128, page_size=64,
                         seed=seed, poison=poison, name="mla_fp8", cache_dtype="fp8")


def mla_verify(poison: bool = True, seed: int = SEED_BASE + 9, cache_dtype: str = "bf16") -> MlaCase:
    """The mla shape with 4 queries per sequence (one token and three drafts
    to verify), causal within the block: 512 query heads over each page."""
    return make_mla_case(ctx_draw=(1024, 8192), batch=16, num_heads=128, page_size=64,
                         seed=seed, poison=poison, name="mla_verify", num_queries=4,
                         cache_dtype=cache_dtype)


NAMED = {"tiny": tiny, "llama": llama, "d256w": d256w, "long": long_ctx, "mla": mla,
         "llama_fp8": llama_fp8, "llama_f32": llama_f32, "d512": d512, "mla_fp8": mla_fp8,
         "mla_verify": mla_verify}
