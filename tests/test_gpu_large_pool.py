"""Pools past 4 GiB: byte offsets above 2^32 in every read and write path.

Each case's pages are moved to pages spread up to the top of a pool larger
than 2^32 bytes, every other page NaN.  Since the result does not depend on
where the pages sit, each decode must equal the same decode over the compact
pool bit for bit, and pass the oracle gate; the inserts must land at the right
rows at the top of the pool and nowhere else.
"""
from __future__ import annotations

import pytest
import torch

from gpu_util import dev_case, run_decode, run_decode_fp8, run_mla
from oracle.compare import compare
from paged_attention_decode_05_amd import binding as pb
from paged_attention_decode_05_amd import workload as wl

pytestmark = pytest.mark.gpu

GIB4 = 1 << 32


def _gate(out, ref, what):
    rep = compare(out, ref)
    print(f"[{what}] {rep}", flush=True)
    assert rep.ok, f"{what}: {rep}"


def _spread(n_small: int, n_big: int) -> torch.Tensor:
    """Big-pool page of small page p: from the top down, evenly spread."""
    step = max(1, (n_big - 1) // max(1, n_small))
    return torch.tensor([n_big - 1 - step * p for p in range(n_small)], dtype=torch.int64)


def _relocate(pool: torch.Tensor, bt: torch.Tensor, n_big: int, fill):
    """(big pool on the device, remapped block table): page p of `pool` goes to
    page _spread(p); the rest of the big pool holds `fill`."""
    where = _spread(pool.shape[0], n_big)
    big = torch.full((n_big,) + tuple(pool.shape[1:]), fill, dtype=pool.dtype, device="cuda")
    big.index_copy_(0, where.cuda(), pool.cuda())
    bt2 = bt.clone()
    live = bt2 >= 0
    bt2[live] = where[bt2[live].long()].to(torch.int32)
    return big, bt2


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_gqa_decode_above_4gib(oracle, kv_dtype):
    kw = dict(kv_dtype="fp8", k_scale=0.0173, v_scale=0.0291) if kv_dtype == "fp8" else {}
    case = wl.make_gqa_case(context_lens=(1, 100, 3000, 7777), num_q_heads=32, num_kv_heads=8,
                            head_dim=128, page_size=32, seed=8600, **kw)
    page_bytes = case.k_pool[0].numel() * case.k_pool.element_size()
    n_big = GIB4 // page_bytes + 4096                  # past 2^32 bytes
    ref, _ = oracle.decode_fp8(case) if kv_dtype == "fp8" else oracle.decode(case)
    run = run_decode_fp8 if kv_dtype == "fp8" else run_decode
    small, small_lse = run(dev_case(case))
    fill = wl.FP8_NAN if kv_dtype == "fp8" else float("nan")
    big = case.to("cpu")
    big.k_pool, bt = _relocate(case.k_pool, case.block_table, n_big, fill)
    big.v_pool, _ = _relocate(case.v_pool, case.block_table, n_big, fill)
    big.block_table = bt
    big.num_pages = n_big
    assert big.k_pool.numel() * big.k_pool.element_size() > GIB4
    assert int(bt.max()) * page_bytes > GIB4 - page_bytes
    dc = big.to("cuda")
    out, lse = run(dc)
    assert torch.equal(out.view(torch.int16), small.view(torch.int16))
    assert torch.equal(lse, small_lse)
    _gate(out, ref, f"{kv_dtype} decode, pages above 4 GiB")
    del big, dc
    _free()


@pytest.mark.parametrize("cache_dtype", ["bf16", "fp8"])
def test_mla_decode_above_4gib(oracle, cache_dtype):
    case = wl.make_mla_case(context_lens=(1, 700, 2049), num_heads=64, page_size=64, seed=8610,
                            cache_dtype=cache_dtype)
    page_bytes = case.cache[0].numel() * case.cache.element_size()
    n_big = GIB4 // page_bytes + 2048
    fill = wl.FP8_NAN if cache_dtype == "fp8" else float("nan")
    if cache_dtype == "fp8":
        ref, _ = oracle.mla_fp8(case)
    else:
        ref, _, _ = oracle.mla(case)

    def run(c):
        if cache_dtype == "bf16":
            return run_mla(c)
        B, H = c.q_nope.shape[0], c.q_nope.shape[1]
        out = torch.full((B, H, c.d_v), float("nan"), dtype=torch.bfloat16, device="cuda")
        n = pb.mla_absorbed_decode_workspace_size(B, H, c.max_pages, c.page_size, 0)
        ws = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")
        pb.mla_absorbed_decode_fp8(c.q_nope, c.q_rope, c.cache, pb.kv_layout(c.cache, "PSR"),
                                   c.w_uk, c.w_uv, c.block_table, c.context_lens, c.scale, out,
                                   ws)
        torch.cuda.synchronize()
        return out.cpu()

    small = run(case.to("cuda"))
    big = case.to("cpu")
    big.cache, big.block_table = _relocate(case.cache, case.block_table, n_big, fill)
    big.num_pages = n_big
    assert big.cache.numel() * big.cache.element_size() > GIB4
    out = run(big.to("cuda"))
    assert torch.equal(out.view(torch.int16), small.view(torch.int16))
    _gate(out, ref, f"MLA {cache_dtype}, pages above 4 GiB")
    del big
    _free()


def test_inserts_above_4gib():
    """K/V and MLA rows (bf16 and FP8) written to the top slots of pools past
    2^32 bytes land there and nowhere else."""
    gen = torch.Generator().manual_seed(8620)
    T = 40
    # K/V pools [P][Hkv][page][D] bf16, 64 KiB pages
    Hkv, D, S = 8, 128, 32
    P = GIB4 // (Hkv * S * D * 2) + 64
    k_pool = torch.zeros(P, Hkv, S, D, dtype=torch.bfloat16, device="cuda")
    v_pool = torch.zeros_like(k_pool)
    slots = torch.tensor([P * S - 1 - 37 * i for i in range(T)], dtype=torch.int64)
    k_new = torch.randn(T, Hkv, D, generator=gen).to(torch.bfloat16)
    v_new = torch.randn(T, Hkv, D, generator=gen).to(torch.bfloat16)
    pb.pa_kv_insert(k_new.cuda(), v_new.cuda(), k_pool, v_pool, pb.kv_layout(k_pool, "PHSD"),
                    slots.cuda())
    torch.cuda.synchronize()
    pages, offs = (slots // S).cuda(), (slots % S).cuda()
    got_k = k_pool[pages, :, offs, :].cpu()
    got_v = v_pool[pages, :, offs, :].cpu()
    assert torch.equal(got_k.view(torch.int16), k_new.view(torch.int16))
    assert torch.equal(got_v.view(torch.int16), v_new.view(torch.int16))
    k_pool[pages, :, offs, :] = 0
    assert int((k_pool != 0).sum()) == 0               # nothing written elsewhere
    del k_pool, v_pool
    _free()
    # MLA caches: bf16 rows of 576 and FP8 rows of 656 bytes, 64-token pages
    kv_c = torch.randn(T, 512, generator=gen).to(torch.bfloat16)
    k_pe = torch.randn(T, 64, generator=gen).to(torch.bfloat16)
    for row, dtype, insert in ((576, torch.bfloat16, pb.mla_cache_insert),
                               (pb.MLA_FP8_ROW, torch.uint8, pb.mla_cache_insert_fp8)):
        esz = 2 if dtype == torch.bfloat16 else 1
        P = GIB4 // (64 * row * esz) + 64
        cache = torch.zeros(P, 64, row, dtype=dtype, device="cuda")
        slots = torch.tensor([P * 64 - 1 - 53 * i for i in range(T)], dtype=torch.int64)
        insert(kv_c.cuda(), k_pe.cuda(), cache, pb.kv_layout(cache, "PSR"), slots.cuda())
        torch.cuda.synchronize()
        pages, offs = (slots // 64).cuda(), (slots % 64).cuda()
        rows = cache[pages, offs, :].cpu()
        if dtype == torch.bfloat16:
            assert torch.equal(rows[:, :512].view(torch.int16), kv_c.view(torch.int16))
            assert torch.equal(rows[:, 512:].view(torch.int16), k_pe.view(torch.int16))
        else:
            assert torch.equal(rows[:, 512:640], k_pe.view(torch.uint8))
            assert int(rows[:, 640:648].min()) >= 1 and int(rows[:, 648:].sum()) == 0
        cache[pages, offs, :] = 0
        assert int((cache != 0).sum()) == 0
        del cache
        _free()
