"""GPU parity of the cache writes (pa_kv_insert, mla_cache_insert) against the
CPU oracle, through the C ABI.

A copy does not round, so the gate is bit equality of the whole pool: the
written slots hold the new rows and every other element is unchanged.  The
slot lists mix distinct valid slots with padding (-1) and out-of-range
slots, which must be skipped.  Insert-then-decode closes the loop with the
attention kernels: rows knocked out of a pool (NaN) and written back by the
insert kernel give a bit-identical decode.
"""
from __future__ import annotations

import pytest
import torch

from gpu_util import run_decode, run_mla
from oracle.compare import compare
from oracle.oracle import _Pool
from paged_attention_decode_05_amd import binding as pb
from paged_attention_decode_05_amd import workload as wl

pytestmark = pytest.mark.gpu


def _bits_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.detach().cpu().contiguous().view(torch.int16),
                       b.detach().cpu().contiguous().view(torch.int16))


def _slots(total: int, n: int, seed: int) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed)
    s = torch.randperm(total, generator=g)[:n].to(torch.int64)
    extra = torch.tensor([-1, total, -5, total + 100], dtype=torch.int64)
    return torch.cat([s[: n // 2], extra, s[n // 2:]])


def _pool_desc(case) -> _Pool:
    ps, hs, ts = case.strides()
    return _Pool(case.num_pages, case.page_size, case.num_kv_heads, case.head_dim, ps, hs, ts)


@pytest.mark.parametrize("layout", ["PHSD", "PSHD"])
@pytest.mark.parametrize("hkv,d", [(1, 128), (2, 128), (8, 128), (2, 256), (4, 64)])
def test_kv_insert_matches_oracle(oracle, layout, hkv, d):
    case = wl.make_gqa_case(context_lens=(100, 300), num_q_heads=hkv, num_kv_heads=hkv,
                            head_dim=d, page_size=32, seed=9800 + hkv + d, layout=layout,
                            poison=False, pool_pages=40)
    total = case.num_pages * case.page_size
    slots = _slots(total, 600, 9801)
    g = torch.Generator().manual_seed(9802)
    k_new = torch.randn(len(slots), hkv, d, generator=g).to(torch.bfloat16)
    v_new = torch.randn(len(slots), hkv, d, generator=g).to(torch.bfloat16)
    ref_k, ref_v = oracle.kv_insert(k_new, v_new, case.k_pool, case.v_pool, _pool_desc(case), slots)
    dc = case.to("cuda")
    pb.pa_kv_insert(k_new.cuda(), v_new.cuda(), dc.k_pool, dc.v_pool, pb.kv_layout(dc.k_pool, layout),
                    slots.cuda())
    torch.cuda.synchronize()
    assert _bits_equal(dc.k_pool, ref_k) and _bits_equal(dc.v_pool, ref_v)


def test_kv_insert_strided_source(oracle):
    """Sources with padded rows ([T, Hkv, D + 24] sliced to D, heads 2 apart)."""
    case = wl.make_gqa_case(context_lens=(64,), num_q_heads=4, num_kv_heads=2, head_dim=128,
                            page_size=16, seed=9810, poison=False, pool_pages=20)
    slots = _slots(case.num_pages * 16, 200, 9811)
    g = torch.Generator().manual_seed(9812)
    big_k = torch.randn(len(slots), 4, 152, generator=g).to(torch.bfloat16)
    big_v = torch.randn(len(slots), 4, 152, generator=g).to(torch.bfloat16)
    k_view, v_view = big_k[:, ::2, :128], big_v[:, ::2, :128]
    ref_k, ref_v = oracle.kv_insert(k_view.contiguous(), v_view.contiguous(), case.k_pool,
                                    case.v_pool, _pool_desc(case), slots)
    dc = case.to("cuda")
    gk, gv = big_k.cuda(), big_v.cuda()
    pb.pa_kv_insert(gk[:, ::2, :128], gv[:, ::2, :128], dc.k_pool, dc.v_pool,
                    pb.kv_layout(dc.k_pool, "PHSD"), slots.cuda())
    torch.cuda.synchronize()
    assert _bits_equal(dc.k_pool, ref_k) and _bits_equal(dc.v_pool, ref_v)


def test_many_tokens_many_blocks(oracle):
    case = wl.make_gqa_case(context_lens=(4000, 4000), num_q_heads=8, num_kv_heads=8,
                            head_dim=128, page_size=32, seed=9820, poison=False)
    total = case.num_pages * case.page_size
    slots = _slots(total, 5000, 9821)
    g = torch.Generator().manual_seed(9822)
    k_new = torch.randn(len(slots), 8, 128, generator=g).to(torch.bfloat16)
    v_new = torch.randn(len(slots), 8, 128, generator=g).to(torch.bfloat16)
    ref_k, ref_v = oracle.kv_insert(k_new, v_new, case.k_pool, case.v_pool, _pool_desc(case), slots)
    dc = case.to("cuda")
    pb.pa_kv_insert(k_new.cuda(), v_new.cuda(), dc.k_pool, dc.v_pool,
                    pb.kv_layout(dc.k_pool, "PHSD"), slots.cuda())
    torch.cuda.synchronize()
    assert _bits_equal(dc.k_pool, ref_k) and _bits_equal(dc.v_pool, ref_v)


def _last_slots(case):
    bt = case.block_table
    ps = case.page_size
    return torch.tensor([int(bt[b, (n - 1) // ps]) * ps + (n - 1) % ps
                         for b, n in enumerate(case.context_lens.tolist())], dtype=torch.int64)


@pytest.mark.parametrize("layout", ["PHSD", "PSHD"])
def test_insert_then_decode(oracle, layout):
    """The new token of every sequence, knocked out and re-inserted, gives the
    same decode bit for bit (and passes the oracle gate)."""
    case = wl.make_gqa_case(context_lens=(1, 31, 32, 33, 700, 2049), num_q_heads=16,
                            num_kv_heads=4, head_dim=128, page_size=32, seed=9830, layout=layout)
    ref, _ = oracle.decode(case)
    base, base_lse = run_decode(case.to("cuda"))
    slots = _last_slots(case)
    dc = case.to("cuda")
    ps = case.page_size
    pages, offs = (slots // ps).tolist(), (slots % ps).tolist()
    if layout == "PHSD":
        k_new = torch.stack([case.k_pool[p, :, o] for p, o in zip(pages, offs)])
        v_new = torch.stack([case.v_pool[p, :, o] for p, o in zip(pages, offs)])
        for p, o in zip(pages, offs):
            dc.k_pool[p, :, o] = float("nan")
            dc.v_pool[p, :, o] = float("nan")
    else:
        k_new = torch.stack([case.k_pool[p, o] for p, o in zip(pages, offs)])
        v_new = torch.stack([case.v_pool[p, o] for p, o in zip(pages, offs)])
        for p, o in zip(pages, offs):
            dc.k_pool[p, o] = float("nan")
            dc.v_pool[p, o] = float("nan")
    pb.pa_kv_insert(k_new.cuda(), v_new.cuda(), dc.k_pool, dc.v_pool,
                    pb.kv_layout(dc.k_pool, layout), slots.cuda())
    out, lse = run_decode(dc)
    assert _bits_equal(out, base) and torch.equal(lse, base_lse)
    assert compare(out, ref).ok


def test_mla_cache_insert_matches_oracle(oracle):
    """Latent and rope parts taken as column slices of one projection output."""
    P, S = 30, 64
    g = torch.Generator().manual_seed(9840)
    cache = torch.randn(P, S, 576, generator=g).to(torch.bfloat16)
    slots = _slots(P * S, 900, 9841)
    proj = torch.randn(len(slots), 640, generator=g).to(torch.bfloat16)   # 512 latent, 64 rope, pad
    kv_c, k_pe = proj[:, :512], proj[:, 512:576]
    ref = oracle.mla_cache_insert(kv_c.contiguous(), k_pe.contiguous(), cache, slots)
    gc = cache.cuda()
    gp = proj.cuda()
    pb.mla_cache_insert(gp[:, :512], gp[:, 512:576], gc, pb.kv_layout(gc, "PSR"), slots.cuda())
    torch.cuda.synchronize()
    assert _bits_equal(gc, ref)


def test_mla_insert_then_decode(oracle):
    case = wl.make_mla_case(context_lens=(1, 64, 65, 500), num_heads=16, page_size=64, seed=9850)
    ref, _, _ = oracle.mla(case)
    base = run_mla(case.to("cuda"))
    slots = _last_slots(case)
    dc = case.to("cuda")
    rows = torch.stack([case.cache[s // 64, s % 64] for s in slots.tolist()])
    for s in slots.tolist():
        dc.cache[s // 64, s % 64] = float("nan")
    pb.mla_cache_insert(rows[:, :512].cuda(), rows[:, 512:].contiguous().cuda(), dc.cache,
                        pb.kv_layout(dc.cache, "PSR"), slots.cuda())
    out = run_mla(dc)
    assert _bits_equal(out, base)
    assert compare(out, ref).ok
