"""Pins that tie the CPU oracle to something other than itself.

Each pin takes an ``Oracle`` handle and raises AssertionError on failure, so
the same pins run against the shipped build (all must pass) and against
builds with a planted mistake (at least one must fail).

  dense_bruteforce     oracle == float64 dense attention over materialised
                       K/V (independent numpy gather and BLAS products)
  single_token         ctx = 1 returns that token's V row exactly, lse = s
  peaky                one score 800 nats above the rest returns its V row
  uniform_scores       q = 0 returns the mean of V over the key range
  page_permutation     relabelling physical pages changes no bit
  gqa_equals_mha       GQA == MHA with each KV head replicated G times
  window_truncation    window W == no window over the last W keys re-paged
  merge_equals_unsplit merge(partials) == one pass; single partition exact;
                       empty -> (0, -inf)
  mla_unabsorbed       absorbed MLA == unabsorbed MLA (float64, < 1e-11)
  nan_canaries         NaN in every slot outside the key ranges changes nothing
  kv_insert_roundtrip  inserted rows read back bit-exact through independent
                       page/offset indexing; padding and out-of-range slots and
                       every other element untouched
  insert_then_decode   rows knocked out of a pool and inserted again at each
                       sequence's last position give a bit-identical decode
  mla_insert_concat    latent ++ rope land in the 576-wide row in that order
  multi_single_query   multi-query decode with one query == decode, bit for bit
  multi_is_shortened   causal query s == decode over the first n - S + 1 + s
                       keys (with and without a window), bit for bit
  multi_noncausal      every non-causal query == decode over the whole context
  multi_bruteforce     multi-query decode == float64 dense causal attention
  e4m3_decode          E4M3 byte values: closed forms from the OCP definition,
                       all 256 bytes == torch.float8_e4m3fn, finite codes
                       strictly increasing
  fp8_equals_bf16      FP8 pools with power-of-two scales == the bf16 oracle on
                       the exactly dequantised pools, bit for bit
  fp8_bruteforce       FP8 decode == float64 dense attention over K/V decoded
                       by torch and scaled (scales not powers of two)
  f32pool_equals_bf16  f32 pools holding bf16 values == the bf16 oracle, bit
                       for bit
  f32pool_bruteforce   f32-pool decode == float64 dense attention (full float32
                       mantissas, windows, both layouts)
  e4m3_encode          E4M3 encoding: hand-computed ties (to the even code),
                       == torch.float8_e4m3fn's conversion over every midpoint
                       and a random sweep, decode(encode(v)) == v on every code
  mla_fp8_insert       FP8 latent rows: each block exponent is the smallest e
                       with 448 * 2^e >= absmax (exact test), element bytes ==
                       torch's conversion of x * 2^-e, rope bits, zero padding,
                       other rows untouched
  mla_fp8_equals_bf16  MLA over an FP8 cache == the bf16 MLA oracle over the
                       cache dequantized by torch, bit for bit
  mla_multi_bruteforce MLA with S queries per sequence (causal and not, bf16
                       and FP8 caches, contexts shorter than S) == float64
                       unabsorbed attention with the in-block mask; one query
                       == the one-query oracle, bit for bit
"""
from __future__ import annotations

import math

import numpy as np
import torch

from brute import dense_attention, gather_rows, key_range, mla_unabsorbed, pool_f64
from oracle.compare import bf16_rne, bits_of_bf16_values, ulp_dist
from paged_attention_decode_05_amd.workload import make_gqa_case, make_mla_case

# float32 envelope for the _f32 instantiation against float64 truth: the
# pages use 1e-4 for f32 attention outputs [vllm.cpp kernel matrix, row
# KERNEL-ATTN-DFLASH-PAGED-BLOCK: f32 1e-4 / bf16 3e-2].
F32_TOL = 1e-4
F64_TOL = 1e-12

SMALL = [
    # (ctx, Hq, Hkv, D, page, layout, window)
    ((1, 5, 37, 100), 4, 2, 8, 4, "PHSD", 0),
    ((0, 16, 17, 64), 8, 2, 128, 16, "PSHD", 0),
    ((3, 33, 99), 3, 3, 8, 32, "PHSD", 0),
    ((40, 100, 7, 64), 4, 1, 16, 8, "PSHD", 13),
    ((100, 50, 1), 8, 2, 128, 32, "PHSD", 50),
]


def _small_cases():
    for i, (ctx, hq, hkv, d, ps, lay, w) in enumerate(SMALL):
        yield make_gqa_case(context_lens=ctx, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                            page_size=ps, seed=7000 + i, layout=lay, window=w)


def dense_bruteforce(o):
    for case in _small_cases():
        ref, ref_lse = dense_attention(case)
        out, lse = o.decode(case, "f64")
        assert np.allclose(out, ref, rtol=0, atol=F64_TOL), np.abs(out - ref).max()
        fin = np.isfinite(ref_lse)
        assert (np.isfinite(lse) == fin).all()
        assert np.allclose(lse[fin], ref_lse[fin], rtol=0, atol=F64_TOL)
        out32, lse32 = o.decode(case, "f32")
        assert np.abs(out32 - ref).max() <= F32_TOL, np.abs(out32 - ref).max()
        assert np.allclose(lse32[fin], ref_lse[fin], rtol=0, atol=F32_TOL)


def single_token(o):
    case = make_gqa_case(context_lens=(1, 1, 1), num_q_heads=8, num_kv_heads=2, head_dim=128,
                         page_size=32, seed=7101)
    V = pool_f64(case.v_pool)
    K = pool_f64(case.k_pool)
    q = case.q.to(torch.float64).numpy()
    bt = case.block_table.numpy()
    for prec in ("f64", "f32"):
        out, lse = o.decode(case, prec)
        for b in range(case.batch):
            for h in range(case.num_q_heads):
                g = h // 4
                v = gather_rows(V, case.layout, bt[b], np.array([0]), 32, g)[0]
                k = gather_rows(K, case.layout, bt[b], np.array([0]), 32, g)[0]
                assert np.array_equal(out[b, h], v), (prec, b, h)
                s = case.scale * float(k @ q[b, h])
                tol = F64_TOL if prec == "f64" else F32_TOL
                assert abs(lse[b, h] - s) <= tol, (prec, lse[b, h], s)


def peaky(o):
    """A score far above the others takes all the weight: q aligned with one
    key at magnitude 800 nats beyond the rest (exp(-800) underflows to 0)."""
    case = make_gqa_case(context_lens=(50,), num_q_heads=1, num_kv_heads=1, head_dim=8,
                         page_size=4, seed=7102)
    V = pool_f64(case.v_pool)
    bt = case.block_table.numpy()
    # keys: all zero except token 17 = e_0; q = 6400 * e_0 (exact in bf16)
    t17 = 17
    page, slot = int(bt[0, t17 // 4]), t17 % 4
    live = (case.k_pool == case.k_pool)                     # keep NaN canaries
    case.k_pool = torch.where(live, torch.zeros_like(case.k_pool), case.k_pool)
    case.k_pool[page, 0, slot, 0] = 1.0
    case.q = torch.zeros_like(case.q)
    case.q[0, 0, 0] = 6400.0
    case.scale = 0.125
    out, lse = o.decode(case, "f64")
    v17 = gather_rows(V, case.layout, bt[0], np.array([t17]), 4, 0)[0]
    assert np.array_equal(out[0, 0], v17)
    assert lse[0, 0] == 800.0


def uniform_scores(o):
    case = make_gqa_case(context_lens=(1, 31, 32, 33, 100), num_q_heads=4, num_kv_heads=2,
                         head_dim=128, page_size=32, seed=7103, window=40)
    case.q = torch.zeros_like(case.q)
    V = pool_f64(case.v_pool)
    bt = case.block_table.numpy()
    out, _ = o.decode(case, "f64")
    out32, _ = o.decode(case, "f32")
    for b, n in enumerate(case.context_lens.tolist()):
        lo, hi = key_range(n, case.window)
        for h in range(case.num_q_heads):
            mean = gather_rows(V, case.layout, bt[b], np.arange(lo, hi), 32, h // 2).mean(axis=0)
            assert np.abs(out[b, h] - mean).max() <= F64_TOL
            # float32 result: within one bf16 step of the exact mean once both are rounded
            a = bits_of_bf16_values(bf16_rne(out32[b, h]))
            r = bits_of_bf16_values(bf16_rne(mean))
            assert ulp_dist(a, r).max() <= 1


def page_permutation(o):
    case = make_gqa_case(context_lens=(1, 31, 32, 33, 64, 100, 685, 1000), num_q_heads=8,
                         num_kv_heads=2, head_dim=128, page_size=32, seed=7104, pool_pages=128,
                         window=300)
    perm = torch.randperm(case.num_pages, generator=torch.Generator().manual_seed(5))
    moved = case.to("cpu")
    moved.k_pool = torch.empty_like(case.k_pool)
    moved.v_pool = torch.empty_like(case.v_pool)
    moved.k_pool[perm] = case.k_pool
    moved.v_pool[perm] = case.v_pool
    bt = case.block_table.clone()
    live = bt >= 0
    bt[live] = perm.to(torch.int32)[bt[live].long()]
    moved.block_table = bt
    for prec in ("f64", "f32"):
        a, la = o.decode(case, prec)
        b, lb = o.decode(moved, prec)
        assert np.array_equal(a, b) and np.array_equal(la, lb), prec


def gqa_equals_mha(o):
    case = make_gqa_case(context_lens=(5, 77, 130), num_q_heads=8, num_kv_heads=2, head_dim=64,
                         page_size=16, seed=7105)
    G = 4
    mha = case.to("cpu")
    mha.k_pool = case.k_pool.repeat_interleave(G, dim=1).contiguous()
    mha.v_pool = case.v_pool.repeat_interleave(G, dim=1).contiguous()
    mha.num_kv_heads = 8
    for prec in ("f64", "f32"):
        a, la = o.decode(case, prec)
        b, lb = o.decode(mha, prec)
        assert np.array_equal(a, b) and np.array_equal(la, lb), prec


def _repage_window(case):
    """Copy keys [lo, n) of every sequence into a fresh pool starting at
    logical token 0, with a fresh block table; window removed."""
    ps = case.page_size
    ctx = case.context_lens.tolist()
    spans = [key_range(n, case.window) for n in ctx]
    new_ctx = [hi - lo for lo, hi in spans]
    fresh = make_gqa_case(context_lens=new_ctx, num_q_heads=case.num_q_heads,
                          num_kv_heads=case.num_kv_heads, head_dim=case.head_dim, page_size=ps,
                          seed=case.seed + 1, layout=case.layout, window=0)
    fresh.q = case.q.clone()
    fresh.scale = case.scale
    for b, (lo, hi) in enumerate(spans):
        for i, t in enumerate(range(lo, hi)):
            sp, ss = int(case.block_table[b, t // ps]), t % ps
            dp, ds = int(fresh.block_table[b, i // ps]), i % ps
            if case.layout == "PHSD":
                fresh.k_pool[dp, :, ds] = case.k_pool[sp, :, ss]
                fresh.v_pool[dp, :, ds] = case.v_pool[sp, :, ss]
            else:
                fresh.k_pool[dp, ds] = case.k_pool[sp, ss]
                fresh.v_pool[dp, ds] = case.v_pool[sp, ss]
    return fresh


def window_truncation(o):
    for lay, seed in (("PHSD", 7106), ("PSHD", 7107)):
        case = make_gqa_case(context_lens=(1, 20, 33, 64, 65, 200), num_q_heads=4,
                             num_kv_heads=1, head_dim=16, page_size=8, seed=seed, layout=lay,
                             window=33)
        fresh = _repage_window(case)
        for prec in ("f64", "f32"):
            a, la = o.decode(case, prec)
            b, lb = o.decode(fresh, prec)
            assert np.array_equal(a, b) and np.array_equal(la, lb), (lay, prec)


def merge_equals_unsplit(o):
    for window, seed in ((0, 7108), (90, 7109)):
        case = make_gqa_case(context_lens=(0, 1, 31, 32, 33, 100, 257), num_q_heads=4,
                             num_kv_heads=2, head_dim=32, page_size=16, seed=seed, window=window)
        ref, ref_lse = o.decode(case, "f64")
        fin = np.isfinite(ref_lse)
        for P in (1, 7, 16, 32, 100, 512):
            maxp = max(1, math.ceil(257 / P))
            po, pm, pl = o.partials(case, P, maxp, "f64")
            out, lse = o.merge(po, pm, pl, case.context_lens, P, window, "f64")
            assert np.abs(out - ref).max() <= F64_TOL, (window, P)
            assert (np.isfinite(lse) == fin).all()
            assert np.abs(lse[fin] - ref_lse[fin]).max() <= F64_TOL
            # partitions past the live count are empty
            for b, n in enumerate(case.context_lens.tolist()):
                lo, hi = key_range(n, window)
                live = math.ceil((hi - lo) / P)
                assert np.all(pm[b, :, live:] == -np.inf) and np.all(pl[b, :, live:] == 0)
                assert np.all(po[b, :, live:] == 0)
        # one partition covering everything: the merge returns it bit for bit
        po, pm, pl = o.partials(case, 4096, 1, "f64")
        out, lse = o.merge(po, pm, pl, case.context_lens, 4096, window, "f64")
        assert np.array_equal(out, ref)
        assert np.array_equal(np.isfinite(lse), fin)
        # a context of 0 has no live partition: out = 0, lse = -inf
        assert np.all(out[0] == 0) and np.all(lse[0] == -np.inf)
    # hand-made partials: every live partition empty -> (0, -inf)
    po = np.ones((1, 1, 3, 4))
    pm = np.full((1, 1, 3), -np.inf)
    pl = np.zeros((1, 1, 3))
    out, lse = o.merge(po, pm, pl, np.array([30]), 10, 0, "f64")
    assert np.all(out == 0) and lse[0, 0] == -np.inf
    # two partitions with closed-form weights: m = (0, ln 3), l = (1, 1)
    po = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    pm = np.array([[[0.0, math.log(3.0)]]])
    pl = np.array([[[1.0, 1.0]]])
    out, lse = o.merge(po, pm, pl, np.array([20]), 10, 0, "f64")
    assert np.allclose(out[0, 0], [0.25, 0.75], atol=1e-15)
    assert abs(lse[0, 0] - math.log(4.0)) <= 1e-15


def mla_unabsorbed(o):
    import brute
    for ctx, heads, ps, seed in (((1, 17, 70), 3, 16, 7110), ((64, 65), 1, 64, 7111)):
        case = make_mla_case(context_lens=ctx, num_heads=heads, page_size=ps, seed=seed)
        ref = brute.mla_unabsorbed(case)
        out, _, _ = o.mla(case, "f64")
        assert np.abs(out - ref).max() < 1e-11, np.abs(out - ref).max()
        out32, _, _ = o.mla(case, "f32")
        assert np.abs(out32 - ref).max() <= F32_TOL * max(1.0, np.abs(ref).max())


def nan_canaries(o):
    for window in (0, 45):
        clean = make_gqa_case(context_lens=(1, 31, 32, 33, 100), num_q_heads=4, num_kv_heads=2,
                              head_dim=32, page_size=16, seed=7112, window=window, poison=False)
        dirty = make_gqa_case(context_lens=(1, 31, 32, 33, 100), num_q_heads=4, num_kv_heads=2,
                              head_dim=32, page_size=16, seed=7112, window=window, poison=True)
        assert torch.isnan(dirty.k_pool.float()).any()
        a, la = o.decode(clean, "f64")
        b, lb = o.decode(dirty, "f64")
        assert not np.isnan(b).any()
        assert np.array_equal(a, b) and np.array_equal(la, lb)
    mclean = make_mla_case(context_lens=(3, 70), num_heads=2, page_size=16, seed=7113, poison=False)
    mdirty = make_mla_case(context_lens=(3, 70), num_heads=2, page_size=16, seed=7113, poison=True)
    a, _, _ = o.mla(mclean, "f64")
    b, _, _ = o.mla(mdirty, "f64")
    assert not np.isnan(b).any() and np.array_equal(a, b)


def _slot(bt_row, t, page_size):
    return int(bt_row[t // page_size]) * page_size + t % page_size


def _row(pool, layout, slot, page_size, g):
    page, off = slot // page_size, slot % page_size
    return pool[page, g, off] if layout == "PHSD" else pool[page, off, g]


def kv_insert_roundtrip(o):
    from oracle.oracle import _Pool
    gen = torch.Generator().manual_seed(7120)
    for layout, Hkv, D, ps in (("PHSD", 2, 16, 8), ("PSHD", 3, 8, 16)):
        case = make_gqa_case(context_lens=(5, 40), num_q_heads=Hkv, num_kv_heads=Hkv, head_dim=D,
                             page_size=ps, seed=7121, layout=layout, poison=False, pool_pages=12)
        total = case.num_pages * ps
        slots = [3, total - 1, -1, 17, total, 40, 2 * ps]       # -1 padding, total out of range
        T = len(slots)
        k_new = torch.randn(T, Hkv, D, generator=gen).to(torch.bfloat16)
        v_new = torch.randn(T, Hkv, D, generator=gen).to(torch.bfloat16)
        ps_, hs, ts = case.strides()
        pool = _Pool(case.num_pages, ps, Hkv, D, ps_, hs, ts)
        k2, v2 = o.kv_insert(k_new, v_new, case.k_pool, case.v_pool, pool, slots)
        touched = torch.zeros(case.k_pool.shape[:3], dtype=torch.bool)
        for i, s in enumerate(slots):
            if not 0 <= s < total:
                continue
            for g in range(Hkv):
                assert torch.equal(_row(k2, layout, s, ps, g).view(torch.int16),
                                   k_new[i, g].view(torch.int16))
                assert torch.equal(_row(v2, layout, s, ps, g).view(torch.int16),
                                   v_new[i, g].view(torch.int16))
                page, off = s // ps, s % ps
                if layout == "PHSD":
                    touched[page, g, off] = True
                else:
                    touched[page, off, g] = True
        keep = ~touched
        assert torch.equal(k2[keep].view(torch.int16), case.k_pool[keep].view(torch.int16))
        assert torch.equal(v2[keep].view(torch.int16), case.v_pool[keep].view(torch.int16))


def insert_then_decode(o):
    from oracle.oracle import _Pool
    for layout in ("PHSD", "PSHD"):
        case = make_gqa_case(context_lens=(1, 17, 32, 33), num_q_heads=4, num_kv_heads=2,
                             head_dim=16, page_size=16, seed=7122, layout=layout, poison=False)
        ref, ref_lse = o.decode(case, "f64")
        bt = case.block_table.numpy()
        slots = [_slot(bt[b], int(n) - 1, 16) for b, n in enumerate(case.context_lens.tolist())]
        k_new = torch.stack([torch.stack([_row(case.k_pool, layout, s, 16, g) for g in range(2)])
                             for s in slots])
        v_new = torch.stack([torch.stack([_row(case.v_pool, layout, s, 16, g) for g in range(2)])
                             for s in slots])
        damaged = case.to("cpu")
        damaged.k_pool = case.k_pool.clone()
        damaged.v_pool = case.v_pool.clone()
        for s in slots:
            for g in range(2):
                _row(damaged.k_pool, layout, s, 16, g).fill_(float("nan"))
                _row(damaged.v_pool, layout, s, 16, g).fill_(float("nan"))
        ps_, hs, ts = case.strides()
        pool = _Pool(case.num_pages, 16, 2, 16, ps_, hs, ts)
        damaged.k_pool, damaged.v_pool = o.kv_insert(k_new, v_new, damaged.k_pool, damaged.v_pool,
                                                     pool, slots)
        out, lse = o.decode(damaged, "f64")
        assert np.array_equal(out, ref) and np.array_equal(lse, ref_lse)


def mla_insert_concat(o):
    gen = torch.Generator().manual_seed(7123)
    P, S, dl, dr = 6, 8, 12, 4
    cache = torch.randn(P, S, dl + dr, generator=gen).to(torch.bfloat16)
    slots = [0, 13, -1, P * S - 1, P * S]
    kv_c = torch.randn(len(slots), dl, generator=gen).to(torch.bfloat16)
    k_pe = torch.randn(len(slots), dr, generator=gen).to(torch.bfloat16)
    out = o.mla_cache_insert(kv_c, k_pe, cache, slots)
    touched = torch.zeros(P, S, dtype=torch.bool)
    for i, s in enumerate(slots):
        if not 0 <= s < P * S:
            continue
        row = out[s // S, s % S]
        assert torch.equal(row[:dl].view(torch.int16), kv_c[i].view(torch.int16))
        assert torch.equal(row[dl:].view(torch.int16), k_pe[i].view(torch.int16))
        touched[s // S, s % S] = True
    assert torch.equal(out[~touched].view(torch.int16), cache[~touched].view(torch.int16))


def _multi_case(S, window, seed, ctx=(2, 5, 33, 70)):
    return make_gqa_case(context_lens=ctx, num_q_heads=4, num_kv_heads=2, head_dim=16,
                         page_size=8, seed=seed, window=window, num_queries=S)


def _single_of(case, s, ctx_shift):
    one = case.to("cpu")
    one.q = (case.q if case.q.dim() == 4 else case.q[:, None])[:, s].contiguous()
    one.context_lens = (case.context_lens - ctx_shift).clamp(min=0).to(torch.int32)
    return one


def multi_single_query(o):
    for causal in (True, False):
        case = _multi_case(1, 0, 7130)
        out, lse = o.decode_multi(case, causal)
        ref, ref_lse = o.decode(_single_of(case, 0, 0))
        assert np.array_equal(out[:, 0], ref) and np.array_equal(lse[:, 0], ref_lse)


def multi_is_shortened(o):
    for window in (0, 20):
        case = _multi_case(3, window, 7131)
        out, lse = o.decode_multi(case, True)
        for s in range(3):
            ref, ref_lse = o.decode(_single_of(case, s, 3 - 1 - s))
            assert np.array_equal(out[:, s], ref) and np.array_equal(lse[:, s], ref_lse), (window, s)


def multi_noncausal(o):
    case = _multi_case(3, 0, 7132)
    out, lse = o.decode_multi(case, False)
    for s in range(3):
        ref, ref_lse = o.decode(_single_of(case, s, 0))
        assert np.array_equal(out[:, s], ref) and np.array_equal(lse[:, s], ref_lse)


def multi_bruteforce(o):
    import brute
    for causal, window in ((True, 0), (True, 6), (False, 0)):
        case = _multi_case(4, window, 7133, ctx=(1, 3, 9, 40))
        case_clean = make_gqa_case(context_lens=(1, 3, 9, 40), num_q_heads=4, num_kv_heads=2,
                                   head_dim=16, page_size=8, seed=7133, window=window,
                                   num_queries=4, poison=False)
        ref, ref_lse = brute.dense_multi(case_clean, causal)
        out, lse = o.decode_multi(case, causal)
        assert np.abs(out - ref).max() < 1e-12, (causal, window, np.abs(out - ref).max())
        fin = np.isfinite(ref_lse)
        assert np.array_equal(fin, np.isfinite(lse))
        assert np.abs(lse[fin] - ref_lse[fin]).max() < 1e-12


def e4m3_decode(o):
    # closed forms of the OCP E4M3 definition (bias 7, subnormals m * 2^-9)
    want = {0x00: 0.0, 0x01: 2.0**-9, 0x07: 7 * 2.0**-9, 0x08: 2.0**-6, 0x30: 0.5,
            0x38: 1.0, 0x3C: 1.5, 0x40: 2.0, 0x77: 240.0, 0x7E: 448.0, 0xB8: -1.0,
            0xFE: -448.0}
    for b, v in want.items():
        assert o.e4m3_value(b) == v, (hex(b), o.e4m3_value(b), v)
    assert math.copysign(1.0, o.e4m3_value(0x80)) == -1.0 and o.e4m3_value(0x80) == 0.0
    assert math.isnan(o.e4m3_value(0x7F)) and math.isnan(o.e4m3_value(0xFF))
    # every byte against torch's decoder
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([o.e4m3_value(b) for b in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin])
    assert np.all(np.diff(got[:0x7F]) > 0)


def _fp8_case(seed, ks, vs, **kw):
    base = dict(context_lens=(0, 1, 5, 37, 100), num_q_heads=4, num_kv_heads=2, head_dim=16,
                page_size=8, window=0)
    base.update(kw)
    return make_gqa_case(seed=seed, kv_dtype="fp8", k_scale=ks, v_scale=vs, **base)


def fp8_equals_bf16(o):
    from brute import fp8_pool_f64
    for layout, window, ks, vs in (("PHSD", 0, 2.0**-6, 2.0**-5), ("PSHD", 30, 2.0**-4, 2.0**-7)):
        c8 = _fp8_case(7140, ks, vs, layout=layout, window=window)
        c16 = c8.to("cpu")
        c16.kv_dtype, c16.k_scale, c16.v_scale = "bf16", 1.0, 1.0
        c16.k_pool = torch.from_numpy(fp8_pool_f64(c8.k_pool, ks)).to(torch.bfloat16)
        c16.v_pool = torch.from_numpy(fp8_pool_f64(c8.v_pool, vs)).to(torch.bfloat16)
        # the dequantised values are exact in bf16 (3 mantissa bits, power-of-two scale)
        back = torch.from_numpy(fp8_pool_f64(c8.k_pool, ks))
        assert torch.equal(c16.k_pool.to(torch.float64).nan_to_num(7.0), back.nan_to_num(7.0))
        out8, lse8 = o.decode_fp8(c8)
        out16, lse16 = o.decode(c16, "f64")
        assert np.array_equal(out8, out16) and np.array_equal(lse8, lse16), (layout, window)


def fp8_bruteforce(o):
    for i, (layout, window) in enumerate((("PHSD", 0), ("PSHD", 0), ("PHSD", 40))):
        c = _fp8_case(7150 + i, 0.0173, 0.0291, layout=layout, window=window, poison=False)
        ref, ref_lse = dense_attention(c)
        cp = _fp8_case(7150 + i, 0.0173, 0.0291, layout=layout, window=window)
        out, lse = o.decode_fp8(cp)
        assert np.abs(out - ref).max() < F64_TOL, np.abs(out - ref).max()
        fin = np.isfinite(ref_lse)
        assert np.array_equal(fin, np.isfinite(lse))
        assert np.abs(lse[fin] - ref_lse[fin]).max() < F64_TOL


def _f32_case(seed, **kw):
    base = dict(context_lens=(0, 1, 5, 37, 100), num_q_heads=4, num_kv_heads=2, head_dim=16,
                page_size=8, window=0)
    base.update(kw)
    return make_gqa_case(seed=seed, kv_dtype="f32", **base)


def f32pool_equals_bf16(o):
    for layout, window in (("PHSD", 0), ("PSHD", 30)):
        c16 = make_gqa_case(context_lens=(0, 1, 5, 37, 100), num_q_heads=4, num_kv_heads=2,
                            head_dim=16, page_size=8, seed=7160, layout=layout, window=window)
        c32 = c16.to("cpu")
        c32.kv_dtype = "f32"
        c32.k_pool = c16.k_pool.to(torch.float32)
        c32.v_pool = c16.v_pool.to(torch.float32)
        out32, lse32 = o.decode_f32pool(c32)
        out16, lse16 = o.decode(c16, "f64")
        assert np.array_equal(out32, out16) and np.array_equal(lse32, lse16), (layout, window)


def f32pool_bruteforce(o):
    for i, (layout, window) in enumerate((("PHSD", 0), ("PSHD", 0), ("PHSD", 40))):
        c = _f32_case(7170 + i, layout=layout, window=window, poison=False)
        ref, ref_lse = dense_attention(c)
        cp = _f32_case(7170 + i, layout=layout, window=window)
        out, lse = o.decode_f32pool(cp)
        assert np.abs(out - ref).max() < F64_TOL, np.abs(out - ref).max()
        fin = np.isfinite(ref_lse)
        assert np.array_equal(fin, np.isfinite(lse))
        assert np.abs(lse[fin] - ref_lse[fin]).max() < F64_TOL


def e4m3_encode(o):
    # hand-computed from the OCP definition: ties go to the even code
    want = {0.0: 0x00, 1.0: 0x38, 1.0625: 0x38, 1.1875: 0x3A, -3.0: 0xC4, 448.0: 0x7E,
            440.0: 0x7E, 432.0: 0x7E, 424.0: 0x7D, 2.0**-10: 0x00, 3 * 2.0**-10: 0x02,
            2.0**-6 - 2.0**-10: 0x08, -(2.0**-9): 0x81, 0.3: 0x2A}
    for v, b in want.items():
        assert o.e4m3_encode(v) == b, (v, hex(o.e4m3_encode(v)), hex(b))
    assert o.e4m3_encode(-0.0) == 0x80
    # every finite code round-trips
    for b in range(256):
        if (b & 0x7F) != 0x7F:
            assert o.e4m3_encode(o.e4m3_value(b)) == b, hex(b)
    # against torch's round-to-nearest-even conversion: every midpoint between
    # neighbouring codes (and its negative) and a random sweep of +-448
    vals = torch.arange(0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64)
    mids = (vals[1:] + vals[:-1]) / 2
    gen = torch.Generator().manual_seed(7190)
    sweep = (torch.rand(4000, generator=gen, dtype=torch.float64) * 2 - 1) * 448.0
    x = torch.cat([mids, -mids, sweep, sweep * 2.0**-8]).to(torch.float32)
    ref = x.to(torch.float8_e4m3fn).view(torch.uint8).tolist()
    got = [o.e4m3_encode(float(v)) for v in x.tolist()]
    bad = [(float(x[i]), got[i], ref[i]) for i in range(len(ref)) if got[i] != ref[i]]
    assert not bad, bad[:5]


def mla_fp8_insert(o):
    gen = torch.Generator().manual_seed(7200)
    T, P, S = 24, 4, 8
    x = torch.randn(T, 512, generator=gen, dtype=torch.float64)
    # per-block magnitudes from 2^-140 to 2^40; one all-zero block; a block
    # whose absmax is exactly 448; a block of exact E4M3 ties at scale 1
    mag = torch.exp2(torch.randint(-140, 41, (T, 8), generator=gen).to(torch.float64))
    x = x * mag.repeat_interleave(64, dim=1)
    x[0, 64:128] = 0.0
    x[1, :64] = 1.0
    x[1, 0] = 448.0
    x[2, :64] = torch.tensor([1.0625, 1.1875, -3.0, 2.0**-10, 3 * 2.0**-10, 432.0, 448.0] * 9 + [1.0])
    kv_c = x.to(torch.bfloat16)
    k_pe = torch.randn(T, 64, generator=gen).to(torch.bfloat16)
    cache = torch.randint(0, 256, (P, S, 656), generator=gen, dtype=torch.int64).to(torch.uint8)
    perm = torch.randperm(P * S, generator=gen)[:T - 2]
    slots = torch.cat([perm, torch.tensor([-1, P * S])])
    new = o.mla_cache_insert_fp8(kv_c, k_pe, cache, slots)
    xs = kv_c.to(torch.float64)
    touched = set()
    for i, sl in enumerate(slots.tolist()):
        if not 0 <= sl < P * S:
            continue
        touched.add(sl)
        row = new[sl // S, sl % S]
        for j in range(8):
            blk = xs[i, 64 * j:64 * (j + 1)]
            e = int(row[640 + j]) - 127
            a = float(blk.abs().max())
            if a == 0.0 or a <= 448.0 * 2.0**-126:
                assert e == -126, (i, j, a, e)
            else:   # the smallest e with 448 * 2^e >= absmax
                assert 448.0 * 2.0**(e - 1) < a <= 448.0 * 2.0**e, (i, j, a, e)
            q = (blk * 2.0**-e).to(torch.float32)
            ref = q.to(torch.float8_e4m3fn).view(torch.uint8)
            assert torch.equal(row[64 * j:64 * (j + 1)], ref), (i, j)
        assert torch.equal(row[512:640], k_pe[i].contiguous().view(torch.uint8))
        assert int(row[648:].sum()) == 0
    s0 = int(slots[0])                  # token 0's zero block 1 takes the clamped exponent
    assert int(new[s0 // S, s0 % S, 641]) == -126 + 127
    for sl in range(P * S):
        if sl not in touched:
            assert torch.equal(new[sl // S, sl % S], cache[sl // S, sl % S]), sl


def mla_fp8_equals_bf16(o):
    from brute import mla_fp8_rows_f64
    for seed, ctx, page in ((7210, (0, 1, 17, 40), 16), (7211, (63, 64, 65), 64)):
        c8 = make_mla_case(context_lens=ctx, num_heads=5, page_size=page, seed=seed,
                           cache_dtype="fp8")
        deq = torch.from_numpy(mla_fp8_rows_f64(c8.cache))
        c16 = c8.to("cpu")
        c16.cache_dtype = "bf16"
        c16.cache = deq.to(torch.bfloat16)
        # the dequantized values are exact in bf16 (4 significant bits, power-of-two scale)
        assert torch.equal(c16.cache.to(torch.float64).nan_to_num(7.0), deq.nan_to_num(7.0))
        out8, lse8 = o.mla_fp8(c8)
        out16, lse16, _ = o.mla(c16, "f64")
        assert np.array_equal(out8, out16) and np.array_equal(lse8, lse16), seed


def mla_multi_bruteforce(o):
    from brute import mla_unabsorbed_multi
    for seed, S, ctx, page, dt in ((7220, 3, (0, 1, 2, 3, 17, 40), 16, "bf16"),
                                   (7221, 4, (2, 63, 64, 65, 130), 64, "fp8"),
                                   (7222, 2, (1, 33), 32, "bf16")):
        case = make_mla_case(context_lens=ctx, num_heads=3, page_size=page, seed=seed,
                             num_queries=S, cache_dtype=dt)
        for causal in (True, False):
            out, lse = o.mla_multi(case, causal)
            ref, ref_lse = mla_unabsorbed_multi(case, causal)
            assert np.abs(out - ref).max() < 1e-11, (seed, causal, np.abs(out - ref).max())
            assert np.array_equal(np.isinf(lse), np.isinf(ref_lse)), (seed, causal)
            fin = np.isfinite(ref_lse)
            assert np.abs(lse[fin] - ref_lse[fin]).max() < 1e-11, (seed, causal)
            if causal:      # the mask is load-bearing: the last query differs from the first
                assert not np.allclose(out[:, 0], out[:, -1])
    one = make_mla_case(context_lens=(5, 70), num_heads=4, page_size=16, seed=7223)
    mq = one.to("cpu")
    mq.q_nope, mq.q_rope = one.q_nope[:, None], one.q_rope[:, None]
    for causal in (True, False):
        a, la = o.mla_multi(mq, causal)
        b, lb, _ = o.mla(one, "f64")
        assert np.array_equal(a[:, 0], b) and np.array_equal(la[:, 0], lb)


PINS = {
    "dense_bruteforce": dense_bruteforce,
    "single_token": single_token,
    "peaky": peaky,
    "uniform_scores": uniform_scores,
    "page_permutation": page_permutation,
    "gqa_equals_mha": gqa_equals_mha,
    "window_truncation": window_truncation,
    "merge_equals_unsplit": merge_equals_unsplit,
    "mla_unabsorbed": mla_unabsorbed,
    "nan_canaries": nan_canaries,
    "kv_insert_roundtrip": kv_insert_roundtrip,
    "insert_then_decode": insert_then_decode,
    "mla_insert_concat": mla_insert_concat,
    "multi_single_query": multi_single_query,
    "multi_is_shortened": multi_is_shortened,
    "multi_noncausal": multi_noncausal,
    "multi_bruteforce": multi_bruteforce,
    "e4m3_decode": e4m3_decode,
    "fp8_equals_bf16": fp8_equals_bf16,
    "fp8_bruteforce": fp8_bruteforce,
    "f32pool_equals_bf16": f32pool_equals_bf16,
    "f32pool_bruteforce": f32pool_bruteforce,
    "e4m3_encode": e4m3_encode,
    "mla_fp8_insert": mla_fp8_insert,
    "mla_fp8_equals_bf16": mla_fp8_equals_bf16,
    "mla_multi_bruteforce": mla_multi_bruteforce,
}


def run_all(o) -> dict:
    """name -> None (passed) or the failure text."""
    res = {}
    for name, fn in PINS.items():
        try:
            fn(o)
            res[name] = None
        except Exception as e:  # noqa: BLE001 -- a planted mistake may fail any way
            res[name] = f"{type(e).__name__}: {e}"
    return res
