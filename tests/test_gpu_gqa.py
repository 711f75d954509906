"""GPU parity of the GQA paged-decode path (pa_decode, pa_decode_splitkv,
pa_merge_lse) against the CPU oracle, through the C ABI.

Gate: oracle.compare (|g - r| <= 2e-2 and <= 2 bf16 ulps, floor 2^-22) on
bf16 outputs; fp32 partials within 1e-5 abs + 1e-5 rel of the float64
oracle (fp32 accumulation over at most a few thousand keys with |v| < 5).
Every pool carries NaN canaries in unused pages, page tails and (with a
window) keys older than the window, so any out-of-range read shows up as NaN.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from gpu_util import dev_case, max_parts_for, run_decode, run_merge, run_splitkv
from oracle.compare import bf16_bits, close_f32, compare
from paged_attention_decode_05_amd import workload as wl

pytestmark = pytest.mark.gpu


def _gate(out, ref, what=""):
    rep = compare(out, ref)
    print(f"[{what}] {rep}", flush=True)
    assert rep.ok, f"{what}: {rep}"
    return rep


def _lse_ok(lse_gpu, lse_ref, what=""):
    g = np.asarray(lse_gpu, np.float64)
    fin = np.isfinite(lse_ref)
    assert (np.isfinite(g) == fin).all(), what
    assert np.all(g[~fin] == -np.inf), what
    if fin.any():
        err = np.abs(g[fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin]))
        assert err.max() <= 2e-6, (what, err.max())


@pytest.mark.parametrize("layout", ["PHSD", "PSHD"])
def test_tiny_parity(oracle, layout):
    case = wl.tiny(layout=layout)
    ref, ref_lse = oracle.decode(case)
    out, lse = run_decode(dev_case(case))
    _gate(out, ref, f"tiny {layout}")
    _lse_ok(lse, ref_lse, "tiny")


def test_single_key_returns_v_row_exactly(oracle):
    """ctx = 1: softmax weight 1, so out must equal that key's V row bit for bit."""
    case = wl.tiny()
    out, lse = run_decode(dev_case(case))
    ref, ref_lse = oracle.decode(case)
    b = 0
    assert int(case.context_lens[b]) == 1
    page = int(case.block_table[b, 0])
    for h in range(case.num_q_heads):
        g = h // (case.num_q_heads // case.num_kv_heads)
        v = case.v_pool[page, g, 0]
        assert torch.equal(out[b, h].view(torch.int16), v.view(torch.int16))
    assert np.abs(lse[b].numpy() - ref_lse[b]).max() <= 2e-6 * max(1, np.abs(ref_lse[b]).max())


def test_uniform_scores_mean_of_v(oracle):
    case = wl.make_gqa_case(context_lens=(1, 31, 32, 33, 64, 100, 685, 1000), num_q_heads=8,
                            num_kv_heads=2, head_dim=128, page_size=32, seed=8001, window=300)
    case.q = torch.zeros_like(case.q)
    ref, _ = oracle.decode(case)
    out, _ = run_decode(dev_case(case))
    _gate(out, ref, "q=0")


def test_peaky_softmax(oracle):
    """q scaled by 8: scores spread over ~+-90 nats, exercising the running-max
    rescale across chunks, waves and partitions."""
    case = wl.make_gqa_case(context_lens=(1000, 4100, 37, 513), num_q_heads=8, num_kv_heads=2,
                            head_dim=128, page_size=32, seed=8002)
    case.q = (case.q.float() * 8).to(torch.bfloat16)
    ref, ref_lse = oracle.decode(case)
    out, lse = run_decode(dev_case(case))
    _gate(out, ref, "peaky")
    _lse_ok(lse, ref_lse, "peaky")


def test_context_zero_gives_zero_and_neg_inf(oracle):
    case = wl.make_gqa_case(context_lens=(0, 5, 0, 64), num_q_heads=4, num_kv_heads=1,
                            head_dim=128, page_size=16, seed=8003, max_pages=8)
    ref, ref_lse = oracle.decode(case)
    out, lse = run_decode(dev_case(case))
    assert torch.all(out[0].float() == 0) and torch.all(out[2].float() == 0)
    assert torch.all(lse[0] == -math.inf) and torch.all(lse[2] == -math.inf)
    _gate(out, ref, "ctx0")


@pytest.mark.parametrize("head_dim,group,kv_heads", [
    (64, 1, 3), (64, 2, 1), (64, 4, 3), (64, 8, 1), (64, 16, 2),
    (128, 1, 3), (128, 2, 3), (128, 4, 1), (128, 8, 3), (128, 16, 1),
    (256, 1, 3), (256, 2, 1), (256, 4, 3), (256, 8, 1), (256, 16, 1),
    # groups that are not a power of two run on the next tile size, padded
    (64, 3, 2), (128, 3, 2), (128, 5, 1), (128, 6, 2), (128, 7, 1), (128, 12, 1),
    (256, 6, 2), (256, 3, 1), (256, 12, 1), (512, 6, 1)])
def test_group_and_head_dim_sweep(oracle, head_dim, group, kv_heads):
    case = wl.make_gqa_case(context_lens=(1, 17, 32, 33, 257, 700), num_q_heads=group * kv_heads,
                            num_kv_heads=kv_heads, head_dim=head_dim, page_size=32,
                            seed=8100 + head_dim + 10 * group + kv_heads)
    ref, ref_lse = oracle.decode(case)
    out, lse = run_decode(dev_case(case))
    _gate(out, ref, f"D{head_dim} G{group} Hkv{kv_heads}")
    _lse_ok(lse, ref_lse)


@pytest.mark.parametrize("page_size,layout", [(16, "PHSD"), (64, "PHSD"), (16, "PSHD"),
                                              (64, "PSHD")])
def test_page_sizes(oracle, page_size, layout):
    case = wl.make_gqa_case(context_lens=(1, 15, 16, 17, 63, 64, 65, 900), num_q_heads=8,
                            num_kv_heads=2, head_dim=128, page_size=page_size, seed=8200 + page_size,
                            layout=layout)
    ref, _ = oracle.decode(case)
    out, _ = run_decode(dev_case(case))
    _gate(out, ref, f"ps{page_size} {layout}")


@pytest.mark.parametrize("window", [1, 31, 32, 33, 100, 4096])
def test_window_starting_mid_page(oracle, window):
    case = wl.make_gqa_case(context_lens=(1, 31, 33, 100, 685, 1000, 5000), num_q_heads=16,
                            num_kv_heads=2, head_dim=256, page_size=32, seed=8300 + window,
                            window=window, q_std=0.5)
    ref, ref_lse = oracle.decode(case)
    out, lse = run_decode(dev_case(case))
    _gate(out, ref, f"window {window}")
    _lse_ok(lse, ref_lse)


@pytest.mark.parametrize("partition_size", [1, 7, 16, 17, 64, 300, 512, 4096])
@pytest.mark.parametrize("window", [0, 90])
def test_splitkv_partials_match_oracle(oracle, partition_size, window):
    case = wl.make_gqa_case(context_lens=(0, 1, 31, 32, 33, 100, 685, 1000), num_q_heads=8,
                            num_kv_heads=2, head_dim=128, page_size=32, seed=8400, window=window)
    dc = dev_case(case)
    mp = max_parts_for(dc, partition_size)
    po, pm, ps = run_splitkv(dc, partition_size, mp)
    rpo, rpm, rps = oracle.partials(case, partition_size, mp)
    ok, err = close_f32(pm.cpu().numpy(), rpm, rtol=2e-6, atol=1e-5)
    assert ok, ("max", err)
    ok, err = close_f32(ps.cpu().numpy(), rps, rtol=1e-5, atol=1e-6)
    assert ok, ("sum", err)
    ok, err = close_f32(po.cpu().numpy(), rpo, rtol=1e-5, atol=1e-5)
    assert ok, ("out", err)
    # the GPU merge of the GPU partials passes the bf16 gate against the oracle
    ref, ref_lse = oracle.decode(case)
    out, lse = run_merge(po, pm, ps, dc.context_lens, partition_size, window)
    _gate(out, ref, f"split P={partition_size} W={window}")
    _lse_ok(lse, ref_lse)


@pytest.mark.parametrize("partition_size,window", [(64, 0), (100, 0), (48, 90)])
def test_splitkv_batch_past_64(oracle, partition_size, window):
    """More than 64 sequences, some with no key: the fixed grid's blocks find
    their partition with a scan of the context lengths 64 sequences at a time,
    partitions with keys first, then the empty ones."""
    rng = np.random.default_rng(9900 + partition_size + window)
    ctx = rng.integers(0, 700, size=100)
    ctx[rng.choice(100, size=9, replace=False)] = 0
    case = wl.make_gqa_case(context_lens=tuple(int(c) for c in ctx), num_q_heads=8,
                            num_kv_heads=2, head_dim=128, page_size=32,
                            seed=9950 + partition_size, window=window)
    dc = dev_case(case)
    mp = max_parts_for(dc, partition_size)
    po, pm, ps = run_splitkv(dc, partition_size, mp)
    rpo, rpm, rps = oracle.partials(case, partition_size, mp)
    ok, err = close_f32(pm.cpu().numpy(), rpm, rtol=2e-6, atol=1e-5)
    assert ok, ("max", err)
    ok, err = close_f32(ps.cpu().numpy(), rps, rtol=1e-5, atol=1e-6)
    assert ok, ("sum", err)
    ok, err = close_f32(po.cpu().numpy(), rpo, rtol=1e-5, atol=1e-5)
    assert ok, ("out", err)
    ref, ref_lse = oracle.decode(case)
    out, lse = run_merge(po, pm, ps, dc.context_lens, partition_size, window)
    _gate(out, ref, f"split B=100 P={partition_size} W={window}")
    _lse_ok(lse, ref_lse)


def test_splitkv_grid_past_65536_blocks(oracle):
    """Small partitions over a wide batch: max_parts x KV heads x batch is
    past 65,536 blocks, so the fixed grid folds its linear block index into
    two grid dimensions."""
    rng = np.random.default_rng(9990)
    ctx = rng.integers(0, 2100, size=64)
    ctx[:2] = (2100, 0)
    case = wl.make_gqa_case(context_lens=tuple(int(c) for c in ctx), num_q_heads=32,
                            num_kv_heads=8, head_dim=128, page_size=32, seed=9991)
    dc = dev_case(case)
    P = 16
    mp = max_parts_for(dc, P)
    assert mp * 8 * 64 > 65536
    po, pm, ps = run_splitkv(dc, P, mp)
    rpo, rpm, rps = oracle.partials(case, P, mp)
    ok, err = close_f32(pm.cpu().numpy(), rpm, rtol=2e-6, atol=1e-5)
    assert ok, ("max", err)
    ok, err = close_f32(ps.cpu().numpy(), rps, rtol=1e-5, atol=1e-6)
    assert ok, ("sum", err)
    ok, err = close_f32(po.cpu().numpy(), rpo, rtol=1e-5, atol=1e-5)
    assert ok, ("out", err)
    ref, ref_lse = oracle.decode(case)
    out, lse = run_merge(po, pm, ps, dc.context_lens, P, 0)
    _gate(out, ref, "split P=16 over 67K blocks")
    _lse_ok(lse, ref_lse)


@pytest.mark.parametrize("group,head_dim", [(3, 128), (6, 256), (12, 64)])
def test_splitkv_partials_padded_group(oracle, group, head_dim):
    """Fixed partitions with a group that is not a power of two: the padding
    heads of the kernel's tile write no partial, so the rows of the next KV
    group (NaN-filled beforehand) hold exactly the oracle's partials."""
    case = wl.make_gqa_case(context_lens=(0, 1, 33, 300, 1000), num_q_heads=2 * group,
                            num_kv_heads=2, head_dim=head_dim, page_size=32,
                            seed=8450 + group, window=700)
    dc = dev_case(case)
    P = 128
    mp = max_parts_for(dc, P)
    po, pm, ps = run_splitkv(dc, P, mp)
    rpo, rpm, rps = oracle.partials(case, P, mp)
    ok, err = close_f32(pm.cpu().numpy(), rpm, rtol=2e-6, atol=1e-5)
    assert ok, ("max", err)
    ok, err = close_f32(ps.cpu().numpy(), rps, rtol=1e-5, atol=1e-6)
    assert ok, ("sum", err)
    ok, err = close_f32(po.cpu().numpy(), rpo, rtol=1e-5, atol=1e-5)
    assert ok, ("out", err)
    ref, ref_lse = oracle.decode(case)
    out, lse = run_merge(po, pm, ps, dc.context_lens, P, case.window)
    _gate(out, ref, f"split G={group} D={head_dim}")
    _lse_ok(lse, ref_lse)


@pytest.mark.parametrize("what,kw", [
    ("tiny", dict(context_lens=(0, 1, 31, 32, 33, 64, 100, 685, 1000), num_q_heads=8,
                  num_kv_heads=2, head_dim=128, page_size=32)),
    ("window d256 G8", dict(context_lens=(1, 33, 700, 5000), num_q_heads=16, num_kv_heads=2,
                            head_dim=256, page_size=32, window=1000, q_std=0.5)),
    ("G6 d128 ps16", dict(context_lens=(0, 17, 4000, 250), num_q_heads=12, num_kv_heads=2,
                          head_dim=128, page_size=16)),
    ("G2 valu", dict(context_lens=(3, 64, 2000), num_q_heads=4, num_kv_heads=2, head_dim=128,
                     page_size=64)),
])
def test_null_workspace(oracle, what, kw):
    """A NULL workspace: one block per (sequence, KV head) row, bf16 written
    directly, no merge; the same gate against the oracle."""
    from paged_attention_decode_05_amd import binding as pb
    case = wl.make_gqa_case(seed=8470 + len(what), **kw)
    dc = dev_case(case)
    B, H, D = dc.q.shape
    out = torch.full((B, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    pb.pa_decode(dc.q, dc.k_pool, dc.v_pool, pb.kv_layout(dc.k_pool, dc.layout), dc.block_table,
                 dc.context_lens, dc.scale, dc.window, out, lse, None)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode(case)
    _gate(out.cpu(), ref, f"no workspace: {what}")
    _lse_ok(lse.cpu(), ref_lse, what)


def test_merge_on_oracle_partials(oracle):
    """The merge kernel alone, fed the oracle's partials rounded to fp32."""
    case = wl.make_gqa_case(context_lens=(0, 1, 100, 257, 1000), num_q_heads=4, num_kv_heads=2,
                            head_dim=256, page_size=16, seed=8500, window=200)
    P, mp = 64, 4
    po, pm, ps = oracle.partials(case, P, mp)
    ref, ref_lse = oracle.merge(po, pm, ps, case.context_lens, P, case.window)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()
    out, lse = run_merge(t(po), t(pm), t(ps), case.context_lens.cuda(), P, case.window)
    _gate(out, ref, "merge only")
    _lse_ok(lse, ref_lse)


def test_single_partition_merge_is_exact():
    """One live partition: the merge returns bf16 of that partial exactly."""
    case = wl.make_gqa_case(context_lens=(5, 300, 511), num_q_heads=8, num_kv_heads=2,
                            head_dim=128, page_size=32, seed=8501)
    dc = dev_case(case)
    po, pm, ps = run_splitkv(dc, 512, 1)
    out, _ = run_merge(po, pm, ps, dc.context_lens, 512, 0)
    want = po[:, :, 0, :].to(torch.bfloat16).cpu()        # torch RNE of the same fp32 values
    assert torch.equal(out.view(torch.int16), want.view(torch.int16))


def test_run_to_run_bit_identical():
    case = wl.make_gqa_case(context_lens=(1, 31, 32, 33, 64, 100, 685, 1000, 3000, 7000),
                            num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=32, seed=8600)
    dc = dev_case(case)
    first, first_lse = run_decode(dc)
    for _ in range(4):
        out, lse = run_decode(dc)
        assert torch.equal(out.view(torch.int16), first.view(torch.int16))
        assert torch.equal(lse, first_lse)


def test_workspace_needs_no_initialisation(oracle):
    """Rows cut into many pieces (one KV head, long rows), merged by the block
    that finishes last: a workspace full of random bytes, reused call after
    call, gives the same bits as a zeroed one, and passes the oracle gate."""
    from paged_attention_decode_05_amd import binding as pb
    case = wl.make_gqa_case(context_lens=(0, 1, 5000, 17, 9000, 0, 4096), num_q_heads=8,
                            num_kv_heads=1, head_dim=128, page_size=16, seed=8610)
    dc = dev_case(case)
    B, H, D = dc.q.shape
    nbytes = pb.pa_decode_workspace_size(B, H, 1, D, dc.max_pages, dc.page_size, dc.window)
    g = torch.Generator(device="cuda").manual_seed(8611)
    junk = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    ref, ref_lse = oracle.decode(case)
    base, base_lse = run_decode(dc)
    _gate(base, ref, "zeroed workspace")
    _lse_ok(base_lse, ref_lse, "zeroed workspace")
    ones = torch.full((nbytes,), 255, dtype=torch.uint8, device="cuda")
    for ws in (junk, junk, ones, ones):
        out, lse = run_decode(dc, workspace=ws)
        assert torch.equal(out.view(torch.int16), base.view(torch.int16))
        assert torch.equal(lse, base_lse)


def test_page_permutation_bit_identical():
    case = wl.make_gqa_case(context_lens=(1, 31, 32, 33, 64, 100, 685, 1000), num_q_heads=8,
                            num_kv_heads=2, head_dim=128, page_size=32, seed=8601, pool_pages=128,
                            window=300)
    perm = torch.randperm(case.num_pages, generator=torch.Generator().manual_seed(9))
    moved = case.to("cpu")
    moved.k_pool = torch.empty_like(case.k_pool)
    moved.v_pool = torch.empty_like(case.v_pool)
    moved.k_pool[perm] = case.k_pool
    moved.v_pool[perm] = case.v_pool
    bt = case.block_table.clone()
    live = bt >= 0
    bt[live] = perm.to(torch.int32)[bt[live].long()]
    moved.block_table = bt
    a, la = run_decode(dev_case(case))
    b, lb = run_decode(dev_case(moved))
    assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)


def test_reverse_interleaved_block_table(oracle):
    """Pages handed out in reverse, interleaved across sequences."""
    case = wl.make_gqa_case(context_lens=(100, 200, 300), num_q_heads=8, num_kv_heads=2,
                            head_dim=128, page_size=16, seed=8602, pool_pages=64, max_pages=19)
    bt = torch.full_like(case.block_table, -1)
    pages = list(range(63, -1, -1))
    need = [math.ceil(n / 16) for n in case.context_lens.tolist()]
    k = 0
    for i in range(max(need)):
        for b in range(3):
            if i < need[b]:
                bt[b, i] = pages[k]
                k += 1
    # rebuild pools so the new table addresses the same logical keys
    moved = case.to("cpu")
    moved.k_pool = torch.full_like(case.k_pool, float("nan"))
    moved.v_pool = torch.full_like(case.v_pool, float("nan"))
    for b in range(3):
        for i in range(need[b]):
            moved.k_pool[int(bt[b, i])] = case.k_pool[int(case.block_table[b, i])]
            moved.v_pool[int(bt[b, i])] = case.v_pool[int(case.block_table[b, i])]
    moved.block_table = bt
    ref, _ = oracle.decode(case)
    out, _ = run_decode(dev_case(moved))
    _gate(out, ref, "reverse-interleaved")


# ---- the named workloads at full size --------------------------------------------


def test_llama_full(oracle):
    case = wl.llama()
    oracle.set_threads(max(1, min(16, oracle.max_threads())))
    ref, ref_lse = oracle.decode(case)
    out, lse = run_decode(dev_case(case))
    _gate(out, ref, "llama bs64 full")
    _lse_ok(lse, ref_lse, "llama")


def test_d256w_full(oracle):
    case = wl.d256w()
    ref, ref_lse = oracle.decode(case)
    out, lse = run_decode(dev_case(case))
    _gate(out, ref, "d256 window full")
    _lse_ok(lse, ref_lse, "d256w")


def test_long_full_splitkv_512(oracle):
    """Long contexts through the explicit two-stage API with 512-key partitions."""
    case = wl.long_ctx()
    dc = dev_case(case)
    mp = max_parts_for(dc, 512)
    po, pm, ps = run_splitkv(dc, 512, mp)
    out, lse = run_merge(po, pm, ps, dc.context_lens, 512, 0)
    ref, ref_lse = oracle.decode(case)
    _gate(out, ref, "long split 512")
    _lse_ok(lse, ref_lse, "long")
    out2, _ = run_decode(dc)
    _gate(out2, ref, "long pa_decode")


@pytest.mark.parametrize("layout", ["PHSD", "PSHD"])
def test_head_dim_64_window_and_two_stage(oracle, layout):
    """head_dim 64 (every group size runs on the matrix cores): a window, 16-key
    pages, and the fixed-partition split + merge against the same oracle."""
    case = wl.make_gqa_case(context_lens=(0, 1, 15, 16, 17, 300, 2049), num_q_heads=16,
                            num_kv_heads=4, head_dim=64, page_size=16, seed=8650, layout=layout,
                            window=500)
    ref, ref_lse = oracle.decode(case)
    dc = dev_case(case)
    out, lse = run_decode(dc)
    _gate(out, ref, f"D64 window {layout}")
    _lse_ok(lse, ref_lse, "D64")
    mp = max_parts_for(dc, 128)
    po, pm, ps = run_splitkv(dc, 128, mp)
    out2, lse2 = run_merge(po, pm, ps, dc.context_lens, 128, case.window)
    _gate(out2, ref, f"D64 two-stage {layout}")
    _lse_ok(lse2, ref_lse, "D64 two-stage")
