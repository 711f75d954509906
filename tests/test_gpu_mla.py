"""GPU parity of absorbed MLA decode (mla_absorbed_decode) against the CPU
oracle, through the C ABI.

Gate: oracle.compare (|g - r| <= 2e-2 and <= 2 bf16 ulps, floor 2^-22) on the
bf16 output [B, H, 128] against the float64 oracle, which keeps q_abs, the
scores, o_lat and the W_UV product unrounded.  The GPU carries q_abs, P and
o_lat as hi + lo bf16 pairs into fp32-accumulating MFMAs, which keeps each
product within a few fp32 ulps.  Every cache carries NaN canaries in unused
pages and the tail of each sequence's last page; the workspace starts as
NaN bytes, so a partial that is read but never written shows up too.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_util import run_mla
from oracle.compare import compare
from paged_attention_decode_05_amd import workload as wl

pytestmark = pytest.mark.gpu


def _gate(out, ref, what=""):
    rep = compare(out, ref)
    print(f"[{what}] {rep}", flush=True)
    assert rep.ok, f"{what}: {rep}"
    return rep


def _case(ctx, heads=16, page_size=64, seed=0, **kw):
    return wl.make_mla_case(context_lens=ctx, num_heads=heads, page_size=page_size, seed=seed,
                            **kw)


def test_small_mixed_lengths(oracle):
    case = _case((1, 63, 64, 65, 300), heads=16, page_size=64, seed=4242)
    ref, _, _ = oracle.mla(case)
    _gate(run_mla(case.to("cuda")), ref, "mla small")


@pytest.mark.parametrize("heads", [1, 3, 16, 17, 32, 33, 48, 80, 100, 128])
def test_head_counts(oracle, heads):
    """Head counts that fill part of a 32-head wave-pair tile, one or both pairs
    of a 64-head block, and spill into a second block (1, 3 and 17 as in the
    test discipline of the kernel matrix's sparse-MLA row)."""
    case = _case((5, 129, 700), heads=heads, page_size=32, seed=9100 + heads)
    ref, _, _ = oracle.mla(case)
    _gate(run_mla(case.to("cuda")), ref, f"mla heads={heads}")


@pytest.mark.parametrize("page_size", [16, 32, 64])
def test_page_sizes(oracle, page_size):
    case = _case((1, 17, 33, 250, 1030), heads=32, page_size=page_size, seed=9200 + page_size)
    ref, _, _ = oracle.mla(case)
    _gate(run_mla(case.to("cuda")), ref, f"mla page={page_size}")


@pytest.mark.parametrize("partition_size", [64, 128, 256, 1024, 4096])
def test_partition_sizes(oracle, partition_size):
    """Explicit partition sizes, from one 64-key granule per block to one block
    per sequence; every live partition count from 1 to 40 occurs."""
    case = _case((1, 64, 65, 1000, 2500), heads=32, page_size=64, seed=9300)
    ref, _, _ = oracle.mla(case)
    _gate(run_mla(case.to("cuda"), partition_size=partition_size), ref,
          f"mla P={partition_size}")


@pytest.mark.parametrize("partition_size", [0, 128])
def test_batch_past_64(oracle, partition_size):
    """100 sequences of seeded lengths 0 .. 400: the split's plan, row search
    and row-slot list go past the first 64 sequences (whose lengths a wave
    holds in registers) into the ones read from memory."""
    rng = np.random.default_rng(9800)
    ctx = tuple(int(x) for x in rng.integers(0, 401, size=100))
    case = _case(ctx, heads=16, page_size=16, seed=9801)
    ref, _, _ = oracle.mla(case)
    _gate(run_mla(case.to("cuda"), partition_size=partition_size), ref,
          f"mla batch=100 P={partition_size}")


def test_empty_context_gives_zero(oracle):
    case = _case((0, 10, 0, 70), heads=16, page_size=16, seed=9400)
    ref, _, _ = oracle.mla(case)
    out = run_mla(case.to("cuda"))
    assert torch.count_nonzero(out[0].float()) == 0 and torch.count_nonzero(out[2].float()) == 0
    _gate(out, ref, "mla empty rows")


def test_single_key_is_projected_latent(oracle):
    """One key: softmax weight 1, so out = W_UV[h] . c_0[0:512] exactly up to rounding."""
    case = _case((1, 1), heads=16, page_size=16, seed=9401)
    lat = case.cache[int(case.block_table[0, 0]), 0, :512].double()
    direct = torch.einsum("hvj,j->hv", case.w_uv.double(), lat).numpy()
    ref, _, _ = oracle.mla(case)
    np.testing.assert_allclose(ref[0], direct, rtol=1e-12, atol=1e-12)
    _gate(run_mla(case.to("cuda")), ref, "mla single key")


@pytest.mark.parametrize("scale", [2.0, 1e-4])
def test_peaky_and_flat_softmax(oracle, scale):
    """scale 2.0 makes score spreads of hundreds (the running-max rescale path
    runs often); scale 1e-4 makes the softmax nearly uniform."""
    case = _case((37, 600, 2049), heads=32, page_size=32, seed=9500, scale=scale)
    ref, _, _ = oracle.mla(case)
    _gate(run_mla(case.to("cuda"), partition_size=256), ref, f"mla scale={scale}")


def test_padded_token_stride(oracle):
    """Cache rows padded to 640 elements: only the first 576 are read."""
    case = _case((3, 90, 513), heads=16, page_size=32, seed=9600)
    ref, _, _ = oracle.mla(case)
    dc = case.to("cuda")
    P, S, R = case.cache.shape
    big = torch.full((P, S, 640), float("nan"), dtype=torch.bfloat16, device="cuda")
    big[:, :, :R] = dc.cache
    dc.cache = big[:, :, :R]
    assert dc.cache.stride() == (S * 640, 640, 1)
    _gate(run_mla(dc), ref, "mla token_stride 640")


def test_run_to_run_bit_identical():
    case = _case((1, 700, 3000, 64), heads=64, page_size=64, seed=9700)
    dc = case.to("cuda")
    first = run_mla(dc)
    for _ in range(3):
        assert torch.equal(run_mla(dc).view(torch.int16), first.view(torch.int16))


def test_page_permutation_bit_identical():
    case = _case((1, 31, 100, 685, 1000), heads=16, page_size=16, seed=9701, pool_pages=160)
    perm = torch.randperm(case.num_pages, generator=torch.Generator().manual_seed(11))
    moved = case.to("cpu")
    moved.cache = torch.empty_like(case.cache)
    moved.cache[perm] = case.cache
    bt = case.block_table.clone()
    live = bt >= 0
    bt[live] = perm.to(torch.int32)[bt[live].long()]
    moved.block_table = bt
    a = run_mla(case.to("cuda"))
    b = run_mla(moved.to("cuda"))
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_mla_full(oracle):
    """The 128-head, batch-16 latent workload (ctx U[1024, 8192], page 64) at full size."""
    case = wl.mla()
    oracle.set_threads(max(1, min(16, oracle.max_threads())))
    ref, _, _ = oracle.mla(case)
    _gate(run_mla(case.to("cuda")), ref, "mla bs16 h128 full")
