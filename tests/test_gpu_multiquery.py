"""GPU parity of multi-query decode (pa_decode_multiquery) against the CPU
oracle, through the C ABI.

Same gate as single-query decode (|g - r| <= 2e-2 and <= 2 bf16 ulps,
floor 2^-22); lse within 2e-6 relative; queries that see no key give 0 and
-inf.  Pools carry NaN canaries outside the union of the queries' key ranges.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle.compare import compare
from paged_attention_decode_05_amd import binding as pb
from paged_attention_decode_05_amd import workload as wl

pytestmark = pytest.mark.gpu


def _run(case, causal, workspace=None):
    if case.q.dim() == 3:                 # one query per sequence: add the query axis
        case = case.to("cpu")
        case.q = case.q[:, None].contiguous()
    dc = case.to("cuda")
    B, S, H, D = dc.q.shape
    out = torch.full((B, S, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, S, H), float("nan"), dtype=torch.float32, device="cuda")
    if workspace is None:
        n = pb.pa_decode_multiquery_workspace_size(B, H, dc.num_kv_heads, D, dc.max_pages,
                                                   dc.page_size, dc.window, S)
        assert n > 0
        workspace = torch.zeros(n, dtype=torch.uint8, device="cuda")
    pb.pa_decode_multiquery(dc.q, dc.k_pool, dc.v_pool, pb.kv_layout(dc.k_pool, dc.layout),
                            dc.block_table, dc.context_lens, dc.scale, dc.window, causal, out,
                            lse, workspace)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _check(oracle, case, causal, what):
    ref, ref_lse = oracle.decode_multi(case, causal)
    out, lse = _run(case, causal)
    rep = compare(out, ref)
    print(f"[{what}] {rep}", flush=True)
    assert rep.ok, f"{what}: {rep}"
    g = lse.numpy().astype(np.float64)
    fin = np.isfinite(ref_lse)
    assert (np.isfinite(g) == fin).all(), what
    if fin.any():
        err = np.abs(g[fin] - ref_lse[fin]) / np.maximum(1.0, np.abs(ref_lse[fin]))
        assert err.max() <= 2e-6, (what, err.max())
    return out, lse


@pytest.mark.parametrize("S", [1, 2, 3, 4])
@pytest.mark.parametrize("causal", [True, False])
def test_queries_and_masks(oracle, S, causal):
    case = wl.make_gqa_case(context_lens=(5, 31, 32, 33, 700, 1500), num_q_heads=16,
                            num_kv_heads=4, head_dim=128, page_size=32, seed=9900 + S,
                            num_queries=S)
    _check(oracle, case, causal, f"S={S} causal={causal}")


@pytest.mark.parametrize("window", [50, 600])
def test_causal_window(oracle, window):
    case = wl.make_gqa_case(context_lens=(3, 64, 65, 1000, 2200), num_q_heads=8, num_kv_heads=2,
                            head_dim=128, page_size=16, seed=9910 + window, window=window,
                            num_queries=3)
    _check(oracle, case, True, f"window={window}")


@pytest.mark.parametrize("S,gq", [(3, 3), (5, 3), (2, 5), (3, 1)])
@pytest.mark.parametrize("causal", [True, False])
def test_padded_virtual_heads(oracle, S, gq, causal):
    """S * Gq virtual heads that are not a power of two (9, 15, 10, 3): the
    tile is padded and the padding heads write nothing (out is NaN-filled
    beforehand, so a stray write would show)."""
    case = wl.make_gqa_case(context_lens=(2, 40, 33, 900, 1700), num_q_heads=2 * gq,
                            num_kv_heads=2, head_dim=128, page_size=32,
                            seed=9960 + 10 * S + gq, num_queries=S)
    _check(oracle, case, causal, f"S={S} Gq={gq} causal={causal}")


def test_null_workspace_multiquery(oracle):
    case = wl.make_gqa_case(context_lens=(1, 2, 64, 1000), num_q_heads=8, num_kv_heads=2,
                            head_dim=128, page_size=16, seed=9970, num_queries=3)
    ref, ref_lse = oracle.decode_multi(case, True)
    dc = case.to("cuda")
    B, S, H, D = dc.q.shape
    out = torch.full((B, S, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, S, H), float("nan"), dtype=torch.float32, device="cuda")
    pb.pa_decode_multiquery(dc.q, dc.k_pool, dc.v_pool, pb.kv_layout(dc.k_pool, dc.layout),
                            dc.block_table, dc.context_lens, dc.scale, dc.window, True, out,
                            lse, None)
    torch.cuda.synchronize()
    rep = compare(out.cpu(), ref)
    assert rep.ok, rep
    g = lse.cpu().numpy().astype(np.float64)
    assert (np.isfinite(g) == np.isfinite(ref_lse)).all()


def test_head_dim_256(oracle):
    case = wl.make_gqa_case(context_lens=(17, 300, 1100), num_q_heads=4, num_kv_heads=2,
                            head_dim=256, page_size=32, seed=9920, num_queries=4)
    _check(oracle, case, True, "d256 S=4")


@pytest.mark.parametrize("causal", [True, False])
def test_head_dim_64(oracle, causal):
    """head_dim 64 (matrix-core routine at every group size): 4 queries of
    GQA-4 fill the 16-column tile; 16-key pages."""
    case = wl.make_gqa_case(context_lens=(1, 17, 300, 2049), num_q_heads=8, num_kv_heads=2,
                            head_dim=64, page_size=16, seed=9925, num_queries=4)
    _check(oracle, case, causal, f"d64 S=4 causal={causal}")


def test_context_shorter_than_queries(oracle):
    """ctx 1 and 2 with S = 4: the early causal queries see no key."""
    case = wl.make_gqa_case(context_lens=(1, 2, 4, 9), num_q_heads=8, num_kv_heads=2,
                            head_dim=128, page_size=16, seed=9930, num_queries=4)
    out, lse = _check(oracle, case, True, "short contexts")
    assert torch.count_nonzero(out[0, :3].float()) == 0 and torch.isinf(lse[0, :3]).all()


def test_one_query_equals_decode():
    case = wl.make_gqa_case(context_lens=(1, 100, 2049), num_q_heads=32, num_kv_heads=8,
                            head_dim=128, page_size=32, seed=9940, num_queries=1)
    multi = case.to("cpu")
    multi.q = case.q[:, None].contiguous()
    out_m, lse_m = _run(multi, True)
    from gpu_util import run_decode
    out, lse = run_decode(case.to("cuda"))
    assert torch.equal(out_m[:, 0].view(torch.int16), out.view(torch.int16))
    assert torch.equal(lse_m[:, 0], lse)


def test_run_to_run_bit_identical():
    case = wl.make_gqa_case(context_lens=(7, 900, 3000), num_q_heads=8, num_kv_heads=2,
                            head_dim=128, page_size=32, seed=9950, num_queries=4)
    a, la = _run(case, True)
    for _ in range(3):
        b, lb = _run(case, True)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)) and torch.equal(la, lb)


def test_verify_bs64(oracle):
    """bs64 llama-shaped verify step: 4 queries per sequence, 32 q / 8 KV heads."""
    case = wl.make_gqa_case(context_lens=(), ctx_draw=(512, 4096), batch=64, num_q_heads=32,
                            num_kv_heads=8, head_dim=128, page_size=32, seed=9960, num_queries=4)
    oracle.set_threads(max(1, min(16, oracle.max_threads())))
    _check(oracle, case, True, "verify bs64 S=4")
