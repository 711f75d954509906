"""pa_decode_noalloc through the C ABI: the library's own device scratch in
place of a caller workspace must give pa_decode's results bit for bit, and
pass the oracle gate, on two calls in a row (the second with a smaller
batch, so the scratch holds the first call's larger contents)."""
from __future__ import annotations

import pytest
import torch

from gpu_util import run_decode
from oracle.compare import compare
from paged_attention_decode_05_amd import binding as pb
from paged_attention_decode_05_amd import workload as wl

pytestmark = pytest.mark.gpu


def _noalloc(dc):
    B, H, D = dc.q.shape
    out = torch.full((B, H, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    pb.pa_decode_noalloc(dc.q, dc.k_pool, dc.v_pool, pb.kv_layout(dc.k_pool, dc.layout),
                         dc.block_table, dc.context_lens, dc.scale, dc.window, out, lse)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def test_noalloc_matches_pa_decode_two_calls(oracle):
    big = wl.make_gqa_case(context_lens=(), ctx_draw=(512, 8192), batch=24, num_q_heads=32,
                           num_kv_heads=8, head_dim=128, page_size=32, seed=8800)
    small = wl.make_gqa_case(context_lens=(0, 1, 31, 33, 700, 5000), num_q_heads=32,
                             num_kv_heads=8, head_dim=128, page_size=32, seed=8801, window=600)
    for case in (big, small):
        print(f"case batch={case.batch} window={case.window}", flush=True)
        dc = case.to("cuda")
        out, lse = _noalloc(dc)
        ref_out, ref_lse = run_decode(dc)
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
        assert torch.equal(lse, ref_lse)
        oracle.set_threads(max(1, min(16, oracle.max_threads())))
        want, _ = oracle.decode(case)
        rep = compare(out, want)
        print(f"[noalloc batch={case.batch}] {rep}", flush=True)
        assert rep.ok, rep


def test_noalloc_full_cu_blocks_two_calls(oracle):
    """head_dim 256, groups of 8: the balanced split's blocks hold all the
    waves of a CU; two calls in a row, the second smaller."""
    big = wl.make_gqa_case(context_lens=(), ctx_draw=(1024, 6000), batch=12, num_q_heads=16,
                           num_kv_heads=2, head_dim=256, page_size=32, seed=8810, window=4096,
                           q_std=0.5)
    small = wl.make_gqa_case(context_lens=(0, 1, 257, 3000, 90), num_q_heads=16, num_kv_heads=2,
                             head_dim=256, page_size=32, seed=8811, window=4096, q_std=0.5)
    for case in (big, small):
        print(f"case D=256 batch={case.batch}", flush=True)
        dc = case.to("cuda")
        out, lse = _noalloc(dc)
        ref_out, ref_lse = run_decode(dc)
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
        assert torch.equal(lse, ref_lse)
        want, _ = oracle.decode(case)
        rep = compare(out, want)
        print(f"[noalloc D=256 batch={case.batch}] {rep}", flush=True)
        assert rep.ok, rep


def test_noalloc_rejects_shapes_past_its_scratch():
    """A plan larger than the 32 MiB array is refused on the host."""
    kv = pb.KvLayout(64, 32, 8, 512, 8 * 32 * 512, 32 * 512, 512)
    need = pb.pa_decode_workspace_size(4096, 128, 8, 512, 64, 32, 0)
    assert need > 32 << 20
    q = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    i = torch.zeros(16, dtype=torch.int32, device="cuda")
    import ctypes as C
    rc = pb.LIB.pa_decode_noalloc(q.data_ptr(), q.data_ptr(), q.data_ptr(), C.byref(kv),
                                  i.data_ptr(), 64, i.data_ptr(), 4096, 128, 64, 0.05, 0,
                                  q.data_ptr(), None, None)
    assert rc == -5 and "scratch" in pb.pa_last_error()
