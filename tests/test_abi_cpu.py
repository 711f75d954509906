"""The C-ABI library without a GPU: it loads, exports every entry point the
header declares, and rejects bad arguments on the host before any launch.

No call here is valid enough to reach a kernel launch: every one fails a
host-side check (the fake device addresses are never dereferenced).  A call
that is valid up to its workspace passes a 1-byte one (a NULL workspace is
a valid mode of the decode entry points, so it would launch).
"""
from __future__ import annotations

import ctypes as C
import os
import re

import pytest

from paged_attention_decode_05_amd import binding as pb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pa_decode.h")

FAKE = 0x10000          # 16-byte aligned address, never dereferenced
PA = {"OK": 0, "NULL": -1, "SHAPE": -2, "UNSUPPORTED": -3, "ALIGN": -4, "WORKSPACE": -5}


def declared_functions():
    text = open(HEADER).read()
    return set(re.findall(r"PA_API\s+[\w\s\*]+?\b(\w+)\s*\(", text))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("pa_decode", "pa_decode_splitkv", "pa_merge_lse", "mla_absorbed_decode"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = C.CDLL(pb.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(pb.EXPORTS) == declared_functions()


def _kv(**kw):
    d = dict(num_pages=128, page_size=32, num_kv_heads=2, head_dim=128,
             page_stride=2 * 32 * 128, head_stride=32 * 128, token_stride=128)
    d.update(kw)
    return pb.KvLayout(**d)


def _decode(kv=None, q=FAKE, k=FAKE, v=FAKE, bt=FAKE, bt_stride=32, ctx=FAKE, batch=8, hq=8,
            maxp=32, scale=0.088, window=0, out=FAKE, lse=None, ws=FAKE, ws_bytes=1):
    kv = kv or _kv()
    return pb.LIB.pa_decode(q, k, v, C.byref(kv), bt, bt_stride, ctx, batch, hq, maxp, scale,
                            window, out, lse, ws, ws_bytes, None)


@pytest.mark.parametrize("field,status", [
    ("q", "NULL"), ("k", "NULL"), ("v", "NULL"), ("bt", "NULL"), ("ctx", "NULL"), ("out", "NULL")])
def test_null_pointers(field, status):
    assert _decode(**{field: None}) == PA[status]
    assert pb.pa_last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), "SHAPE"), (dict(hq=7), "SHAPE"), (dict(maxp=0), "SHAPE"),
    (dict(scale=0.0), "SHAPE"), (dict(scale=float("nan")), "SHAPE"),
    (dict(scale=float("inf")), "SHAPE"), (dict(bt_stride=16), "SHAPE"),
    (dict(batch=70000), "SHAPE"),
    (dict(kv=_kv(head_dim=96, token_stride=96, head_stride=32 * 96, page_stride=2 * 32 * 96)),
     "UNSUPPORTED"),
    (dict(hq=64), "UNSUPPORTED"),                                  # 32 q heads per KV head
    (dict(hq=34), "UNSUPPORTED"),                                  # 17 q heads per KV head
    (dict(kv=_kv(page_size=8)), "UNSUPPORTED"),
    (dict(kv=_kv(token_stride=132)), "ALIGN"),
    (dict(kv=_kv(page_stride=4100)), "ALIGN"),
    (dict(q=FAKE + 8), "ALIGN"), (dict(k=FAKE + 2), "ALIGN"),
    (dict(out=FAKE + 4), "ALIGN"),
    (dict(), "WORKSPACE"),
    (dict(ws=FAKE, ws_bytes=100), "WORKSPACE"),
    (dict(ws=FAKE + 16, ws_bytes=1 << 30), "ALIGN"),
])
def test_decode_rejections(kw, status):
    assert _decode(**kw) == PA[status], pb.pa_last_error()
    assert pb.pa_last_error()


def test_head_dim_512_accepted():
    """head_dim 512 takes groups 1-16; every such call is valid up to the
    too-small workspace, for bf16 and f32 pools."""
    kv = _kv(head_dim=512, num_kv_heads=1, token_stride=512, head_stride=32 * 512,
             page_stride=32 * 512)
    for hq in (1, 2, 4, 8, 16):
        assert _decode(kv=kv, hq=hq) == PA["WORKSPACE"], pb.pa_last_error()
    assert _decode(kv=kv, hq=32) == PA["UNSUPPORTED"]
    f = pb.LIB.pa_decode_f32
    assert f(FAKE, FAKE, FAKE, C.byref(kv), FAKE, 32, FAKE, 8, 16, 32, 0.044, 0, FAKE, None,
             FAKE, 1, None) == PA["WORKSPACE"], pb.pa_last_error()


@pytest.mark.parametrize("head_dim", [64, 128, 256, 512])
def test_every_group_1_to_16_accepted(head_dim):
    """Any 1..16 q heads per KV head runs on the kernel built for the next
    power of two; the workspace is sized for that padded group."""
    kv = _kv(head_dim=head_dim, num_kv_heads=1, token_stride=head_dim,
             head_stride=32 * head_dim, page_stride=32 * head_dim)
    for g in range(1, 17):
        assert _decode(kv=kv, hq=g) == PA["WORKSPACE"], (g, pb.pa_last_error())
        padded = 1 << (g - 1).bit_length()
        assert pb.pa_decode_workspace_size(8, g, 1, head_dim, 32, 32, 0) == \
            pb.pa_decode_workspace_size(8, padded, 1, head_dim, 32, 32, 0)
    assert _decode(kv=kv, hq=17) == PA["UNSUPPORTED"]
    assert pb.pa_decode_workspace_size(8, 17, 1, head_dim, 32, 32, 0) == 0
    need = pb.pa_decode_workspace_size(8, 16, 1, 512, 32, 32, 0)
    slots = 8 + 2048
    base = slots * 16 * 514 * 4 + 8 * 4
    assert base <= need < base + 1024


def test_workspace_alignment_checked_last():
    need = pb.pa_decode_workspace_size(8, 8, 2, 128, 32, 32, 0)
    assert need > 0
    assert _decode(ws=FAKE + 16, ws_bytes=need) == PA["ALIGN"]


def test_workspace_and_partition_plan():
    # suggested two-stage partition: bs64 32q/8kv d128, 256 pages of 32 -> 512 keys
    assert pb.pa_decode_partition_size(64, 32, 8, 128, 256, 32, 0) == 512
    # pa_decode's balanced split: one fp32 partial slot per (row, block) segment,
    # rows + 2048 slots of G*(D+2) floats, and a 4-byte record per row
    need = pb.pa_decode_workspace_size(64, 32, 8, 128, 256, 32, 0)
    rows = 64 * 8
    slots = rows + 2048
    base = slots * 4 * 130 * 4 + rows * 4
    assert base <= need < base + 1024
    # a window bounds the keys, hence the partitions
    p = pb.pa_decode_partition_size(32, 16, 2, 256, 512, 32, 4096)
    assert p >= 128 and 4096 % p == 0
    assert pb.pa_decode_workspace_size(0, 8, 2, 128, 32, 32, 0) == 0
    assert pb.pa_decode_workspace_size(8, 8, 2, 96, 32, 32, 0) == 0


def _split(P=512, maxparts=2, window=0, po=FAKE, pm=FAKE, ps=FAKE, maxp=32):
    kv = _kv()
    return pb.LIB.pa_decode_splitkv(FAKE, FAKE, FAKE, C.byref(kv), FAKE, 32, FAKE, 8, 8, maxp,
                                    0.088, window, P, maxparts, po, pm, ps, None)


def test_splitkv_rejections():
    assert _split(po=None) == PA["NULL"]
    assert _split(P=0) == PA["SHAPE"]
    assert _split(P=512, maxparts=1) == PA["SHAPE"]            # 1024 keys need 2
    assert _split(P=100, maxparts=9, window=1000) == PA["SHAPE"]      # 1000 keys need 10
    assert _split(po=FAKE + 4) == PA["ALIGN"]


def test_merge_rejections():
    f = pb.LIB.pa_merge_lse
    assert f(None, FAKE, FAKE, FAKE, 8, 8, 128, 512, 2, 0, FAKE, None, None) == PA["NULL"]
    assert f(FAKE, FAKE, FAKE, FAKE, 8, 8, 96, 512, 2, 0, FAKE, None, None) == PA["UNSUPPORTED"]
    assert f(FAKE, FAKE, FAKE, FAKE, 8, 8, 128, 0, 2, 0, FAKE, None, None) == PA["SHAPE"]
    assert f(FAKE, FAKE, FAKE, FAKE, 8, 8, 128, 512, 2, 0, FAKE + 2, None, None) == PA["ALIGN"]


def _mla(cache=None, heads=128, P=0, ws=None, ws_bytes=0, **kw):
    cache = cache or pb.KvLayout(1300, 64, 1, 576, 64 * 576, 0, 576)
    args = dict(qn=FAKE, qr=FAKE, c=FAKE, wuk=FAKE, wuv=FAKE, bt=FAKE, ctx=FAKE, out=FAKE)
    args.update(kw)
    return pb.LIB.mla_absorbed_decode(args["qn"], args["qr"], args["c"], C.byref(cache),
                                      args["wuk"], args["wuv"], args["bt"], 128, args["ctx"], 16,
                                      heads, 128, 0.072, P, args["out"], ws, ws_bytes, None)


def test_mla_rejections():
    assert _mla(qn=None) == PA["NULL"]
    assert _mla(heads=100) == PA["WORKSPACE"]             # any head count: padded tiles
    assert _mla(cache=pb.KvLayout(1300, 64, 1, 512, 64 * 512, 0, 512)) == PA["UNSUPPORTED"]
    assert _mla(P=100) == PA["SHAPE"]
    assert _mla(cache=pb.KvLayout(1300, 64, 1, 576, 64 * 580, 0, 580)) == PA["ALIGN"]
    assert _mla(wuv=FAKE + 8) == PA["ALIGN"]
    assert _mla() == PA["WORKSPACE"]
    assert pb.mla_absorbed_decode_workspace_size(16, 128, 128, 64, 0) > 0
    assert pb.mla_absorbed_decode_workspace_size(16, 100, 128, 64, 0) > 0
    assert pb.mla_absorbed_decode_workspace_size(16, 0, 128, 64, 0) == 0


def test_mla_fp8_rejections():
    """FP8 latent rows are 656 bytes with byte strides in multiples of 16;
    the bf16 row size is refused and vice versa."""
    f8 = pb.KvLayout(1300, 64, 1, 656, 64 * 656, 0, 656)

    def dec(cache, **kw):
        a = dict(qn=FAKE, out=FAKE)
        a.update(kw)
        return pb.LIB.mla_absorbed_decode_fp8(a["qn"], FAKE, FAKE, C.byref(cache), FAKE, FAKE,
                                              FAKE, 128, FAKE, 16, 128, 128, 0.072, 0, a["out"],
                                              None, 0, None)
    assert dec(f8) == PA["WORKSPACE"], pb.pa_last_error()
    assert dec(f8, qn=None) == PA["NULL"]
    assert dec(pb.KvLayout(1300, 64, 1, 576, 64 * 576, 0, 576)) == PA["UNSUPPORTED"]
    assert dec(pb.KvLayout(1300, 64, 1, 656, 64 * 664, 0, 664)) == PA["ALIGN"]   # 664 % 16
    assert dec(pb.KvLayout(1300, 64, 1, 656, 64 * 672, 0, 672)) == PA["WORKSPACE"]
    assert _mla(cache=f8) == PA["UNSUPPORTED"]            # the bf16 entry point
    ins = pb.LIB.mla_cache_insert_fp8
    assert ins(None, 512, FAKE, 64, FAKE, C.byref(f8), FAKE, 4, None) == PA["NULL"]
    assert ins(FAKE, 512, FAKE, 64, FAKE, C.byref(f8), FAKE, 0, None) == PA["OK"]
    assert ins(FAKE, 500, FAKE, 64, FAKE, C.byref(f8), FAKE, 0, None) == PA["ALIGN"]
    assert ins(FAKE, 512, FAKE, 64, FAKE, C.byref(pb.KvLayout(100, 64, 1, 576, 64 * 576, 0, 576)),
               FAKE, 0, None) == PA["UNSUPPORTED"]
    assert ins(FAKE, 512, FAKE, 64, FAKE, C.byref(pb.KvLayout(100, 64, 1, 656, 64 * 640, 0, 640)),
               FAKE, 0, None) == PA["SHAPE"]             # token_stride < 656


def test_mla_multiquery_rejections():
    """num_queries outside 1..16, or a workspace sized for fewer query heads,
    is refused before any launch; FP8 and bf16 rows go to their own entry."""
    bf = pb.KvLayout(1300, 64, 1, 576, 64 * 576, 0, 576)
    f8 = pb.KvLayout(1300, 64, 1, 656, 64 * 656, 0, 656)

    def dec(cache=bf, S=4, causal=1, H=128, ws=0, fn=pb.LIB.mla_absorbed_decode_multiquery):
        return fn(FAKE, FAKE, FAKE, C.byref(cache), FAKE, FAKE, FAKE, 128, FAKE, 16, H, S, causal,
                  128, 0.072, 0, FAKE, FAKE if ws else None, ws, None)
    assert dec() == PA["WORKSPACE"], pb.pa_last_error()
    assert "512" in pb.pa_last_error()                    # the query heads the size is for
    assert dec(S=0) == PA["SHAPE"] and dec(S=17) == PA["SHAPE"]
    assert dec(S=16, H=4096) == PA["SHAPE"]               # 65536 query heads
    assert dec(H=24) == PA["WORKSPACE"]                   # any head count
    n1 = pb.mla_absorbed_decode_workspace_size(16, 128, 128, 64, 0)
    n4 = pb.mla_absorbed_decode_workspace_size(16, 512, 128, 64, 0)
    assert 0 < n1 < n4
    assert dec(ws=n1) == PA["WORKSPACE"]
    assert dec(cache=f8) == PA["UNSUPPORTED"]
    assert dec(cache=f8, fn=pb.LIB.mla_absorbed_decode_multiquery_fp8) == PA["WORKSPACE"]
    assert dec(cache=bf, fn=pb.LIB.mla_absorbed_decode_multiquery_fp8) == PA["UNSUPPORTED"]


def _ins(kv=None, n=4, ts=256, hs=128, **kw):
    kv = kv or _kv()
    a = dict(k=FAKE, v=FAKE, kp=FAKE, vp=FAKE, sl=FAKE)
    a.update(kw)
    return pb.LIB.pa_kv_insert(a["k"], a["v"], ts, hs, a["kp"], a["vp"], C.byref(kv), a["sl"], n,
                               None)


def test_kv_insert_rejections():
    assert _ins(k=None) == PA["NULL"]
    assert _ins(sl=None) == PA["NULL"]
    assert _ins(n=-1) == PA["SHAPE"]
    assert _ins(kv=_kv(head_dim=12, token_stride=16)) == PA["UNSUPPORTED"]
    assert _ins(ts=260) == PA["ALIGN"]
    assert _ins(kv=_kv(token_stride=132)) == PA["ALIGN"]           # not a multiple of 8
    assert _ins(kv=_kv(token_stride=64)) == PA["SHAPE"]            # rows would overlap
    assert _ins(hs=64) == PA["SHAPE"]
    assert _ins(vp=FAKE + 8) == PA["ALIGN"]
    # zero tokens is a valid no-op: nothing is launched
    assert _ins(n=0) == PA["OK"]


def _mins(cache=None, n=4, cs=512, ps=64, **kw):
    cache = cache or pb.KvLayout(100, 64, 1, 576, 64 * 576, 0, 576)
    a = dict(c=FAKE, pe=FAKE, kc=FAKE, sl=FAKE)
    a.update(kw)
    return pb.LIB.mla_cache_insert(a["c"], cs, a["pe"], ps, a["kc"], C.byref(cache), a["sl"], n,
                                   None)


def test_mla_cache_insert_rejections():
    assert _mins(c=None) == PA["NULL"]
    assert _mins(n=-2) == PA["SHAPE"]
    assert _mins(cache=pb.KvLayout(100, 64, 1, 512, 64 * 512, 0, 512)) == PA["UNSUPPORTED"]
    assert _mins(cache=pb.KvLayout(100, 64, 2, 576, 64 * 576, 0, 576)) == PA["UNSUPPORTED"]
    assert _mins(cs=500) == PA["ALIGN"]
    assert _mins(cs=504) == PA["SHAPE"]
    assert _mins(ps=56) == PA["SHAPE"]
    assert _mins(pe=FAKE + 4) == PA["ALIGN"]
    assert _mins(n=0) == PA["OK"]


def test_multiquery_rejections_and_sizes():
    kv = _kv()
    f = pb.LIB.pa_decode_multiquery
    args = lambda S, heads=8: (FAKE, FAKE, FAKE, C.byref(kv), FAKE, 32, FAKE, 8, heads, S, 1, 32,
                               0.088, 0, FAKE, None, FAKE, 1, None)
    assert f(*args(0)) == PA["SHAPE"]
    assert f(*args(17)) == PA["SHAPE"]
    assert f(*args(5)) == PA["UNSUPPORTED"]      # 5 queries x 4 heads per KV head = 20
    assert f(*args(4)) == PA["WORKSPACE"]        # 4 x 4 = 16: supported, workspace too small
    assert f(*args(5, heads=6)) == PA["WORKSPACE"]   # 5 x 3 = 15
    ws = pb.pa_decode_multiquery_workspace_size
    assert ws(8, 8, 2, 128, 32, 32, 0, 3) == ws(8, 8, 2, 128, 32, 32, 0, 4) > 0
    assert ws(8, 6, 2, 128, 32, 32, 0, 5) == ws(8, 8, 2, 128, 32, 32, 0, 4)
    assert ws(8, 8, 2, 128, 32, 32, 0, 1) == pb.pa_decode_workspace_size(8, 8, 2, 128, 32, 32, 0)
    assert ws(8, 8, 2, 128, 32, 32, 0, 0) == 0


def test_fp8_rejections():
    f = pb.LIB.pa_decode_fp8
    kv8 = _kv(page_stride=2 * 32 * 128, head_stride=32 * 128, token_stride=128)
    def call(kv=kv8, ks=0.02, vs=0.03, scale=0.088):
        return f(FAKE, FAKE, FAKE, C.byref(kv), FAKE, 32, FAKE, 8, 8, 32, scale, ks, vs, 0, FAKE,
                 None, FAKE, 1, None)
    assert call(kv=_kv(token_stride=136, head_stride=32 * 136, page_stride=2 * 32 * 136)) == PA["ALIGN"]
    assert call(ks=0.0) == PA["SHAPE"]
    assert call(vs=float("nan")) == PA["SHAPE"]
    assert call(ks=1e38, scale=1e3) == PA["SHAPE"]            # scale * k_scale overflows
    assert call() == PA["WORKSPACE"]                          # valid up to the workspace
    # bf16 pools need 8-element strides, FP8 pools 16-element ones
    kv_b = _kv(token_stride=136, head_stride=32 * 136, page_stride=2 * 32 * 136)
    assert _decode(kv=kv_b) == PA["WORKSPACE"]


def test_f32_pool_rejections():
    f = pb.LIB.pa_decode_f32
    def call(kv):
        return f(FAKE, FAKE, FAKE, C.byref(kv), FAKE, 32, FAKE, 8, 8, 32, 0.088, 0, FAKE, None,
                 FAKE, 1, None)
    assert call(_kv(head_dim=256, token_stride=256, head_stride=32 * 256,
                    page_stride=2 * 32 * 256)) == PA["WORKSPACE"]
    assert call(_kv(head_dim=96, token_stride=96, head_stride=32 * 96,
                    page_stride=2 * 32 * 96)) == PA["UNSUPPORTED"]
    assert call(_kv(token_stride=130, head_stride=32 * 130, page_stride=2 * 32 * 130)) == PA["ALIGN"]
    # 4-element strides are 16-byte rows for f32: valid up to the workspace
    assert call(_kv(token_stride=132, head_stride=32 * 132, page_stride=2 * 32 * 132)) == PA["WORKSPACE"]
    # one page must stay below 2^32 bytes: 2^30 f32 elements is 2^32 bytes
    assert call(_kv(page_stride=2**30)) == PA["SHAPE"]
    assert call(_kv(page_stride=2**30 - 4)) == PA["WORKSPACE"]


def test_noalloc_host_checks():
    """pa_decode_noalloc validates like pa_decode, and refuses shapes whose
    plan exceeds its 32 MiB scratch before touching the device."""
    f = pb.LIB.pa_decode_noalloc
    kv = _kv()
    assert f(None, FAKE, FAKE, C.byref(kv), FAKE, 32, FAKE, 8, 8, 32, 0.088, 0, FAKE, None,
             None) == PA["NULL"]
    assert f(FAKE, FAKE, FAKE, C.byref(kv), FAKE, 32, FAKE, 8, 7, 32, 0.088, 0, FAKE, None,
             None) == PA["SHAPE"]
    big = pb.KvLayout(64, 32, 8, 512, 8 * 32 * 512, 32 * 512, 512)
    assert pb.pa_decode_workspace_size(4096, 128, 8, 512, 64, 32, 0) > 32 << 20
    assert f(FAKE, FAKE, FAKE, C.byref(big), FAKE, 64, FAKE, 4096, 128, 64, 0.05, 0, FAKE, None,
             None) == PA["WORKSPACE"]
    assert "scratch" in pb.pa_last_error()
