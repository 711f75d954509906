"""Independent float64 brute force used to pin the oracle.

Written separately from the oracle (numpy fancy indexing instead of pointer
and stride arithmetic, BLAS products instead of ascending loops), so a
mistake in the oracle's gather, head map, window or softmax shows up as a
disagreement here.
"""
from __future__ import annotations

import numpy as np
import torch


def pool_f64(pool: torch.Tensor) -> np.ndarray:
    return pool.detach().cpu().to(torch.float64).numpy()


def gather_rows(pool: np.ndarray, layout: str, bt_row: np.ndarray, t: np.ndarray,
                page_size: int, g: int) -> np.ndarray:
    """Rows of KV head g for logical tokens t: [len(t), D]."""
    pages = bt_row[t // page_size]
    slots = t % page_size
    if layout == "PHSD":
        return pool[pages, g, slots, :]
    return pool[pages, slots, g, :]


def key_range(n: int, window: int) -> tuple[int, int]:
    return (max(0, n - window) if window > 0 else 0), n


def fp8_pool_f64(pool: torch.Tensor, scale: float) -> np.ndarray:
    """Values of an E4M3 byte pool times its scale, decoded by torch."""
    return pool.detach().cpu().contiguous().view(torch.float8_e4m3fn).to(torch.float64).numpy() * scale


def mla_fp8_rows_f64(rows: torch.Tensor, d_lat: int = 512, d_rope: int = 64) -> np.ndarray:
    """Values [P, S, d_lat + d_rope] of FP8 latent-cache rows (uint8): the
    E4M3 latent decoded by torch times 2^(scale byte - 127) of its 64-block,
    then the bf16 rope part."""
    r = rows.detach().cpu().contiguous()
    lat = r[..., :d_lat].contiguous().view(torch.float8_e4m3fn).to(torch.float64)
    sb = r[..., d_lat + 2 * d_rope:d_lat + 2 * d_rope + d_lat // 64].to(torch.float64)
    lat = lat * torch.exp2(sb - 127.0).repeat_interleave(64, dim=-1)
    rope = r[..., d_lat:d_lat + 2 * d_rope].contiguous().view(torch.bfloat16).to(torch.float64)
    return torch.cat([lat, rope], dim=-1).numpy()


def dense_attention(case, window=None):
    """(out [B,Hq,D], lse [B,Hq]) in float64 over materialised K/V."""
    w = case.window if window is None else window
    if getattr(case, "kv_dtype", "bf16") == "fp8":
        K = fp8_pool_f64(case.k_pool, case.k_scale)
        V = fp8_pool_f64(case.v_pool, case.v_scale)
    elif getattr(case, "kv_dtype", "bf16") == "f32":
        K = case.k_pool.detach().cpu().to(torch.float64).numpy()
        V = case.v_pool.detach().cpu().to(torch.float64).numpy()
    else:
        K = pool_f64(case.k_pool)
        V = pool_f64(case.v_pool)
    q = case.q.to(torch.float64).numpy()
    bt = case.block_table.numpy()
    ctx = case.context_lens.numpy()
    B, H, D = q.shape
    G = H // case.num_kv_heads
    out = np.zeros((B, H, D))
    lse = np.full((B, H), -np.inf)
    for b in range(B):
        lo, n = key_range(int(ctx[b]), w)
        if n <= lo:
            continue
        t = np.arange(lo, n)
        for g in range(case.num_kv_heads):
            Kb = gather_rows(K, case.layout, bt[b], t, case.page_size, g)
            Vb = gather_rows(V, case.layout, bt[b], t, case.page_size, g)
            for h in range(g * G, (g + 1) * G):
                s = case.scale * (Kb @ q[b, h])
                mx = s.max()
                e = np.exp(s - mx)
                out[b, h] = (e @ Vb) / e.sum()
                lse[b, h] = mx + np.log(e.sum())
    return out, lse


def mla_unabsorbed(case):
    """MLA evaluated without absorption: per head, materialise
    k_t = [W_UK[h] c_t[:d_lat] ; c_t[d_lat:]] and v_t = W_UV[h] c_t[:d_lat],
    then plain softmax attention of q = [q_nope ; q_rope]."""
    C = case.cache.detach().cpu().to(torch.float64).numpy()
    qn = case.q_nope.to(torch.float64).numpy()
    qr = case.q_rope.to(torch.float64).numpy()
    Wuk = case.w_uk.to(torch.float64).numpy()   # [H, d_nope, d_lat]
    Wuv = case.w_uv.to(torch.float64).numpy()   # [H, d_v, d_lat]
    bt = case.block_table.numpy()
    ctx = case.context_lens.numpy()
    B, H = qn.shape[:2]
    out = np.zeros((B, H, case.d_v))
    for b in range(B):
        n = int(ctx[b])
        if n == 0:
            continue
        t = np.arange(n)
        rows = C[bt[b][t // case.page_size], t % case.page_size, :]    # [n, 576]
        lat, rope = rows[:, :case.d_lat], rows[:, case.d_lat:]
        for h in range(H):
            k_nope = lat @ Wuk[h].T          # [n, d_nope]
            v = lat @ Wuv[h].T               # [n, d_v]
            k = np.concatenate([k_nope, rope], axis=1)
            q = np.concatenate([qn[b, h], qr[b, h]])
            s = case.scale * (k @ q)
            e = np.exp(s - s.max())
            out[b, h] = (e @ v) / e.sum()
    return out


def mla_unabsorbed_multi(case, causal: bool):
    """(out [B,S,H,d_v], lse [B,S,H]) in float64 for an MLA case whose q is
    [B, S, H, *] (or [B, H, *], S = 1), over a bf16 or FP8 cache, without
    absorption: per head k_t = [W_UK[h] c_t[:d_lat] ; c_t[d_lat:]] and
    v_t = W_UV[h] c_t[:d_lat]; query s of sequence b sees keys
    t <= n - S + s (causal) or t < n."""
    if case.cache_dtype == "fp8":
        C = mla_fp8_rows_f64(case.cache, case.d_lat, case.d_rope)
    else:
        C = case.cache.detach().cpu().to(torch.float64).numpy()
    qn = case.q_nope.to(torch.float64).numpy()
    qr = case.q_rope.to(torch.float64).numpy()
    if qn.ndim == 3:
        qn, qr = qn[:, None], qr[:, None]
    Wuk = case.w_uk.to(torch.float64).numpy()
    Wuv = case.w_uv.to(torch.float64).numpy()
    bt = case.block_table.numpy()
    ctx = case.context_lens.numpy()
    B, S, H = qn.shape[:3]
    out = np.zeros((B, S, H, case.d_v))
    lse = np.full((B, S, H), -np.inf)
    for b in range(B):
        n = int(ctx[b])
        for s in range(S):
            hi = n - S + s + 1 if causal else n
            if hi <= 0:
                continue
            t = np.arange(hi)
            rows = C[bt[b][t // case.page_size], t % case.page_size, :]
            lat, rope = rows[:, :case.d_lat], rows[:, case.d_lat:]
            for h in range(H):
                k = np.concatenate([lat @ Wuk[h].T, rope], axis=1)
                v = lat @ Wuv[h].T
                sc = case.scale * (k @ np.concatenate([qn[b, s, h], qr[b, s, h]]))
                m = sc.max()
                e = np.exp(sc - m)
                out[b, s, h] = (e @ v) / e.sum()
                lse[b, s, h] = m + np.log(e.sum())
    return out, lse


def dense_multi(case, causal: bool):
    """(out [B,S,Hq,D], lse [B,S,Hq]) in float64 for a multi-query case:
    query s of sequence b sees keys t <= n - S + s (causal) or t < n, and
    with a window only the last `window` of them."""
    K = pool_f64(case.k_pool)
    V = pool_f64(case.v_pool)
    q = case.q.to(torch.float64).numpy()
    bt = case.block_table.numpy()
    ctx = case.context_lens.numpy()
    B, S, H, D = q.shape
    G = H // case.num_kv_heads
    out = np.zeros((B, S, H, D))
    lse = np.full((B, S, H), -np.inf)
    for b in range(B):
        n = int(ctx[b])
        for s in range(S):
            hi = min(n, n - S + s + 1) if causal else n
            lo = max(0, hi - case.window) if case.window > 0 else 0
            if hi <= lo:
                continue
            t = np.arange(lo, hi)
            for h in range(H):
                k = gather_rows(K, case.layout, bt[b], t, case.page_size, h // G)
                v = gather_rows(V, case.layout, bt[b], t, case.page_size, h // G)
                sc = case.scale * (k @ q[b, s, h])
                m = sc.max()
                e = np.exp(sc - m)
                out[b, s, h] = (e @ v) / e.sum()
                lse[b, s, h] = m + np.log(e.sum())
    return out, lse
