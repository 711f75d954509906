#!/usr/bin/env python3
"""Decode-attention benchmark: µs per call and KV-read bandwidth on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama]

One step = one pa_decode call (balanced split-KV kernel + LSE merge kernel)
over one batch of the synthetic workload, inputs resident in HBM.  The timed
region is bracketed by torch.cuda.synchronize() on both sides and measured
with HIP events on the stream the kernels are launched on (torch's current
stream, whose handle is passed through the C ABI).

value = algorithmic K+V bytes per call / mean time per call  (GB/s, 1e9 B/s)
  algorithmic bytes = sum over sequences of attended keys * 2 (K and V)
                      * num_kv_heads * head_dim * 2 B
roofline: the same bytes / the mean duration of one pa_decode call (balanced
  split-KV kernel + merge kernel), from HIP events around each of K calls on
  the launch stream; the rocprofv3 kernel trace splits it.

--workload mla times mla_absorbed_decode on the 128-head latent workload
instead (absorb + split + merge/W_UV kernels); its bytes are the latent rows
read plus W_UK, W_UV, q and out, and its flops the four contractions.
cpu_baseline: the CPU oracle (float64, the parity reference) on the whole
  workload, all host threads, on the same byte definition.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, 2.5 PFLOP/s
METRIC = "decode-attn µs/call + KV-read GB/s (% of MI355X HBM peak), d128 GQA bs64"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama",
                    choices=["tiny", "llama", "d256w", "long", "mla", "verify", "insert",
                             "llama_fp8", "llama_f32", "d512", "mla_fp8", "mla_verify",
                             "mla_verify_fp8", "long_splitkv"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run K device-to-device copies of a 1 GiB buffer instead (reference "
                         "kernel of known traffic for the HBM byte counters); prints one JSON line")
    ap.add_argument("--rotate", type=int, default=1,
                    help="input sets to rotate through (for workloads that fit in the 256 MB "
                         "Infinity Cache)")
    return ap.parse_args()


def main() -> int:
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              "(this build has no multi-GPU path)", file=sys.stderr)
        return 2
    import torch

    from paged_attention_decode_05_amd import binding as pb
    from paged_attention_decode_05_amd import workload as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    if a.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(a.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": a.steps}), flush=True)
        return 0
    if a.workload in ("mla", "mla_fp8", "mla_verify", "mla_verify_fp8"):
        return bench_mla(a, torch, pb, wl, dev)
    if a.workload == "verify":
        return bench_verify(a, torch, pb, wl, dev)
    if a.workload == "insert":
        return bench_insert(a, torch, pb, wl, dev)
    if a.workload == "long_splitkv":
        return bench_splitkv(a, torch, pb, wl, dev)
    log(f"generating workload {a.workload} (seeded) ...")
    t0 = time.time()
    cases = [wl.NAMED[a.workload](poison=False, seed=wl.SEED_BASE + 100 * i + {
        "tiny": 1, "llama": 2, "d256w": 3, "long": 4, "llama_fp8": 5, "llama_f32": 6,
        "d512": 7}[a.workload])
        for i in range(a.rotate)]
    dcs = [c.to(dev) for c in cases]
    log(f"  {time.time() - t0:.1f}s; pool pages {cases[0].num_pages}, "
        f"sum ctx {int(cases[0].context_lens.sum())}")
    c0 = cases[0]
    B, H, D = c0.q.shape
    Hkv = c0.num_kv_heads
    kv_bytes = [c.kv_bytes() for c in cases]
    ws_bytes = pb.pa_decode_workspace_size(B, H, Hkv, D, c0.max_pages, c0.page_size, c0.window)
    ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
    kvl = [pb.kv_layout(d.k_pool, d.layout) for d in dcs]

    fp8 = c0.kv_dtype == "fp8"
    f32 = c0.kv_dtype == "f32"

    def step(i):
        d = dcs[i % len(dcs)]
        if f32:
            pb.pa_decode_f32(d.q, d.k_pool, d.v_pool, kvl[i % len(dcs)], d.block_table,
                             d.context_lens, d.scale, d.window, out, None, ws)
        elif fp8:
            pb.pa_decode_fp8(d.q, d.k_pool, d.v_pool, kvl[i % len(dcs)], d.block_table,
                             d.context_lens, d.scale, d.k_scale, d.v_scale, d.window, out, None, ws)
        else:
            pb.pa_decode(d.q, d.k_pool, d.v_pool, kvl[i % len(dcs)], d.block_table,
                         d.context_lens, d.scale, d.window, out, None, ws)

    stream = torch.cuda.current_stream()
    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"timing {a.steps} pa_decode calls ...")
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(a.steps):
        step(i)
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    ms_per_step = total_ms / a.steps
    mean_bytes = sum(kv_bytes[i % len(cases)] for i in range(a.steps)) / a.steps
    gbs = mean_bytes / (ms_per_step * 1e-3) / 1e9

    # The dominant work is the balanced split-KV kernel; pa_decode launches it
    # and the merge kernel inside one C call, so the per-launch figure brackets
    # the whole call with HIP events on the launch stream (an upper bound on
    # the split kernel's own duration).
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(a.steps)]
    torch.cuda.synchronize()
    for i in range(a.steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    call_ms = [e[0].elapsed_time(e[1]) for e in ev]
    call_mean = statistics.fmean(call_ms)
    achieved = mean_bytes / (call_mean * 1e-3) / 1e9

    cpu = None
    if not a.no_cpu:
        cpu = cpu_baseline(cases[0])

    res = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_call": round(ms_per_step * 1e3, 2),
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "storage_dtype": "e4m3 (one scale per pool)" if fp8 else ("f32" if f32 else "bf16"),
        "data": "synthetic",
        "config": {
            "workload": {"llama": "llama3-8b-shaped decode, bs64, 32q/8kv heads, d128, page 32, "
                                  "ctx U[512,8192]",
                         "tiny": "tiny paged decode, 8 seqs, 8q/2kv, d128, page 32",
                         "d256w": "d256 GQA-8 sliding window 4096, bs32",
                         "d512": "head_dim-512 GQA-8 decode, bs64, 16q/2kv heads, page 32, "
                                 "ctx U[512,8192]",
                         "long": "long context bs4, ctx 32K-128K, d128",
                         "llama_fp8": "llama3-8b-shaped decode over an FP8 (E4M3) KV cache, bs64, "
                                      "32q/8kv heads, d128, page 32, ctx U[512,8192]",
                         "llama_f32": "llama3-8b-shaped decode over an f32 KV cache, bs64, "
                                      "32q/8kv heads, d128, page 32, ctx U[512,8192]"}[a.workload],
            "batch": B, "num_q_heads": H, "num_kv_heads": Hkv, "head_dim": D,
            "page_size": c0.page_size, "window": c0.window,
            "sum_context": int(c0.context_lens.sum()), "pool_pages": c0.num_pages,
            "split": "balanced (equal K/V bytes per block)", "kv_bytes_per_call": int(mean_bytes),
            "input_sets_rotated": a.rotate, "layout": c0.layout,
        },
        "call_us": {"mean": round(call_mean * 1e3, 2),
                    "p10": round(sorted(call_ms)[len(call_ms) // 10] * 1e3, 2),
                    "p90": round(sorted(call_ms)[(9 * len(call_ms)) // 10] * 1e3, 2)},
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": (recorded_traffic({"llama": "pa_decode_llama_bs64",
                                          "llama_fp8": "pa_decode_fp8_llama_bs64",
                                          "d512": "pa_decode_d512_bs64"}[a.workload])
                        if a.workload in ("llama", "llama_fp8", "d512") and a.rotate == 1 else None),
            "kernel": ("pa_decode_fp8" if fp8 else "pa_decode_f32" if f32 else "pa_decode") +
                      " call: balanced_split_kernel + balanced_merge_kernel",
            "algorithmic_bytes_per_launch": int(mean_bytes),
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)
    return 0


def recorded_traffic(profile: str):
    """HBM bytes per call from the PMC summary profiles/<profile>.md (FETCH_SIZE
    and WRITE_SIZE scaled by a 1 GiB copy), or None when the kernel sources
    it lists have changed since the counters were taken."""
    import hashlib
    import re
    path = os.path.join(ROOT, "profiles", profile + ".md")
    try:
        text = open(path).read()
    except OSError:
        return None
    m_t = re.search(r"^traffic_bytes_per_call: (\d+)$", text, re.M)
    m_s = re.search(r"^sources: (.+)$", text, re.M)
    m_h = re.search(r"^sources_sha256: ([0-9a-f]{64})$", text, re.M)
    if not (m_t and m_s and m_h):
        return None
    h = hashlib.sha256()
    for f in m_s.group(1).split():
        try:
            h.update(open(os.path.join(ROOT, "paged_attention_decode_05_amd", "csrc", f), "rb").read())
        except OSError:
            return None
    return int(m_t.group(1)) if h.hexdigest() == m_h.group(1) else None


def _time_calls(torch, stream, step, steps):
    """Mean per-call ms from HIP events around each call on the launch stream,
    plus the list of per-call times."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = [e[0].elapsed_time(e[1]) for e in ev]
    return statistics.fmean(ms), ms


def _timed(a, torch, step):
    stream = torch.cuda.current_stream()
    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(a.steps):
        step(i)
    stop.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(stop) / a.steps
    call_mean, call_ms = _time_calls(torch, stream, step, a.steps)
    return ms_per_step, call_mean, call_ms


def _line(a, metric, nbytes, ms_per_step, call_mean, call_ms, config, kernel, extra=None):
    gbs = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (call_mean * 1e-3) / 1e9
    res = {"metric": metric, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
           "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_per_step, 5),
           "us_per_call": round(ms_per_step * 1e3, 2),
           "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "f32", "storage_dtype": "bf16",
           "data": "synthetic", "config": config,
           "call_us": {"mean": round(call_mean * 1e3, 2),
                       "p10": round(sorted(call_ms)[len(call_ms) // 10] * 1e3, 2),
                       "p90": round(sorted(call_ms)[(9 * len(call_ms)) // 10] * 1e3, 2)},
           "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                        "kernel": kernel, "algorithmic_bytes_per_launch": int(nbytes)},
           "cpu_baseline": None}
    if extra:
        res.update(extra)
    print(json.dumps(res), flush=True)
    return 0


def bench_verify(a, torch, pb, wl, dev) -> int:
    """Speculative-decoding verify step: the llama-shaped bs64 batch with 4
    causal queries per sequence through pa_decode_multiquery."""
    S = 4
    log("generating workload verify (seeded) ...")
    case = wl.make_gqa_case(context_lens=(), ctx_draw=(512, 8192), batch=64, num_q_heads=32,
                            num_kv_heads=8, head_dim=128, page_size=32, seed=wl.SEED_BASE + 6,
                            num_queries=S, poison=False, name="verify")
    dc = case.to(dev)
    B, _, H, D = dc.q.shape
    out = torch.empty_like(dc.q)
    ws = torch.zeros(pb.pa_decode_multiquery_workspace_size(B, H, 8, D, dc.max_pages, 32, 0, S),
                     dtype=torch.uint8, device=dev)
    kv = pb.kv_layout(dc.k_pool, dc.layout)

    def step(i):
        pb.pa_decode_multiquery(dc.q, dc.k_pool, dc.v_pool, kv, dc.block_table, dc.context_lens,
                                dc.scale, 0, True, out, None, ws)

    ms, mean, calls = _timed(a, torch, step)
    return _line(a, "verify-step decode-attn GB/s (4 causal queries per sequence), d128 GQA bs64",
                 case.kv_bytes(), ms, mean, calls,
                 {"workload": "llama3-8b-shaped verify step, bs64, 4 causal queries per sequence, "
                              "32q/8kv heads, d128, page 32, ctx U[512,8192]",
                  "sum_context": int(case.context_lens.sum()), "num_queries": S},
                 "pa_decode_multiquery call: balanced_split_kernel<128,16> + merge")


def bench_insert(a, torch, pb, wl, dev) -> int:
    """KV insert of an 8192-token chunk (32q/8kv heads, d128) into the
    llama-shaped pools at random free slots."""
    T = 8192
    log("generating workload insert (seeded) ...")
    case = wl.llama(poison=False)
    dc = case.to(dev)
    g = torch.Generator().manual_seed(wl.SEED_BASE + 7)
    total = case.num_pages * case.page_size
    slots = torch.randperm(total, generator=g)[:T].to(torch.int64).to(dev)
    k_new = torch.randn(T, 8, 128, generator=g).to(torch.bfloat16).to(dev)
    v_new = torch.randn(T, 8, 128, generator=g).to(torch.bfloat16).to(dev)
    kv = pb.kv_layout(dc.k_pool, dc.layout)

    def step(i):
        pb.pa_kv_insert(k_new, v_new, dc.k_pool, dc.v_pool, kv, slots)

    ms, mean, calls = _timed(a, torch, step)
    nbytes = 2 * (2 * T * 8 * 128 * 2)          # K and V rows read once and written once
    return _line(a, "KV insert GB/s (rows read + written), 8192 tokens x 8 KV heads x d128",
                 nbytes, ms, mean, calls,
                 {"workload": "KV insert of an 8192-token chunk into the llama-shaped pools",
                  "tokens": T}, "pa_kv_insert call: kv_insert_kernel")


def bench_splitkv(a, torch, pb, wl, dev) -> int:
    """The long-context workload through the fixed-partition path: 512-key
    partitions, per-partition (max, sum, partial out) in fp32 from
    pa_decode_splitkv, then pa_merge_lse in ascending partition order."""
    P = 512
    log("generating workload long (seeded) ...")
    case = wl.long_ctx(poison=False)
    dc = case.to(dev)
    B, H, D = case.q.shape
    maxp = (int(case.context_lens.max()) + P - 1) // P
    part_out = torch.empty((B, H, maxp, D), dtype=torch.float32, device=dev)
    part_max = torch.empty((B, H, maxp), dtype=torch.float32, device=dev)
    part_sum = torch.empty((B, H, maxp), dtype=torch.float32, device=dev)
    out = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
    kv = pb.kv_layout(dc.k_pool, dc.layout)

    def step(i):
        pb.pa_decode_splitkv(dc.q, dc.k_pool, dc.v_pool, kv, dc.block_table, dc.context_lens,
                             dc.scale, dc.window, P, maxp, part_out, part_max, part_sum)
        pb.pa_merge_lse(part_out, part_max, part_sum, dc.context_lens, P, dc.window, out)

    ms, mean, calls = _timed(a, torch, step)
    return _line(a, METRIC, case.kv_bytes(), ms, mean, calls,
                 {"workload": "long context bs4, ctx 32K-128K, d128, fixed 512-key partitions",
                  "batch": B, "num_q_heads": H, "num_kv_heads": case.num_kv_heads, "head_dim": D,
                  "page_size": case.page_size, "sum_context": int(case.context_lens.sum()),
                  "partition_size": P, "max_partitions": maxp,
                  "partial_bytes_written": int(part_out.numel() * 4 + 2 * part_max.numel() * 4)},
                 "pa_decode_splitkv + pa_merge_lse calls: split_kernel + merge_kernel")


def bench_mla(a, torch, pb, wl, dev) -> int:
    fp8 = a.workload.endswith("_fp8")
    verify = a.workload.startswith("mla_verify")
    log(f"generating workload {a.workload} (seeded) ...")
    if verify:
        def make(poison, seed):
            return wl.mla_verify(poison=poison, seed=seed, cache_dtype="fp8" if fp8 else "bf16")
        base = wl.SEED_BASE + 9
    else:
        make = wl.mla_fp8 if fp8 else wl.mla
        base = wl.SEED_BASE + (8 if fp8 else 5)
    cases = [make(poison=False, seed=base + 100 * i) for i in range(a.rotate)]
    case = cases[0]
    dcs = [c.to(dev) for c in cases]
    B, H, S = case.batch, case.num_heads, case.num_queries
    out = torch.empty(((B, S, H) if verify else (B, H)) + (case.d_v,), dtype=torch.bfloat16,
                      device=dev)
    ws = torch.empty(max(pb.mla_absorbed_decode_workspace_size(B, S * H, c.max_pages, c.page_size,
                                                               0)
                         for c in cases), dtype=torch.uint8, device=dev)
    layouts = [pb.kv_layout(d.cache, "PSR") for d in dcs]

    if verify:
        def decode(*args):
            pb.mla_absorbed_decode_multiquery(*args, causal=True)
    else:
        decode = pb.mla_absorbed_decode_fp8 if fp8 else pb.mla_absorbed_decode

    def step(i):
        dc = dcs[i % len(dcs)]
        decode(dc.q_nope, dc.q_rope, dc.cache, layouts[i % len(dcs)], dc.w_uk, dc.w_uv,
               dc.block_table, dc.context_lens, dc.scale, out, ws)

    stream = torch.cuda.current_stream()
    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(a.steps):
        step(i)
    stop.record(stream)
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(stop) / a.steps
    call_mean, call_ms = _time_calls(torch, stream, step, a.steps)
    def flops_of(c):
        # keys seen per query head, summed: under the causal mask query s of S
        # sees n - S + 1 + s keys
        n = c.context_lens.to(torch.int64)
        k = int(sum((n - S + 1 + s).clamp(min=0).sum() for s in range(S))) if verify \
            else int(n.sum())
        return 2 * B * S * H * c.d_nope * c.d_lat + 2 * H * k * (c.d_lat + c.d_rope) \
            + 2 * H * k * c.d_lat + 2 * B * S * H * c.d_lat * c.d_v
    # mean over the calls of the timed loops (input set i % rotate)
    nbytes = int(round(sum(cases[i % len(cases)].algorithmic_bytes() for i in range(a.steps)) / a.steps))
    flops = int(round(sum(flops_of(cases[i % len(cases)]) for i in range(a.steps)) / a.steps))
    keys = int(case.context_lens.sum())
    gbs = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (call_mean * 1e-3) / 1e9
    cpu = None
    if not a.no_cpu:
        from oracle.oracle import Oracle
        o = Oracle()
        threads = oracle_threads()

        def run(c):
            if verify:
                o.mla_multi(c, True)
            elif fp8:
                o.mla_fp8(c)
            else:
                o.mla(c, "f64")

        o.set_threads(threads)
        t = time.time()
        run(case)
        sec = time.time() - t
        # one thread: the first 2 sequences (the oracle's time is linear in the keys)
        sub = case.to("cpu")
        sub.q_nope, sub.q_rope = case.q_nope[:2].contiguous(), case.q_rope[:2].contiguous()
        sub.block_table, sub.context_lens = case.block_table[:2].contiguous(), case.context_lens[:2].contiguous()
        o.set_threads(1)
        t = time.time()
        run(sub)
        sec1 = time.time() - t
        o.set_threads(threads)
        cpu = {"value": round(case.algorithmic_bytes() / sec / 1e9, 3), "unit": "GB/s", "cores": threads,
               "kind": "oracle", "sample": f"whole workload ({B} seqs, {keys} keys), float64 "
                                           "oracle, one run", "seconds_per_call": round(sec, 3),
               "one_core": {"value": round(sub.algorithmic_bytes() / sec1 / 1e9, 3), "unit": "GB/s",
                            "seconds": round(sec1, 3),
                            "sample": f"first 2 sequences ({int(sub.context_lens.sum())} keys), "
                                      "one run, their bytes on the same definition"},
               "host": host_info()}
    mflops = flops / (call_mean * 1e-3) / 1e12
    if verify:
        # query heads x keys dominate: the contraction over the latent cache
        roof = {"bound": "mfma", "achieved": round(mflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(mflops / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": recorded_traffic("mla_verify_fp8_bs16_s4_h128" if fp8
                                            else "mla_verify_bs16_s4_h128")
                if a.rotate == 1 else None,
                "kernel": ("mla_absorbed_decode_multiquery_fp8" if fp8 else
                           "mla_absorbed_decode_multiquery") +
                          " call: absorb + split + merge/W_UV kernels",
                "algorithmic_flops_per_launch": flops,
                "hbm_gbs": round(achieved, 1)}
    else:
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": recorded_traffic("mla_absorbed_decode_fp8_bs16_h128" if fp8
                                            else "mla_absorbed_decode_bs16_h128")
                if a.rotate == 1 else None,
                "kernel": ("mla_absorbed_decode_fp8" if fp8 else "mla_absorbed_decode") +
                          " call: absorb + split + merge/W_UV kernels",
                "algorithmic_bytes_per_launch": nbytes,
                "mfma_tflops": round(mflops, 2)}
    what = ("absorbed MLA verify, 4 causal queries per sequence, " if verify else
            "absorbed MLA decode, ")
    res = {
        "metric": ("absorbed-MLA verify µs/call + TFLOP/s, bs16 S4 h128" if verify else
                   "absorbed-MLA decode µs/call + latent GB/s, bs16 h128"),
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms_per_step, 5),
        "us_per_call": round(ms_per_step * 1e3, 2),
        "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "storage_dtype": ("e4m3 latent (one power-of-two scale per 64) + bf16 rope, 656 B/token"
                          if fp8 else "bf16"),
        "data": "synthetic",
        "config": {"workload": what + ("over an FP8 latent cache, " if fp8 else "") +
                               "bs16, 128 heads, 512+64 latent, page 64, ctx U[1024,8192]",
                   "sum_context": keys, "input_sets_rotated": a.rotate,
                   "algorithmic_bytes": nbytes, "algorithmic_flops": flops},
        "call_us": {"mean": round(call_mean * 1e3, 2),
                    "p10": round(sorted(call_ms)[len(call_ms) // 10] * 1e3, 2),
                    "p90": round(sorted(call_ms)[(9 * len(call_ms)) // 10] * 1e3, 2)},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)
    return 0


def host_info():
    """CPU model and logical CPU count of the host the bench runs on."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "cpu_count": os.cpu_count()}


def oracle_threads():
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    # the GPU machine grants 16 host threads per GPU (OMP_NUM_THREADS)
    return max(1, min(threads, int(os.environ.get("OMP_NUM_THREADS", "16") or 16)))


def cpu_baseline(case):
    """The CPU oracle (float64 gate instantiation, unmodified) on the whole
    workload with every host thread, repeated until about 10 s of wall time or
    3 runs; reports the median on the same byte definition as the GPU.  Then
    one run of the whole workload on one thread."""
    from oracle.oracle import Oracle
    o = Oracle()
    threads = oracle_threads()

    def run():
        if case.kv_dtype == "fp8":
            o.decode_fp8(case)
        elif case.kv_dtype == "f32":
            o.decode_f32pool(case)
        else:
            o.decode(case, "f64")

    o.set_threads(threads)
    times = []
    t_all = time.time()
    while len(times) < 3 or (time.time() - t_all < 10 and len(times) < 10):
        t = time.time()
        run()
        times.append(time.time() - t)
    med = statistics.median(times)
    o.set_threads(1)
    t = time.time()
    run()
    one = time.time() - t
    o.set_threads(threads)
    return {"value": round(case.kv_bytes() / med / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"whole workload ({case.batch} seqs, {int(case.context_lens.sum())} keys), "
                      f"float64 oracle, median of {len(times)} runs",
            "seconds_per_call": round(med, 3),
            "one_core": {"value": round(case.kv_bytes() / one / 1e9, 3), "unit": "GB/s",
                         "seconds_per_call": round(one, 3), "sample": "whole workload, one run"},
            "host": host_info()}


if __name__ == "__main__":
    sys.exit(main())
