#!/usr/bin/env python3
"""Decode-attention benchmark: µs per call and KV-read bandwidth on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama]

One step = one call of the workload's entry point (pa_decode by default: the
balanced split-KV kernel and the LSE merge kernel) over one batch of the
synthetic workload, inputs resident in HBM.  The timed region is K calls back
to back, bracketed by torch.cuda.synchronize() and HIP events on the stream the
kernels are launched on (torch's current stream, whose handle is passed through
the C ABI).

value        algorithmic bytes per call / (timed region / K)        (GB/s, 1e9 B/s)
             bytes = attended keys x 2 (K and V) x num_kv_heads x head_dim x
             element size, summed over sequences (the MLA workloads: latent rows
             read once + W_UK + W_UV + q + out)
roofline     one definition for every workload: the algorithmic bytes (or, for the
             MFMA-bound MLA split kernel, flops) of one call divided by the mean
             duration of that call's dominant kernel, which the library times with
             two HIP events attached to that kernel's launch (pa_profile_next:
             hipExtLaunchKernelGGL stamps them as the kernel starts and ends, the
             clock of a rocprofv3 kernel trace); averaged over K calls.  `traffic` is the HBM
             byte count of that kernel from the rocprofv3 FETCH_SIZE / WRITE_SIZE
             summary under profiles/, or null when the kernel sources changed
             since the counters were taken.
parity       the same call's output against the float64 oracle (oracle.compare:
             |g - r| <= 2e-2 and <= 2 bf16 ulps, floor 2^-22), with the number of
             elements that pass only through the floor
cpu_baseline the fp32 oracle (the f64 gate where the oracle has no fp32 form) on
             the whole workload with the host threads granted per GPU, and on one
             thread; same byte definition

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, 2.5 PFLOP/s
METRIC = "decode-attn µs/call + KV-read GB/s (% of MI355X HBM peak), d128 GQA bs64"

GQA = {   # name -> (generator, seed offset, description)
    "tiny": ("tiny", 1, "tiny paged decode, 8 seqs, 8q/2kv, d128, page 32"),
    "llama": ("llama", 2, "llama3-8b-shaped decode, bs64, 32q/8kv heads, d128, page 32, "
                          "ctx U[512,8192]"),
    "d256w": ("d256w", 3, "d256 GQA-8 sliding window 4096, bs32, 16q/2kv heads, page 32, "
                          "ctx U[1024,16384]"),
    "long": ("long_ctx", 4, "long context bs4, ctx 32K-128K, 32q/8kv heads, d128, page 32"),
    "llama_fp8": ("llama_fp8", 5, "llama3-8b-shaped decode over an FP8 (E4M3) KV cache, bs64, "
                                  "32q/8kv heads, d128, page 32, ctx U[512,8192]"),
    "llama_f32": ("llama_f32", 6, "llama3-8b-shaped decode over an f32 KV cache, bs64, "
                                  "32q/8kv heads, d128, page 32, ctx U[512,8192]"),
    "d512": ("d512", 7, "head_dim-512 GQA-8 decode, bs64, 16q/2kv heads, page 32, "
                        "ctx U[512,8192]"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="llama",
                    choices=sorted(GQA) + ["mla", "mla_fp8", "mla_verify", "mla_verify_fp8",
                                           "verify", "insert", "long_splitkv"])
    ap.add_argument("--no-cpu", action="store_true",
                    help="skip the CPU-oracle baseline and the parity check")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run K device-to-device copies of a 1 GiB buffer instead (reference "
                         "kernel of known traffic for the HBM byte counters); prints one JSON line")
    ap.add_argument("--rotate", type=int, default=1,
                    help="input sets to rotate through (for workloads that fit in the 256 MB "
                         "Infinity Cache)")
    return ap.parse_args()


# ---- timing --------------------------------------------------------------------------


class Timing:
    """Back-to-back calls (ms_per_step), then per-call events: around the whole
    call and, through the library's hook, around its dominant kernel."""

    def __init__(self, torch, pb, a, step):
        self.torch, self.pb = torch, pb
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
        self.ms_per_step = start.elapsed_time(stop) / a.steps
        call = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(a.steps)]
        kern = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(a.steps)]
        for e0, e1 in kern:            # materialise the events' handles
            e0.record(stream)
            e1.record(stream)
        torch.cuda.synchronize()
        for i in range(a.steps):
            call[i][0].record(stream)
            pb.pa_profile_next(kern[i][0].cuda_event, kern[i][1].cuda_event)
            step(i)
            call[i][1].record(stream)
        torch.cuda.synchronize()
        pb.pa_profile_next(None, None)
        self.call_ms = [e0.elapsed_time(e1) for e0, e1 in call]
        self.kern_ms = [e0.elapsed_time(e1) for e0, e1 in kern]
        self.call_mean = statistics.fmean(self.call_ms)
        self.kern_mean = statistics.fmean(self.kern_ms)

    def call_us(self):
        s = sorted(self.call_ms)
        return {"mean": round(self.call_mean * 1e3, 2), "p10": round(s[len(s) // 10] * 1e3, 2),
                "p90": round(s[(9 * len(s)) // 10] * 1e3, 2)}


def recorded_traffic(profile: str):
    """HBM bytes per launch of the dominant kernel from the PMC summary
    profiles/<profile>.md (FETCH_SIZE and WRITE_SIZE scaled by a 1 GiB copy), or
    None when the kernel sources it lists have changed since the counters were
    taken."""
    path = os.path.join(ROOT, "profiles", profile + ".md")
    try:
        text = open(path).read()
    except OSError:
        return None
    m_t = re.search(r"^traffic_bytes_per_launch: (\d+)$", text, re.M)
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


def roofline(t: Timing, kernel: str, profile: str | None, rotate: int, nbytes=None, flops=None):
    """The dominant kernel against its roofline: HBM (GB/s) when nbytes is given,
    dense bf16 MFMA (TFLOP/s) when flops is."""
    sec = t.kern_mean * 1e-3
    traffic = recorded_traffic(profile) if (profile and rotate == 1) else None
    if flops is not None:
        ach = flops / sec / 1e12
        r = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
             "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
             "algorithmic_flops_per_launch": int(flops)}
    else:
        ach = nbytes / sec / 1e9
        r = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
             "algorithmic_bytes_per_launch": int(nbytes)}
    r.update({"kernel": kernel, "kernel_us": round(t.kern_mean * 1e3, 2),
              "definition": "algorithmic work of one call / mean duration of its dominant kernel "
                            "(HIP events attached by the library to that kernel's launch, "
                            "stamped as it starts and ends on the launch stream)"})
    return r


def line(a, metric, nbytes, t: Timing, config, roof, extra=None, dtype="f32",
         storage="bf16", parity=None, cpu=None):
    gbs = nbytes / (t.ms_per_step * 1e-3) / 1e9
    res = {"metric": metric, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1,
           "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(t.ms_per_step, 5),
           "us_per_call": round(t.ms_per_step * 1e3, 2),
           "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": dtype, "storage_dtype": storage,
           "data": "synthetic", "config": config, "call_us": t.call_us(), "roofline": roof,
           "parity": parity, "cpu_baseline": cpu}
    if extra:
        res.update(extra)
    print(json.dumps(res), flush=True)
    return 0


# ---- oracle: parity and the CPU baseline ---------------------------------------------


def host_info():
    """CPU model and logical CPU count of the host the bench runs on."""
    model = "unknown"
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_model": model, "cpu_count": os.cpu_count()}


def oracle_threads():
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    # the GPU machine grants 16 host threads per GPU (OMP_NUM_THREADS)
    return max(1, min(threads, int(os.environ.get("OMP_NUM_THREADS", "16") or 16)))


def parity_of(out_cpu, ref):
    from oracle.compare import compare
    rep = compare(out_cpu, ref)
    return {"gate": "|g-r| <= 2e-2 and <= 2 bf16 ulp vs the float64 oracle (floor 2^-22)",
            "ok": rep.ok, "elements": rep.n, "max_abs": rep.max_abs, "max_ulp": rep.max_ulp,
            "bitwise_pct": round(rep.bitwise_pct, 4), "fail": rep.n_fail,
            "pass_only_by_floor": rep.n_fail_unfloored - rep.n_fail}


def cpu_timed(run, nbytes, what, sample):
    """The oracle on the granted host threads (median of >= 3 runs, about 10 s at
    most), then once on one thread."""
    from oracle.oracle import Oracle
    o = Oracle()
    threads = oracle_threads()
    o.set_threads(threads)
    times, t_all = [], time.time()
    while len(times) < 3 or (time.time() - t_all < 10 and len(times) < 10):
        t = time.time()
        run(o)
        times.append(time.time() - t)
    med = statistics.median(times)
    o.set_threads(1)
    t = time.time()
    run(o)
    one = time.time() - t
    o.set_threads(threads)
    return {"value": round(nbytes / med / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "oracle": what, "sample": sample + f", median of {len(times)} runs",
            "seconds_per_call": round(med, 4),
            "one_core": {"value": round(nbytes / one / 1e9, 3), "unit": "GB/s",
                         "seconds_per_call": round(one, 4), "sample": sample + ", one run"},
            "host": host_info()}


# ---- workloads -----------------------------------------------------------------------


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
    if a.workload.startswith("mla"):
        return bench_mla(a, torch, pb, wl, dev)
    if a.workload == "verify":
        return bench_verify(a, torch, pb, wl, dev)
    if a.workload == "insert":
        return bench_insert(a, torch, pb, wl, dev)
    if a.workload == "long_splitkv":
        return bench_splitkv(a, torch, pb, wl, dev)
    return bench_gqa(a, torch, pb, wl, dev)


def bench_gqa(a, torch, pb, wl, dev) -> int:
    gen, seed_off, desc = GQA[a.workload]
    log(f"generating workload {a.workload} (seeded) ...")
    t0 = time.time()
    cases = [getattr(wl, gen)(poison=False, seed=wl.SEED_BASE + 100 * i + seed_off)
             for i in range(a.rotate)]
    dcs = [c.to(dev) for c in cases]
    log(f"  {time.time() - t0:.1f}s; pool pages {cases[0].num_pages}, "
        f"sum ctx {int(cases[0].context_lens.sum())}")
    c0 = cases[0]
    B, H, D = c0.q.shape
    Hkv = c0.num_kv_heads
    ws = torch.zeros(pb.pa_decode_workspace_size(B, H, Hkv, D, c0.max_pages, c0.page_size,
                                                 c0.window), dtype=torch.uint8, device=dev)
    out = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
    kvl = [pb.kv_layout(d.k_pool, d.layout) for d in dcs]
    fp8, f32 = c0.kv_dtype == "fp8", c0.kv_dtype == "f32"

    def step(i):
        d, kv = dcs[i % len(dcs)], kvl[i % len(dcs)]
        if f32:
            pb.pa_decode_f32(d.q, d.k_pool, d.v_pool, kv, d.block_table, d.context_lens, d.scale,
                             d.window, out, None, ws)
        elif fp8:
            pb.pa_decode_fp8(d.q, d.k_pool, d.v_pool, kv, d.block_table, d.context_lens, d.scale,
                             d.k_scale, d.v_scale, d.window, out, None, ws)
        else:
            pb.pa_decode(d.q, d.k_pool, d.v_pool, kv, d.block_table, d.context_lens, d.scale,
                         d.window, out, None, ws)

    log(f"timing {a.steps} calls ...")
    t = Timing(torch, pb, a, step)
    nbytes = sum(cases[i % len(cases)].kv_bytes() for i in range(a.steps)) / a.steps
    entry = "pa_decode_fp8" if fp8 else "pa_decode_f32" if f32 else "pa_decode"
    kname = f"balanced_split_kernel<{D}, {1 << (H // Hkv - 1).bit_length()}, {c0.kv_dtype}>"
    roof = roofline(t, f"{entry}: {kname}",
                    {"llama": "pa_decode_llama_bs64", "llama_fp8": "pa_decode_fp8_llama_bs64",
                     "llama_f32": "pa_decode_f32_llama_bs64", "d512": "pa_decode_d512_bs64",
                     "d256w": "pa_decode_d256w_bs32", "long": "pa_decode_long_bs4",
                     "tiny": "pa_decode_tiny"}.get(a.workload),
                    a.rotate, nbytes=nbytes)
    parity = cpu = None
    if not a.no_cpu:
        step(0)
        torch.cuda.synchronize()
        got = out.cpu()
        from oracle.oracle import Oracle
        o = Oracle()
        o.set_threads(oracle_threads())
        ref = (o.decode_fp8(c0) if fp8 else o.decode_f32pool(c0) if f32 else o.decode(c0))[0]
        parity = parity_of(got, ref)
        if fp8:
            run, what = (lambda o: o.decode_fp8(c0)), "float64 (the oracle has no fp32 FP8 form)"
        elif f32:
            run, what = (lambda o: o.decode_f32pool(c0)), "float64 (the oracle has no fp32 form for f32 pools)"
        else:
            run, what = (lambda o: o.decode(c0, "f32")), "fp32"
        cpu = cpu_timed(run, c0.kv_bytes(), what,
                        f"whole workload ({c0.batch} seqs, {int(c0.context_lens.sum())} keys)")
    config = {"workload": desc, "batch": B, "num_q_heads": H, "num_kv_heads": Hkv,
              "head_dim": D, "page_size": c0.page_size, "window": c0.window,
              "sum_context": int(c0.context_lens.sum()), "pool_pages": c0.num_pages,
              "split": "balanced (equal K/V bytes per block)", "kv_bytes_per_call": int(nbytes),
              "input_sets_rotated": a.rotate, "layout": c0.layout}
    storage = "e4m3 (one scale per pool)" if fp8 else ("f32" if f32 else "bf16")
    return line(a, METRIC, nbytes, t, config, roof, storage=storage, parity=parity, cpu=cpu)


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

    t = Timing(torch, pb, a, step)
    nbytes = case.kv_bytes()
    roof = roofline(t, "pa_decode_multiquery: balanced_split_kernel<128, 16, bf16>",
                    "pa_decode_verify_bs64_s4", a.rotate, nbytes=nbytes)
    parity = None
    if not a.no_cpu:
        from oracle.oracle import Oracle
        o = Oracle()
        o.set_threads(oracle_threads())
        parity = parity_of(out.cpu(), o.decode_multi(case, True)[0])
    return line(a, "verify-step decode-attn GB/s (4 causal queries per sequence), d128 GQA bs64",
                nbytes, t, {"workload": "llama3-8b-shaped verify step, bs64, 4 causal queries per "
                                        "sequence, 32q/8kv heads, d128, page 32, ctx U[512,8192]",
                            "sum_context": int(case.context_lens.sum()), "num_queries": S},
                roof, parity=parity)


def bench_insert(a, torch, pb, wl, dev) -> int:
    """KV insert of an 8192-token chunk (8 KV heads, d128) into the llama-shaped
    pools at random free slots."""
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

    t = Timing(torch, pb, a, step)
    nbytes = 2 * (2 * T * 8 * 128 * 2)          # K and V rows read once and written once
    roof = roofline(t, "pa_kv_insert: kv_insert_kernel", "pa_kv_insert_8192", a.rotate, nbytes=nbytes)
    return line(a, "KV insert GB/s (rows read + written), 8192 tokens x 8 KV heads x d128",
                nbytes, t, {"workload": "KV insert of an 8192-token chunk into the llama-shaped "
                                        "pools", "tokens": T}, roof, dtype="u16 copy")


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

    # the hook arms the first call of the step: pa_decode_splitkv's split kernel
    t = Timing(torch, pb, a, step)
    nbytes = case.kv_bytes()
    roof = roofline(t, "pa_decode_splitkv: split_kernel<128, 4>", "pa_decode_splitkv_long_bs4",
                    a.rotate, nbytes=nbytes)
    parity = None
    if not a.no_cpu:
        from oracle.oracle import Oracle
        o = Oracle()
        o.set_threads(oracle_threads())
        parity = parity_of(out.cpu(), o.decode(case)[0])
    return line(a, METRIC, nbytes, t,
                {"workload": "long context bs4, ctx 32K-128K, d128, fixed 512-key partitions",
                 "batch": B, "num_q_heads": H, "num_kv_heads": case.num_kv_heads, "head_dim": D,
                 "page_size": case.page_size, "sum_context": int(case.context_lens.sum()),
                 "partition_size": P, "max_partitions": maxp,
                 "partial_bytes_written": int(part_out.numel() * 4 + 2 * part_max.numel() * 4)},
                roof, parity=parity)


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
        base = wl.SEED_BASE + 5   # FP8 and bf16 caches over the same draws
    cases = [make(poison=False, seed=base + 100 * i) for i in range(a.rotate)]
    case = cases[0]
    dcs = [c.to(dev) for c in cases]
    B, H, S = case.batch, case.num_heads, case.num_queries
    out = torch.empty(((B, S, H) if verify else (B, H)) + (case.d_v,), dtype=torch.bfloat16,
                      device=dev)
    ws = torch.empty(max(pb.mla_absorbed_decode_workspace_size(B, S * H, c.max_pages, c.page_size, 0)
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

    t = Timing(torch, pb, a, step)

    def keys_seen(c):
        # query heads' keys summed: under the causal mask query s of S sees n - S + 1 + s
        n = c.context_lens.to(torch.int64)
        return int(sum((n - S + 1 + s).clamp(min=0).sum() for s in range(S))) if verify \
            else int(n.sum())

    def split_flops(c):   # the latent contractions: 576-deep scores and 512-wide P.V
        return 2 * H * keys_seen(c) * (c.d_lat + c.d_rope) + 2 * H * keys_seen(c) * c.d_lat

    def call_flops(c):
        return 2 * B * S * H * c.d_nope * c.d_lat + split_flops(c) + 2 * B * S * H * c.d_lat * c.d_v

    avg = lambda f: sum(f(cases[i % len(cases)]) for i in range(a.steps)) / a.steps
    nbytes = avg(lambda c: c.algorithmic_bytes())
    entry = ("mla_absorbed_decode_multiquery" if verify else "mla_absorbed_decode") + \
        ("_fp8" if fp8 else "")
    kname = f"{entry}: mla_split_kernel<{'true' if fp8 else 'false'}, {'true' if verify else 'false'}>"
    prof = ("mla_verify" if verify else "mla_absorbed_decode") + ("_fp8" if fp8 else "") + \
        ("_bs16_s4_h128" if verify else "_bs16_h128")
    roof = roofline(t, kname, prof, a.rotate, flops=avg(split_flops))
    roof["hbm_gbs_of_call_bytes"] = round(nbytes / (t.kern_mean * 1e-3) / 1e9, 1)
    parity = cpu = None
    if not a.no_cpu:
        from oracle.oracle import Oracle
        o = Oracle()
        o.set_threads(oracle_threads())
        if verify:
            ref = o.mla_multi(case, True)[0]
        elif fp8:
            ref = o.mla_fp8(case)[0]
        else:
            ref = o.mla(case, "f64")[0]
        step(0)
        torch.cuda.synchronize()
        parity = parity_of(out.cpu(), ref)
        if not verify:
            sub = case.to("cpu")     # the first 2 sequences: a bounded sample
            sub.q_nope, sub.q_rope = case.q_nope[:2].contiguous(), case.q_rope[:2].contiguous()
            sub.block_table = case.block_table[:2].contiguous()
            sub.context_lens = case.context_lens[:2].contiguous()
            if fp8:
                run, what = (lambda o: o.mla_fp8(sub)), "float64 (the oracle has no fp32 FP8 form)"
            else:
                run, what = (lambda o: o.mla(sub, "f32")), "fp32"
            cpu = cpu_timed(run, sub.algorithmic_bytes(), what,
                            f"first 2 sequences ({int(sub.context_lens.sum())} keys), their "
                            "bytes on the same definition")
    what = ("absorbed MLA verify, 4 causal queries per sequence, " if verify else
            "absorbed MLA decode, ")
    return line(a, ("absorbed-MLA verify µs/call + TFLOP/s, bs16 S4 h128" if verify else
                    "absorbed-MLA decode µs/call + latent GB/s, bs16 h128"), nbytes, t,
                {"workload": what + ("over an FP8 latent cache, " if fp8 else "") +
                             "bs16, 128 heads, 512+64 latent, page 64, ctx U[1024,8192]",
                 "sum_context": int(case.context_lens.sum()), "input_sets_rotated": a.rotate,
                 "algorithmic_bytes": int(nbytes), "algorithmic_flops": int(avg(call_flops)),
                 "mfma_tflops_of_call": round(avg(call_flops) / (t.ms_per_step * 1e-3) / 1e12, 1)},
                roof, storage=("e4m3 latent (one power-of-two scale per 64) + bf16 rope, 656 B/token"
                               if fp8 else "bf16"), parity=parity, cpu=cpu)


if __name__ == "__main__":
    sys.exit(main())
