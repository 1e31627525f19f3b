"""Benchmark: hybrid-batch attention microseconds per iteration on one MI355X, and the achieved
fraction of the max(MFMA, HBM) roofline.

    python bench.py [--steps K] [--warmup W] [--workload N] [--mode fused] [--legs 2,3,4]

One step = one pod_attn_run over the whole hybrid batch (host planning, plan upload, prefill
tiles + decode split-KV + combine), inputs resident in HBM.  Prints ONE JSON line.

The measured workload (``value``, ``roofline``) is the largest single-GPU one: Llama-3-8B heads
(32 query / 8 KV heads, head_dim 128, bf16, 16-token pages), one 512-token prefill chunk at
offset 32256 plus 256 decodes at context 32768, over a randomly permuted 2^20-page (64 GiB) pool.
``value`` is the median per-step wall time of exactly K timed steps after a warm-up of W steps
and at least 0.2 s of GPU work.  Beside it:
  * modes: the same workload in the separate and two-stream modes;
  * legs: the Llama-2-7B-, Llama-3-8B- and Yi-6B-shaped workloads, each in every mode, with at
    least 0.1 s of timed steps per mode and the roofline fraction of the median kernel time;
  * kv_append: the step preceded by the KV append of every row's new K/V (pod_attn_run_append);
  * small_q_extend: a speculative-verification step (4-token extends) with the extends on the
    decode path and on the prefill-tile path;
  * fp8_kv: the measured and the Llama-2-7B-shaped workloads with an FP8 E4M3 cache;
  * cpu_baseline: the fp64 oracle on a bounded sample of the measured workload, scaled.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "hybrid-batch attention µs/iter + fraction of max(MFMA,HBM) roofline, 1 GPU"
PEAK_HBM = 8.0e12            # B/s, MI355X
PEAK_MFMA = {"bf16": 2.5e15, "fp32": 157.3e12}   # dense FLOP/s, MI355X


def algorithmic_work(spec):
    """Bytes and FLOPs the method must move / do (not what a kernel happens to do):
    K and V read once per KV head per live context token, q read and out written once, one
    int32 block-table entry per live page (and, for an FP8 cache, its two float scales per KV
    head); 4*D FLOPs per visible (query head, key) pair."""
    eb = spec.elem_bytes
    D, Hq, Hkv = spec.head_dim, spec.num_q_heads, spec.num_kv_heads
    ctx = spec.seq_ctx()
    kv = sum(ctx) * Hkv * D * eb * 2
    qo = spec.total_q * Hq * D * spec.q_elem_bytes * 2
    bt = sum(-(-c // 16) for c in ctx) * (4 + (8 * Hkv if spec.dtype == "fp8" else 0))
    pairs_pf = 0
    for L, c in zip(spec.prefill_q_len, spec.prefill_ctx_len):
        o = c - L
        pairs_pf += L * o + L * (L + 1) // 2
    pairs_dc = sum(spec.decode_ctx_len)
    pairs = Hq * (pairs_pf + pairs_dc)
    return {"bytes": kv + qo + bt, "kv_bytes": kv, "flops": 4 * D * pairs, "pairs": pairs,
            "pairs_prefill": Hq * pairs_pf, "pairs_decode": Hq * pairs_dc}


def _ctx_desc(ctx):
    return f"{ctx[0]}" if len(set(ctx)) == 1 else f"{min(ctx)}..{max(ctx)}, mean {sum(ctx) / len(ctx):.0f}"


def workload_desc(spec):
    if len(spec.prefill_q_len) <= 4:
        pre = ", ".join(f"{L}@{c - L}" for L, c in zip(spec.prefill_q_len, spec.prefill_ctx_len))
    else:                                   # many chunks: one entry per chunk length
        by_len = {}
        for L, c in zip(spec.prefill_q_len, spec.prefill_ctx_len):
            by_len.setdefault(L, []).append(c)
        pre = ", ".join(f"{len(v)}x{L} (ctx {_ctx_desc(v)})" for L, v in sorted(by_len.items(), reverse=True))
    dc = spec.decode_ctx_len
    dec = f"{len(dc)} (ctx {_ctx_desc(dc)})" if dc else "0"
    return {"workload": f"{spec.name}: hybrid batch, prefill chunks [{pre}] + {dec} decodes",
            "heads_q_kv_dim": [spec.num_q_heads, spec.num_kv_heads, spec.head_dim],
            "page_tokens": 16, "pool_pages": spec.num_pages, "pages": "random permutation",
            "dtype": spec.dtype}


WARM_FLOOR_S = 0.2           # untimed GPU work before any timed mode, whatever --warmup says
MIN_TIMED_S = 0.1            # the comparison legs time at least this much GPU work per mode


def time_mode(torch, h, b, meta, out, ws, steps, warmup, new=None, scaled=False, min_timed_s=0.0):
    """Time one handle on one batch.  Untimed warm-up: ``warmup`` runs, then more until at least
    WARM_FLOOR_S of GPU time has run (the first mode timed in a process otherwise meets a GPU
    still coming up from host-side input generation).  Timed: ``steps`` runs (more when
    ``min_timed_s`` asks for a longer window), each bracketed by wall events on the launch stream
    and by the library's one-shot kernel events (pod_attn_set_kernel_events).  Returns the
    per-step wall and kernel times (ms) and the warm-up count.  With new = (k_new, v_new) every
    run first appends those tokens (pod_attn_run_append); scaled runs an FP8 cache with its scales
    (pod_attn_run_scaled)."""
    stream = torch.cuda.current_stream()

    def one():
        if scaled:
            h.run_scaled(b.q, b.k_pool, b.v_pool, b.k_scale, b.v_scale, b.block_tables, meta, out, ws)
        elif new is None:
            h.run(b.q, b.k_pool, b.v_pool, b.block_tables, meta, out, ws)
        else:
            h.run_append(b.q, new[0], new[1], b.k_pool, b.v_pool, b.block_tables, meta, out, ws)

    def batch_ms(n):
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n):
            one()
        z.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(z)

    warm, warm_ms = max(1, warmup), 0.0
    warm_ms += batch_ms(warm)
    while warm_ms < WARM_FLOOR_S * 1e3:
        per = warm_ms / warm
        n = max(1, math.ceil((WARM_FLOOR_S * 1e3 - warm_ms) / per))
        warm_ms += batch_ms(n)
        warm += n
    per = warm_ms / warm
    if min_timed_s > 0:
        steps = max(steps, math.ceil(min_timed_s * 1e3 / per))
    walls = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ks = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, z in ks:             # torch creates the HIP events on first record; the library re-records them
        a.record(stream)
        z.record(stream)
    for e in walls:
        e.record(stream)
    torch.cuda.synchronize()
    walls[0].record(stream)
    for i in range(steps):
        h.set_kernel_events(*ks[i])
        one()
        walls[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = [walls[i].elapsed_time(walls[i + 1]) for i in range(steps)]
    kern = [a.elapsed_time(z) for a, z in ks]
    return {"steps": steps, "warmup_runs": warm, "total_ms": walls[0].elapsed_time(walls[-1]),
            "wall_ms": wall, "kernel_ms": kern}


def summarize(t, t_roof_s=None):
    """Median / mean / min per-step wall and kernel microseconds of a time_mode result, and the
    roofline fraction of the median kernel time when a bound is given."""
    r = {"us_per_iter": round(statistics.median(t["wall_ms"]) * 1e3, 2),
         "us_per_iter_mean": round(t["total_ms"] / t["steps"] * 1e3, 2),
         "kernel_us": round(statistics.median(t["kernel_ms"]) * 1e3, 2),
         "kernel_us_mean": round(statistics.mean(t["kernel_ms"]) * 1e3, 2),
         "kernel_us_min": round(min(t["kernel_ms"]) * 1e3, 2),
         "steps": t["steps"], "timed_ms": round(t["total_ms"], 1)}
    if t_roof_s is not None:
        r["frac"] = round(t_roof_s / (statistics.median(t["kernel_ms"]) / 1e3), 4)
    return r


def measured_peaks(torch, B):
    """This GPU's HBM read rate and dense bf16 MFMA rate, from the library's probes
    (pod_attn_probe_hbm_read over an 8 GiB buffer, pod_attn_probe_mfma): each probe runs untimed
    for at least 0.2 s, then the median of individually timed launches (HIP events on the launch
    stream).  Called before any workload is allocated: measured, an 8 GiB buffer allocated right
    after tens of GiB were returned to the driver reads about 4% slower, warm-up or not."""
    stream = torch.cuda.current_stream()
    nbytes = 8 << 30
    buf = torch.empty(nbytes // 4, dtype=torch.int32, device="cuda")
    isink = torch.empty(B.PROBE_WGS, dtype=torch.int32, device="cuda")
    fsink = torch.empty(4 * B.PROBE_WGS, dtype=torch.float32, device="cuda")
    iters = 2048

    def timed(fn, reps, warm_s=0.2):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < warm_s:
            fn()
            torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, z in ev:
            a.record(stream)
            fn()
            z.record(stream)
        torch.cuda.synchronize()
        return statistics.median(a.elapsed_time(z) for a, z in ev) / 1e3

    t_hbm = timed(lambda: B.probe_hbm_read(buf, isink, stream), 15)
    flops = B.probe_mfma(iters, fsink, stream)
    t_mfma = timed(lambda: B.probe_mfma(iters, fsink, stream), 9)
    del buf
    return {"hbm_read_gbps": round(nbytes / t_hbm / 1e9, 1), "mfma_bf16_tflops": round(flops / t_mfma / 1e12, 1),
            "how": "library probes, median of timed launches after 0.2 s of untimed ones: streaming read of 8 GiB "
                   "in 16 KiB blocks, two in flight per wave; 4096x4 waves x 8 chains of bf16 32x32x16 MFMA"}


def measured_traffic(kernel_name, workload_name):
    """HBM bytes per launch from the committed counter record (FETCH_SIZE + WRITE_SIZE, each
    calibrated on a plain copy), or None when absent or taken on different kernel sources."""
    from hybrid_prefill_decode_paged_amd.profiling import kernel_source_hash
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_name}_{workload_name}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return rec["traffic_bytes_per_dispatch"]


def cpu_baseline(b, budget_s=12.0):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload: whole decode
    sequences (all heads) and blocks of 32 prefill rows (all heads), until about budget_s of
    CPU work; scaled to the full workload by its visible (head, key) pair count."""
    import numpy as np
    import torch
    from oracle import attention as orc

    spec = b.spec

    class Pages:
        def __init__(self, t):
            self.t = t

        def __getitem__(self, idx):
            sel = self.t[torch.as_tensor(np.asarray(idx, dtype=np.int64), device=self.t.device)].cpu()
            return sel.view(torch.int16).numpy() if spec.dtype == "bf16" else sel.numpy()

    q = b.q.cpu()
    qraw = q.view(torch.int16).numpy() if spec.dtype == "bf16" else q.numpy()
    prob = orc.HybridProblem(qraw, Pages(b.k_pool), Pages(b.v_pool), b.block_tables_host, b.prefill_q_start,
                             b.prefill_ctx_len, b.decode_ctx_len, spec.num_q_heads, spec.num_kv_heads,
                             spec.dtype, spec.softmax_scale)
    Hq = spec.num_q_heads
    t_dc = t_pf = 0.0
    pairs_dc = pairs_pf = 0
    n_dc = n_pf_rows = 0
    start = time.perf_counter()
    i = 0
    while i < spec.num_decode and time.perf_counter() - start < budget_s / 2:
        s = spec.num_prefill + i
        t = time.perf_counter()
        prob.sequence_output(s)
        t_dc += time.perf_counter() - t
        pairs_dc += Hq * spec.decode_ctx_len[i]
        n_dc += 1
        i += 1
    start = time.perf_counter()
    for p in range(spec.num_prefill):
        rows = prob.seq_rows(p)
        for a in range(0, len(rows), 32):
            if time.perf_counter() - start >= budget_s / 2:
                break
            blk = rows[a:a + 32]
            t = time.perf_counter()
            prob.rows_output(p, blk)
            t_pf += time.perf_counter() - t
            pairs_pf += Hq * sum(prob.row_info(int(r))[1] + 1 for r in blk)
            n_pf_rows += len(blk)
    w = algorithmic_work(spec)
    est = 0.0
    if pairs_dc:
        est += t_dc / pairs_dc * w["pairs_decode"]
    if pairs_pf:
        est += t_pf / pairs_pf * w["pairs_prefill"]
    threads = os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        nt = [d.get("num_threads", 0) for d in threadpool_info() if d.get("user_api") == "blas"]
        if nt:
            threads = max(nt)
    except Exception:
        pass
    return {"value": round(est * 1e6, 1), "unit": "us/iter", "cores": threads, "kind": "oracle",
            "sample": (f"{n_dc} whole decode sequences + {n_pf_rows} prefill rows, all {Hq} heads "
                       f"({t_dc + t_pf:.1f} s of fp64 numpy incl. page copies to host), "
                       f"scaled by visible (head,key) pairs to the full batch")}


def roofline_of(spec):
    """Algorithmic work of a workload and its max(MFMA, HBM) bound (seconds, bound name)."""
    work = algorithmic_work(spec)
    peak_mfma = PEAK_MFMA["fp32" if spec.dtype == "fp32" else "bf16"]
    t_math, t_mem = work["flops"] / peak_mfma, work["bytes"] / PEAK_HBM
    return work, max(t_math, t_mem), ("hbm" if t_mem >= t_math else "mfma"), peak_mfma


def run_modes(torch, binding, gen, spec, b, modes, steps, warmup, min_timed_s, t_roof_s, say):
    """Time every mode of ``modes`` on one resident batch; returns ({mode: summary}, {mode: stats},
    {mode: raw time_mode result})."""
    meta = binding.BatchMeta.from_batch(b)
    res, stats, raw = {}, {}, {}
    for mode in modes:
        h = binding.PodAttention(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.dtype, mode,
                                 scale=spec.softmax_scale)
        ws = torch.empty(h.workspace_size(meta), dtype=torch.uint8, device="cuda")
        out = torch.empty_like(b.q)
        say(f"timing {spec.name} mode={mode}")
        t = time_mode(torch, h, b, meta, out, ws, steps, warmup, scaled=spec.dtype == "fp8",
                      min_timed_s=min_timed_s)
        res[mode] = summarize(t, t_roof_s)
        res[mode]["warmup_runs"] = t["warmup_runs"]
        stats[mode] = h.stats()
        raw[mode] = t
        del ws, out
        h.close()
    return res, stats, raw


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", type=int, default=5,
                    help="1..5; 5 (Llama-3-8B heads, 512-token chunk + 256 decodes at 32K) is the measured workload")
    ap.add_argument("--mode", default="fused", choices=["fused", "separate", "streams"])
    ap.add_argument("--legs", default="2,3,4",
                    help="other workloads timed in every mode beside the headline ('' for none)")
    ap.add_argument("--no-compare", action="store_true", help="skip timing the other two modes of the headline workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-append", action="store_true", help="skip timing the KV-append variant")
    ap.add_argument("--no-extend", action="store_true", help="skip timing the small-q extend workload")
    ap.add_argument("--no-fp8", action="store_true", help="skip timing the FP8-cache variant")
    ap.add_argument("--no-peaks", action="store_true", help="skip the HBM / MFMA probes")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy 3 times (counter calibration)")
    ap.add_argument("--calibrate-mfma", action="store_true",
                    help="only run the library's dense bf16 MFMA probe 3 times (counter calibration)")
    args = ap.parse_args()
    if args.calibrate_mfma:
        import torch
        from hybrid_prefill_decode_paged_amd import binding
        binding.load()
        sink = torch.empty(4 * binding.PROBE_WGS, dtype=torch.float32, device="cuda")
        for _ in range(3):
            flops = binding.probe_mfma(2048, sink)
        torch.cuda.synchronize()
        print(f"mfma probe 3 x {flops:.4g} FLOP", flush=True)
        return
    if args.calibrate_copy:
        import torch
        x = torch.full((1 << 30,), 3, dtype=torch.uint8, device="cuda")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print("copied 3 x 1 GiB", flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(a hybrid batch would shard by sequence or KV head, one process per GPU, with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from hybrid_prefill_decode_paged_amd import binding
    from hybrid_prefill_decode_paged_amd import inputs as gen

    def say(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    binding.load()
    torch.cuda.set_device(0)
    # the probes run first, before the workloads' tens of GiB are allocated
    peaks = None
    if not args.no_peaks:
        say("measuring this GPU's HBM read and MFMA rates")
        peaks = measured_peaks(torch, binding)
    spec = gen.config_spec(args.workload)
    say(f"generating {spec.name}: {spec.num_pages} pages")
    b = gen.make_batch(spec, "cuda")
    torch.cuda.synchronize()
    work, t_roof_s, bound, peak_mfma = roofline_of(spec)

    # ---- the headline: the asked mode on the measured workload, exactly --steps timed runs
    modes = [args.mode] + ([] if args.no_compare else [m for m in ("fused", "separate", "streams") if m != args.mode])
    results, stats, raw = {}, {}, {}
    for i, mode in enumerate(modes):
        r, st, rw = run_modes(torch, binding, gen, spec, b, [mode], args.steps, args.warmup,
                              0.0 if i == 0 else MIN_TIMED_S, t_roof_s, say)
        results.update(r)
        stats.update(st)
        raw.update(rw)
    head = raw[args.mode]

    # ---- the other workloads, each in every mode, >= MIN_TIMED_S of timed steps per mode
    legs = {}
    for idx in [int(x) for x in args.legs.split(",") if x.strip()]:
        if idx == args.workload:
            continue
        ls = gen.config_spec(idx)
        say(f"generating {ls.name}: {ls.num_pages} pages")
        lb = gen.make_batch(ls, "cuda")
        lw, lroof, lbound, _ = roofline_of(ls)
        r, _, _ = run_modes(torch, binding, gen, ls, lb, ["fused", "separate", "streams"], args.steps,
                            args.warmup, MIN_TIMED_S, lroof, say)
        legs[ls.name] = {"workload": workload_desc(ls)["workload"], "t_roof_us": round(lroof * 1e6, 2),
                         "bound": lbound, "algorithmic_bytes": lw["bytes"], "algorithmic_flops": lw["flops"],
                         "modes": r,
                         "fused_vs_separate": round(r["separate"]["us_per_iter"] / r["fused"]["us_per_iter"], 4)}
        del lb
        torch.cuda.empty_cache()

    append = None
    if not args.no_append:
        # The same step preceded by the KV append of every query row's new K/V (the tokens
        # drawn once; rewriting them each step moves the same bytes).
        k_new, v_new = gen.new_tokens(spec, spec.seed + 7, "cuda")
        meta = binding.BatchMeta.from_batch(b)
        append = {"append_bytes": 2 * 2 * spec.total_q * spec.num_kv_heads * spec.head_dim * spec.elem_bytes}
        for mode in ("fused", "separate"):
            h = binding.PodAttention(spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.dtype, mode,
                                     scale=spec.softmax_scale)
            ws = torch.empty(h.workspace_size(meta), dtype=torch.uint8, device="cuda")
            out = torch.empty_like(b.q)
            say(f"timing mode={mode} with KV append")
            t = time_mode(torch, h, b, meta, out, ws, args.steps, args.warmup, new=(k_new, v_new),
                          min_timed_s=MIN_TIMED_S)
            r = summarize(t, t_roof_s)
            if mode in results:
                r["extra_us_vs_no_append"] = round(r["us_per_iter"] - results[mode]["us_per_iter"], 2)
            r["units"] = h.stats()["num_append_units"]
            append[mode] = r
            del ws, out
            h.close()
        del k_new, v_new

    extend = None
    if not args.no_extend:
        # Small-q extends: a speculative-verification step shaped like the Llama-3-8B workload
        # (128 sequences extending by 4 tokens each, plus its 2048-token chunk), fused mode,
        # with the extends on the decode path (default) and on the prefill-tile path.
        xs = gen.spec_verify_spec(4)
        say(f"generating {xs.name}: {xs.num_pages} pages")
        xb = gen.make_batch(xs, "cuda")
        xmeta = binding.BatchMeta.from_batch(xb)
        _, x_roof, _, _ = roofline_of(xs)
        extend = {"workload": workload_desc(xs)["workload"], "t_roof_us": round(x_roof * 1e6, 2)}
        for name, emax in (("decode_path", 0), ("tile_path", -1)):
            h = binding.PodAttention(xs.num_q_heads, xs.num_kv_heads, xs.head_dim, xs.dtype, "fused",
                                     scale=xs.softmax_scale, extend_max_q=emax)
            ws = torch.empty(h.workspace_size(xmeta), dtype=torch.uint8, device="cuda")
            out = torch.empty_like(xb.q)
            say(f"timing small-q extends on the {name}")
            t = time_mode(torch, h, xb, xmeta, out, ws, args.steps, args.warmup, min_timed_s=MIN_TIMED_S)
            extend[name] = summarize(t, x_roof)
            extend[name]["small_extends"] = h.stats()["num_small_extends"]
            del ws, out
            h.close()
        del xb
        torch.cuda.empty_cache()

    fp8 = None
    if not args.no_fp8 and spec.dtype == "bf16":
        # Workloads with their cache in FP8 E4M3 (per-(page, KV head) scales, bf16 q/out), fused
        # and separate: half the K/V bytes of the decode stream.  The measured workload and the
        # Llama-2-7B-shaped one.
        fp8 = {}
        for idx in sorted({args.workload, 2}):
            fs = gen.fp8_spec(idx)
            say(f"generating {fs.name}: {fs.num_pages} pages")
            fb = gen.make_batch(fs, "cuda")
            fw, f_roof, _, _ = roofline_of(fs)
            r, _, _ = run_modes(torch, binding, gen, fs, fb, ["fused", "separate"], args.steps, args.warmup,
                                MIN_TIMED_S, f_roof, say)
            fp8[fs.name] = {"workload": workload_desc(fs)["workload"], "algorithmic_bytes": fw["bytes"],
                            "t_roof_us": round(f_roof * 1e6, 2), "modes": r}
            del fb
            torch.cuda.empty_cache()

    # ---- roofline of the dominant kernel: algorithmic work / its median launch duration
    kern_s = statistics.median(head["kernel_ms"]) / 1e3
    if bound == "hbm":
        achieved, peak, unit = work["bytes"] / kern_s / 1e9, PEAK_HBM / 1e9, "GB/s"
    else:
        achieved, peak, unit = work["flops"] / kern_s / 1e12, peak_mfma / 1e12, "TFLOP/s"
    st = stats[args.mode]
    kernel_name = "pod_fused_kernel" if args.mode == "fused" else f"{args.mode} kernels"
    traffic = measured_traffic(kernel_name, spec.name)
    if peaks is not None:
        # the dominant kernel's rate against this GPU's own ceiling (context beside frac)
        if bound == "hbm" or spec.dtype != "fp32":
            measured = peaks["hbm_read_gbps"] if bound == "hbm" else peaks["mfma_bf16_tflops"]
            peaks["dominant_kernel_fraction_of_measured"] = round(achieved / measured, 4)
    line = {
        "metric": METRIC,
        "value": round(statistics.median(head["wall_ms"]) * 1e3, 2),
        "unit": "us/iter",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["total_ms"] / head["steps"], 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded N(0,1)*0.5 values, seeded page permutation)",
        "config": workload_desc(spec),
        "value_is": "median per-step wall time of the timed steps (events on the launch stream); "
                    "ms_per_step is their mean",
        "warmup_runs": head["warmup_runs"],
        "roofline": {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel": kernel_name, "kernel_us_median": round(kern_s * 1e6, 2),
                     "algorithmic_bytes": work["bytes"], "algorithmic_flops": work["flops"],
                     "t_roof_us": round(t_roof_s * 1e6, 2),
                     "roof_fraction_of_step": round(t_roof_s / (statistics.median(head["wall_ms"]) / 1e3), 4)},
        "modes": results,
        "fused_vs_separate": (round(results["separate"]["us_per_iter"] / results["fused"]["us_per_iter"], 4)
                              if "separate" in results and "fused" in results else None),
        "legs": legs,
        "kv_append": append,
        "small_q_extend": extend,
        "fp8_kv": fp8,
        "measured_rates": peaks,
        "plan": {k: st[k] for k in ("num_prefill_items", "num_decode_items", "num_combine_groups",
                                    "decode_split_tokens", "prefill_max_splits", "grid_wgs", "wgs_per_cu",
                                    "num_cus", "vgprs_per_lane", "lds_bytes_per_wg", "mode_used", "prefill_wg_budget",
                                    "fallback_reason", "host_plan_us")},
    }
    if not args.no_cpu_baseline:
        say("timing the CPU oracle on a sample")
        line["cpu_baseline"] = cpu_baseline(b, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
