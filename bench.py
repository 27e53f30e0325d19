"""Benchmark of the absorbed-MLA split-KV decode on one MI355X.

One step = the whole hot path on one batch: the split-KV decode launch (partials) and
the LSE combine launch, through the C ABI, on inputs already resident in HBM.  The
default workload is the paged FP8 batch B=64, H=128, q_len=1, seq_len uniform in
[1024, 32768], page size 64 (seeded, synthetic).  Prints ONE JSON line on stdout.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Algorithmic counts (per step): flops = 2 * (576 + 512) * H * sum over requests and
queries of the tokens each query sees; bytes = visible cache rows (576 FP8 bytes per
token) + Q + QPE + O (bf16) + LSE (fp32) + one int32 block-table entry per page read.

Roofline.  The binding roof of the decode kernel is max(bytes / HBM peak, flops / MFMA
peak of the contraction's own operand type): FP8 MFMA (5.0 PFLOP/s) for the FP8 cache,
whose products run on FP8 matrix cores, bf16 MFMA (2.5 PFLOP/s) for the bf16 cache and
f16 MFMA (2.5 PFLOP/s) for the NVFP4 cache, whose exact dequantised values and weights run
on f16 operands.  The fraction is quoted against the published peaks and, beside them, against
ceilings measured in the same run (a stream-read kernel and MFMA loops,
libmla_ceiling.so).

Timing.  Before the warm-up, steps run for --settle-ms of wall time so that the clocks
have settled (the first launches on a fresh GPU run ~20% slower); the settle steps are
reported apart from the warm-up.  The decode and combine launches are bracketed with
HIP events on the launch stream; per-launch decode times go to stderr.  Workloads whose
streamed bytes would fit twice in the 256 MB MALL are flushed between steps by reading
a 1 GiB buffer (a read leaves the caches holding clean lines; a write would leave
dirty ones whose write-back then competes with the decode's own reads); their value and
times then come from the events (the wall clock includes the flush), and their warm
time is reported too.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0                          # MI355X HBM3E, published
PEAK_TFLOPS = {"bf16": 2500.0, "f16": 2500.0, "fp8": 5000.0}   # MI355X dense MFMA, published
MALL_BYTES = 256 << 20
METRIC = "MLA decode KV GB/s + TFLOP/s (% roofline), B=64 H=128 paged fp8"
# operand type of each paged cache format's matrix-core products
CONTRACTION = {0: "bf16", 1: "fp8", 2: "f16", 3: "fp8"}
ARITHMETIC = {
    0: "bf16 MFMA (bf16 query, bf16 weights), fp32 accumulation",
    1: "FP8 MFMA on the raw FP8 cache: the bf16 query as an exact two-term E4M3 split, the softmax weights "
       "(per-row, per-tile power-of-two scale) as two E4M3 terms (~8 significant bits), fp32 accumulation",
    2: "f16 MFMA on the NVFP4 cache dequantised exactly to f16 (the bf16 query as f16 after a per-row "
       "power-of-two scale, the weights in f16), fp32 accumulation",
    3: "FP8 MFMA: query rounded to E4M3, weights as two E4M3 terms, fp32 accumulation",
}
KERNEL_SOURCES = ("mla_split_kv_02_amd/csrc/mla_kernels.hip", "mla_split_kv_02_amd/csrc/mla_internal.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_counts(w):
    import numpy as np
    n = w.seq_lens.astype(np.int64)
    vis = sum(np.maximum(n - w.q_len + i + 1, 0) for i in range(w.q_len))  # per request
    flops = 2.0 * (576 + 512) * w.H * float(vis.sum())
    from workloads.gen import row_bytes
    kv = float(n.sum()) * row_bytes(w.fmt)
    rows = w.B * w.q_len * w.H
    qbytes = rows * (512 + 64) * 2
    obytes = rows * 512 * 2 + rows * 4
    tbytes = 4.0 * float(((n + w.page_size - 1) // w.page_size).sum())
    return flops, kv + qbytes + obytes + tbytes, kv


def traffic_from_profiles(workload: str, src_hash: str, kernel: str = "decode_paged", variant: str | None = None):
    """HBM bytes per decode launch (FETCH_SIZE and WRITE_SIZE, each scaled by what the
    counter reads for a copy kernel of known size) from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None.  variant: the name
    of another decode kernel the same profiled runs launched (the benchmark's variants)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}.{workload}.counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_sha") != src_hash:
        return None
    if variant is not None:
        return d.get("variant_hbm_bytes_per_launch", {}).get(variant)
    return d.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s: float):
    """The float64 oracle, as it stands, on requests of the same batch taken in order
    until about budget_s seconds of CPU work."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    q, qpe = w.q_f64()
    done_flops, used, t0 = 0.0, 0, time.perf_counter()
    for b in range(w.B):
        if time.perf_counter() - t0 > budget_s and used > 0:
            break
        oracle.paged_decode_request(q[b], qpe[b], w.cache, w.fmt, w.kv_scale, w.page_size, w.page_stride,
                                    w.block_tables[b], int(w.seq_lens[b]), w.sm_scale)
        n = int(w.seq_lens[b])
        done_flops += 2.0 * (576 + 512) * w.H * sum(max(n - w.q_len + i + 1, 0) for i in range(w.q_len))
        used += 1
    dt = time.perf_counter() - t0
    return {"value": round(done_flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"requests 0..{used - 1} of the same batch ({used} of {w.B}), float64 numpy, {dt:.1f} s",
            "cpu_model": cpu_model()}


def copy_calibration(torch, dev, nbytes: int, steps: int):
    """Known-traffic kernels for the HBM counters: fill writes nbytes, copy reads nbytes
    and writes nbytes.  Buffers are far larger than the last-level caches."""
    x = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    for _ in range(steps):
        x.fill_(7)
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "steps": steps}), flush=True)


def measure_ceilings(torch, dev):
    """On-box ceilings: a 2 GiB stream read (GB/s) and MFMA loops, bf16 and FP8
    (TFLOP/s), each the median of several launches timed with events."""
    import numpy as np
    from mla_split_kv_02_amd import ceiling

    def timed(fn, reps):
        st = torch.cuda.current_stream(dev)
        fn()  # warm
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(st)
            fn()
            b.record(st)
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return float(np.median(ts))

    nbytes = 2 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(3)
    blocks = 256 * 8
    out = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
    t_read = timed(lambda: ceiling.stream_read(buf, out, blocks), 7)
    del buf
    res = {"hbm_stream_read_GBps": round(nbytes / t_read / 1e9, 1)}
    mb = 1024  # 4 wavefronts per SIMD
    mout = torch.empty(mb * 4, dtype=torch.float32, device=dev)
    for name, kind, iters in (("bf16", ceiling.MFMA_BF16, 2000), ("f16", ceiling.MFMA_F16, 2000),
                              ("fp8", ceiling.MFMA_FP8, 1000)):
        flops = mb * 4 * iters * 4 * ceiling.lib().mla_ceiling_mfma_flops(kind)
        t = timed(lambda: ceiling.mfma(kind, iters, mout, mb), 5)
        res[f"mfma_{name}_TFLOPs"] = round(flops / t / 1e12, 1)
    # the clock the MFMA loop implies (published peaks assume 2.4 GHz)
    res["mfma_clock_GHz"] = round(res["mfma_bf16_TFLOPs"] / PEAK_TFLOPS["bf16"] * 2.4, 3)
    torch.cuda.synchronize()
    return res


def roofline(flops, nbytes, t_ms, contraction, ceilings, traffic):
    """Fraction of the binding roof for a kernel of `flops` / `nbytes` taking t_ms."""
    peak = PEAK_TFLOPS[contraction]
    t_hbm = nbytes / (HBM_PEAK_GBPS * 1e9)
    t_mfma = flops / (peak * 1e12)
    if t_hbm >= t_mfma:
        a = nbytes / (t_ms * 1e-3) / 1e9
        r = {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
             "frac": round(a / HBM_PEAK_GBPS, 4), "traffic": traffic, "contraction": contraction}
        m = ceilings.get("hbm_stream_read_GBps") if ceilings else None
    else:
        a = flops / (t_ms * 1e-3) / 1e12
        r = {"bound": "mfma", "achieved": round(a, 3), "peak": peak, "unit": "TFLOP/s",
             "frac": round(a / peak, 4), "traffic": traffic, "contraction": contraction}
        m = ceilings.get(f"mfma_{contraction}_TFLOPs") if ceilings else None
    r["roof_us"] = round(max(t_hbm, t_mfma) * 1e6, 2)
    r["algorithmic_bytes"] = int(nbytes)
    r["algorithmic_flops"] = float(flops)
    if m:
        r["measured_peak"] = m
        r["frac_of_measured"] = round(a / m, 4)
    return r


def settle(step, torch, ms: float):
    """Run steps for about `ms` of wall time (clocks settle); returns (steps, ms)."""
    t0, n = time.perf_counter(), 0
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(10):
            step()
            n += 1
        torch.cuda.synchronize()
    return n, round((time.perf_counter() - t0) * 1e3, 1)


def timed_steps(torch, steps, decode, combine, flush_buf=None):
    """K steps with events around each launch; returns (wall_s, decode_ms[], combine_ms[]).
    Without a flush, consecutive steps share their boundary event (two event records per
    step: each record between two launches adds a few microseconds to the stream); with
    one, each step has its own three, so the flush stays outside the timed launches."""
    E = lambda: torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if flush_buf is None:
        ev = [E() for _ in range(2 * steps + 1)]
        ev[0].record()
        for k in range(steps):
            decode()
            ev[2 * k + 1].record()
            combine()
            ev[2 * k + 2].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return (wall, [ev[2 * k].elapsed_time(ev[2 * k + 1]) for k in range(steps)],
                [ev[2 * k + 1].elapsed_time(ev[2 * k + 2]) for k in range(steps)])
    ev = [[E() for _ in range(3)] for _ in range(steps)]
    for k in range(steps):
        flush_buf[1].copy_(flush_buf[0].max())  # reads the whole buffer
        ev[k][0].record()
        decode()
        ev[k][1].record()
        combine()
        ev[k][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [e[0].elapsed_time(e[1]) for e in ev], [e[1].elapsed_time(e[2]) for e in ev]


def log_launches(name, ts):
    import numpy as np
    t = np.array(ts)
    log(f"[bench] {name} per launch (ms): min {t.min():.4f} p10 {np.percentile(t, 10):.4f} median "
        f"{np.median(t):.4f} p90 {np.percentile(t, 90):.4f} max {t.max():.4f}; first "
        f"{', '.join(f'{x:.4f}' for x in t[:5])}; last {', '.join(f'{x:.4f}' for x in t[-3:])}")


def run(args, w, mla, torch, np, gen):
    dev = torch.device("cuda:0")
    t16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    paged = w.__class__.__name__ == "PagedInputs"
    if paged:
        q, qpe = t16(w.q), t16(w.qpe)
        cache = torch.from_numpy(w.cache).to(dev)
        bt = torch.from_numpy(w.block_tables).to(dev)
        sl = torch.from_numpy(w.seq_lens).to(dev)
        G = args.num_splits or mla.plan_paged(mla.device_num_cus(0), w.B, w.q_len, w.H)
        call = mla.PagedCall(q, qpe, cache, w.fmt, bt, sl, w.page_size, w.page_stride, w.kv_scale, w.sm_scale,
                             num_splits=G)
        decode, combine = call.partials, call.combine
        flops, nbytes, kvbytes = algorithmic_counts(w)
        fmt = w.fmt
        cfg = {"workload": args.workload, "B": w.B, "H": w.H, "q_len": w.q_len, "page_size": w.page_size,
               "kv_format": gen.FMT_NAMES[w.fmt], "tokens": int(w.seq_lens.sum()), "num_splits": G}
        log(f"[bench] B={w.B} H={w.H} q_len={w.q_len} tokens={int(w.seq_lens.sum())} num_splits={G} "
            f"flops={flops:.3e} bytes={nbytes:.3e}")
    else:
        q, qpe, kv, kpe = (t16(a) for a in (w.q, w.qpe, w.kv, w.kpe))
        L = gen.WORKLOADS[args.workload].get("kv_len_per_split")
        op, lp, L = mla.decode_splitkv(q, qpe, kv, kpe, w.sm_scale, L)
        o, lse = mla.splitkv_combine(op, lp)
        decode = lambda: mla.decode_splitkv(q, qpe, kv, kpe, w.sm_scale, L, o_part=op, lse_part=lp)
        combine = lambda: mla.splitkv_combine(op, lp, o=o, lse=lse)
        flops = 2.0 * (576 + 512) * w.H * w.B * w.S
        kvbytes = 2.0 * 576 * w.B * w.S
        nbytes = kvbytes + w.B * w.H * (576 * 2 + 512 * 2 + 4)
        fmt = 0
        cfg = {"workload": args.workload, "B": w.B, "H": w.H, "S_kv": w.S, "q_len": 1, "kv_format": "bf16",
               "kv_len_per_split": L, "num_splits": int(op.shape[2])}
    step = lambda: (decode(), combine())
    flush = {"on": True, "off": False}.get(args.flush, kvbytes < 2 * MALL_BYTES)
    # [0]: 1 GiB read before each timed step, [1]: where the read's result goes
    flush_buf = (torch.ones(1 << 28, dtype=torch.int32, device=dev), torch.zeros((), dtype=torch.int32, device=dev)) \
        if flush else None

    n_settle, settle_ms = settle(step, torch, args.settle_ms)
    log(f"[bench] settle: {n_settle} steps in {settle_ms} ms")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")

    wall, dec_ms, comb_ms = timed_steps(torch, args.steps, decode, combine, flush_buf)
    dec = float(np.mean(dec_ms))
    comb = float(np.mean(comb_ms))
    log_launches("decode", dec_ms)
    log(f"[bench] timed {args.steps} steps: {wall / args.steps * 1e3:.4f} ms/step wall"
        f"{' (incl. flush)' if flush else ''}, decode {dec:.4f} ms, combine {comb:.4f} ms")
    if flush:
        # value from the launches themselves: the wall clock includes the flush writes
        ms_step = dec + comb
        _, wdec, wcomb = timed_steps(torch, args.steps, decode, combine, None)
        cfg["warm_decode_ms"] = round(float(np.mean(wdec)), 5)
        cfg["warm_combine_ms"] = round(float(np.mean(wcomb)), 5)
        cfg["value_from"] = "hip events (decode + combine), L2/MALL flushed (1 GiB read) before each step"
    else:
        ms_step = wall / args.steps * 1e3
        cfg["value_from"] = "wall clock over the timed steps"

    ceilings = {}
    if not args.no_ceilings:
        ceilings = measure_ceilings(torch, dev)
        log(f"[bench] ceilings: {ceilings}")
    contraction = CONTRACTION[fmt]
    src_hash = kernel_source_hash()
    traffic = traffic_from_profiles(args.workload, src_hash, "decode_paged" if paged else "decode_contig")
    roof = roofline(flops, nbytes, dec, contraction, ceilings, traffic)

    value = flops / (ms_step * 1e-3) / 1e12
    cfg.update({"arithmetic": ARITHMETIC[fmt], "decode_ms": round(dec, 5), "combine_ms": round(comb, 5),
                "decode_ms_median": round(float(np.median(dec_ms)), 5),
                "kv_GBps": round(nbytes / (ms_step * 1e-3) / 1e9, 1),
                "settle": {"steps": n_settle, "ms": settle_ms}, "flush_between_steps": flush,
                "kernel_source_sha": src_hash})
    if fmt == 1:
        # the split path runs each product as two FP8 MFMA terms: twice the algorithmic
        # flops on FP8 matrix cores, i.e. the matrix-core time of a bf16 contraction
        a = flops / (dec * 1e-3) / 1e12
        roof["bf16_rate_view"] = {"achieved_TFLOPs": round(a, 3), "peak": PEAK_TFLOPS["bf16"],
                                  "frac": round(a / PEAK_TFLOPS["bf16"], 4),
                                  "note": "algorithmic flops against the bf16 MFMA peak: the rate the two-term "
                                          "FP8 products execute at"}
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": contraction, "data": "synthetic", "config": cfg, "roofline": roof,
    }
    if ceilings:
        out["ceilings"] = ceilings
    if paged and fmt == gen.FMT_FP8 and not args.no_variant:
        out["fp8_query_variant"] = time_fp8_query_variant(mla, torch, np, w, q, qpe, cache, bt, sl, G, args, flops,
                                                          nbytes, ceilings)
    if paged and not args.no_variant:
        out["fixed_splits_variant"] = time_fixed_splits(mla, torch, np, w, q, qpe, cache, bt, sl, args, flops, nbytes,
                                                        ceilings, flush_buf)
    if paged and not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (oracle, ~{args.cpu_seconds:.0f} s)")
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def time_fp8_query_variant(mla, torch, np, w, q, qpe, cache, bt, sl, G, args, flops, nbytes, ceilings):
    """The same pages decoded as format 3 (query rounded to E4M3, FP8-MFMA scores): same
    steps, same timing, reported beside the headline (which keeps the bf16 query)."""
    call = mla.PagedCall(q, qpe, cache, mla.MLA_KV_FP8_E4M3_QFP8, bt, sl, w.page_size, w.page_stride, w.kv_scale,
                         w.sm_scale, num_splits=G)
    for _ in range(max(args.warmup, 20)):
        call.partials()
        call.combine()
    wall, dec_ms, _ = timed_steps(torch, args.steps, call.partials, call.combine)
    ms_step = wall / args.steps * 1e3
    dec = float(np.mean(dec_ms))
    log(f"[bench] fp8-query variant: {ms_step:.4f} ms/step, decode {dec:.4f} ms")
    return {"kv_format": "fp8_e4m3, query rounded to e4m3", "arithmetic": ARITHMETIC[3],
            "ms_per_step": round(ms_step, 5), "value": round(flops / (ms_step * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
            "decode_ms": round(dec, 5),
            "roofline": roofline(flops, nbytes, dec, "fp8", ceilings,
                                 traffic_from_profiles(args.workload, kernel_source_hash(), "decode_paged",
                                                       f"decode_paged_kernel<{mla.MLA_KV_FP8_E4M3_QFP8}>"))}


def time_fixed_splits(mla, torch, np, w, q, qpe, cache, bt, sl, args, flops, nbytes, ceilings, flush_buf):
    """The same pages through the fixed-length split interface (mla_plan_paged_splits on the
    host lengths, then mla_paged_decode_splits): every split covers kv_len_per_split tokens,
    so the longest request sets the time.  Same flush and event timing as the headline."""
    dev = q.device
    L, _ = mla.plan_paged_splits(mla.device_num_cus(0), w.B, w.q_len, w.seq_lens.tolist(), w.page_size)
    ns = -(-w.max_blocks * w.page_size // L)
    ws = torch.empty(mla.paged_splits_workspace_bytes(w.B, w.q_len, w.H, ns), dtype=torch.uint8, device=dev)
    o = torch.empty((w.B, w.q_len, w.H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.B, w.q_len, w.H), dtype=torch.float32, device=dev)
    run = lambda: mla.paged_decode_splits(q, qpe, cache, w.fmt, bt, sl, w.page_size, w.page_stride, w.kv_scale,
                                          w.sm_scale, kv_len_per_split=L, max_splits=ns, workspace=ws, o=o, lse=lse)
    for _ in range(max(args.warmup, 20)):
        run()
    _, ms, _ = timed_steps(torch, args.steps, run, lambda: None, flush_buf)
    t = float(np.mean(ms))
    log(f"[bench] fixed splits (L={L}, {ns} splits): decode + combine {t:.4f} ms")
    return {"kv_len_per_split": L, "max_splits": ns, "ms_per_step": round(t, 5),
            "value": round(flops / (t * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
            "value_from": "hip events around both launches" + (", caches flushed before each step" if flush_buf
                                                               is not None else "")}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="wall time of untimed steps before the warm-up, for the clocks to settle")
    ap.add_argument("--workload", default="paged_fp8_b64_h128_s1k_32k")
    ap.add_argument("--num-splits", type=int, default=None)
    ap.add_argument("--flush", choices=("auto", "on", "off"), default="auto",
                    help="read 1 GiB between timed steps (auto: when the cache would fit twice in the MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-variant", action="store_true",
                    help="skip the extra timings (FP8-query variant on FP8 workloads; fixed-length splits)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="instead of the decode, run torch's fill and copy kernels on buffers of this many MiB "
                         "(known HBM bytes, used to scale the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this decode path is built and measured on a single MI355X "
              f"(--gpus {args.gpus} was asked for); a multi-GPU decode would split the requests' token "
              f"ranges across GPUs and merge their partials with the same LSE combine, which is not built.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mla_split_kv_02_amd as mla
    from workloads import gen

    dev = torch.device("cuda:0")
    if args.copy_calibration_mib:
        copy_calibration(torch, dev, args.copy_calibration_mib << 20, args.steps)
        return
    log(f"[bench] generating {args.workload}")
    w = gen.make_workload(args.workload)
    run(args, w, mla, torch, np, gen)


if __name__ == "__main__":
    main()
