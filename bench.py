"""Benchmark of the absorbed-MLA paged decode on one MI355X.

One step = the whole hot path on one batch: the split-KV decode launch (partials) and
the LSE combine launch, through the C ABI, on inputs already resident in HBM.  The
default workload is the paged FP8 batch B=64, H=128, q_len=1, seq_len uniform in
[1024, 32768], page size 64 (seeded, synthetic).  Prints ONE JSON line on stdout.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

Algorithmic counts (per step): flops = 2 * (576 + 512) * H * sum over requests and
queries of the tokens each query sees; bytes = visible cache rows (576 FP8 bytes per
token) + Q + QPE + O (bf16) + LSE (fp32) + one int32 block-table entry per page read.
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

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
METRIC = "MLA decode KV GB/s + TFLOP/s (% roofline), B=64 H=128 paged fp8"
# what each paged cache format computes in
ARITHMETIC = {
    0: "bf16 MFMA (bf16 query, bf16 weights), fp32 accumulation",
    1: "bf16 query and softmax weights as exact two-term E4M3 splits on FP8 MFMA with the raw FP8 cache, "
       "fp32 accumulation",
    2: "bf16 MFMA on the NVFP4 cache dequantised exactly to bf16, fp32 accumulation",
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


def traffic_from_profiles(workload: str, src_hash: str, kernel: str = "decode_paged"):
    """HBM bytes per decode launch (FETCH_SIZE and WRITE_SIZE, each scaled by what the
    counter reads for a copy kernel of known size) from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kernel}.{workload}.counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_sha") != src_hash:
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(w, budget_s: float):
    """The float64 oracle, as it stands, on requests of the same batch taken in order
    until about budget_s seconds of CPU work."""
    import numpy as np
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
            "sample": f"requests 0..{used - 1} of the same batch ({used} of {w.B}), float64 numpy, {dt:.1f} s"}


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


# Score flops run at the FP8 rate and output flops at the bf16 rate in the FP8-query
# variant (its output product is two FP8 terms, the bf16 rate's time): per (row, token)
# pair 1152 flops at 5.0 PFLOP/s and 1024 at 2.5 PFLOP/s.
MFMA_FP8_PEAK_TFLOPS = 5000.0
MIXED_PEAK_TFLOPS = 2176.0 / (1152.0 / MFMA_FP8_PEAK_TFLOPS + 1024.0 / MFMA_BF16_PEAK_TFLOPS)


def time_fp8_query_variant(mla, torch, w, q, qpe, cache, bt, sl, G, args, flops):
    """The same pages decoded as format 3 (query rounded to E4M3, FP8-MFMA scores): same
    steps, same timing, reported beside the headline (which is the bf16-query path)."""
    call = mla.PagedCall(q, qpe, cache, mla.MLA_KV_FP8_E4M3_QFP8, bt, sl, w.page_size, w.page_stride, w.kv_scale,
                         w.sm_scale, num_splits=G)
    for _ in range(args.warmup):
        call.partials()
        call.combine()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        ev[k][0].record()
        call.partials()
        ev[k][1].record()
        call.combine()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) / args.steps * 1e3
    dec = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    dec_tflops = flops / (dec * 1e-3) / 1e12
    log(f"[bench] fp8-query variant: {ms_step:.4f} ms/step, decode {dec:.4f} ms")
    return {"kv_format": "fp8_e4m3, query rounded to e4m3 (FP8-MFMA scores; output product as on the FP8 path: "
                         "weights split into two E4M3 terms on FP8 MFMA)",
            "ms_per_step": round(ms_step, 5), "value": round(flops / (ms_step * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
            "decode_ms": round(dec, 5),
            "roofline": {"bound": "mfma", "achieved": round(dec_tflops, 3), "peak": round(MIXED_PEAK_TFLOPS, 1),
                         "unit": "TFLOP/s", "frac": round(dec_tflops / MIXED_PEAK_TFLOPS, 4),
                         "peak_note": "score flops at the fp8 peak, output flops at the bf16 peak (two FP8 terms)"}}


def run_contig(args, w, mla, torch, np, gen):
    """Contiguous split-KV decode (bf16 cache, q_len 1): one step is mla_decode_splitkv
    followed by mla_splitkv_combine, with the planner's split (fixed at 128 tokens for the
    tiny workload, as its definition states)."""
    dev = torch.device("cuda:0")
    t16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    q, qpe, kv, kpe = (t16(a) for a in (w.q, w.qpe, w.kv, w.kpe))
    L = gen.WORKLOADS[args.workload].get("kv_len_per_split")
    op, lp, L = mla.decode_splitkv(q, qpe, kv, kpe, w.sm_scale, L)
    o, lse = mla.splitkv_combine(op, lp)
    flops = 2.0 * (576 + 512) * w.H * w.B * w.S
    kvb = 2.0 * 576 * w.B * w.S
    nbytes = kvb + w.B * w.H * (576 * 2 + 512 * 2 + 4)
    for _ in range(args.warmup):
        mla.decode_splitkv(q, qpe, kv, kpe, w.sm_scale, L, o_part=op, lse_part=lp)
        mla.splitkv_combine(op, lp, o=o, lse=lse)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        ev[k][0].record()
        mla.decode_splitkv(q, qpe, kv, kpe, w.sm_scale, L, o_part=op, lse_part=lp)
        ev[k][1].record()
        mla.splitkv_combine(op, lp, o=o, lse=lse)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) / args.steps * 1e3
    dec = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    traffic = traffic_from_profiles(args.workload, kernel_source_hash(), "decode_contig")
    if flops / nbytes >= ridge:
        a = flops / (dec * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(a, 3), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(a / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic}
    else:
        a = nbytes / (dec * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(a / HBM_PEAK_GBPS, 4), "traffic": traffic}
    out = {
        "metric": METRIC, "value": round(flops / (ms_step * 1e-3) / 1e12, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "B": w.B, "H": w.H, "S_kv": w.S, "q_len": 1, "kv_format": "bf16",
                   "kv_len_per_split": L, "num_splits": int(op.shape[2]), "decode_ms": round(dec, 5),
                   "kv_GBps": round(kvb / (ms_step * 1e-3) / 1e9, 1), "kernel_source_sha": kernel_source_hash()},
        "roofline": roof,
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the clocks take a few tens of milliseconds of load to settle (the first ~20 launches
    # run ~20% slower), so the default warm-up is ~0.2 s of steps; the whole run stays < 1 s
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", default="paged_fp8_b64_h128_s1k_32k")
    ap.add_argument("--num-splits", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-variant", action="store_true",
                    help="skip the extra timing of the FP8-query variant on FP8 workloads")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="instead of the decode, run torch's fill and copy kernels on buffers of this many MiB "
                         "(known HBM bytes, used to scale the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this decode path is built and measured on a single MI355X "
              f"(--gpus {args.gpus} was asked for); see the design notes for how it would shard.", file=sys.stderr)
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
    if w.__class__.__name__ != "PagedInputs":
        return run_contig(args, w, mla, torch, np, gen)
    t16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    q, qpe = t16(w.q), t16(w.qpe)
    cache = torch.from_numpy(w.cache).to(dev)
    bt = torch.from_numpy(w.block_tables).to(dev)
    sl = torch.from_numpy(w.seq_lens).to(dev)
    num_cus = mla.device_num_cus(0)
    G = args.num_splits or mla.plan_paged(num_cus, w.B, w.q_len, w.H)
    call = mla.PagedCall(q, qpe, cache, w.fmt, bt, sl, w.page_size, w.page_stride, w.kv_scale, w.sm_scale,
                         num_splits=G)
    flops, nbytes, kvbytes = algorithmic_counts(w)
    log(f"[bench] B={w.B} H={w.H} q_len={w.q_len} tokens={int(w.seq_lens.sum())} num_splits={G} "
        f"flops={flops:.3e} bytes={nbytes:.3e}")

    for _ in range(args.warmup):
        call.partials()
        call.combine()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        ev[k][0].record()
        call.partials()
        ev[k][1].record()
        call.combine()
        ev[k][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec_ms = [e[0].elapsed_time(e[1]) for e in ev]
    comb_ms = [e[1].elapsed_time(e[2]) for e in ev]
    ms_step = wall / args.steps * 1e3
    dec_avg = sum(dec_ms) / len(dec_ms)
    log(f"[bench] timed {args.steps} steps: {ms_step:.4f} ms/step wall, decode {dec_avg:.4f} ms "
        f"(min {min(dec_ms):.4f}, max {max(dec_ms):.4f}), combine {sum(comb_ms) / len(comb_ms):.4f} ms")

    value = flops / (ms_step * 1e-3) / 1e12
    kv_gbps = nbytes / (ms_step * 1e-3) / 1e9
    dec_tflops = flops / (dec_avg * 1e-3) / 1e12
    intensity = flops / nbytes
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    src_hash = kernel_source_hash()
    traffic = traffic_from_profiles(args.workload, src_hash)
    if intensity >= ridge:
        roof = {"bound": "mfma", "achieved": round(dec_tflops, 3), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(dec_tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": traffic}
        if w.fmt == gen.FMT_FP8:
            # the FP8 cache path runs each product as two FP8 MFMA terms (exact E4M3 splits of
            # the bf16 query and of the weights): twice the algorithmic flops at twice the rate
            roof["peak_note"] = ("bf16 dense MFMA peak; the FP8 cache path executes 2x these flops on FP8 MFMA "
                                 "(two-term E4M3 operand splits), the same fraction of the 5.0 PFLOP/s FP8 peak")
    else:
        dec_gbps = nbytes / (dec_avg * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(dec_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(dec_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic}

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "B": w.B, "H": w.H, "q_len": w.q_len, "page_size": w.page_size,
                   "kv_format": gen.FMT_NAMES[w.fmt], "tokens": int(w.seq_lens.sum()), "num_splits": G,
                   "arithmetic": ARITHMETIC[w.fmt],
                   "decode_ms": round(dec_avg, 5), "combine_ms": round(sum(comb_ms) / len(comb_ms), 5),
                   "kv_GBps": round(kv_gbps, 1), "kv_GBps_frac_of_hbm": round(kv_gbps / HBM_PEAK_GBPS, 4),
                   "step_TFLOPs_frac_of_bf16_mfma": round(value / MFMA_BF16_PEAK_TFLOPS, 4),
                   "kernel_source_sha": src_hash},
        "roofline": roof,
    }
    if w.fmt == gen.FMT_FP8 and not args.no_variant:
        out["fp8_query_variant"] = time_fp8_query_variant(mla, torch, w, q, qpe, cache, bt, sl, G, args, flops)
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (oracle, ~{args.cpu_seconds:.0f} s)")
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
