#!/usr/bin/env python3
"""MLA decode benchmark on one MI355X.

A step is one pass of the whole decode hot path over one batch: mla_decode
(page walk, HBM->LDS latent tiles, score MFMAs, online softmax, output MFMAs,
split epilogue) followed by mla_combine (LSE merge).  Inputs are seeded and
synthetic and already resident in HBM when the timed region starts; the
latent cache and queries are rotated over enough copies that the 256 MB
Infinity Cache cannot serve them from one step to the next.

Prints one JSON line (see --help).  --gpus above 1 is refused: this build
runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
MALL_BYTES = 256 << 20
FLOP_PER_QROW_ROW = 2 * 128 * 576 + 2 * 128 * 512   # scores + output per (query token, cache row)
DEFAULT_WORKLOAD = "batched_b32_l1k_4k"


def row_bytes(cache_dtype: str) -> int:
    # bf16: 576 x 2 B; fp8: 512 B e4m3 + 4 fp32 scales + 64 bf16 rope values
    return 1152 if cache_dtype == "bf16" else 512 + 16 + 128


def algorithmic_work(inp):
    """Bytes the method must move and MFMA flops it must do for one step."""
    lens = inp.seq_lens.to(dtype=__import__("torch").int64)
    rows = int(lens.sum())
    qrows = inp.batch * inp.s_q * 128
    nbytes = rows * row_bytes(inp.cache_dtype) + qrows * 576 * 2 + qrows * (512 + 1) * 4
    nbytes += inp.batch * 4 + (0 if inp.block_table is None else inp.block_table.numel() * 4)
    vis = 0
    for s in range(inp.s_q):
        vis += int((lens - inp.s_q + s + 1).clamp(min=0).sum())
    flops = vis * FLOP_PER_QROW_ROW
    return rows, nbytes, flops


def measured_traffic(workload: str):
    """HBM bytes per decode launch from the committed rocprofv3 FETCH_SIZE and
    WRITE_SIZE passes (profiles/decode_traffic.json, scaled by the copy
    calibration), or None when they were taken on other kernels (the SHA-256
    of both kernels' generated assembly differs) or not for this workload."""
    path = os.path.join(ROOT, "profiles", "decode_traffic.json")
    try:
        rec = json.load(open(path))
        sha = kernels_sha256()
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sha256") != sha or workload not in rec.get("workloads", {}):
        return None
    return rec["workloads"][workload]["bytes"]


def kernels_sha256() -> str:
    """SHA-256 of the assembly the generator emits for the bf16 and the e4m3
    decode kernels (what the library embeds)."""
    import hashlib
    import importlib.util
    gen = os.path.join(ROOT, "mla_latent_kv_39_amd", "csrc", "gen_decode_gfx950.py")
    spec = importlib.util.spec_from_file_location("_gen_decode_for_sha", gen)
    g = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(g)
    return hashlib.sha256((g.kernel(False) + g.kernel(True)).encode()).hexdigest()


def cpu_baseline(inp, budget_s: float):
    """The fp64 oracle on a bounded sample of the same workload: whole
    sequences in order (repeating the batch if it ends first) until about
    budget_s seconds of CPU work."""
    from oracle import mla_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    O.decode_one(inp, 0, 0, heads=list(range(8)))  # warm-up
    t0 = time.perf_counter()
    rows = 0
    done = 0
    while time.perf_counter() - t0 <= budget_s:
        b = done % inp.batch
        for s in range(inp.s_q):
            O.decode_one(inp, b, s)
        rows += int(inp.seq_lens[b])
        done += 1
    dt = time.perf_counter() - t0
    passes = f", {done / inp.batch:.1f} passes over the batch" if done > inp.batch else ""
    return {"value": rows / dt, "unit": "cache-tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{min(done, inp.batch)} of {inp.batch} sequences{passes} ({rows} cache rows, all heads "
                      f"and query tokens), {dt:.1f} s, numpy fp64 on the host"}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--num-splits", type=int, default=0, help="0: the library's hint")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (20 times), to scale HBM counters")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU layout is "
              "described, not built", file=sys.stderr)
        return 2

    import torch
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(20):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": 20}))
        return 0
    import mla_latent_kv_39_amd as mla
    from mla_latent_kv_39_amd.runner import DecodeWorkspace
    from mla_inputs import make_inputs

    print(f"[bench] generating {args.workload} (seed {args.seed})", file=sys.stderr, flush=True)
    inp = make_inputs(args.workload, seed=args.seed)
    rows, nbytes, flops = algorithmic_work(inp)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    # the partition count only changes how the work is cut (the merge is exact): fill the GPU
    splits = args.num_splits or mla.mla_num_splits_hint(0, inp.batch, inp.s_q, inp.max_blocks)

    # rotate enough copies of cache + queries that the MALL cannot hold them across steps
    footprint = inp.cache.numel() * inp.cache.element_size() + inp.q_absorbed.numel() * 2 + inp.q_rope.numel() * 2
    if inp.cache_scales is not None:
        footprint += inp.cache_scales.numel() * 4 + inp.cache_rope.numel() * 2
    copies = 1 if footprint > 2 * MALL_BYTES else int(math.ceil((1 << 30) / footprint)) + 1
    print(f"[bench] rows={rows} bytes={nbytes/1e6:.1f}MB flops={flops/1e9:.1f}G splits={splits} copies={copies}",
          file=sys.stderr, flush=True)
    sets = []
    for _ in range(copies):
        if inp.cache_dtype == "bf16":
            cache = mla.LatentCache(mla.MLA_CACHE_BF16, inp.cache.to(dev))
        else:
            cache = mla.LatentCache(mla.MLA_CACHE_FP8_E4M3, inp.cache.to(dev), inp.cache_scales.to(dev),
                                    inp.cache_rope.to(dev))
        sets.append((inp.q_absorbed.to(dev), inp.q_rope.to(dev), cache))
    seq_lens = inp.seq_lens.to(dev)
    table = None if inp.block_table is None else inp.block_table.to(dev)
    ws = DecodeWorkspace(inp.batch, inp.s_q, splits, device=dev)
    stream = torch.cuda.current_stream()

    def decode(i):
        qa, qr, cache = sets[i % copies]
        mla.mla_decode(qa, qr, cache, table, seq_lens, inp.scale, splits, ws.partial_out, ws.partial_lse,
                       ws.out, ws.lse, max_blocks_per_seq=inp.max_blocks, stream=stream)

    def step(i):
        decode(i)
        mla.mla_combine(ws.partial_out, ws.partial_lse, seq_lens, splits, ws.out, ws.lse, stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # whole steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps
    # the dominant kernel alone, same launches back to back
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for i in range(args.steps):
        decode(i)
    k1.record(stream)
    torch.cuda.synchronize()
    ms_decode = k0.elapsed_time(k1) / args.steps
    print(f"[bench] step {ms_step*1e3:.1f} us, decode kernel {ms_decode*1e3:.1f} us", file=sys.stderr, flush=True)

    value = rows / (ms_step * 1e-3)
    intensity = flops / nbytes
    bound = "hbm" if intensity < (MFMA_BF16_PEAK_TFLOPS * 1e12) / (HBM_PEAK_GBS * 1e9) else "mfma"
    if bound == "hbm":
        achieved = nbytes / (ms_decode * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None}
    else:
        achieved = flops / (ms_decode * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None}

    roof["traffic"] = measured_traffic(args.workload)
    result = {
        "metric": "MLA decode cache-tokens/s and achieved HBM GB/s (% of roofline), 1 MI355X",
        "value": round(value, 1), "unit": "cache-tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": inp.batch, "s_q": inp.s_q, "cache_rows": rows,
                   "layout": "contiguous" if inp.block_table is None else "paged64",
                   "cache_dtype": inp.cache_dtype, "num_splits": splits, "rotated_copies": copies,
                   "step_gbs": round(nbytes / (ms_step * 1e-3) / 1e9, 1),
                   "decode_kernel_us": round(ms_decode * 1e3, 2),
                   "algorithmic_bytes": nbytes, "mfma_flops": flops},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
