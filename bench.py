#!/usr/bin/env python3
"""MLA decode benchmark on one MI355X.

A step is one pass of the whole decode hot path over one batch: mla_decode
(page walk, HBM->LDS latent tiles, score MFMAs, online softmax, output MFMAs,
split epilogue) followed by mla_combine (LSE merge).  Inputs are seeded and
synthetic and already resident in HBM when the timed region starts; the
latent cache and queries are rotated over enough copies that the 256 MB
Infinity Cache cannot serve them from one step to the next.

The headline workload (default: the MTP batch, B=128 with two query tokens
over 4096..8192 cached rows, the largest of the five) gives `value`; every
other workload is timed the same way in the same run and reported under
config.workloads, so that one run measures all five.

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

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
MALL_BYTES = 256 << 20
FLOP_PER_QROW_ROW = 2 * 128 * 576 + 2 * 128 * 512   # scores + output per (query token, cache row)
DEFAULT_WORKLOAD = "mtp_b128_sq2_l4k_8k"
ALL_WORKLOADS = ("single_b1_l128", "batched_b32_l1k_4k", "paged_b64_l256_32k", "mtp_b128_sq2_l4k_8k",
                 "fp8_b4_l128k")


def row_bytes(cache_dtype: str) -> int:
    # bf16: 576 x 2 B; fp8: 512 B e4m3 + 4 fp32 scales + 64 bf16 rope values
    return 1152 if cache_dtype == "bf16" else 512 + 16 + 128


def algorithmic_work(inp):
    """Bytes the method must move and MFMA flops it must do for one step."""
    import torch
    lens = inp.seq_lens.to(dtype=torch.int64)
    rows = int(lens.sum())
    qrows = inp.batch * inp.s_q * 128
    nbytes = rows * row_bytes(inp.cache_dtype) + qrows * 576 * 2 + qrows * (512 + 1) * 4
    nbytes += inp.batch * 4 + (0 if inp.block_table is None else inp.block_table.numel() * 4)
    vis = 0
    for s in range(inp.s_q):
        vis += int((lens - inp.s_q + s + 1).clamp(min=0).sum())
    flops = vis * FLOP_PER_QROW_ROW
    return rows, nbytes, flops


def binding_bound(nbytes, flops):
    intensity = flops / nbytes
    return "hbm" if intensity < (MFMA_BF16_PEAK_TFLOPS * 1e12) / (HBM_PEAK_GBS * 1e9) else "mfma"


def roofline_frac(bound, nbytes, flops, seconds):
    if bound == "hbm":
        return nbytes / seconds / 1e9 / HBM_PEAK_GBS
    return flops / seconds / 1e12 / MFMA_BF16_PEAK_TFLOPS


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


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


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
            "cpu_model": cpu_model(),
            "sample": f"{min(done, inp.batch)} of {inp.batch} sequences{passes} ({rows} cache rows, all heads "
                      f"and query tokens), {dt:.1f} s, numpy fp64 on the host"}


def measure(workload: str, steps: int, warmup: int, num_splits: int = 0, seed: int = 0, min_warm_s: float = 0.0):
    """Time `steps` decode steps (decode + combine) and `steps` decode
    launches alone on one stream with HIP events; returns a dict.  The
    untimed warm-up runs `warmup` steps, and then more until `min_warm_s`
    seconds have passed on the GPU (short steps need more than a hundred to
    leave the slow first milliseconds behind)."""
    import torch

    import mla_latent_kv_39_amd as mla
    from mla_latent_kv_39_amd.runner import DecodeWorkspace
    from mla_inputs import make_inputs

    print(f"[bench] generating {workload} (seed {seed})", file=sys.stderr, flush=True)
    inp = make_inputs(workload, seed=seed)
    rows, nbytes, flops = algorithmic_work(inp)
    dev = torch.device("cuda", 0)
    # the partition count only changes how the work is cut (the merge is exact):
    # the workload's own, else the library's hint that fills the GPU
    splits = num_splits or inp.num_splits or mla.mla_num_splits_hint(0, inp.batch, inp.s_q, inp.max_blocks)

    # rotate enough copies of cache + queries that the MALL cannot hold them across steps
    footprint = inp.cache.numel() * inp.cache.element_size() + inp.q_absorbed.numel() * 2 + inp.q_rope.numel() * 2
    if inp.cache_scales is not None:
        footprint += inp.cache_scales.numel() * 4 + inp.cache_rope.numel() * 2
    copies = 1 if footprint > 2 * MALL_BYTES else int(math.ceil((1 << 30) / footprint)) + 1
    print(f"[bench] {workload}: rows={rows} bytes={nbytes/1e6:.1f}MB flops={flops/1e9:.1f}G splits={splits} "
          f"copies={copies}", file=sys.stderr, flush=True)
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

    # one prepared step per rotated copy: descriptors built once, so the host
    # launches faster than a short step runs
    prepared = [mla.PreparedStep(qa, qr, cache, table, seq_lens, inp.scale, ws.out, ws.lse, ws.partial_out,
                                 ws.partial_lse) for qa, qr, cache in sets]
    handle = int(stream.cuda_stream)

    def decode(i):
        prepared[i % copies].decode(handle)

    def step(i):
        prepared[i % copies](handle)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < min_warm_s:
        for i in range(50):
            step(i)
        torch.cuda.synchronize()
    # whole steps back to back, bracketed by two events on the stream the
    # kernels run on: the timed region
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    for i in range(steps):
        step(i)
    s1.record(stream)
    torch.cuda.synchronize()
    ms_step = s0.elapsed_time(s1) / steps
    # the spread of single steps (p10 / p50 / p90) from a second pass with an
    # event between every two steps; each event adds ~2-3 us to a step, so
    # these run above ms_step on short steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record(stream)
    for i in range(steps):
        step(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
    pct = {f"p{q}": per_step[min(steps - 1, (q * steps) // 100)] for q in (10, 50, 90)}
    # the dominant kernel alone, same launches back to back
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record(stream)
    for i in range(steps):
        decode(i)
    k1.record(stream)
    torch.cuda.synchronize()
    ms_decode = k0.elapsed_time(k1) / steps
    del sets, ws, prepared
    torch.cuda.empty_cache()
    bound = binding_bound(nbytes, flops)
    res = {"workload": workload, "inp": inp, "rows": rows, "bytes": nbytes, "flops": flops, "splits": splits,
           "copies": copies, "ms_step": ms_step, "ms_decode": ms_decode, "bound": bound, "step_pct": pct,
           "frac_decode": roofline_frac(bound, nbytes, flops, ms_decode * 1e-3),
           "frac_step": roofline_frac(bound, nbytes, flops, ms_step * 1e-3)}
    print(f"[bench] {workload}: step {ms_step*1e3:.1f} us, decode kernel {ms_decode*1e3:.1f} us, "
          f"{bound}-bound fraction {res['frac_decode']:.3f} (decode) {res['frac_step']:.3f} (step)",
          file=sys.stderr, flush=True)
    return res


def copy_bandwidth(mib: int = 1024, reps: int = 20) -> float:
    """GB/s of a plain device-to-device copy of `mib` MiB (bytes read plus
    bytes written per second): the HBM rate a streaming kernel can reach."""
    import torch
    n = mib << 20
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return round(gbs, 1)


def measure_next_rows(batch: int, s_q: int, steps: int, warmup: int, hidden: int = 7168, seed: int = 0):
    """Time the steps around the decode for one decode step of `batch`
    sequences x `s_q` tokens (query absorption + RoPE, output absorption,
    KV projection of the new tokens, cache append), each alone with HIP events
    on the launch stream, inputs rotated past the Infinity Cache.  All four
    are bound by HBM bytes (intensity well under the ridge)."""
    import torch

    import mla_latent_kv_39_amd as mla
    from mla_latent_kv_39_amd.runner import DecodeWorkspace  # noqa: F401
    g = torch.Generator().manual_seed(seed)
    dev = torch.device("cuda", 0)
    T = batch * s_q
    stream = torch.cuda.current_stream()
    lens = torch.randint(4096, 8193, (batch,), generator=g, dtype=torch.int32)
    mb = 8192 // 64
    table = torch.randperm(batch * mb, generator=g).to(torch.int32).reshape(batch, mb)

    def rnd(*shape, dtype=torch.bfloat16, scale=1.0):
        return (torch.randn(shape, generator=g) * scale).to(dtype).to(dev)

    def timed(fn, nbytes, flops, name, result):
        """`steps` calls captured in a HIP graph and replayed, so that the
        time is the kernels' and not the host's launch rate (the small
        kernels here run for less than a Python call takes); the graph's last
        result must equal an eager call's."""
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(steps):
                fn(i)
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        s = e0.elapsed_time(e1) / steps * 1e-3
        replayed = result().clone()
        fn(steps - 1)
        torch.cuda.synchronize()
        if not torch.equal(replayed, result()):
            raise RuntimeError(f"{name}: graph replay differs from an eager call")
        del graph
        rec = {"us": round(s * 1e6, 2), "algorithmic_bytes": nbytes, "mfma_flops": flops,
               "gbs": round(nbytes / s / 1e9, 1), "bound": binding_bound(nbytes, max(flops, 1)),
               "frac": round(roofline_frac(binding_bound(nbytes, max(flops, 1)), nbytes, flops, s), 4)}
        print(f"[bench] {name}: {rec['us']} us, {rec['gbs']} GB/s, {rec['bound']} fraction {rec['frac']}",
              file=sys.stderr, flush=True)
        return rec

    def copies_for(nbytes):
        return max(1, min(16, int(math.ceil((1 << 30) / max(nbytes, 1))) + 1))

    out = {"tokens": T, "hidden": hidden}
    # query side
    w_uk_t = rnd(128, 512, 128, scale=512 ** -0.5)
    qb = T * 128 * (128 + 64) * 2
    n = copies_for(qb + T * 128 * 576 * 2)
    qs = [(rnd(batch, s_q, 128, 128), rnd(batch, s_q, 128, 64)) for _ in range(n)]
    qa = torch.empty((batch, s_q, 128, 512), dtype=torch.bfloat16, device=dev)
    qr = torch.empty((batch, s_q, 128, 64), dtype=torch.bfloat16, device=dev)
    lens_d = lens.to(dev)
    out["absorb_query"] = timed(lambda i: mla.mla_absorb_query(qs[i % n][0], qs[i % n][1], w_uk_t, lens_d, qa, qr),
                                qb + w_uk_t.numel() * 2 + T * 128 * 576 * 2 + batch * 4,
                                2 * T * 128 * 128 * 512, "absorb_query", lambda: torch.cat([qa.flatten(), qr.flatten()]))
    del qs
    # output side
    w_uv = rnd(128, 128, 512, scale=512 ** -0.5)
    ob = T * 128 * 512 * 4
    n = copies_for(ob)
    ols = [rnd(batch, s_q, 128, 512, dtype=torch.float32, scale=0.3) for _ in range(n)]
    vals = torch.empty((batch, s_q, 128, 128), device=dev)
    out["absorb_output"] = timed(lambda i: mla.mla_absorb_output(ols[i % n], w_uv, vals),
                                 ob + w_uv.numel() * 2 + T * 128 * 128 * 4, 2 * T * 128 * 512 * 128, "absorb_output",
                                 lambda: vals)
    del ols
    # KV projection of the new tokens
    w_kv = rnd(576, hidden, scale=hidden ** -0.5)
    hb = T * hidden * 2
    n = copies_for(hb + w_kv.numel() * 2)
    hs = [rnd(T, hidden) for _ in range(n)]
    w_kvs = [w_kv] + [w_kv.clone() for _ in range(n - 1)]
    kv = torch.empty((T, 576), device=dev)
    kvb, kvf = hb + w_kv.numel() * 2 + T * 576 * 4, 2 * T * hidden * 576
    splits = mla.mla_kv_project_splits(T, hidden)
    ws = torch.empty((splits, T, 576), device=dev)
    out["kv_project"] = timed(lambda i: mla.mla_kv_project_split(hs[i % n], w_kvs[i % n], kv, ws),
                              kvb, kvf, "kv_project", lambda: kv)
    out["kv_project"]["splits"] = splits
    out["kv_project_unsplit"] = timed(lambda i: mla.mla_kv_project(hs[i % n], w_kvs[i % n], kv),
                                      kvb, kvf, "kv_project_unsplit", lambda: kv)
    del ws
    del hs, w_kvs
    # cache append into a bf16 paged cache of the same batch shape
    rows = torch.zeros((batch * mb, 64, 576), dtype=torch.bfloat16, device=dev)
    cache = mla.LatentCache(mla.MLA_CACHE_BF16, rows)
    table_d = table.to(dev)
    kv3 = kv.view(batch, s_q, 576)
    out["cache_append"] = timed(lambda i: mla.mla_cache_append(kv3, lens_d, table_d, cache),
                                T * 576 * 4 + T * 1152 + batch * 4 + T * 4, 0, "cache_append", lambda: rows)
    return out


def summary(r):
    """The per-workload record of config.workloads."""
    s = r["ms_step"] * 1e-3
    return {"step_us": round(r["ms_step"] * 1e3, 2), "decode_us": round(r["ms_decode"] * 1e3, 2),
            **{f"step_us_{k}": round(v * 1e3, 2) for k, v in r["step_pct"].items()},
            "combine_us_est": round((r["ms_step"] - r["ms_decode"]) * 1e3, 2),
            "cache_tokens_per_s": round(r["rows"] / s, 1), "step_gbs": round(r["bytes"] / s / 1e9, 1),
            "step_tflops": round(r["flops"] / s / 1e12, 1), "bound": r["bound"],
            "frac_decode": round(r["frac_decode"], 4), "frac_step": round(r["frac_step"], 4),
            "num_splits": r["splits"], "cache_dtype": r["inp"].cache_dtype, "rows": r["rows"],
            "algorithmic_bytes": r["bytes"], "mfma_flops": r["flops"],
            "decode_traffic_bytes": measured_traffic(r["workload"])}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100,
                    help="untimed steps first: a cold GPU runs its first ~30 MTP steps through a clock transient")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, help="the headline workload")
    ap.add_argument("--only", action="store_true", help="time the headline workload only")
    ap.add_argument("--around-only", action="store_true",
                    help="time only the steps around the decode (absorption, projection, cache append) for "
                         "the headline workload's batch shape, and print their record")
    ap.add_argument("--num-splits", type=int, default=0, help="0: the workload's, else the library's hint")
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
    torch.cuda.set_device(0)

    if args.around_only:
        from mla_inputs import get_workload
        wl = get_workload(args.workload)
        print(json.dumps(measure_next_rows(wl["batch"], wl["s_q"], args.steps, args.warmup)), flush=True)
        return 0
    head = measure(args.workload, args.steps, args.warmup, args.num_splits, args.seed)
    others = {}
    if not args.only:
        for w in ALL_WORKLOADS:
            if w != args.workload:
                others[w] = summary(measure(w, args.steps, args.warmup, 0, args.seed, min_warm_s=0.25))
    inp = head["inp"]
    next_rows = None if args.only else measure_next_rows(inp.batch, inp.s_q, args.steps, args.warmup)
    copy_gbs = copy_bandwidth()
    ms_step, ms_decode = head["ms_step"], head["ms_decode"]
    nbytes, flops = head["bytes"], head["flops"]
    if head["bound"] == "hbm":
        achieved = nbytes / (ms_decode * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        achieved = flops / (ms_decode * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s"}
    roof["frac"] = round(head["frac_decode"], 4)
    roof["traffic"] = measured_traffic(args.workload)
    roof["step_frac"] = round(head["frac_step"], 4)
    workloads = {args.workload: summary(head), **others}
    result = {
        "metric": "MLA decode cache-tokens/s and achieved HBM GB/s (% of roofline), 1 MI355X",
        "value": round(head["rows"] / (ms_step * 1e-3), 1), "unit": "cache-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        # the arithmetic: bf16 MFMA with fp32 accumulation; an e4m3 cache is widened exactly to bf16
        "dtype": "bf16" if inp.cache_dtype == "bf16" else "fp8_e4m3",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": inp.batch, "s_q": inp.s_q, "cache_rows": head["rows"],
                   "layout": "contiguous" if inp.block_table is None else "paged64",
                   "cache_dtype": inp.cache_dtype, "num_splits": head["splits"], "rotated_copies": head["copies"],
                   "step_gbs": round(nbytes / (ms_step * 1e-3) / 1e9, 1),
                   "step_tflops": round(flops / (ms_step * 1e-3) / 1e12, 1),
                   "query_row_pairs_per_s": round(flops / FLOP_PER_QROW_ROW / (ms_step * 1e-3), 1),
                   "decode_kernel_us": round(ms_decode * 1e3, 2),
                   **{f"step_us_{k}": round(v * 1e3, 2) for k, v in head["step_pct"].items()},
                   "copy_gbs": copy_gbs,
                   "step_gbs_of_copy": round(nbytes / (ms_step * 1e-3) / 1e9 / copy_gbs, 4),
                   "algorithmic_bytes": nbytes, "mfma_flops": flops, "workloads": workloads,
                   "around_the_decode": next_rows},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_budget)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
