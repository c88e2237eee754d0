"""Throughput of the CSA2 attention step on one MI355X.

One step = one csa2_decode call over the whole batch: indexer scores for every
query over its reachable compressed entries, per-query top-512, and the
64-head single-softmax attention over 128 window rows + 512 selected rows.
Default workload: 64 independent decode queries at context 65,536 with
compress ratio 4 (16,384 candidates each), bf16 KV, fp32 indexer keys; inputs
are seeded synthetic N(0, 1) data, resident in HBM before timing starts.

Prints ONE JSON line.  Besides the contract fields it carries
  roofline:     the dominant kernel (the indexer scan) against HBM bandwidth,
                its duration measured here with HIP events on the launch stream;
  cpu_baseline: the CPU oracle timed on a bounded sample of the same workload;
  step_us:      medians of per-step HIP-event times, warm (back to back) and
                cold (a 1 GiB fill before each step evicts the last-level cache).
The default warm-up (100 untimed steps) outlasts the clock ramp of the first
~20 ms of sustained work, so the timed steps see the steady state.
--config 2 times the 4,096-query prefill chunk instead (one csa2_prefill per
step; the roofline is then the attention's against the bf16 MFMA peak).
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA2 attended queries/sec (64h×512, 128+512 keys) + % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
INDEX_KEY_BYTES = 128 * 4    # one fp32 index key row per scanned candidate
MXFP4_KEY_BYTES = 64 + 4     # one MXFP4 index key row: 64 code bytes + 4 E8M0 scales
INDEX_Q_BYTES = 128 * 4      # one fp32 indexer query per query
PROFILE_DIR = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILE_DIR, "index_scores_decode_64x16384_traffic.json")
INDEX_SRC = os.path.join(ROOT, "sparse_long_context_amd", "csrc", "index_scores.hip")
ATTN_TRAFFIC_FILE = os.path.join(PROFILE_DIR, "attend_mq_prefill_4096_traffic.json")
ATTN_SRC = os.path.join(ROOT, "sparse_long_context_amd", "csrc", "attend_mq.hip")
# (kernel name fragment, record file, kernel source, workload, bench arguments of the counter runs)
TRAFFIC_KERNELS = {
    "index": ("index_scores_decode", TRAFFIC_FILE, INDEX_SRC, "decode, 64 queries x 16,384 candidates",
              "--no-cpu-baseline --copy-probe --steps 3 --warmup 1"),
    "attend": ("attend_mq_kernel", ATTN_TRAFFIC_FILE, ATTN_SRC, "prefill chunk, 4,096 queries x 640 entries",
               "--config 2 --no-cpu-baseline --copy-probe --steps 3 --warmup 1"),
}
COPY_PROBE_BYTES = 512 << 20


def source_digest(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def workload_desc(inp, storage="native"):
    d = inp["dims"]
    kv = "bf16" if d["kv_dtype"] == 0 else "fp8 e4m3 + ue8m0/32"
    keys = "fp32"
    if storage == "fp4":
        kv, keys = "fp4 e2m1 + e4m3/16", "mxfp4 (e2m1 + e8m0/32)"
    return {
        "workload": (f"decode, {inp['B']} queries, context {int(inp['pos'][0]) + 1}, compress ratio "
                     f"{int(inp['ratio'][0])} -> {int(inp['pool_len'][0])} candidates each, window "
                     f"{d['window']}, top-{d['index_topk']}, {d['n_heads']} heads x {d['head_dim']}, {kv} KV, "
                     f"{keys} indexer keys dim {d['index_dim']}"),
        "queries_per_step": int(inp["B"]),
        "candidates_per_query": int(inp["pool_len"][0]),
        "window": d["window"], "index_topk": d["index_topk"], "kv": kv, "index_keys": keys,
    }


def traffic_from_profile(which="index"):
    """HBM bytes per launch of a kernel (the decode indexer, or the prefill
    attention) from committed rocprofv3 PMC counters, if they were taken on
    the current kernel source."""
    _, path, src, _, _ = TRAFFIC_KERNELS[which]
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256_16") != source_digest(src):
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_probe(torch):
    """Plain streaming kernels of known size, for scaling the HBM byte
    counters: a fill writes COPY_PROBE_BYTES, a sum reads them."""
    src = torch.empty(COPY_PROBE_BYTES // 4, dtype=torch.float32, device="cuda")
    for _ in range(3):
        src.fill_(1.0)
        float(src.sum())
    torch.cuda.synchronize()


def summarize_traffic(fetch_csv, write_csv, which="index"):
    """Per-launch HBM bytes of a kernel from rocprofv3 counter CSVs.

    FETCH_SIZE and WRITE_SIZE are in KiB per dispatch.  Each is scaled by what
    the counter reads for a plain streaming kernel of COPY_PROBE_BYTES (a sum
    that reads exactly that many bytes, a fill that writes them), so the result
    is in true bytes."""
    import csv

    def per_kernel(path, counter):
        vals = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    kname, out_path, src, workload, run_args = TRAFFIC_KERNELS[which]
    out = {}
    for path, counter in ((fetch_csv, "FETCH_SIZE"), (write_csv, "WRITE_SIZE")):
        v = per_kernel(path, counter)
        idx = [x for k, xs in v.items() if kname in k for x in xs]
        # the probe's streaming kernel for this counter: the sum reads, the fill writes
        probe = "reduce_kernel" if counter == "FETCH_SIZE" else "FillFunctor"
        # (the cold-step flush is a 1 GiB fill: twice the probe, so it is not
        # taken; FETCH_SIZE reports about half the bytes read on this part)
        cpy = [x for k, xs in v.items() if probe in k for x in xs
               if 0.3 * COPY_PROBE_BYTES < x * 1024 < 1.5 * COPY_PROBE_BYTES]
        if not idx or not cpy:
            raise SystemExit(f"{path}: no {kname} or copy dispatches with {counter}")
        scale = COPY_PROBE_BYTES / (1024.0 * (sum(cpy) / len(cpy)))
        out[counter] = {"kib_per_launch": sum(idx) / len(idx), "copy_kib": sum(cpy) / len(cpy), "scale": scale,
                        "bytes_per_launch": scale * 1024.0 * sum(idx) / len(idx), "launches": len(idx)}
    rec = {"kernel": kname, "workload": workload,
           "kernel_source_sha256_16": source_digest(src),
           "hbm_bytes_per_launch": round(out["FETCH_SIZE"]["bytes_per_launch"] + out["WRITE_SIZE"]["bytes_per_launch"]),
           "fetch": out["FETCH_SIZE"], "write": out["WRITE_SIZE"],
           "commands": ["rocprofv3 --pmc FETCH_SIZE -d <dir> -o fetch --output-format csv -- python3 bench.py " + run_args,
                        "rocprofv3 --pmc WRITE_SIZE -d <dir> -o write --output-format csv -- python3 bench.py " + run_args]}
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def cpu_baseline(inp, min_seconds=10.0, max_seconds=30.0):
    """Oracle over whole passes of the batch until at least min_seconds."""
    from oracle import oracle as O
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    n = 0
    passes = 0
    t0 = time.perf_counter()
    while True:
        O.decode_batch(inp)
        n += inp["B"]
        passes += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or el >= max_seconds:
            break
    return {"value": n / el, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"{passes} passes over the {inp['B']}-query batch ({n} queries, {el:.1f} s, fp64 oracle, "
                      f"OpenMP over queries)"}


def step_medians(torch, fn, steps, stream):
    """Median of per-step HIP-event times of fn (microseconds): warm, back to
    back with no flush; cold, with a 1 GiB fill before each step, which evicts
    the last-level cache (256 MB) so every input comes from HBM again."""
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    out = {}
    for mode in ("warm", "cold"):
        ts = []
        for _ in range(steps):
            if mode == "cold":
                flush.fill_(1.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            ts.append(1000.0 * e0.elapsed_time(e1))
        ts.sort()
        out[mode + "_median_us"] = round(ts[len(ts) // 2], 2)
    del flush
    return out


def bench_prefill(args):
    """The prefill chunk (4,096 queries of one sequence at positions
    126,976..131,071, compress ratio 8): one step = one csa2_prefill call."""
    import torch
    from sparse_long_context_amd import csa2, synth
    print("[bench] generating the prefill chunk", file=sys.stderr, flush=True)
    pf = synth.config(2)
    w = csa2.PrefillWorkload(pf)
    stream = torch.cuda.current_stream()
    T = w.T
    for _ in range(args.warmup):
        w.prefill()
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        w.prefill()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    # the attention on its own (the dominant kernel): the same batch through
    # csa2_attend, launched back to back between two HIP events
    inp = synth.prefill_as_batch(pf)
    dw = csa2.DecodeWorkload(inp)
    dw.topk.copy_(w.topk)
    attend = lambda: csa2.csa2_attend(dw.dims, T, dw.batch, dw.q, dw.win_kv, dw.win_scale, dw.comp_kv,  # noqa: E731
                                      dw.comp_scale, dw.topk, None, dw.out, dw.lse, None, 0)
    for _ in range(args.warmup):
        attend()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        attend()
    e1.record(stream)
    torch.cuda.synchronize()
    attn_us = 1000.0 * e0.elapsed_time(e1) / args.steps
    step_us = step_medians(torch, w.prefill, min(args.steps, 20), stream)
    if args.copy_probe:
        copy_probe(torch)
    ent = int(inp["win_len"].sum()) + T * pf["dims"]["index_topk"]
    attn_flops = 4.0 * 64 * 512 * ent
    achieved = attn_flops / (attn_us * 1e-6) / 1e12
    d = pf["dims"]
    gather_bytes = ent * d["head_dim"] * 2 + T * d["n_heads"] * d["head_dim"] * (2 + 4)
    line = {
        "metric": METRIC, "value": round(T * args.steps / wall, 1), "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": (f"prefill chunk, {T} queries at positions {int(pf['pos0'])}..{int(pf['pos0']) + T - 1}, "
                                f"compress ratio {int(pf['ratio'])} -> {int(pf['pool_len'])} pool rows, window "
                                f"{d['window']}, top-{d['index_topk']}, {d['n_heads']} heads x {d['head_dim']}, bf16 KV, "
                                f"fp32 indexer keys dim {d['index_dim']}"),
                   "queries_per_step": T, "pool_rows": int(pf["pool_len"]), "window": d["window"],
                   "index_topk": d["index_topk"], "kv": "bf16", "index_keys": "fp32"},
        "roofline": {"bound": "mfma", "kernel": "attend_mq_kernel", "achieved": round(achieved, 1),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic_from_profile("attend"), "algorithmic_flops_per_launch": attn_flops,
                     "avg_launch_us": round(attn_us, 2)},
        "stages_us": {"attend": round(attn_us, 2)},
        # the same launch against HBM bandwidth, every entry's row counted once
        # per use (as if gathered from HBM) plus q and the fp32 output: most
        # rows in fact come from the last-level cache (a 16 MiB pool)
        "attend_gather": {"achieved": round(gather_bytes / (attn_us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": round(gather_bytes / (attn_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                          "bytes_per_launch": gather_bytes},
        "step_us": step_us,
        "gpu": torch.cuda.get_device_name(0),
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline_prefill(pf, inp)
    print(json.dumps(line), flush=True)


def cpu_baseline_prefill(pf, inp, min_seconds=10.0):
    """Oracle over groups of 64 consecutive prefill queries (scores against
    the shared pool, top-512, attention) until at least min_seconds."""
    import numpy as np
    from oracle import oracle as O
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    n = 0
    t0 = time.perf_counter()
    start = 0
    while True:
        qs = np.arange(start, start + 64) % pf["T"]
        O.decode_batch(inp, qs)
        n += len(qs)
        start += 64
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    return {"value": n / el, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"{n} of the chunk's queries in groups of 64 ({el:.1f} s, fp64 oracle, OpenMP over queries)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the clocks ramp for the first ~20 ms of sustained work (the prefill
    # attention measured 499 us after 5 warm-up launches, 454 us after 100),
    # so the default warm-up runs 100 untimed steps (and 100 launches before
    # each stage's timing) to time the steady state
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", type=int, default=1,
                    help="workload index: decode 1, 3 or 4, or 2 (the 4,096-query prefill chunk)")
    ap.add_argument("--storage", choices=("native", "fp4"), default="native",
                    help="fp4: the same workload with its KV rows re-stored as FP4 (E4M3 scale per 16) and its index "
                         "keys as MXFP4, quantized on the GPU by the library's own quantizers before timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain %d MiB fill and sum (for scaling rocprofv3 byte counters)" % (COPY_PROBE_BYTES >> 20))
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of 'bench.py --copy-probe' "
                         "into a kernel's HBM bytes per launch, and exit")
    ap.add_argument("--traffic-kernel", choices=sorted(TRAFFIC_KERNELS), default="index",
                    help="with --traffic-from: the decode indexer (index) or the prefill attention (attend)")
    args = ap.parse_args()
    if args.traffic_from:
        summarize_traffic(*args.traffic_from, which=args.traffic_kernel)
        return
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}); the decode batch "
              "shards by sequence with no exchange, so N GPUs would each run this same step on their own "
              "queries.", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_long_context_amd import csa2, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.config not in (1, 2, 3, 4):
        print("bench.py times the workloads 1, 2, 3 or 4", file=sys.stderr)
        sys.exit(2)
    if args.config == 2:
        if args.storage != "native":
            print("--storage fp4 re-stores decode workloads only", file=sys.stderr)
            sys.exit(2)
        bench_prefill(args)
        return
    print(f"[bench] generating workload {args.config}", file=sys.stderr, flush=True)
    inp = synth.config(args.config)
    w = csa2.DecodeWorkload(inp)
    stream = torch.cuda.current_stream()
    B = w.B
    if args.storage == "fp4":
        if inp["dims"]["kv_dtype"] != 0:
            print("--storage fp4 re-stores bf16 workloads (1 or 4)", file=sys.stderr)
            sys.exit(2)
        print("[bench] re-storing KV as FP4 and index keys as MXFP4 on the GPU", file=sys.stderr, flush=True)
        for name, scname in (("win_kv", "win_scale"), ("comp_kv", "comp_scale")):
            src = getattr(w, name).view(torch.bfloat16).float()
            rows = src.shape[0]
            codes = torch.empty((rows, 256), dtype=torch.uint8, device="cuda")
            scales = torch.empty((rows, 32), dtype=torch.uint8, device="cuda")
            csa2.csa2_quantize_fp4_kv(rows, 512, src, codes, scales)
            setattr(w, name, codes)
            setattr(w, scname, scales)
            del src
        rows = w.idx_k.shape[0]
        kc = torch.empty((rows, 64), dtype=torch.uint8, device="cuda")
        ks = torch.empty((rows, 4), dtype=torch.uint8, device="cuda")
        csa2.csa2_quantize_mxfp4(rows, 128, w.idx_k, kc, ks)
        w.idx_k, w.idx_k_scale = kc, ks
        w.dims.kv_dtype, w.dims.index_key_dtype = 2, 1
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    for _ in range(args.warmup):
        w.decode()
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        w.decode()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    value = B * args.steps / wall

    # per-kernel durations: each of the three stage entry points launched
    # `steps` times back to back between two HIP events on the launch stream
    # (the same kernels and launch shapes csa2_decode issues)
    stride = (w.max_cand + 63) // 64 * 64  # the row stride csa2_decode uses for its own score buffer
    scores = torch.empty((B, stride), dtype=torch.float32, device="cuda")
    stages = [
        lambda: csa2.csa2_index_scores(w.dims, B, w.batch, w.idx_q, w.idx_w, w.idx_k, scores, stride,
                                       idx_k_scale=w.idx_k_scale),
        lambda: csa2.csa2_topk(w.dims, B, w.batch, scores, stride, w.topk),
        lambda: csa2.csa2_attend(w.dims, B, w.batch, w.q, w.win_kv, w.win_scale, w.comp_kv, w.comp_scale, w.topk,
                                 w.sink, w.out, w.lse, w.ws, w.ws_bytes),
    ]
    stage_us = []
    for fn in stages:
        for _ in range(args.warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        stage_us.append(1000.0 * e0.elapsed_time(e1) / args.steps)
    step_us = step_medians(torch, w.decode, args.steps, stream)
    if args.copy_probe:
        copy_probe(torch)

    n_cand = int(sum(min(int(p), (int(pos) + 1) // int(r)) for p, pos, r, m in
                     zip(inp["pool_len"], inp["pos"], inp["ratio"], inp["mode"]) if m == 0 and r > 0))
    n_full = int((inp["mode"] == 0).sum())
    key_bytes = MXFP4_KEY_BYTES if args.storage == "fp4" else INDEX_KEY_BYTES
    idx_bytes = n_cand * key_bytes + n_full * INDEX_Q_BYTES
    achieved = idx_bytes / (stage_us[0] * 1e-6) / 1e9
    traffic = traffic_from_profile() if (args.config == 1 and args.storage == "native") else None
    roofline = {"bound": "hbm", "kernel": "index_scores_decode" if args.storage == "native" else "index_scores_decode_mx", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "algorithmic_bytes_per_launch": idx_bytes,
                "avg_launch_us": round(stage_us[0], 2)}
    # the attention contraction on its own: 2 x (64 x entries x 512) MACs per query
    ent = 0
    for b in range(B):
        nv = min(int(inp["pool_len"][b]), (int(inp["pos"][b]) + 1) // max(int(inp["ratio"][b]), 1))
        sel = min(512, nv) if inp["mode"][b] in (0, 1) else (int((inp["sel_in"][b] >= 0).sum())
                                                            if inp["mode"][b] == 2 else 0)
        ent += int(inp["win_len"][b]) + sel
    attn_flops = 4.0 * 64 * 512 * ent
    attend_tflops = attn_flops / (stage_us[2] * 1e-6) / 1e12

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": workload_desc(inp, args.storage),
        "roofline": roofline,
        "stages_us": {"index_scores": round(stage_us[0], 2), "topk": round(stage_us[1], 2),
                      "attend": round(stage_us[2], 2)},
        "attend_mfma": {"achieved": round(attend_tflops, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(attend_tflops / BF16_PEAK_TFLOPS, 4)},
        "step_us": step_us,
        "gpu": torch.cuda.get_device_name(0),
    }
    if not args.no_cpu_baseline and args.storage == "native":
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(inp)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
