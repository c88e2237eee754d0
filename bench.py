"""Throughput of the CSA2 attention step on one MI355X.

Headline workload (the default): the prefill chunk of 4,096 query tokens of one
sequence at positions 126,976..131,071 of a 131,072-token context, compress
ratio 8 (a pool of 16,384 compressed rows), each query with its own causal
128-row window and its own top-512 from the indexer, 64 heads x 512 dims, bf16
KV, fp32 index keys.  One step = one csa2_prefill call over the whole chunk:
indexer scores, per-query top-512, and the 64-head single-softmax attention
over 128 window rows + 512 selected rows.  Inputs are seeded synthetic N(0, 1)
data, resident in HBM before timing starts.

Prints ONE JSON line.  Besides the contract fields it carries
  roofline:     the dominant kernel (the prefill attention) against the bf16
                MFMA peak, its duration measured here with HIP events on the
                launch stream (a csa2_prefill call in Reuse mode over the same
                selections: the attention and a 2-4 us descriptor kernel);
  cpu_baseline: the CPU oracle timed on a bounded sample of the same workload
                (all host threads), with the host's CPU model and a
                single-thread rate;
  step_us:      medians of per-step HIP-event times, warm (back to back) and
                cold (a 1 GiB fill before each step evicts the last-level cache);
  workloads:    the decode batches (64 x 16,384 bf16; 256 x 16,384 fp8 at 1M
                context; 128 mixed-mode ragged queries; the first re-stored as
                FP4 KV + MXFP4 keys), each with its step time, queries/s, stage
                times and its indexer against HBM bandwidth (--no-extras skips).
Before the warm-up steps the GPU runs ~50 ms of plain fills, past the clock ramp
of the first ~20 ms of sustained work, so the timed steps see the steady state.
--config 1, 3 or 4 makes one decode batch the headline instead.
"""
import argparse
import ctypes
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
FP32_MFMA_TFLOPS = 157.3     # MI355X fp32 matrix, published
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
              "--config 1 --no-cpu-baseline --copy-probe --steps 3 --warmup 1"),
    "attend": ("attend_mq_kernel<false>", ATTN_TRAFFIC_FILE, ATTN_SRC, "prefill chunk, 4,096 queries x 640 entries",
               "--no-extras --no-cpu-baseline --copy-probe --steps 3 --warmup 1"),
}
COPY_PROBE_BYTES = 512 << 20
KV_NAMES = {0: "bf16", 1: "fp8 e4m3 + ue8m0/32", 2: "fp4 e2m1 + e4m3/16"}


def say(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def source_digest(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profile(which):
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


def gather_probe(torch):
    """Rate of random 1 KiB row gathers per CU and over the chip (the bf16
    attention's access pattern), by LDS DMA and by loads into registers, from
    regions of 2 MiB (L2-resident), 16 MiB (the prefill pool) and 512 MiB,
    with libcsa2_probe.so; one JSON line."""
    import ctypes
    import numpy as np
    from sparse_long_context_amd import build as B
    if not os.path.exists(B.PROBE_LIB):
        raise RuntimeError(f"{B.PROBE_LIB} is not built; run __graft_entry__.build() first")
    L = ctypes.CDLL(B.PROBE_LIB)
    L.csa2_probe_gather.restype = ctypes.c_int
    L.csa2_probe_gather.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    nrows, per_wave, reps = 1 << 19, 1024, 5
    rows = torch.zeros(nrows * 256, dtype=torch.int32, device="cuda")  # 512 MiB of 1 KiB rows
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    rng = np.random.default_rng(1)
    out = {"probe": "random 1 KiB row gathers, one workgroup per CU, each wave two batches of 8 rows in flight",
           "cus": n_cu, "rows_per_wave": per_wave, "results": []}
    for region, span in (("2 MiB", 2048), ("16 MiB", 16384), ("512 MiB", nrows)):
        idx_np = rng.integers(0, span, size=n_cu * 8 * per_wave).astype(np.int32)
        assert idx_np.min() >= 0 and idx_np.max() < nrows
        idx = torch.from_numpy(idx_np).cuda()
        for mode, name in ((0, "lds_dma"), (1, "registers")):
            for waves in (4, 8):
                def go():
                    rc = L.csa2_probe_gather(mode, waves, n_cu, rows.data_ptr(), idx.data_ptr(), per_wave,
                                             sink.data_ptr(), ctypes.c_void_p(stream.cuda_stream))
                    if rc != 0:
                        raise RuntimeError(f"csa2_probe_gather: hipError {rc}")
                go()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(reps):
                    go()
                e1.record(stream)
                torch.cuda.synchronize()
                us = e0.elapsed_time(e1) * 1000.0 / reps
                gbs = n_cu * waves * per_wave * 1024.0 / (us * 1e-6) / 1e9
                out["results"].append({"region": region, "path": name, "waves_per_cu": waves,
                                       "us_per_launch": round(us, 1), "gb_s": round(gbs, 1),
                                       "gb_s_per_cu": round(gbs / n_cu, 1)})
        del idx
    print(json.dumps(out), flush=True)


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

    def probe_of(counter):
        return "reduce_kernel" if counter == "FETCH_SIZE" else "FillFunctor"

    kname, out_path, src, workload, run_args = TRAFFIC_KERNELS[which]
    out = {}
    for path, counter in ((fetch_csv, "FETCH_SIZE"), (write_csv, "WRITE_SIZE")):
        v = per_kernel(path, counter)
        idx = [x for k, xs in v.items() if kname in k for x in xs]
        # the probe's streaming kernel for this counter: the sum reads, the fill
        # writes.  A counter reports either the true bytes or half of them on
        # this part (FETCH_SIZE: half), so the probe dispatches are those within
        # 10% of the probe's size or of half of it, the full-size ones when both
        # occur; the other fills (the clock ramp's 192 MiB, the cold-step flush's
        # 1 GiB) fall in neither window.
        near = {1.0: [], 0.5: []}
        for k, xs in v.items():
            if probe_of(counter) in k:
                for x in xs:
                    for f in near:
                        if abs(x * 1024 - f * COPY_PROBE_BYTES) < 0.1 * f * COPY_PROBE_BYTES:
                            near[f].append(x)
        cpy = near[1.0] or near[0.5]
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


# ---- CPU baseline (the oracle, as it stands) ---------------------------------

def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _omp_threads(n):
    """Set the OpenMP thread count of the process (the oracle's libgomp)."""
    try:
        ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))
        return True
    except OSError:
        return False


def _timed_oracle(run, per_call, min_seconds, max_calls):
    n = calls = 0
    t0 = time.perf_counter()
    while True:
        run(calls)
        n += per_call
        calls += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or calls >= max_calls:
            return n, el


def cpu_baseline(run, per_call, what, min_seconds=10.0, single_seconds=3.0):
    """run(i) executes the oracle on the i-th group of per_call queries.  All
    host threads first (at least min_seconds), then one thread."""
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    n, el = _timed_oracle(run, per_call, min_seconds, 10 ** 9)
    rec = {"value": round(n / el, 1), "unit": "queries/s", "cores": threads, "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": f"{n} queries of {what} in groups of {per_call} ({el:.1f} s, fp64 oracle, OpenMP over "
                     f"queries on {threads} threads)"}
    if _omp_threads(1):
        n1, el1 = _timed_oracle(run, per_call, single_seconds, 10 ** 9)
        _omp_threads(threads)
        rec["single_thread"] = {"value": round(n1 / el1, 2), "unit": "queries/s",
                                "sample": f"{n1} queries ({el1:.1f} s, one thread)"}
    return rec


# ---- timing helpers -----------------------------------------------------------

def ramp_clocks(torch, ms=50.0):
    """About `ms` of plain fills, so the clocks leave their idle state before
    the warm-up steps."""
    # 192 MiB: a size the traffic counters' probe windows never take
    buf = torch.empty(48 << 20, dtype=torch.float32, device="cuda")
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1000.0 < ms:
        for _ in range(20):
            buf.fill_(1.0)
        torch.cuda.synchronize()
    del buf


def timed(torch, fn, n, stream):
    """Average microseconds per call of fn over n calls back to back between
    two HIP events on the launch stream."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(n):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return 1000.0 * e0.elapsed_time(e1) / n


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


def headline_steps(torch, fn, n_queries, steps, warmup, stream):
    """W untimed steps, then exactly K timed steps between a synchronize and
    two HIP events; returns (queries/s over the wall clock, ms per step)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    say(f"timing {steps} steps")
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        fn()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return n_queries * steps / wall, ev0.elapsed_time(ev1) / steps


# ---- the prefill chunk ----------------------------------------------------------

def prefill_desc(pf):
    d = pf["dims"]
    T = int(pf["T"])
    return (f"prefill chunk, {T} queries at positions {int(pf['pos0'])}..{int(pf['pos0']) + T - 1}, compress "
            f"ratio {int(pf['ratio'])} -> {int(pf['pool_len'])} pool rows, window {d['window']}, "
            f"top-{d['index_topk']}, {d['n_heads']} heads x {d['head_dim']}, {KV_NAMES[d['kv_dtype']]} KV, "
            f"fp32 indexer keys dim {d['index_dim']}")


def bench_prefill(args, torch, stream):
    import numpy as np
    from sparse_long_context_amd import csa2, synth
    say("generating the prefill chunk")
    pf = synth.config(2)
    w = csa2.PrefillWorkload(pf)
    T = w.T
    ramp_clocks(torch)
    value, ms_step = headline_steps(torch, w.prefill, T, args.steps, args.warmup, stream)
    # the attention on its own (the dominant kernel), one launch per call:
    # csa2_attend over the chunk as a batch of Reuse queries, each with the
    # window rows and the selection the step gave it (query t at p = pos0 + t
    # reads raw rows max(win_pos0, p - W + 1) .. p, as the chunk's descriptor
    # kernel derives them), unsplit as in the step
    d = pf["dims"]
    pos = int(pf["pos0"]) + np.arange(T, dtype=np.int64)
    lo = np.maximum(int(pf["win_pos0"]), pos - d["window"] + 1)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    rb = {"pos": dev(pos), "mode": dev(np.full(T, synth.MODE_REUSE, np.int32)),
          "ratio": dev(np.full(T, int(pf["ratio"]), np.int32)), "win_row0": dev(lo - int(pf["win_pos0"])),
          "win_len": dev((pos - lo + 1).astype(np.int32)), "pool_row0": dev(np.zeros(T, np.int64)),
          "pool_len": dev(np.full(T, int(pf["pool_len"]), np.int32))}
    batch = csa2.Batch(csa2._p(rb["pos"]), csa2._p(rb["mode"]), csa2._p(rb["ratio"]), csa2._p(rb["win_row0"]),
                       csa2._p(rb["win_len"]), csa2._p(rb["pool_row0"]), csa2._p(rb["pool_len"]), None, None, 0)
    out = torch.empty_like(w.out)
    lse = torch.empty_like(w.lse)
    ws_bytes = csa2.csa2_workspace_size(w.dims, T, 0)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")

    def attend(rope=None, ws_=None, ws_bytes_=0):
        csa2.csa2_attend(w.dims, T, batch, w.q, w.win_kv, None, w.comp_kv, None, w.topk, None, out, lse, ws_,
                         ws_bytes_, stream=stream, rope=rope)

    for _ in range(max(args.warmup, 20)):
        attend()
    attn_us = timed(torch, attend, max(args.steps, 20), stream)
    # the output de-rotation (64 rope dims at offset 448, theta 160,000):
    # fused into the attention's writes (its cos / sin rows need the
    # workspace), and as its own pass over the output
    inv_t = torch.from_numpy(160000.0 ** (-np.arange(32, dtype=np.float64) / 32.0)).cuda()
    rope = csa2.out_rope(448, 64, inv_t)
    attn_rope_us = timed(torch, lambda: attend(rope, ws, ws_bytes), max(args.steps, 20), stream)
    derot_us = timed(torch, lambda: csa2.csa2_derotate(w.dims, T, rb["pos"], 448, 64, inv_t, out),
                     max(args.steps, 20), stream)
    # the indexer on its own: the chunk's scores into a buffer of the step's stride
    stride = (int(pf["pool_len"]) + 63) // 64 * 64
    scores = torch.empty((T, stride), dtype=torch.float32, device="cuda")
    for _ in range(max(args.warmup, 20)):
        w.index_scores(scores, stride)
    scores_us = timed(torch, lambda: w.index_scores(scores, stride), max(args.steps, 20), stream)
    # the top-K on its own, over those scores (the same descriptors as Full queries)
    full = csa2.Batch(csa2._p(rb["pos"]), csa2._p(dev(np.full(T, synth.MODE_FULL, np.int32))), csa2._p(rb["ratio"]),
                      csa2._p(rb["win_row0"]), csa2._p(rb["win_len"]), csa2._p(rb["pool_row0"]),
                      csa2._p(rb["pool_len"]), None, None, int(pf["pool_len"]))
    sel_t = torch.empty_like(w.topk)
    topk = lambda: csa2.csa2_topk(w.dims, T, full, scores, stride, sel_t, stream=stream)  # noqa: E731
    for _ in range(max(args.warmup, 20)):
        topk()
    topk_us = timed(torch, topk, max(args.steps, 20), stream)
    del scores, sel_t
    step_us = step_medians(torch, w.prefill, min(args.steps, 20), stream)
    if args.copy_probe:
        copy_probe(torch)
    # entries per query: its window rows (128 everywhere here: the raw rows
    # reach 127 positions before the chunk) plus its 512 selected rows
    sel = w.topk.cpu().numpy()
    win_rows = T * d["window"]
    ent = win_rows + int((sel >= 0).sum())
    attn_flops = 4.0 * d["n_heads"] * d["head_dim"] * ent
    # indexer: one 128-long fp32 FMA chain per (query, reachable candidate)
    idx_flops = 2.0 * d["index_dim"] * sum(min(int(pf["pool_len"]), (int(pf["pos0"]) + t + 1) // int(pf["ratio"]))
                                           for t in range(T))
    achieved = attn_flops / (attn_us * 1e-6) / 1e12
    gather_bytes = ent * d["head_dim"] * 2 + T * d["n_heads"] * d["head_dim"] * (2 + 4)
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": prefill_desc(pf), "queries_per_step": T, "pool_rows": int(pf["pool_len"]),
                   "window": d["window"], "index_topk": d["index_topk"], "kv": "bf16", "index_keys": "fp32"},
        "roofline": {"bound": "mfma", "kernel": "attend_mq_kernel", "achieved": round(achieved, 1),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic_from_profile("attend"), "algorithmic_flops_per_launch": attn_flops,
                     "avg_launch_us": round(attn_us, 2)},
        # each stage timed alone: the attention (csa2_attend), the chunk's
        # scores (csa2_prefill_index_scores, with the 2-5 us descriptor
        # kernel), the top-K over them (csa2_topk); select = the step less the
        # attention
        "stages_us": {"attend": round(attn_us, 2), "select": round(1000.0 * ms_step - attn_us, 2),
                      "index_scores": round(scores_us, 2), "topk": round(topk_us, 2)},
        "index_scores_mfma": {"achieved": round(idx_flops / (scores_us * 1e-6) / 1e12, 1), "peak": FP32_MFMA_TFLOPS,
                              "unit": "TFLOP/s",
                              "frac": round(idx_flops / (scores_us * 1e-6) / 1e12 / FP32_MFMA_TFLOPS, 4)},
        # the same launch against HBM bandwidth, every entry's row counted once
        # per use (as if gathered from HBM) plus q and the fp32 output: most
        # rows in fact come from the last-level cache (a 16 MiB pool)
        "attend_gather": {"achieved": round(gather_bytes / (attn_us * 1e-6) / 1e9, 1), "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": round(gather_bytes / (attn_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                          "bytes_per_launch": gather_bytes},
        "output_derotation_us": {"attend_fused": round(attn_rope_us, 2), "attend_plain": round(attn_us, 2),
                                 "separate_pass": round(derot_us, 2)},
        "step_us": step_us,
        "gpu": torch.cuda.get_device_name(0),
    }
    del out, lse, ws
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import oracle as O
        say("timing the CPU oracle")
        per = 64
        cpu = cpu_baseline(lambda i: O.prefill_chunk(pf, (np.arange(per) + per * i) % T), per,
                           "the chunk (scores against the shared 16,384-row pool, top-512, attention)")
    del w
    torch.cuda.empty_cache()
    return line, cpu


# ---- decode batches ------------------------------------------------------------

def decode_desc(inp, storage):
    d = inp["dims"]
    kv = KV_NAMES[d["kv_dtype"]] if storage == "native" else KV_NAMES[2]
    keys = "fp32" if storage == "native" else "mxfp4 (e2m1 + e8m0/32)"
    B = int(inp["B"])
    modes = inp["mode"]
    if len(set(int(m) for m in modes)) == 1 and len(set(int(p) for p in inp["pos"])) == 1:
        what = (f"decode, {B} queries, context {int(inp['pos'][0]) + 1}, compress ratio {int(inp['ratio'][0])} -> "
                f"{int(inp['pool_len'][0])} candidates each")
    else:
        ctx = inp["pos"] + 1
        nf, nr, nw = (int((modes == m).sum()) for m in (0, 2, 3))
        full = modes == 0
        nv = [min(int(pl), (int(p) + 1) // int(r)) for pl, p, r in
              zip(inp["pool_len"][full], inp["pos"][full], inp["ratio"][full])]
        what = (f"decode, {B} mixed-mode queries ({nf} Full, {nr} Reuse, {nw} window-only), contexts "
                f"{int(ctx.min())}..{int(ctx.max())}, compress ratio 4 -> {min(nv)}..{max(nv)} candidates per "
                f"Full query")
    idx = f"{keys} indexer keys dim {d['index_dim']}"
    if d["index_heads"] > 1:
        idx += f", {d['index_heads']} ReLU index heads with per-head weights"
    return {"workload": f"{what}, window {d['window']}, top-{d['index_topk']}, {d['n_heads']} heads x "
                        f"{d['head_dim']}, {kv} KV, {idx}",
            "queries_per_step": B, "window": d["window"], "index_topk": d["index_topk"], "kv": kv,
            "index_keys": keys}


def restore_fp4(torch, csa2, w):
    """Re-store a bf16 workload's KV rows as FP4 and its index keys as MXFP4
    with the library's own quantizers (on the GPU, before timing)."""
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


def bench_decode(torch, stream, inp, storage, steps, warmup, copy_probe_run=False):
    from sparse_long_context_amd import csa2
    w = csa2.DecodeWorkload(inp)
    B = w.B
    if storage == "fp4":
        restore_fp4(torch, csa2, w)
    value, ms_step = headline_steps(torch, w.decode, B, steps, warmup, stream)
    # per-kernel durations: each stage entry point launched back to back
    # between two HIP events on the launch stream (the same kernels and
    # launch shapes csa2_decode issues)
    stride = (w.max_cand + 63) // 64 * 64  # the row stride csa2_decode uses for its own score buffer
    scores = torch.empty((B, max(stride, 1)), dtype=torch.float32, device="cuda")
    stages = {
        "index_scores": lambda: csa2.csa2_index_scores(w.dims, B, w.batch, w.idx_q, w.idx_w, w.idx_k, scores,
                                                       stride, idx_k_scale=w.idx_k_scale),
        "topk": lambda: csa2.csa2_topk(w.dims, B, w.batch, scores, stride, w.topk, workspace=w.ws,
                                       workspace_bytes=w.ws_bytes),
        "attend": lambda: csa2.csa2_attend(w.dims, B, w.batch, w.q, w.win_kv, w.win_scale, w.comp_kv, w.comp_scale,
                                           w.topk, w.sink, w.out, w.lse, w.ws, w.ws_bytes),
    }
    stage_us = {}
    for name, fn in stages.items():
        for _ in range(max(warmup, 20)):
            fn()
        stage_us[name] = timed(torch, fn, max(steps, 20), stream)
    step_us = step_medians(torch, w.decode, min(max(steps, 10), 20), stream)
    if copy_probe_run:
        copy_probe(torch)
    full = inp["mode"] == 0
    n_cand = int(sum(min(int(p), (int(pos) + 1) // int(r)) for p, pos, r in
                     zip(inp["pool_len"][full], inp["pos"][full], inp["ratio"][full])))
    key_bytes = MXFP4_KEY_BYTES if storage == "fp4" else INDEX_KEY_BYTES
    idx_bytes = n_cand * key_bytes + int(full.sum()) * INDEX_Q_BYTES
    achieved = idx_bytes / (stage_us["index_scores"] * 1e-6) / 1e9
    hi = int(inp["dims"]["index_heads"])
    idx_flops = 2.0 * 128 * hi * n_cand
    ent = 0
    for b in range(B):
        nv = min(int(inp["pool_len"][b]), (int(inp["pos"][b]) + 1) // max(int(inp["ratio"][b]), 1))
        m = int(inp["mode"][b])
        sel = min(512, nv) if m in (0, 1) else (int((inp["sel_in"][b] >= 0).sum()) if m == 2 else 0)
        ent += int(inp["win_len"][b]) + sel
    attn_flops = 4.0 * 64 * 512 * ent
    attend_tflops = attn_flops / (stage_us["attend"] * 1e-6) / 1e12
    res = {
        "value": round(value, 1), "unit": "queries/s", "ms_per_step": round(ms_step, 4),
        # the arithmetic: fp32 index scores (FP4 keys widened exactly), bf16
        # matrix products in the attention (fp8 / FP4 rows widened exactly)
        "dtype": "fp32+bf16", "config": decode_desc(inp, storage),
        "roofline": {"bound": "hbm", "kernel": "index_scores_decode" if storage == "native" else "index_scores_decode_mx",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_launch": idx_bytes,
                     "avg_launch_us": round(stage_us["index_scores"], 2)},
        "stages_us": {k: round(v, 2) for k, v in stage_us.items()},
        # the indexer's fixed-order fp32 chains (H_I x 128 FMAs per candidate)
        # against the fp32 matrix peak (they run on the matrix cores for
        # 17 to 32 heads, on the vector units otherwise)
        "index_scores_fp32": {"index_heads": hi, "achieved": round(idx_flops / (stage_us["index_scores"] * 1e-6) / 1e12, 2),
                              "peak": FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                              "frac": round(idx_flops / (stage_us["index_scores"] * 1e-6) / 1e12 / FP32_MFMA_TFLOPS, 4)},
        "attend_mfma": {"achieved": round(attend_tflops, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(attend_tflops / BF16_PEAK_TFLOPS, 4)},
        "step_us": step_us,
    }
    del w, scores
    torch.cuda.empty_cache()
    return res


EXTRAS = [("decode_full_64x16384", 1, "native"), ("decode_fp8_256x16384_ctx1M", 3, "native"),
          ("mixed_128_ragged", 4, "native"), ("decode_full_64x16384_fp4_storage", 1, "fp4")]


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2,
                    help="headline workload: 2 (the 4,096-query prefill chunk, default) or a decode batch 1, 3, 4")
    ap.add_argument("--storage", choices=("native", "fp4"), default="native",
                    help="with --config 1 or 4: KV rows re-stored as FP4 (E4M3 scale per 16) and index keys as "
                         "MXFP4, quantized on the GPU by the library's own quantizers before timing")
    ap.add_argument("--index-heads", type=int, default=1,
                    help="with --config 1, 3 or 4: the pages' indexer form (this many ReLU heads with drawn per-head "
                         "weights) instead of the workloads' one plain-dot head")
    ap.add_argument("--no-extras", action="store_true", help="time the headline workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain %d MiB fill and sum (for scaling rocprofv3 byte counters)" % (COPY_PROBE_BYTES >> 20))
    ap.add_argument("--gather-probe", action="store_true",
                    help="only measure the rate of random 1 KiB row gathers (libcsa2_probe.so) and print it")
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
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}); decode batches shard "
              "by sequence with no exchange, and a long sequence by pool position with one all-gather of "
              "(score, row) pairs and one merge of softmax partials, so each GPU would run this same step on "
              "its own share.", file=sys.stderr)
        sys.exit(2)
    if args.config not in (1, 2, 3, 4):
        print("bench.py times the workloads 1, 2, 3 or 4", file=sys.stderr)
        sys.exit(2)
    if args.index_heads != 1 and args.config == 2:
        print("--index-heads applies to the decode workloads (1, 3, 4)", file=sys.stderr)
        sys.exit(2)
    if args.storage == "fp4" and args.config not in (1, 4):
        print("--storage fp4 re-stores the bf16 decode workloads (1 or 4)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from sparse_long_context_amd import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.gather_probe:
        gather_probe(torch)
        return
    stream = torch.cuda.current_stream()

    if args.config == 2:
        line, cpu = bench_prefill(args, torch, stream)
    else:
        say(f"generating workload {args.config}")
        inp = synth.config(args.config, index_heads=args.index_heads)
        ramp_clocks(torch)
        res = bench_decode(torch, stream, inp, args.storage, args.steps, args.warmup, args.copy_probe)
        line = {"metric": METRIC, "value": res["value"], "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
                "warmup": args.warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True,
                "scaling": "weak", "vs_baseline": None, "dtype": res["dtype"], "data": "synthetic",
                "config": res["config"], "roofline": dict(res["roofline"]), "stages_us": res["stages_us"],
                "attend_mfma": res["attend_mfma"], "index_scores_fp32": res["index_scores_fp32"],
                "step_us": res["step_us"], "gpu": torch.cuda.get_device_name(0)}
        line["roofline"]["traffic"] = (traffic_from_profile("index")
                                       if (args.config == 1 and args.storage == "native" and args.index_heads == 1)
                                       else None)
        cpu = None
        if not args.no_cpu_baseline:
            from oracle import oracle as O
            say("timing the CPU oracle")
            per = min(64, int(inp["B"]))
            cpu = cpu_baseline(lambda i: O.decode_batch(inp, (np.arange(per) + per * i) % inp["B"]), per,
                               f"the {inp['B']}-query batch")
        del inp
    if cpu is not None:
        line["cpu_baseline"] = cpu

    if args.config == 2 and not args.no_extras:
        extras = {}
        for name, idx, storage in EXTRAS:
            try:
                say(f"extra workload {name}: generating")
                inp = synth.config(idx)
                extras[name] = bench_decode(torch, stream, inp, storage, max(args.steps, 20), max(args.warmup, 20))
                # the counters were taken on workload 1's indexer (fp32 keys)
                extras[name]["roofline"]["traffic"] = (traffic_from_profile("index")
                                                       if (idx == 1 and storage == "native") else None)
                del inp
            except Exception as e:  # an extra never hides the headline
                extras[name] = {"error": repr(e)}
            say(f"extra workload {name}: {json.dumps(extras[name].get('value'))} queries/s")
        line["workloads"] = extras
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
