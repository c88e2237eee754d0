"""Runs the oracle and the synthetic generator over small cases that reach
every entry point, under the sanitized builds that test_sanitizers_cpu.py
makes (it sets CSA2_ORACLE_LIB / CSA2_SYNTH_LIB and preloads the sanitizer
runtime).  Any sanitizer finding aborts the process."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import oracle as O  # noqa: E402
from sparse_long_context_amd import synth  # noqa: E402

assert O.LIB_PATH == os.environ["CSA2_ORACLE_LIB"] and synth.SYNTH_LIB == os.environ["CSA2_SYNTH_LIB"]


def step(name):
    print("exercise:", name, flush=True)


def fp4(inp):
    out = dict(inp, dims=dict(inp["dims"], kv_dtype=synth.KV_FP4))
    for src, sc in (("win_kv", "win_scale"), ("comp_kv", "comp_scale")):
        out[src], out[sc] = O.quant_fp4kv(synth.bf16_bits_to_f32(inp[src]))
    return out


step("decode batches: four modes, bf16 / fp8 / FP4 rows, sink, scale, weights, ReLU heads, Reindex lists")
ctx = [1, 5, 40, 300, 1000, 2000, 77, 513]
modes = [synth.MODE_FULL, synth.MODE_REINDEX, synth.MODE_REUSE, synth.MODE_WINDOW] * 2
ratios = [4, 4, 4, 0, 8, 4, 4, 0]
for kv in (synth.KV_BF16, synth.KV_FP8):
    dims = synth.default_dims(kv_dtype=kv, index_heads=4, index_relu=1, index_topk=16, window=8)
    inp = synth.add_reindex_lists(synth.decode_batch(7, ctx, modes, ratios, dims=dims, weights=True), 7)
    for case in ([inp, fp4(inp)] if kv == synth.KV_BF16 else [inp]):
        sel, out, lse = O.decode_batch(case, np.arange(len(ctx)), sink=np.linspace(-1, 1, 64).astype(np.float32),
                                       scale=0.5)
        assert np.isfinite(out).all()

step("prefill chunks: Full with a replay cut, Window")
dims = synth.default_dims(index_topk=16, window=8)
pf = synth.prefill_chunk(8, 12, 40, 4, 11, dims=dims, win_pos0=36)
O.prefill_chunk(pf)
O.prefill_chunk(dict(pf, mode=synth.MODE_WINDOW))

step("top-k with ties and -0, candidate pool, compressor and its decode step, de-rotation")
rng = np.random.default_rng(1)
sc = rng.integers(-3, 3, 500).astype(np.float32)
sc[::7] = -0.0
O.topk(sc, 37, 400)
O.candidate_pool(rng.standard_normal(300).astype(np.float32), 16, 4)
c = rng.standard_normal((12, 24)).astype(np.float32)
g = rng.standard_normal((12, 24)).astype(np.float32)
w = np.ones(24, np.float32)
O.compress(c, g, w, 4)
kvs = np.zeros((2, 4, 24), np.float32)
scs = np.zeros((2, 4, 24), np.float32)
out = np.zeros((2, 24), np.float32)
for p in range(6):
    O.compress_step(np.array([p, p + 3]), c[[p, p + 3]], g[[p, p + 3]], kvs, scs, w, 4, out)
O.derotate(rng.standard_normal((4, 64)).astype(np.float32), 1234, 0.5 ** np.arange(4), 56, 8)

step("quantizers and decoders")
x = (rng.standard_normal((3, 64)) * np.array([1e-8, 1.0, 1e4])[:, None]).astype(np.float32)
O.quant_fp4kv(x)
codes, scales = O.quant_mxfp4(x)
O.dequant_mxfp4(codes, scales)
print("exercise: done", flush=True)
