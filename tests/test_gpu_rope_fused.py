"""GPU parity of the output de-rotation fused into the attention's writes
("DeepSeek-V4.1-Flash on WASTE", What is new, 1. CSA2: the rope dims of the
attention output turn back by the query's own rotation).

With a csa2_out_rope descriptor every output kernel writes its rope pairs
already turned: the all-heads bf16 kernel (unsplit, and split then merged),
the head-group fp8 / FP4 kernel, the all-heads fp8 / FP4 kernel (unsplit and
split), in decode and in prefill.  Each case must equal, bit for bit, the
unfused output turned afterwards by csa2_derotate (the two share one fp64
rotation), leave lse and the selections untouched, and match the oracle's
output de-rotated by the oracle within the parity tolerance.  The layouts
cover the model's (offset 448, 64 dims), one that crosses the 256-dim
boundary (192, 128), and one whose pairs start mid-column (254, 4).
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import oracle as O  # noqa: E402
from sparse_long_context_amd import csa2, synth  # noqa: E402
from parity_util import TOL, normwise  # noqa: E402

pytestmark = pytest.mark.gpu

LAYOUTS = [(448, 64), (192, 128), (254, 4)]


def say(*a):
    print("[gpu-rope]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa2.lib()
    yield
    torch.cuda.synchronize()


def inv_freq(dims):
    # plain RoPE schedule with theta 160,000 over the rope dims
    return 160000.0 ** (-np.arange(dims // 2, dtype=np.float64) * 2.0 / dims)


def with_fp4_kv(inp):
    out = dict(inp, dims=dict(inp["dims"], kv_dtype=synth.KV_FP4))
    for src, sc in (("win_kv", "win_scale"), ("comp_kv", "comp_scale")):
        codes, scales = O.quant_fp4kv(synth.bf16_bits_to_f32(inp[src]))
        out[src], out[sc] = codes, scales
    return out


def decode_inputs(kv, B, seed):
    ctx = synth.uniform_int(seed, 1, B, 1024, 262144)
    modes = [(synth.MODE_FULL, synth.MODE_REUSE, synth.MODE_WINDOW, synth.MODE_FULL)[i % 4] for i in range(B)]
    ratios = [4 if m != synth.MODE_WINDOW else 0 for m in modes]
    dims = synth.default_dims(kv_dtype=synth.KV_BF16 if kv == synth.KV_FP4 else kv)
    inp = synth.decode_batch(seed, ctx, modes, ratios, dims=dims, pool_cap=3000)
    return with_fp4_kv(inp) if kv == synth.KV_FP4 else inp


def fused_vs_separate(run, n, pos_t, dims, off, rd):
    """run(rope) -> (out, lse, sel) tensors; returns the fused output (numpy)."""
    inv = inv_freq(rd)
    inv_t = torch.from_numpy(inv).cuda()
    out0, lse0, sel0 = (x.clone() for x in run(None))
    torch.cuda.synchronize()
    out1, lse1, sel1 = run(csa2.out_rope(off, rd, inv_t))
    torch.cuda.synchronize()
    out1, lse1, sel1 = out1.clone(), lse1.clone(), sel1.clone()
    csa2.csa2_derotate(dims, n, pos_t, off, rd, inv_t, out0)
    torch.cuda.synchronize()
    a, b = out1.cpu().numpy(), out0.cpu().numpy()
    if not np.array_equal(a.view(np.uint32), b.view(np.uint32)):
        bad = np.argwhere(a.view(np.uint32) != b.view(np.uint32))
        raise AssertionError(f"fused output differs from the separate pass at {len(bad)} places, first {bad[:4]}")
    assert np.array_equal(lse1.cpu().numpy(), lse0.cpu().numpy())
    assert np.array_equal(sel1.cpu().numpy(), sel0.cpu().numpy())
    return a, inv


@pytest.mark.parametrize("kv,B,layout", [
    (synth.KV_BF16, 300, 0),   # all-heads bf16, unsplit
    (synth.KV_BF16, 24, 1),    # all-heads bf16, entries split and merged
    (synth.KV_FP8, 24, 2),     # head groups
    (synth.KV_FP8, 100, 0),    # all-heads fp8, split and merged
    (synth.KV_FP8, 300, 1),    # all-heads fp8, unsplit
    (synth.KV_FP4, 24, 1),     # head groups, FP4 rows
    (synth.KV_FP4, 300, 2),    # all-heads FP4, unsplit
])
def test_decode_fused_derotation(kv, B, layout):
    off, rd = LAYOUTS[layout]
    say(f"decode kv={kv} B={B} rope=({off},{rd})")
    inp = decode_inputs(kv, B, 70 + B + kv)
    w = csa2.DecodeWorkload(inp, sink=synth.normal_f32(71, 1, (64,)))

    def run(rope):
        w.decode(rope=rope)
        return w.out, w.lse, w.topk

    got, inv = fused_vs_separate(run, B, w.pos, w.dims, off, rd)
    qs = np.arange(0, B, max(1, B // 6))
    sel_o, out_o, _ = O.decode_batch(inp, qs, sink=synth.normal_f32(71, 1, (64,)))
    for i, b in enumerate(qs):
        want = O.derotate(out_o[i].astype(np.float32), int(inp["pos"][b]), inv, off, rd)
        err = normwise(got[b], want)
        assert err <= TOL[kv], f"query {b}: normwise error {err:.3e}"


@pytest.mark.parametrize("kv,T,layout", [
    (synth.KV_BF16, 300, 0),
    (synth.KV_BF16, 40, 1),
    (synth.KV_FP8, 160, 2),
])
def test_prefill_fused_derotation(kv, T, layout):
    off, rd = LAYOUTS[layout]
    say(f"prefill kv={kv} T={T} rope=({off},{rd})")
    pf = synth.prefill_chunk(80 + T, T, 20000, 4, 5000, dims=synth.default_dims(kv_dtype=kv))
    w = csa2.PrefillWorkload(pf)

    def run(rope):
        w.prefill(rope=rope)
        return w.out, w.lse, w.topk

    pos_t = torch.arange(pf["pos0"], pf["pos0"] + T, dtype=torch.int64, device="cuda")
    got, inv = fused_vs_separate(run, T, pos_t, w.dims, off, rd)
    qs = np.array([0, T // 2, T - 1])
    _, out_o, _ = O.prefill_chunk(pf, qs)
    for i, t in enumerate(qs):
        want = O.derotate(out_o[i].astype(np.float32), int(pf["pos0"] + t), inv, off, rd)
        err = normwise(got[t], want)
        assert err <= TOL[kv], f"query {t}: normwise error {err:.3e}"


def test_attend_fused_derotation_needs_a_workspace():
    # csa2_attend: with no workspace every query runs unsplit and a rope
    # descriptor is refused; with csa2_workspace_size(dims, B, 0) bytes the
    # output leaves de-rotated
    off, rd = LAYOUTS[0]
    inp = decode_inputs(synth.KV_BF16, 20, 90)
    w = csa2.DecodeWorkload(inp)
    w.decode()
    torch.cuda.synchronize()
    inv_t = torch.from_numpy(inv_freq(rd)).cuda()
    with pytest.raises(csa2.Csa2Error) as e:
        csa2.csa2_attend(w.dims, w.B, w.batch, w.q, w.win_kv, w.win_scale, w.comp_kv, w.comp_scale, w.topk, w.sink,
                         w.out, w.lse, None, 0, rope=csa2.out_rope(off, rd, inv_t))
    assert e.value.status == csa2.CSA2_ERR_WORKSPACE
    nbytes = csa2.csa2_workspace_size(w.dims, w.B, 0)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def run(rope):
        csa2.csa2_attend(w.dims, w.B, w.batch, w.q, w.win_kv, w.win_scale, w.comp_kv, w.comp_scale, w.topk, w.sink,
                         w.out, w.lse, ws, nbytes, rope=rope)
        return w.out, w.lse, w.topk

    fused_vs_separate(run, w.B, w.pos, w.dims, off, rd)
