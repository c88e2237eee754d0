"""GPU parity of the FP4 storage formats: FP4 main KV (E2M1 codes, one E4M3
scale per 16 values) and MXFP4 index keys (E2M1 codes, one E8M0 scale per 32).

The FP4 bytes every comparison uses are written by the oracle's quantizer from
fp32 values (the bf16 rows of the seeded workloads, widened), so both paths read
identical inputs.  The HIP quantizers are checked separately, byte for byte,
against the oracle's.  FP4 values are exact in bf16, so the attention meets
the bf16 bar (normwise 1e-2); index scores over the decoded keys, and hence
the selections, match bit for bit.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import oracle as O  # noqa: E402
from sparse_long_context_amd import csa2, synth  # noqa: E402
from parity_util import compare_decode as compare, compare_prefill  # noqa: E402

pytestmark = pytest.mark.gpu



def say(*a):
    print("[gpu-fp4]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa2.lib()
    yield
    torch.cuda.synchronize()


def with_fp4_kv(inp):
    """The batch with its bf16 KV rows re-stored as FP4 (oracle quantizer)."""
    out = dict(inp, dims=dict(inp["dims"], kv_dtype=synth.KV_FP4))
    for src, sc in (("win_kv", "win_scale"), ("comp_kv", "comp_scale")):
        codes, scales = O.quant_fp4kv(synth.bf16_bits_to_f32(inp[src]))
        out[src], out[sc] = codes, scales
    return out


def with_mxfp4_keys(inp):
    codes, scales = O.quant_mxfp4(inp["idx_k"])
    return dict(inp, idx_k=codes, idx_k_scale=scales, dims=dict(inp["dims"], index_key_dtype=synth.IDXK_MXFP4))


def run_decode(inp):
    w = csa2.DecodeWorkload(inp)
    w.decode()
    torch.cuda.synchronize()
    return w.topk.cpu().numpy(), w.out.cpu().numpy(), w.lse.cpu().numpy()


def small_dims(**kw):
    d = synth.default_dims()
    d.update(kw)
    return d


def test_quantizers_match_the_oracle_byte_for_byte():
    rng = np.random.default_rng(31)
    kv = (rng.standard_normal((777, 512)) * np.exp(rng.uniform(-7, 7, (777, 1)))).astype(np.float32)
    kv[5, 32:48] = 0.0                                   # all-zero block: scale 2^-9
    kv[6] *= 1e4                                         # amax / 6 above 448: saturating scale and codes
    s = np.float32(0.375)                                # exact E4M3; amax 6 s gives exactly this scale
    mids = np.array([6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0, 0.5],
                    np.float32)
    kv[7, :16] = mids * s                                # every E2M1 rounding tie, both signs
    keys = (rng.standard_normal((999, 128)) * np.exp(rng.uniform(-20, 20, (999, 1)))).astype(np.float32)
    keys[3, 32:64] = 0.0
    mids32 = np.concatenate([mids, mids[::-1]])
    keys[4, :32] = mids32 * np.float32(2.0 ** -3)        # amax / 6 = 2^-3 exactly: ties at the E8M0 scale
    for name, x, fn, oq, blk in (("fp4 kv", kv, csa2.csa2_quantize_fp4_kv, O.quant_fp4kv, 16),
                                 ("mxfp4", keys, csa2.csa2_quantize_mxfp4, O.quant_mxfp4, 32)):
        say(f"quantizer {name}: {x.shape}")
        src = torch.from_numpy(x).cuda()
        codes = torch.empty((x.shape[0], x.shape[1] // 2), dtype=torch.uint8, device="cuda")
        scales = torch.empty((x.shape[0], x.shape[1] // blk), dtype=torch.uint8, device="cuda")
        fn(x.shape[0], x.shape[1], src, codes, scales)
        torch.cuda.synchronize()
        c_o, s_o = oq(x)
        assert np.array_equal(scales.cpu().numpy(), s_o), name
        assert np.array_equal(codes.cpu().numpy(), c_o), name


def test_decode_fp4_kv_and_mxfp4_keys():
    ctx = [1000, 4096 + 4 * 300 + 3, 70001, 4 * 513, 2, 12345]
    inp = synth.decode_batch(32, ctx, [synth.MODE_FULL] * len(ctx), [4] * len(ctx), dims=small_dims())
    inp = with_mxfp4_keys(with_fp4_kv(inp))
    say("decode FP4 KV + MXFP4 keys, B =", inp["B"])
    sg, og, lg = run_decode(inp)
    say(f"  worst normwise error {compare(inp, sg, og, lg):.2e}")


def test_decode_fp4_kv_all_heads_kernel():
    # more than 64 queries: the all-heads kernel, entries split over workgroups
    ctx = [20000] * 3 + [300] * 63
    inp = synth.decode_batch(33, ctx, [0] * 3 + [3] * 63, [4] * 3 + [0] * 63, dims=small_dims())
    inp = with_fp4_kv(inp)
    say("decode FP4 KV, B =", inp["B"])
    sg, og, lg = run_decode(inp)
    compare(inp, sg, og, lg, queries=[0, 1, 2, 3, 65])


def test_decode_mxfp4_keys_reindex_and_heads():
    ctx = [9000, 9000, 9000, 300, 50000, 20000]
    modes = [0, 1, 2, 0, 1, 1]
    dims = small_dims(index_heads=3, index_relu=1)
    inp = synth.decode_batch(34, ctx, modes, [4] * len(ctx), dims=dims)
    synth.add_reindex_lists(inp, 34, frac=0.3)
    inp = with_mxfp4_keys(inp)
    say("decode MXFP4 keys, 3 ReLU index heads, Reindex lists")
    sg, og, lg = run_decode(inp)
    compare(inp, sg, og, lg)


def test_prefill_fp4_kv_and_mxfp4_keys():
    pos0, T, m = 6000, 300, 8
    pf = synth.prefill_chunk(35, T, pos0, m, (pos0 + T) // m, dims=small_dims(), win_pos0=pos0 - 40)
    pf = with_mxfp4_keys(with_fp4_kv(pf))
    say("prefill T=300 FP4 KV + MXFP4 keys")
    w = csa2.PrefillWorkload(pf)
    w.prefill()
    torch.cuda.synchronize()
    compare_prefill(pf, w.topk.cpu().numpy(), w.out.cpu().numpy(), w.lse.cpu().numpy())


def test_full_size_decode_fp4():
    """The 64-query, 16,384-candidate decode workload with its KV rows in FP4 and
    its index keys in MXFP4: the HIP quantizers reproduce the oracle's bytes at
    full size, and every query matches the oracle."""
    say("building config 1")
    inp = synth.config(1)
    for src, fn, blk, nb in (("comp_kv", csa2.csa2_quantize_fp4_kv, 16, 512), ("idx_k", csa2.csa2_quantize_mxfp4, 32, 128)):
        x = synth.bf16_bits_to_f32(inp[src]) if src == "comp_kv" else inp[src]
        rows = x.shape[0]
        say(f"quantizing {src} on the GPU: {rows} rows")
        xs = torch.from_numpy(np.ascontiguousarray(x)).cuda()
        codes = torch.empty((rows, nb // 2), dtype=torch.uint8, device="cuda")
        scales = torch.empty((rows, nb // blk), dtype=torch.uint8, device="cuda")
        fn(rows, nb, xs, codes, scales)
        torch.cuda.synchronize()
        c_g, s_g = codes.cpu().numpy(), scales.cpu().numpy()
        del xs, codes, scales
        torch.cuda.empty_cache()
        c_o, s_o = (O.quant_fp4kv if src == "comp_kv" else O.quant_mxfp4)(x)
        assert np.array_equal(s_g, s_o) and np.array_equal(c_g, c_o), src
        del c_g, s_g, c_o, s_o
    inp = with_mxfp4_keys(with_fp4_kv(inp))
    say("config 1 in FP4 / MXFP4: running")
    sg, og, lg = run_decode(inp)
    torch.cuda.empty_cache()
    say("oracle on all 64 queries")
    worst = compare(inp, sg, og, lg)
    say(f"  worst normwise error {worst:.2e}")
    for b in range(inp["B"]):
        v = sg[b][sg[b] >= 0]
        assert len(v) == 512 and (np.diff(v) > 0).all()
    assert np.isfinite(og).all()


def test_mxfp4_scores_at_extreme_scale_bytes():
    """MXFP4 index scores bit for bit against the oracle's fmaf chain over the
    decoded keys, with E8M0 scale bytes at both ends: 0 and 1 (products down to
    2^-128, subnormal), 2 and 252 (the first and last bytes whose products are
    all normal), 253 and 254 (codes kept at most 3 and 1.5, so the keys stay
    finite), among ordinary bytes near 127.  The query's last 32 dims (the
    block that carries the largest scales) are tiny, so no score overflows."""
    rng = np.random.default_rng(4711)
    ctx = [4 * 3000, 4 * 1500 + 3, 4 * 777]
    inp = synth.decode_batch(77, ctx, [synth.MODE_FULL] * 3, [4] * 3, dims=small_dims())
    rows = inp["idx_k"].shape[0]
    codes = rng.integers(0, 256, size=(rows, 64), dtype=np.uint8)
    scales = rng.integers(118, 136, size=(rows, 4), dtype=np.uint8)
    lowb = np.array([0, 1, 2], np.uint8)
    scales[:, :3] = np.where(rng.random((rows, 3)) < 0.4, rng.choice(lowb, size=(rows, 3)), scales[:, :3])
    top = rng.choice(np.array([252, 253, 254, 127], np.uint8), size=rows)
    scales[:, 3] = top
    # block 3 (bytes 48..63 of a row's codes): magnitude codes 0..5 (|v| <= 3)
    # under byte 253, 0..3 (|v| <= 1.5) under byte 254, so 6 * 2^126 and
    # 2 * 2^127 never occur
    blk3 = codes[:, 48:].copy()
    lo, hi = blk3 & 0xF, blk3 >> 4
    for lim, byte in ((5, 253), (3, 254)):
        sel = top == byte
        lo[sel] = (lo[sel] & 8) | np.minimum(lo[sel] & 7, lim)
        hi[sel] = (hi[sel] & 8) | np.minimum(hi[sel] & 7, lim)
    codes[:, 48:] = (hi << 4) | lo
    q = inp["idx_q"].copy()
    q[..., 96:] *= np.float32(2.0 ** -100)
    inp = dict(inp, idx_q=q, idx_k=codes, idx_k_scale=scales,
               dims=dict(inp["dims"], index_key_dtype=synth.IDXK_MXFP4))
    keys = O.dequant_mxfp4(codes, scales)
    assert np.isfinite(keys).all()
    w = csa2.DecodeWorkload(inp)
    stride = w.max_cand + 4
    sc = torch.full((w.B, stride), float("nan"), device="cuda")
    say("MXFP4 scores at scale bytes 0..2 and 252..254")
    csa2.csa2_index_scores(w.dims, w.B, w.batch, w.idx_q, w.idx_w, w.idx_k, sc, stride, idx_k_scale=w.idx_k_scale)
    torch.cuda.synchronize()
    got = sc.cpu().numpy()
    for b in range(w.B):
        p0, pl = int(inp["pool_row0"][b]), int(inp["pool_len"][b])
        nv = O.n_valid(inp["pos"][b], 4, synth.MODE_FULL, pl)
        ref, _, _ = O.index_scores(q[b].reshape(1, -1), keys[p0:p0 + pl], n=nv)
        assert np.isfinite(ref).all()
        assert got[b, :nv].tobytes() == ref.tobytes(), f"query {b}"
