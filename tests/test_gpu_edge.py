"""GPU parity of the boundary's edge cases and of the pages' own indexer form.

* Every Full / Reindex row of topk_idx is written, also when nothing can be
  scored (max_candidates 0, an empty pool): all -1, attention over the window.
* A Reindex query in a batch without lists scores an empty list.
* fp8 scale bytes 0, 1 and 2 (2^-127 .. 2^-125) decode like any other.
* The lightning indexer of the pages ("Reading Notes of DeepSeek-V4.1-Flash",
  3f C2 Step 2): several index heads, ReLU, per-head weights, fp32 keys, in
  decode and in prefill; scores bit-exact, selections bit-exact.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import oracle as O  # noqa: E402
from sparse_long_context_amd import csa2, synth  # noqa: E402
from parity_util import compare_decode, compare_prefill, normwise  # noqa: E402

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-edge]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa2.lib()
    yield
    torch.cuda.synchronize()


def dims(**kw):
    d = synth.default_dims()
    d.update(kw)
    return d


def window_only_reference(inp, b):
    w0, wl = int(inp["win_row0"][b]), int(inp["win_len"][b])
    sc = inp.get("win_scale")
    return O.attend_query(inp["q"][b], inp["win_kv"][w0:w0 + wl], None, None, kv_dtype=inp["dims"]["kv_dtype"],
                          win_scales=None if sc is None else sc[w0:w0 + wl])


@pytest.mark.parametrize("kv", [synth.KV_BF16, synth.KV_FP8])
def test_decode_topk_written_when_nothing_is_scored(kv):
    # max_candidates = 0 although the pools hold rows: no candidate is
    # considered, so the selections are all -1 whatever the buffer held before
    inp = synth.decode_batch(81 + kv, [5000, 3000, 700], [0, 1, 0], [4, 4, 4], dims=dims(kv_dtype=kv))
    synth.add_reindex_lists(inp, 81)
    w = csa2.DecodeWorkload(inp)
    w.batch.max_candidates = 0
    w.topk.copy_(torch.arange(512, dtype=torch.int32, device="cuda").expand(w.B, 512))
    say("decode, max_candidates 0, kv", kv)
    w.decode()
    torch.cuda.synchronize()
    sel, out = w.topk.cpu().numpy(), w.out.cpu().numpy()
    assert (sel == -1).all()
    for b in range(w.B):
        ref, _ = window_only_reference(inp, b)
        assert normwise(out[b], ref) <= 1e-2 if kv == synth.KV_BF16 else 3e-2


def test_prefill_topk_written_with_an_empty_pool():
    pos0, T = 2000, 70
    pf = synth.prefill_chunk(83, T, pos0, 4, 0, dims=dims())  # Full mode, pool of 0 rows
    w = csa2.PrefillWorkload(pf)
    w.topk.copy_(torch.arange(512, dtype=torch.int32, device="cuda").expand(T, 512))
    say("prefill, empty pool")
    w.prefill()
    torch.cuda.synchronize()
    assert (w.topk.cpu().numpy() == -1).all()
    compare_prefill(pf, w.topk.cpu().numpy(), w.out.cpu().numpy(), w.lse.cpu().numpy())


def test_reindex_query_without_lists_is_an_empty_list():
    inp = synth.decode_batch(84, [4000, 4000], [0, 1], [4, 4], dims=dims())
    w = csa2.DecodeWorkload(inp)  # no cand_off / cand_idx: the Reindex query has no list
    assert w.cand_off is None
    w.topk.copy_(torch.arange(512, dtype=torch.int32, device="cuda").expand(w.B, 512))
    say("Reindex query with NULL lists")
    w.decode()
    torch.cuda.synchronize()
    sel, out = w.topk.cpu().numpy(), w.out.cpu().numpy()
    assert (sel[1] == -1).all()
    ref, _ = window_only_reference(inp, 1)
    assert normwise(out[1], ref) <= 1e-2
    compare_decode(inp, sel, out, w.lse.cpu().numpy(), queries=[0])


@pytest.mark.parametrize("B", [8, 70])  # four head-group workgroups per query; all-heads workgroups
def test_fp8_scale_bytes_0_1_2(B):
    """Reuse queries without window rows whose selected rows carry the smallest
    UE8M0 scales (2^-127 .. 2^-125): the output is a weighted mean of those rows,
    so it is exactly as small and any mis-decoded scale shows at full size."""
    n = 3 * B
    inp = synth.decode_batch(85, [4 * n] * B, [synth.MODE_REUSE] * B, [4] * B, dims=dims(kv_dtype=synth.KV_FP8),
                             win_len=[0] * B, pool_cap=n)
    rng = np.random.default_rng(85)
    sel = np.full((B, 512), -1, np.int32)
    for b in range(B):
        k = 1 + b % 3  # one, two or three entries
        sel[b, :k] = np.sort(rng.choice(n, size=k, replace=False))
    inp["sel_in"] = sel
    sc = inp["comp_scale"]
    sc[:] = rng.integers(0, 3, size=sc.shape, dtype=np.uint8)  # bytes 0, 1, 2 only
    say(f"fp8 scale bytes 0..2, B={B}")
    w = csa2.DecodeWorkload(inp)
    w.decode()
    torch.cuda.synchronize()
    out = w.out.cpu().numpy()
    assert np.abs(out).max() < 2.0 ** -110 and np.abs(out).max() > 0
    compare_decode(inp, w.topk.cpu().numpy(), out, w.lse.cpu().numpy())


@pytest.mark.parametrize("hi", [4, 16, 32])
def test_indexer_heads_relu_weights_decode(hi):
    """H_I heads, ReLU, per-head weights drawn N(0, 1), fp32 keys: scores equal
    the oracle's bit for bit (Full and Reindex), and the whole step matches."""
    ctx = [4096 + 4 * 37, 999, 20000, 3, 9000, 65536]
    modes = [0, 1, 0, 0, 1, 0]
    inp = synth.decode_batch(90 + hi, ctx, modes, [4] * len(ctx), dims=dims(index_heads=hi, index_relu=1),
                             weights=True)
    synth.add_reindex_lists(inp, 90 + hi, frac=0.4)
    say(f"indexer {hi} heads, ReLU, weights")
    w = csa2.DecodeWorkload(inp)
    stride = w.max_cand + 5
    scores = torch.full((w.B, stride), float("nan"), device="cuda")
    csa2.csa2_index_scores(w.dims, w.B, w.batch, w.idx_q, w.idx_w, w.idx_k, scores, stride)
    torch.cuda.synchronize()
    sg = scores.cpu().numpy()
    for b in range(w.B):
        p0, pl = int(inp["pool_row0"][b]), int(inp["pool_len"][b])
        keys = inp["idx_k"][p0:p0 + pl]
        nv = O.n_valid(inp["pos"][b], 4, modes[b], pl)
        if modes[b] == 0:
            ref, _, _ = O.index_scores(inp["idx_q"][b], keys, w=inp["idx_w"][b], relu=True, n=nv)
            got = sg[b, :nv]
        else:
            lst = inp["cand_idx"][inp["cand_off"][b]:inp["cand_off"][b + 1]]
            ref, _, _ = O.index_scores(inp["idx_q"][b], keys, w=inp["idx_w"][b], relu=True, cand=lst)
            ref = np.where(lst < nv, ref, -np.inf).astype(np.float32)
            got = sg[b, :len(lst)]
        assert got.tobytes() == ref.tobytes(), f"query {b}"
    w.decode()
    torch.cuda.synchronize()
    compare_decode(inp, w.topk.cpu().numpy(), w.out.cpu().numpy(), w.lse.cpu().numpy())


@pytest.mark.parametrize("hi,mode", [(32, synth.MODE_FULL), (4, synth.MODE_REINDEX), (1, synth.MODE_FULL)])
def test_indexer_heads_relu_weights_prefill(hi, mode):
    pos0, T, m = 6000, 300, 8
    pool = (pos0 + T) // m
    pf = synth.prefill_chunk(95 + hi, T, pos0, m, pool, dims=dims(index_heads=hi, index_relu=1), mode=mode,
                             weights=True, win_pos0=pos0 - 50)
    if mode == synth.MODE_REINDEX:
        offs, parts = np.zeros(T + 1, np.int64), []
        for t in range(T):
            s = synth.sample_distinct(95, 3000 + t, pool, 600)
            parts.append(s)
            offs[t + 1] = offs[t] + len(s)
        pf["cand_off"], pf["cand_idx"] = offs, np.concatenate(parts).astype(np.int32)
    say(f"prefill indexer {hi} heads, ReLU, weights, mode {mode}")
    w = csa2.PrefillWorkload(pf)
    w.prefill()
    torch.cuda.synchronize()
    compare_prefill(pf, w.topk.cpu().numpy(), w.out.cpu().numpy(), w.lse.cpu().numpy())


def _prefill_scores(pf):
    w = csa2.PrefillWorkload(pf)
    pool = int(pf["pool_len"])
    stride = (pool + 3) // 4 * 4 + 4  # a multiple of 4 past the cap, so slots after it are checked
    scores = torch.full((w.T, stride), float("nan"), device="cuda")
    w.index_scores(scores, stride)
    torch.cuda.synchronize()
    return scores.cpu().numpy()


@pytest.mark.parametrize("relu,weights,T", [(0, False, 300), (1, True, 300), (0, False, 129)])
def test_prefill_index_scores_bit_exact(relu, weights, T):
    """The chunk's matrix-core scores equal the oracle's fixed-order fp32
    scores bit for bit, over ragged query and candidate tiles, with the causal
    limit per query (slots past it untouched)."""
    pos0, m = 6003, 8
    pool = (pos0 + T) // m  # the last queries reach every row, the first ones fewer
    pf = synth.prefill_chunk(120 + relu, T, pos0, m, pool, dims=dims(index_relu=relu), weights=weights)
    say(f"prefill scores T={T} pool={pool} relu={relu} weights={weights}")
    sg = _prefill_scores(pf)
    for t in range(T):
        nv = O.n_valid(pos0 + t, m, 0, pool)
        ref, _, _ = O.index_scores(pf["idx_q"][t], pf["idx_k"], w=None if pf["idx_w"] is None else pf["idx_w"][t],
                                   relu=bool(relu), n=nv)
        assert sg[t, :nv].tobytes() == ref.tobytes(), f"query {t}"
        assert np.isnan(sg[t, nv:]).all(), f"query {t}: slots past its reachable count were written"


def test_prefill_index_scores_full_size_sampled():
    """The 4,096-query chunk (several tiles per workgroup): the scores of two
    whole 128-query bands and the first and last query of every other band
    against the oracle's, bit for bit."""
    pf = synth.config(2)
    say("prefill scores, 4,096 x 16,384")
    sg = _prefill_scores(pf)
    qs = sorted({0, 1, 4095, 4094} | {128 * k for k in range(0, 32, 2)} | {128 * k + 127 for k in range(1, 32, 2)}
                | set(range(1920, 2048)) | set(range(3968, 4096)))
    for t in qs:
        nv = O.n_valid(int(pf["pos0"]) + t, 8, 0, 16384)
        ref, _, _ = O.index_scores(pf["idx_q"][t], pf["idx_k"], n=nv)
        assert sg[t, :nv].tobytes() == ref.tobytes(), f"query {t}"


@pytest.mark.parametrize("kind", ["denormal_sums", "large", "cancelling", "small_integers"])
def test_prefill_index_scores_adversarial_bit_exact(kind):
    """The chunk's matrix-core chain against the oracle's fmaf chain where a
    single rounding per step matters most: partial sums in the fp32 denormal
    range, magnitudes near 2^110, pairs that cancel to the last bit, and small
    integers whose sums are exact."""
    pos0, T, m = 5000, 260, 4
    pool = (pos0 + T) // m
    pf = synth.prefill_chunk(130, T, pos0, m, pool, dims=dims())
    q, k = pf["idx_q"].astype(np.float64), pf["idx_k"].astype(np.float64)
    if kind == "denormal_sums":
        q, k = q * 2.0 ** -64, k * 2.0 ** -66
    elif kind == "large":
        q, k = q * 2.0 ** 56, k * 2.0 ** 54
    elif kind == "cancelling":
        k[:, 1::2] = k[:, 0::2] * (1.0 + 2.0 ** -20)
        q[:, 1::2] = -q[:, 0::2]
    else:
        q, k = np.trunc(q * 8), np.trunc(k * 8)
    pf["idx_q"], pf["idx_k"] = q.astype(np.float32), k.astype(np.float32)
    say(f"prefill scores, adversarial inputs: {kind}")
    sg = _prefill_scores(pf)
    for t in range(T):
        nv = O.n_valid(pos0 + t, m, 0, pool)
        ref, _, _ = O.index_scores(pf["idx_q"][t], pf["idx_k"], n=nv)
        assert sg[t, :nv].tobytes() == ref.tobytes(), f"query {t}"
