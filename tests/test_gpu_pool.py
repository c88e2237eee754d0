"""GPU parity of the hierarchical candidate pool (Reading Notes of
DeepSeek-V4.1-Flash, 3f C3; PocketLLM page, the candidate source layer's
block selection with the still-filling block pinned): the pool lists must
match the oracle's exactly, and a Reindex layer searching them must match the
oracle end to end."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import oracle as O  # noqa: E402
from sparse_long_context_amd import csa2, synth  # noqa: E402

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-pool]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa2.lib()
    yield
    torch.cuda.synchronize()


def gpu_pool(w, bs, top):
    B, stride = w.B, w.max_cand
    scores = torch.empty((B, stride), dtype=torch.float32, device="cuda")
    csa2.csa2_index_scores(w.dims, B, w.batch, w.idx_q, w.idx_w, w.idx_k, scores, stride, idx_k_scale=w.idx_k_scale)
    ws_bytes = csa2.csa2_candidate_pool_workspace_size(B, w.max_cand, bs, top)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    off = torch.empty(B + 1, dtype=torch.int64, device="cuda")
    idx = torch.empty((B, bs * top), dtype=torch.int32, device="cuda")
    csa2.csa2_candidate_pool(B, w.batch, scores, stride, bs, top, off, idx, ws, ws_bytes)
    torch.cuda.synchronize()
    return off.cpu().numpy(), idx.cpu().numpy()


def oracle_pool(inp, b, bs, top):
    n = O.n_valid(inp["pos"][b], inp["ratio"][b], inp["mode"][b], inp["pool_len"][b])
    r0 = int(inp["pool_row0"][b])
    s32, _, _ = O.index_scores(inp["idx_q"][b].reshape(1, -1), inp["idx_k"][r0:r0 + n] if n else
                               np.zeros((1, 128), np.float32), n=n)
    return O.candidate_pool(s32[:n], bs, top)


@pytest.mark.parametrize("bs,top", [(8, 2048), (4, 3), (8, 100)])
def test_candidate_pool_matches_oracle(bs, top):
    # entry counts around block boundaries, below one block, and (with ratio 4
    # at 600,000) 150,000 entries = 18,750 blocks, past the register top-k
    ctx = [4 * 17 + 3, 4 * 64, 4 * 5, 4 * 1000 + 7, 600_000, 4 * 16384 + 8, 3]
    modes = [0, 0, 0, 0, 0, 0, 0]
    inp = synth.decode_batch(41, ctx, modes, [4] * len(ctx), dims=synth.default_dims())
    inp = dict(inp)
    # a Reuse query in the batch gets an empty pool
    inp["mode"] = inp["mode"].copy()
    inp["mode"][2] = synth.MODE_REUSE
    w = csa2.DecodeWorkload(inp)
    say(f"pool bs={bs} top={top}, entries", [O.n_valid(p, r, m, l) for p, r, m, l in
                                            zip(inp["pos"], inp["ratio"], inp["mode"], inp["pool_len"])])
    off, idx = gpu_pool(w, bs, top)
    cap = bs * top
    assert np.array_equal(off, np.arange(w.B + 1) * cap)
    for b in range(w.B):
        if inp["mode"][b] != synth.MODE_FULL:
            assert (idx[b] == -1).all()
            continue
        want = oracle_pool(inp, b, bs, top)
        assert np.array_equal(idx[b], want), f"query {b}"


def test_reindex_layer_over_the_pool():
    """Layer 1 (Full) builds the pool; layer 2 (Reindex, its own index queries)
    selects its top-512 inside it and attends: parity with the oracle running
    the same two steps."""
    ctx = [4 * 20000 + 5, 4 * 3000, 4 * 9001 + 2]
    inp = synth.decode_batch(42, ctx, [0] * 3, [4] * 3, dims=synth.default_dims())
    w = csa2.DecodeWorkload(inp)
    off, idx = gpu_pool(w, 8, 256)  # 2,048-entry pools: narrower than the reachable range
    lists_o = [oracle_pool(inp, b, 8, 256) for b in range(3)]
    for b in range(3):
        assert np.array_equal(idx[b], lists_o[b])
    # layer 2: Reindex over the pool with fresh index queries
    l2 = dict(inp)
    l2["mode"] = np.full(3, synth.MODE_REINDEX, np.int32)
    l2["idx_q"] = synth.normal_f32(42, 900, inp["idx_q"].shape)
    l2["cand_off"] = np.arange(4, dtype=np.int64) * 2048
    l2["cand_idx"] = np.concatenate(lists_o).astype(np.int32)
    w2 = csa2.DecodeWorkload(l2)
    w2.decode()
    torch.cuda.synchronize()
    sel_o, out_o, lse_o = O.decode_batch(l2)
    sg, og = w2.topk.cpu().numpy(), w2.out.cpu().numpy()
    for b in range(3):
        assert np.array_equal(sg[b], sel_o[b])
        assert set(sg[b][sg[b] >= 0]) <= set(lists_o[b][lists_o[b] >= 0])
        err = float(np.abs(og[b] - out_o[b]).max()) / float(np.abs(out_o[b]).max())
        assert err <= 1e-2
