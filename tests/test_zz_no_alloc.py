"""csa2_decode_static, the decode entry point that allocates nothing (its
scratch is the library's static device array): through the C ABI, two calls in
a row, the second with a smaller batch, each equal to csa2_decode's results on
the same inputs (selections, outputs and log-sum-exps bit for bit) and to the
oracle's within the parity bar; a batch whose scratch would exceed the static
size is refused before anything runs."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from sparse_long_context_amd import csa2, synth  # noqa: E402
from parity_util import compare_decode  # noqa: E402

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-no-alloc]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa2.lib()
    yield
    torch.cuda.synchronize()


def run_static(w):
    csa2.csa2_decode_static(w.dims, w.B, w.batch, w.q, w.idx_q, w.idx_w, w.idx_k, w.win_kv, w.win_scale, w.comp_kv,
                            w.comp_scale, w.topk, w.sink, w.out, w.lse, idx_k_scale=w.idx_k_scale)


def batch_of(seed, B, kv):
    ctx = synth.uniform_int(seed, 99, B, 300, 120000)
    modes = [(0, 1, 2, 3)[i % 4] for i in range(B)]
    ratios = [0 if m == 3 else 4 for m in modes]
    inp = synth.decode_batch(seed, ctx, modes, ratios, dims=synth.default_dims(kv_dtype=kv))
    return synth.add_reindex_lists(inp, seed, frac=0.3)


@pytest.mark.parametrize("kv", [synth.KV_BF16, synth.KV_FP8])
def test_static_scratch_matches_decode_twice(kv):
    # bf16: both batches split their entries (partials in the scratch); fp8:
    # 70 queries take the all-heads kernel with splits, 6 the head groups
    for i, B in enumerate((40, 6) if kv == synth.KV_BF16 else (70, 6)):  # the second call smaller
        inp = batch_of(110 + 10 * kv + i, B, kv)
        w = csa2.DecodeWorkload(inp)
        assert csa2.csa2_workspace_size(w.dims, w.B, w.max_cand) <= csa2.CSA2_STATIC_SCRATCH_BYTES
        say(f"kv {kv} call {i}: B={B}, max candidates {w.max_cand}")
        w.decode()
        torch.cuda.synchronize()
        ref = (w.topk.clone(), w.out.clone(), w.lse.clone())
        stale = ref[0].cpu().numpy().copy()
        stale[np.isin(inp["mode"], (0, 1))] = -7  # rows the call must write
        w.topk.copy_(torch.from_numpy(stale))
        w.out.fill_(float("nan"))
        w.lse.fill_(float("nan"))
        run_static(w)
        torch.cuda.synchronize()
        assert torch.equal(w.topk, ref[0])
        assert torch.equal(w.out, ref[1]) and torch.equal(w.lse.nan_to_num(), ref[2].nan_to_num())
        compare_decode(inp, w.topk.cpu().numpy(), w.out.cpu().numpy(), w.lse.cpu().numpy())


def test_static_scratch_refuses_a_batch_past_its_size():
    d = csa2.Dims.from_dict(synth.default_dims())
    fake = 0x1000  # never dereferenced: the size check fails before any launch
    b = csa2.Batch(fake, fake, fake, fake, fake, fake, fake, None, None, 16384)
    B = 1100  # 1,100 x 16,384 fp32 scores = 72 MB > 64 MiB
    assert csa2.csa2_workspace_size(d, B, 16384) > csa2.CSA2_STATIC_SCRATCH_BYTES
    st = csa2.lib().csa2_decode_static(csa2.C.byref(d), B, csa2.C.byref(b), fake, fake, None, fake, None, fake, None,
                                       fake, None, fake, None, fake, None, None, None)
    assert st == csa2.CSA2_ERR_WORKSPACE
