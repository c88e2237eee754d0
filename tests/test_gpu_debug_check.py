"""The device-side precondition check (CSA2_DEBUG_CHECK=1, include/csa2.h):
a clean call gives the release results; each broken precondition returns
CSA2_ERR_PRECONDITION with its bit and leaves the outputs untouched (nothing
but the check ran).  Every broken value here is one the check reads before any
compute kernel would: no kernel reads outside the rows its descriptors name."""
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from sparse_long_context_amd import csa2, synth  # noqa: E402

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-debug-check]", *a, file=sys.stderr, flush=True)


@pytest.fixture(autouse=True)
def _debug_on():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa2.lib()
    old = os.environ.get("CSA2_DEBUG_CHECK")
    os.environ["CSA2_DEBUG_CHECK"] = "1"
    yield
    if old is None:
        del os.environ["CSA2_DEBUG_CHECK"]
    else:
        os.environ["CSA2_DEBUG_CHECK"] = old
    torch.cuda.synchronize()


def workload(kv=synth.KV_BF16, seed=101):
    dims = synth.default_dims(kv_dtype=kv)
    inp = synth.decode_batch(seed, [5000, 3000, 900, 400], [0, 1, 2, 3], [4, 4, 4, 0], dims=dims)
    synth.add_reindex_lists(inp, seed)
    return inp


def expect_refused(w, bit, call=None):
    w.out.fill_(float("nan"))
    with pytest.raises(csa2.Csa2Error) as e:
        (call or w.decode)()
    assert e.value.status == csa2.CSA2_ERR_PRECONDITION
    assert csa2.csa2_last_precondition() & bit, hex(csa2.csa2_last_precondition())
    torch.cuda.synchronize()
    assert torch.isnan(w.out).all()  # untouched


def test_clean_call_matches_release():
    inp = workload()
    w = csa2.DecodeWorkload(inp)
    say("clean decode under the check")
    w.decode()
    torch.cuda.synchronize()
    assert csa2.csa2_last_precondition() == 0
    o1, s1 = w.out.clone(), w.topk.clone()
    del os.environ["CSA2_DEBUG_CHECK"]
    w.decode()
    torch.cuda.synchronize()
    os.environ["CSA2_DEBUG_CHECK"] = "1"
    assert torch.equal(o1, w.out) and torch.equal(s1, w.topk)


def test_bad_mode():
    inp = workload()
    inp["mode"] = inp["mode"].copy()
    inp["mode"][3] = 7
    say("mode 7")
    expect_refused(csa2.DecodeWorkload(inp), csa2.CSA2_PRE_MODE)


def test_window_longer_than_the_window_size():
    inp = workload()
    inp["win_len"] = inp["win_len"].copy()
    inp["win_len"][0] = 129
    say("win_len 129")
    expect_refused(csa2.DecodeWorkload(inp), csa2.CSA2_PRE_DESC)


def test_reindex_list_out_of_order():
    inp = workload()
    o0, o1 = inp["cand_off"][1], inp["cand_off"][2]
    assert o1 - o0 >= 2
    inp["cand_idx"] = inp["cand_idx"].copy()
    inp["cand_idx"][o0], inp["cand_idx"][o0 + 1] = inp["cand_idx"][o0 + 1], inp["cand_idx"][o0]
    say("Reindex list swapped")
    expect_refused(csa2.DecodeWorkload(inp), csa2.CSA2_PRE_LIST)


def test_reuse_selection_past_the_pool():
    inp = workload()
    inp["sel_in"] = inp["sel_in"].copy()
    inp["sel_in"][2, 0] = int(inp["pool_len"][2])  # one past the last row
    say("Reuse index = pool_len")
    expect_refused(csa2.DecodeWorkload(inp), csa2.CSA2_PRE_SEL)


def test_attend_checks_every_attended_selection():
    inp = workload()
    w = csa2.DecodeWorkload(inp)
    w.decode()
    w.topk[0, 5] = -2
    say("attend with a -2 entry")
    expect_refused(w, csa2.CSA2_PRE_SEL, call=lambda: csa2.csa2_attend(
        w.dims, w.B, w.batch, w.q, w.win_kv, w.win_scale, w.comp_kv, w.comp_scale, w.topk, None, w.out, w.lse,
        w.ws, w.ws_bytes))


def test_fp8_scale_byte_255_in_a_window_row():
    inp = workload(kv=synth.KV_FP8)
    inp["win_scale"] = inp["win_scale"].copy()
    inp["win_scale"][int(inp["win_row0"][1]) + 3, 7] = 255
    say("fp8 window scale 255")
    expect_refused(csa2.DecodeWorkload(inp), csa2.CSA2_PRE_KV_SCALE)


def test_non_finite_index_key():
    inp = workload()
    inp["idx_k"] = inp["idx_k"].copy()
    inp["idx_k"][int(inp["pool_row0"][0]) + 17, 3] = np.inf
    say("index key inf")
    expect_refused(csa2.DecodeWorkload(inp), csa2.CSA2_PRE_INDEX)


def test_prefill_reuse_selection_checked():
    pos0, T = 3000, 40
    pf = synth.prefill_chunk(102, T, pos0, 4, (pos0 + T) // 4, mode=synth.MODE_REUSE)
    sel = np.full((T, 512), -1, np.int32)
    sel[:, :10] = np.arange(10)
    sel[7, 3] = 10 ** 6
    pf["sel_in"] = sel
    w = csa2.PrefillWorkload(pf)
    say("prefill Reuse index 10^6")
    expect_refused(w, csa2.CSA2_PRE_SEL, call=w.prefill)
