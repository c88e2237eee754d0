"""Host-side checks of the C-ABI library: it loads, exports every entry point
include/csa2.h declares, and rejects bad arguments before launching anything.
No call here reaches a kernel launch."""
import ctypes as C
import os
import re

import pytest

from sparse_long_context_amd import csa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "csa2.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_documented_entry_points():
    names = declared_functions()
    for n in ["csa2_index_scores", "csa2_topk", "csa2_attend", "csa2_decode", "csa2_prefill",
              "csa2_workspace_size", "csa2_prefill_workspace_size", "csa2_status_str", "csa2_abi_version",
              "csa2_last_hip_error", "csa2_quantize_fp4_kv", "csa2_quantize_mxfp4"]:
        assert n in names, n


def test_library_exports_every_declared_symbol():
    L = csa2.lib()
    for n in declared_functions():
        assert hasattr(L, n), n
    assert set(declared_functions()) == set(csa2.EXPORTS)
    assert csa2.csa2_abi_version() == 4
    assert csa2.status_str(0) == "ok"


def dims(**kw):
    d = dict(n_heads=64, head_dim=512, window=128, index_topk=512, index_dim=128, index_heads=1,
             index_relu=0, kv_dtype=0, softmax_scale=1.0)
    d.update(kw)
    return csa2.Dims.from_dict(d)


FAKE = 0x1000  # never dereferenced: validation fails before any launch


def batch(**kw):
    b = csa2.Batch(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 16)
    for k, v in kw.items():
        setattr(b, k, v)
    return b


@pytest.mark.parametrize("kw,status", [
    (dict(n_heads=32), csa2.CSA2_ERR_UNSUPPORTED),
    (dict(head_dim=256), csa2.CSA2_ERR_UNSUPPORTED),
    (dict(index_dim=64), csa2.CSA2_ERR_UNSUPPORTED),
    (dict(index_topk=513), csa2.CSA2_ERR_UNSUPPORTED),
    (dict(window=129), csa2.CSA2_ERR_UNSUPPORTED),
    (dict(index_heads=65), csa2.CSA2_ERR_UNSUPPORTED),
    (dict(index_topk=0), csa2.CSA2_ERR_INVALID_ARG),
    (dict(window=-1), csa2.CSA2_ERR_INVALID_ARG),
    (dict(kv_dtype=3), csa2.CSA2_ERR_INVALID_ARG),
    (dict(index_key_dtype=2), csa2.CSA2_ERR_INVALID_ARG),
    (dict(index_relu=2), csa2.CSA2_ERR_INVALID_ARG),
    (dict(softmax_scale=float("nan")), csa2.CSA2_ERR_INVALID_ARG),
])
def test_bad_dims_rejected_everywhere(kw, status):
    d = dims(**kw)
    with pytest.raises(csa2.Csa2Error) as e:
        csa2.csa2_workspace_size(d, 4, 100)
    assert e.value.status == status
    with pytest.raises(csa2.Csa2Error) as e:
        csa2.csa2_decode(d, 4, batch(), FAKE, FAKE, None, FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE, None,
                         FAKE, 1 << 30, stream=0)
    assert e.value.status == status


def test_bad_arguments_rejected_before_launch():
    d = dims()
    E = csa2.Csa2Error
    with pytest.raises(E) as e:  # negative batch
        csa2.csa2_index_scores(d, -1, batch(), FAKE, None, FAKE, FAKE, 16, stream=0)
    assert e.value.status == csa2.CSA2_ERR_INVALID_ARG
    with pytest.raises(E) as e:  # missing descriptor array
        csa2.csa2_topk(d, 2, batch(pos=None), FAKE, 16, FAKE, stream=0)
    assert e.value.status == csa2.CSA2_ERR_INVALID_ARG
    with pytest.raises(E) as e:  # stride below the candidate bound
        csa2.csa2_index_scores(d, 2, batch(), FAKE, None, FAKE, FAKE, 15, stream=0)
    assert e.value.status == csa2.CSA2_ERR_INVALID_ARG
    with pytest.raises(E) as e:  # list offsets without a list
        csa2.csa2_topk(d, 2, batch(cand_off=FAKE), FAKE, 16, FAKE, stream=0)
    assert e.value.status == csa2.CSA2_ERR_INVALID_ARG
    with pytest.raises(E) as e:  # fp8 without scale planes
        csa2.csa2_attend(dims(kv_dtype=1), 2, batch(), FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE, None, None,
                         0, stream=0)
    assert e.value.status == csa2.CSA2_ERR_INVALID_ARG
    with pytest.raises(E) as e:  # no output
        csa2.csa2_attend(d, 2, batch(), FAKE, FAKE, None, FAKE, None, FAKE, None, None, None, None, 0, stream=0)
    assert e.value.status == csa2.CSA2_ERR_INVALID_ARG
    with pytest.raises(E) as e:  # workspace too small
        csa2.csa2_decode(d, 2, batch(), FAKE, FAKE, None, FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE, None,
                         FAKE, 16, stream=0)
    assert e.value.status == csa2.CSA2_ERR_WORKSPACE
    with pytest.raises(E) as e:  # attend: workspace given but too small (40 bf16 queries split four ways)
        csa2.csa2_attend(d, 40, batch(), FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE, None, FAKE, 16, stream=0)
    assert e.value.status == csa2.CSA2_ERR_WORKSPACE


def test_fused_derotation_descriptor_is_validated():
    # odd offset, odd or too many dims, past the head, no frequencies: refused
    # before anything is launched
    d = dims()
    for off, rd, f in [(447, 64, FAKE), (448, 63, FAKE), (256, 130, FAKE), (480, 64, FAKE), (448, 64, None),
                       (-2, 4, FAKE)]:
        r = csa2.OutRope(off, rd, f)
        with pytest.raises(csa2.Csa2Error) as e:
            csa2.csa2_attend(d, 2, batch(), FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE, None, None, 0,
                             stream=0, rope=r)
        assert e.value.status == csa2.CSA2_ERR_INVALID_ARG
        with pytest.raises(csa2.Csa2Error) as e:
            csa2.csa2_decode(d, 2, batch(), FAKE, FAKE, None, FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE, None,
                             FAKE, 1 << 30, stream=0, rope=r)
        assert e.value.status == csa2.CSA2_ERR_INVALID_ARG
        desc = csa2.PrefillDesc(1000, 10, csa2.MODE_FULL, 4, 250, 900, None, None, 0)
        with pytest.raises(csa2.Csa2Error) as e:
            csa2.csa2_prefill(d, desc, FAKE, FAKE, None, FAKE, FAKE, None, FAKE, None, FAKE, None, FAKE, None,
                              FAKE, 1 << 30, stream=0, rope=r)
        assert e.value.status == csa2.CSA2_ERR_INVALID_ARG
    # zero rope dims turn nothing: a valid descriptor (an empty batch is a no-op)
    csa2.csa2_attend(d, 0, batch(), None, None, None, None, None, None, None, None, None, None, 0, stream=0,
                     rope=csa2.OutRope(448, 0, None))


def test_prefill_descriptor_validation():
    d = dims()
    desc = csa2.PrefillDesc(1000, 10, csa2.MODE_FULL, 4, 250, 900, None, None, 0)
    assert csa2.csa2_prefill_workspace_size(d, desc) > 0
    for bad in [dict(win_pos0=1001), dict(n_queries=-1), dict(mode=7), dict(compress_ratio=-2),
                dict(mode=csa2.MODE_REINDEX)]:
        dd = csa2.PrefillDesc(1000, 10, csa2.MODE_FULL, 4, 250, 900, None, None, 0)
        for k, v in bad.items():
            setattr(dd, k, v)
        with pytest.raises(csa2.Csa2Error) as e:
            csa2.csa2_prefill_workspace_size(d, dd)
        assert e.value.status == csa2.CSA2_ERR_INVALID_ARG


def test_zero_sized_calls_are_noops():
    d = dims()
    csa2.csa2_index_scores(d, 0, batch(), None, None, None, None, 0, stream=0)
    csa2.csa2_topk(d, 0, batch(), None, 0, None, stream=0)
    csa2.csa2_attend(d, 0, batch(), None, None, None, None, None, None, None, None, None, None, 0, stream=0)
    assert csa2.csa2_workspace_size(d, 0, 0) >= 0


def test_storage_format_arguments_are_validated():
    E = csa2.Csa2Error
    for kw in (dict(kv_dtype=3), dict(kv_dtype=-1), dict(index_key_dtype=2)):
        with pytest.raises(E) as e:
            csa2.csa2_workspace_size(dims(**kw), 4, 100)
        assert e.value.status == csa2.CSA2_ERR_INVALID_ARG
    # MXFP4 keys without their scale plane
    with pytest.raises(E) as e:
        csa2.csa2_index_scores(dims(index_key_dtype=1), 2, batch(), FAKE, None, FAKE, FAKE, 16, stream=0)
    assert e.value.status == csa2.CSA2_ERR_INVALID_ARG
    # FP4 KV without its scale plane
    with pytest.raises(E) as e:
        csa2.csa2_attend(dims(kv_dtype=2), 2, batch(), FAKE, FAKE, None, None, None, FAKE, None, FAKE, None,
                         None, 0, stream=0)
    assert e.value.status == csa2.CSA2_ERR_INVALID_ARG
    # quantizers: block multiples, null pointers, negative sizes; zero rows is a no-op
    for fn, bad_d in ((csa2.csa2_quantize_fp4_kv, 24), (csa2.csa2_quantize_mxfp4, 48)):
        for args in ((4, bad_d, FAKE, FAKE, FAKE), (4, 0, FAKE, FAKE, FAKE), (-1, 64, FAKE, FAKE, FAKE),
                     (4, 64, None, FAKE, FAKE), (4, 64, FAKE, None, FAKE), (4, 64, FAKE, FAKE, None)):
            with pytest.raises(E) as e:
                fn(*args, stream=0)
            assert e.value.status == csa2.CSA2_ERR_INVALID_ARG, (fn, args)
        fn(0, 64, None, None, None, stream=0)


def test_candidate_pool_arguments_are_validated():
    E = csa2.Csa2Error
    for args in ((4, 100, 0, 8), (4, 100, 65, 8), (4, 100, 8, 0), (4, 100, 8, 65537), (-1, 100, 8, 8), (4, -1, 8, 8)):
        with pytest.raises(E) as e:
            csa2.csa2_candidate_pool_workspace_size(*args)
        assert e.value.status == csa2.CSA2_ERR_INVALID_ARG, args
    assert csa2.csa2_candidate_pool_workspace_size(4, 100, 8, 16) > 0
    with pytest.raises(E) as e:  # no output lists
        csa2.csa2_candidate_pool(2, batch(), FAKE, 16, 8, 16, None, FAKE, FAKE, 1 << 20, stream=0)
    assert e.value.status == csa2.CSA2_ERR_INVALID_ARG
    with pytest.raises(E) as e:  # stride below max_candidates
        csa2.csa2_candidate_pool(2, batch(), FAKE, 15, 8, 16, FAKE, FAKE, FAKE, 1 << 20, stream=0)
    assert e.value.status == csa2.CSA2_ERR_INVALID_ARG
    with pytest.raises(E) as e:  # workspace too small
        csa2.csa2_candidate_pool(2, batch(), FAKE, 16, 8, 16, FAKE, FAKE, FAKE, 16, stream=0)
    assert e.value.status == csa2.CSA2_ERR_WORKSPACE


def test_compress_and_derotate_arguments_are_validated():
    E = csa2.Csa2Error
    for args in ((4, 0, 512), (4, 2, 0), (4, 2, 1025), (-1, 2, 512)):
        with pytest.raises(E) as e:
            csa2.csa2_compress(*args, FAKE, FAKE, FAKE, 1e-6, FAKE, stream=0)
        assert e.value.status == csa2.CSA2_ERR_INVALID_ARG, args
    for bad in ((FAKE, None, FAKE, FAKE), (None, FAKE, FAKE, FAKE), (FAKE, FAKE, None, FAKE), (FAKE, FAKE, FAKE, None)):
        with pytest.raises(E) as e:
            csa2.csa2_compress(4, 2, 512, bad[0], bad[1], bad[2], 1e-6, bad[3], stream=0)
        assert e.value.status == csa2.CSA2_ERR_INVALID_ARG
    with pytest.raises(E) as e:
        csa2.csa2_compress(4, 2, 512, FAKE, FAKE, FAKE, -1.0, FAKE, stream=0)
    assert e.value.status == csa2.CSA2_ERR_INVALID_ARG
    csa2.csa2_compress(0, 2, 512, None, None, None, 1e-6, None, stream=0)
    # the decode step: sizes, eps, and every array it needs (states and gate
    # logits only above ratio 1)
    for args in ((4, 0, 512), (4, 2, 0), (4, 2, 1025), (-1, 2, 512)):
        with pytest.raises(E) as e:
            csa2.csa2_compress_step(*args, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1e-6, FAKE, FAKE, stream=0)
        assert e.value.status == csa2.CSA2_ERR_INVALID_ARG, args
    for k in range(8):
        ptrs = [FAKE] * 8
        ptrs[k] = None
        with pytest.raises(E) as e:
            csa2.csa2_compress_step(4, 2, 512, *ptrs[:6], 1e-6, *ptrs[6:], stream=0)
        assert e.value.status == csa2.CSA2_ERR_INVALID_ARG, k
    with pytest.raises(E) as e:
        csa2.csa2_compress_step(4, 2, 512, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, float("nan"), FAKE, FAKE, stream=0)
    assert e.value.status == csa2.CSA2_ERR_INVALID_ARG
    csa2.csa2_compress_step(0, 2, 512, None, None, None, None, None, None, 1e-6, None, None, stream=0)
    d = dims()
    for args in ((2, 448, 63), (2, 449, 64), (2, 0, 130), (2, -1, 64), (-1, 448, 64)):
        with pytest.raises(E) as e:
            csa2.csa2_derotate(d, args[0], FAKE, args[1], args[2], FAKE, FAKE, stream=0)
        assert e.value.status == csa2.CSA2_ERR_INVALID_ARG, args
    with pytest.raises(E) as e:
        csa2.csa2_derotate(d, 2, None, 448, 64, FAKE, FAKE, stream=0)
    assert e.value.status == csa2.CSA2_ERR_INVALID_ARG


def test_precondition_status_and_word():
    """The debug-check status has its own message; the word starts at 0, and
    host-invalid arguments are refused before any device check runs (no GPU is
    touched here), whether or not CSA2_DEBUG_CHECK is set."""
    assert "precondition" in csa2.status_str(csa2.CSA2_ERR_PRECONDITION)
    assert csa2.csa2_last_precondition() == 0
    L = csa2.lib()
    old = os.environ.get("CSA2_DEBUG_CHECK")
    os.environ["CSA2_DEBUG_CHECK"] = "1"
    try:
        d, b = dims(), batch()
        assert L.csa2_topk(C.byref(d), 2, C.byref(b), None, 16, None, None, 0, None) == csa2.CSA2_ERR_INVALID_ARG
        assert L.csa2_attend(C.byref(dims(n_heads=8)), 2, C.byref(b), FAKE, None, None, None, None, FAKE, None,
                             FAKE, None, None, 0, None, None) == csa2.CSA2_ERR_UNSUPPORTED
        # an empty batch is a no-op: nothing to check, nothing launched
        assert L.csa2_topk(C.byref(d), 0, C.byref(b), None, 0, None, None, 0, None) == csa2.CSA2_OK
        assert csa2.csa2_last_precondition() == 0
    finally:
        if old is None:
            del os.environ["CSA2_DEBUG_CHECK"]
        else:
            os.environ["CSA2_DEBUG_CHECK"] = old
    # the header's bits are the binding's
    src = open(os.path.join(ROOT, "include", "csa2.h")).read()
    for name in ("MODE", "DESC", "LIST", "SEL", "KV_SCALE", "INDEX"):
        m = re.search(r"#define CSA2_PRE_%s (\d+)u" % name, src)
        assert m and int(m.group(1)) == getattr(csa2, "CSA2_PRE_" + name), name


def test_gather_probe_library_validates_before_launching():
    # the measurement aid behind bench.py --gather-probe (not part of the ABI):
    # built beside libcsa2.so, it refuses a bad mode, wave count or row count
    # (hipErrorInvalidValue = 1) before any launch
    from sparse_long_context_amd import build as B
    if not os.path.exists(B.PROBE_LIB):
        pytest.skip("libcsa2_probe.so is built by __graft_entry__.build()")
    L = C.CDLL(B.PROBE_LIB)
    f = L.csa2_probe_gather
    f.restype = C.c_int
    f.argtypes = [C.c_int, C.c_int, C.c_int, C.c_void_p, C.c_void_p, C.c_int, C.c_void_p, C.c_void_p]
    assert f(2, 4, 1, FAKE, FAKE, 8, FAKE, None) == 1      # mode
    assert f(0, 6, 1, FAKE, FAKE, 8, FAKE, None) == 1      # waves
    assert f(0, 4, 0, FAKE, FAKE, 8, FAKE, None) == 1      # workgroups
    assert f(1, 8, 1, FAKE, FAKE, 12, FAKE, None) == 1     # rows per wave, a multiple of 8
