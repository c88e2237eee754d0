"""ctypes front end of the CPU oracle (liboracle.so, built from csa2_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py``; never by the product path.

Every function here is marshalling: the arithmetic lives in csa2_oracle.c,
which follows the pages step by step (see the comments there), including the
compositions over a decode batch (``decode_batch``) and over a prefill chunk
(``prefill_chunk``, which derives each query's window itself) in the pages'
order: reachability -> scores -> top-K -> one softmax over the window rows and
the selected compressed rows.
"""
import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# CSA2_ORACLE_LIB names another build of the same source (the sanitizer test's)
LIB_PATH = os.environ.get("CSA2_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")

MODE_FULL, MODE_REINDEX, MODE_REUSE, MODE_WINDOW = 0, 1, 2, 3
KV_BF16, KV_FP8, KV_FP4 = 0, 1, 2
IDXK_F32, IDXK_MXFP4 = 0, 1

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build
            build.build()
        L = C.CDLL(LIB_PATH)
        P = C.c_void_p
        i32, i64, dbl = C.c_int32, C.c_int64, C.c_double
        L.csa2o_bf16_to_f64.argtypes = [C.c_uint16, C.POINTER(dbl)]
        L.csa2o_e4m3_to_f64.argtypes = [C.c_uint8, C.POINTER(dbl)]
        L.csa2o_ue8m0_to_f64.argtypes = [C.c_uint8, C.POINTER(dbl)]
        for f in (L.csa2o_bf16_to_f64, L.csa2o_e4m3_to_f64, L.csa2o_ue8m0_to_f64):
            f.restype = C.c_int
        L.csa2o_e2m1_to_f64.argtypes = [C.c_uint8, C.POINTER(dbl)]
        L.csa2o_e2m1_to_f64.restype = C.c_int
        L.csa2o_e2m1_encode.argtypes = [dbl]
        L.csa2o_e2m1_encode.restype = C.c_uint8
        L.csa2o_f32_to_e4m3.argtypes = [C.c_float, C.POINTER(C.c_uint8)]
        L.csa2o_f32_to_e4m3.restype = C.c_int
        for f in (L.csa2o_quant_fp4kv, L.csa2o_quant_mxfp4):
            f.argtypes = [P, i64, P, P]
            f.restype = C.c_int
        L.csa2o_dequant_mxfp4.argtypes = [P, P, i64, P]
        L.csa2o_dequant_mxfp4.restype = C.c_int
        L.csa2o_compress.argtypes = [i64, i32, i32, P, P, P, dbl, P]
        L.csa2o_compress.restype = C.c_int
        L.csa2o_compress_step.argtypes = [i32, i32, i32, P, P, P, P, P, P, dbl, P, P]
        L.csa2o_compress_step.restype = C.c_int
        L.csa2o_derotate.argtypes = [i32, i32, i32, i32, P, i64, P]
        L.csa2o_derotate.restype = C.c_int
        L.csa2o_candidate_pool.argtypes = [P, i64, i32, i32, P]
        L.csa2o_candidate_pool.restype = C.c_int
        L.csa2o_n_valid.argtypes = [i64, i32, i32, i64]
        L.csa2o_n_valid.restype = i64
        L.csa2o_window_range.argtypes = [i64, i32, i64, C.POINTER(i64), C.POINTER(i64)]
        L.csa2o_window_range.restype = C.c_int
        L.csa2o_index_scores.argtypes = [i32, i32, P, P, i32, P, i64, P, i64, P, P, P]
        L.csa2o_index_scores.restype = C.c_int
        L.csa2o_topk.argtypes = [P, P, i64, i64, i32, P]
        L.csa2o_topk.restype = C.c_int
        L.csa2o_attend_core.argtypes = [i32, i32, i64, P, P, P, P, dbl, P, P]
        L.csa2o_attend_core.restype = C.c_int
        L.csa2o_attend_query.argtypes = [i32, i32, i32, P, P, P, i64, P, P, i64, P, i32, P, dbl, P, P]
        L.csa2o_attend_query.restype = C.c_int
        L.csa2o_select_query.argtypes = [i32, i64, i32, i64, i32, i32, P, P, i32, P, P, i64, i32, P, P]
        L.csa2o_select_query.restype = i64
        L.csa2o_decode_batch.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, dbl,
                                         P, P, P, P, P, P, P, P, P,
                                         P, P, P, P, P, P, P, i32, P, P, P, P, P, P]
        L.csa2o_decode_batch.restype = C.c_int
        L.csa2o_prefill_chunk.argtypes = [i32, P, i64, i32, i32, i64, i64, i64, i32, i32, i32, i32, i32, i32,
                                          i32, i32, dbl, P, P, P, P, P, P, P, P, P, i32, P, P, P, P, P, P]
        L.csa2o_prefill_chunk.restype = C.c_int
        _lib = L
    return _lib


class OracleError(RuntimeError):
    pass


def _check(rc):
    if rc < 0:
        raise OracleError(f"oracle refused the input (code {rc})")
    return rc


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


# --- O0 decoders --------------------------------------------------------------

def bf16_to_f64(code):
    out = C.c_double()
    _check(lib().csa2o_bf16_to_f64(int(code), C.byref(out)))
    return out.value


def e4m3_to_f64(code):
    out = C.c_double()
    _check(lib().csa2o_e4m3_to_f64(int(code), C.byref(out)))
    return out.value


def ue8m0_to_f64(code):
    out = C.c_double()
    _check(lib().csa2o_ue8m0_to_f64(int(code), C.byref(out)))
    return out.value


def e2m1_to_f64(code):
    out = C.c_double()
    _check(lib().csa2o_e2m1_to_f64(int(code) & 15, C.byref(out)))
    return out.value


def e2m1_encode(v):
    """Nearest E2M1 code (4 bits) to v, ties to even, saturating at 6."""
    return int(lib().csa2o_e2m1_encode(float(v)))


def f32_to_e4m3(v):
    out = C.c_uint8()
    _check(lib().csa2o_f32_to_e4m3(float(np.float32(v)), C.byref(out)))
    return int(out.value)


def quant_fp4kv(x):
    """FP4 main-KV quantizer over the last axis (a multiple of 16): returns
    (codes uint8 [..., n/2], E4M3 scales uint8 [..., n/16])."""
    x = np.ascontiguousarray(x, np.float32)
    n = x.shape[-1]
    codes = np.empty(x.shape[:-1] + (n // 2,), np.uint8)
    scales = np.empty(x.shape[:-1] + (n // 16,), np.uint8)
    _check(lib().csa2o_quant_fp4kv(_ptr(x), x.size, _ptr(codes), _ptr(scales)))
    return codes, scales


def quant_mxfp4(x):
    """MXFP4 quantizer over the last axis (a multiple of 32): returns
    (codes uint8 [..., n/2], E8M0 scales uint8 [..., n/32])."""
    x = np.ascontiguousarray(x, np.float32)
    n = x.shape[-1]
    codes = np.empty(x.shape[:-1] + (n // 2,), np.uint8)
    scales = np.empty(x.shape[:-1] + (n // 32,), np.uint8)
    _check(lib().csa2o_quant_mxfp4(_ptr(x), x.size, _ptr(codes), _ptr(scales)))
    return codes, scales


def dequant_mxfp4(codes, scales):
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), np.float32)
    _check(lib().csa2o_dequant_mxfp4(_ptr(codes), _ptr(scales), out.size, _ptr(out)))
    return out


# --- O1 / window ------------------------------------------------------------

def n_valid(pos, ratio, mode, pool_len):
    return _check(lib().csa2o_n_valid(int(pos), int(ratio), int(mode), int(pool_len)))


def window_range(pos, w, replay_start):
    lo, cnt = C.c_int64(), C.c_int64()
    _check(lib().csa2o_window_range(int(pos), int(w), int(replay_start), C.byref(lo), C.byref(cnt)))
    return lo.value, cnt.value


# --- O3 / O4 ----------------------------------------------------------------

def index_scores(q, keys, w=None, relu=False, cand=None, n=None):
    """q [H_I, D_I] f32; keys [rows, D_I] f32.  Returns (s32, s64, bound)."""
    q = _c(q, np.float32)
    keys = _c(keys, np.float32)
    w = _c(w, np.float32)
    h_i, d_i = q.shape
    cand = _c(cand, np.int32)
    if n is None:
        n = keys.shape[0] if cand is None else cand.shape[0]
    s32 = np.empty(n, np.float32)
    s64 = np.empty(n, np.float64)
    bnd = np.empty(n, np.float64)
    _check(lib().csa2o_index_scores(h_i, d_i, _ptr(q), _ptr(w), int(bool(relu)), _ptr(keys),
                                    keys.shape[0], _ptr(cand), n, _ptr(s32), _ptr(s64), _ptr(bnd)))
    return s32, s64, bnd


def topk(scores, k, n_valid_=None, pos_of=None):
    scores = _c(scores, np.float32)
    pos_of = _c(pos_of, np.int32)
    n = scores.shape[0]
    if n_valid_ is None:
        n_valid_ = n if pos_of is None else (int(pos_of.max()) + 1 if n else 0)
    out = np.empty(k, np.int32)
    _check(lib().csa2o_topk(_ptr(scores), _ptr(pos_of), n, int(n_valid_), int(k), _ptr(out)))
    return out


# --- O6 ----------------------------------------------------------------------

def attend_core(q, kmat, vmat, sink=None, scale=1.0):
    """fp64 single softmax: q [H, D], kmat/vmat [E, D].  Returns (out [H, D], lse [H])."""
    q = _c(q, np.float64)
    h, d = q.shape
    kmat = _c(kmat, np.float64).reshape(-1, d)
    vmat = _c(vmat, np.float64).reshape(-1, d)
    sink = _c(sink, np.float64)
    out = np.empty((h, d), np.float64)
    lse = np.empty(h, np.float64)
    _check(lib().csa2o_attend_core(h, d, kmat.shape[0], _ptr(q), _ptr(kmat), _ptr(vmat), _ptr(sink),
                                   float(scale), _ptr(out), _ptr(lse)))
    return out, lse


def attend_query(q_bf16, win_rows, pool_rows, sel, kv_dtype=KV_BF16, win_scales=None,
                 pool_scales=None, sink=None, scale=1.0):
    """One query's two-source attention.

    q_bf16 [H, D] uint16; win_rows [win_len, D] (uint16 bf16, or uint8 e4m3 with
    win_scales [win_len, D/32] uint8, or uint8 [win_len, D/2] FP4 codes with
    win_scales [win_len, D/16] E4M3); pool_rows likewise; sel int32 list of
    pool rows (-1 skipped).  Returns (out f32 [H, D], lse f32 [H]).
    """
    q = _c(q_bf16, np.uint16)
    h, d = q.shape
    rdt = np.uint16 if kv_dtype == KV_BF16 else np.uint8
    w = d // 2 if kv_dtype == KV_FP4 else d
    win_rows = np.zeros((0, w), rdt) if win_rows is None else _c(win_rows, rdt).reshape(-1, w)
    pool_rows = np.zeros((0, w), rdt) if pool_rows is None else _c(pool_rows, rdt).reshape(-1, w)
    win_scales = _c(win_scales, np.uint8)
    pool_scales = _c(pool_scales, np.uint8)
    sel = np.zeros(0, np.int32) if sel is None else _c(sel, np.int32)
    sink = _c(sink, np.float32)
    out = np.empty((h, d), np.float32)
    lse = np.empty(h, np.float32)
    _check(lib().csa2o_attend_query(h, d, kv_dtype, _ptr(q), _ptr(win_rows), _ptr(win_scales),
                                    win_rows.shape[0], _ptr(pool_rows), _ptr(pool_scales),
                                    pool_rows.shape[0], _ptr(sel), sel.shape[0], _ptr(sink),
                                    float(scale), _ptr(out), _ptr(lse)))
    return out, lse


def select_query(mode, pos, ratio, pool_len, idx_q, idx_k, k, idx_w=None, relu=False, cand=None, scores=False):
    """Reachability + scores + top-K for one Full/Reindex query.  Returns int32
    [k], or (int32 [k], f32 scores of the scored candidates in candidate
    order: the reachable pool rows, or the reachable listed rows) with
    scores=True."""
    idx_q = _c(idx_q, np.float32)
    h_i, d_i = idx_q.shape
    idx_k = _c(idx_k, np.float32)
    idx_w = _c(idx_w, np.float32)
    cand = _c(cand, np.int32)
    out = np.empty(k, np.int32)
    sc = np.empty(max(int(pool_len), 0 if cand is None else cand.shape[0], 1), np.float32) if scores else None
    n = _check(lib().csa2o_select_query(int(mode), int(pos), int(ratio), int(pool_len), h_i, d_i,
                                        _ptr(idx_q), _ptr(idx_w), int(bool(relu)), _ptr(idx_k), _ptr(cand),
                                        0 if cand is None else cand.shape[0], int(k), _ptr(out), _ptr(sc)))
    return (out, sc[:n]) if scores else out


def compress(c, g, w, m, eps=1e-20):
    """Compressor over n_groups * m tokens: c, g f32 [n_groups * m, d] (g None
    for m == 1), w f32 [d] -> f32 [n_groups, d]."""
    c = _c(c, np.float32)
    g = _c(g, np.float32)
    w = _c(w, np.float32)
    d = c.shape[-1]
    n = c.shape[0] // m
    out = np.empty((n, d), np.float32)
    _check(lib().csa2o_compress(n, int(m), d, _ptr(c), _ptr(g), _ptr(w), float(eps), _ptr(out)))
    return out


def compress_step(pos, c_new, g_new, kv_state, score_state, w, m, out, eps=1e-20):
    """One decode step of the compressor for B sequences: pos int64 [B], c_new,
    g_new f32 [B, d] (g_new None for m == 1); kv_state, score_state f32
    [B, m, d] and out f32 [B, d] are updated in place.  Returns emit_idx int32
    [B] (-1 where the step closes no group)."""
    pos = _c(pos, np.int64)
    c_new = _c(c_new, np.float32)
    g_new = _c(g_new, np.float32)
    w = _c(w, np.float32)
    for a in (kv_state, score_state, out):
        assert a is None or (a.dtype == np.float32 and a.flags.c_contiguous)
    B, d = c_new.shape
    emit = np.empty(B, np.int32)
    _check(lib().csa2o_compress_step(B, int(m), d, _ptr(pos), _ptr(c_new), _ptr(g_new), _ptr(kv_state),
                                     _ptr(score_state), _ptr(w), float(eps), _ptr(out), _ptr(emit)))
    return emit


def derotate(out_h_d, pos, inv_freq, rope_off=448, rope_dims=64):
    """De-rotate one query's output [H, D] (copy returned)."""
    o = np.array(out_h_d, np.float32, copy=True, order="C")
    f = _c(inv_freq, np.float64)
    _check(lib().csa2o_derotate(o.shape[0], o.shape[1], int(rope_off), int(rope_dims), _ptr(f), int(pos), _ptr(o)))
    return o


def candidate_pool(scores, block_size=8, top_blocks=2048):
    """Hierarchical candidate pool of one query from its Full-layer scores over
    its reachable entries: int32 [top_blocks * block_size], ascending, -1 padded."""
    s = _c(scores, np.float32)
    out = np.empty(top_blocks * block_size, np.int32)
    _check(lib().csa2o_candidate_pool(_ptr(s), s.size, int(block_size), int(top_blocks), _ptr(out)))
    return out


def decode_batch(inp, queries=None, sink=None, scale=1.0):
    """Run the oracle over a decode batch described like the HIP library's
    batch (see sparse_long_context_amd.synth): dict of numpy arrays.  ``queries``
    restricts the run to a subset (indices into the batch).  Returns
    (sel int32 [n, K], out f32 [n, H, D], lse f32 [n, H])."""
    d = inp["dims"]
    qs = np.arange(inp["B"]) if queries is None else np.asarray(queries)
    n = len(qs)
    H, D, K, HI, DI = d["n_heads"], d["head_dim"], d["index_topk"], d["index_heads"], d["index_dim"]
    kvd = d["kv_dtype"]
    take = lambda name: np.ascontiguousarray(inp[name][qs])  # noqa: E731
    pos, mode, ratio = take("pos").astype(np.int64), take("mode").astype(np.int32), take("ratio").astype(np.int32)
    win_row0, win_len = take("win_row0").astype(np.int64), take("win_len").astype(np.int32)
    pool_row0, pool_len = take("pool_row0").astype(np.int64), take("pool_len").astype(np.int32)
    q = take("q")
    idx_q = take("idx_q")
    idx_w = None if inp.get("idx_w") is None else take("idx_w")
    sel = np.full((n, K), -1, np.int32)
    if inp.get("sel_in") is not None:
        sel[:] = take("sel_in")
    cand_off = cand_idx = None
    if inp.get("cand_off") is not None:
        offs = inp["cand_off"]
        parts = [inp["cand_idx"][offs[b]:offs[b + 1]] for b in qs]
        cand_off = np.zeros(n + 1, np.int64)
        cand_off[1:] = np.cumsum([len(p) for p in parts])
        cand_idx = np.ascontiguousarray(np.concatenate(parts) if parts else np.zeros(0), np.int32)
    out = np.empty((n, H, D), np.float32)
    lse = np.empty((n, H), np.float32)
    sink = _c(sink, np.float32)
    rc = lib().csa2o_decode_batch(
        n, H, D, K, HI, DI, int(d["index_relu"]), kvd, float(scale),
        _ptr(pos), _ptr(mode), _ptr(ratio), _ptr(win_row0), _ptr(win_len), _ptr(pool_row0), _ptr(pool_len),
        _ptr(cand_off), _ptr(cand_idx), _ptr(q), _ptr(inp["win_kv"]), _ptr(inp.get("win_scale")),
        _ptr(inp["comp_kv"]), _ptr(inp.get("comp_scale")), _ptr(idx_q), _ptr(idx_w),
        int(d.get("index_key_dtype", IDXK_F32)), _ptr(inp["idx_k"]), _ptr(inp.get("idx_k_scale")),
        _ptr(sink), _ptr(sel), _ptr(out), _ptr(lse))
    _check(rc)
    return sel, out, lse


# --- trace (the CSA2_TRACE=1 line format of the HIP library) -------------------

def fnv1a64(data):
    """64-bit FNV-1a of a bytes object."""
    h = 0xcbf29ce484222325
    for byte in data:
        h = ((h ^ byte) * 0x100000001b3) & 0xFFFFFFFFFFFFFFFF
    return h


def trace_lines(call, score_rows, sel_rows, out, lse):
    """The checksum lines of one call: score_rows, the scores of each Full /
    Reindex query in candidate order; sel_rows [r, K] int32, the top-K rows the
    call writes; out [n, H, D] and lse [n, H] of all its queries."""
    vals = [np.asarray(r, np.float32) for r in score_rows]
    vals = np.concatenate(vals) if vals else np.zeros(0, np.float32)
    vals = vals[np.isfinite(vals)].astype(np.float64)
    finite = len(vals)
    total = float(np.cumsum(vals)[-1]) if finite else 0.0  # one addition after another, in order
    sel_rows = np.ascontiguousarray(sel_rows, np.int32).reshape(-1, np.shape(sel_rows)[-1] if len(sel_rows) else 1)
    chosen = int((sel_rows >= 0).sum())
    h = fnv1a64(sel_rows.astype("<i4").tobytes())
    o = np.asarray(out, np.float32).ravel().astype(np.float64)
    lv = np.asarray(lse, np.float32).ravel()
    fin = np.isfinite(lv)
    return [f"csa2-trace {call} scores finite={finite} sum={total:.17g}",
            f"csa2-trace {call} topk rows={len(sel_rows)} chosen={chosen} fnv1a={h:016x}",
            f"csa2-trace {call} attend out_sum={o.sum():.6e} out_abs={np.abs(o).sum():.6e} "
            f"lse_sum={lv[fin].astype(np.float64).sum():.6e} lse_ninf={int((~fin).sum())}"]


def decode_trace(inp, sink=None, scale=1.0):
    """The oracle's trace lines for a whole decode batch (fp32 index keys)."""
    d = inp["dims"]
    sel, out, lse = decode_batch(inp, sink=sink, scale=scale)
    rows, sels = [], []
    for b in range(inp["B"]):
        md = int(inp["mode"][b])
        if md not in (MODE_FULL, MODE_REINDEX):
            continue
        p0, pl = int(inp["pool_row0"][b]), int(inp["pool_len"][b])
        cand = None
        if md == MODE_REINDEX:
            offs = inp.get("cand_off")
            cand = np.zeros(0, np.int32) if offs is None else inp["cand_idx"][offs[b]:offs[b + 1]]
        hi = d["index_heads"]
        _, sc = select_query(md, int(inp["pos"][b]), int(inp["ratio"][b]), pl, inp["idx_q"][b].reshape(hi, -1),
                             inp["idx_k"][p0:p0 + pl], d["index_topk"],
                             idx_w=None if inp.get("idx_w") is None else inp["idx_w"][b], relu=d["index_relu"],
                             cand=cand, scores=True)
        rows.append(sc)
        sels.append(sel[b])
    return trace_lines("decode", rows, np.array(sels, np.int32).reshape(len(sels), -1), out, lse)


def prefill_trace(pf, sink=None, scale=1.0):
    """The oracle's trace lines for a whole prefill chunk (fp32 index keys)."""
    d = pf["dims"]
    sel, out, lse = prefill_chunk(pf, sink=sink, scale=scale)
    md = int(pf["mode"])
    rows = []
    if md in (MODE_FULL, MODE_REINDEX):
        hi = d["index_heads"]
        for t in range(int(pf["T"])):
            cand = None
            if md == MODE_REINDEX:
                offs = pf.get("cand_off")
                cand = np.zeros(0, np.int32) if offs is None else pf["cand_idx"][offs[t]:offs[t + 1]]
            _, sc = select_query(md, int(pf["pos0"]) + t, int(pf["ratio"]), int(pf["pool_len"]),
                                 pf["idx_q"][t].reshape(hi, -1), pf["idx_k"], d["index_topk"],
                                 idx_w=None if pf.get("idx_w") is None else pf["idx_w"][t], relu=d["index_relu"],
                                 cand=cand, scores=True)
            rows.append(sc)
    sels = sel if md in (MODE_FULL, MODE_REINDEX) else sel[:0]
    return trace_lines("prefill", rows, sels, out, lse)


def prefill_chunk(pf, queries=None, sink=None, scale=1.0):
    """Run the oracle over a prefill chunk (dict from ``synth.prefill_chunk``):
    T queries of one sequence at pos0 .. pos0+T-1 sharing its raw window rows
    (row r at position win_pos0 + r), pool and index keys.  Each query's window,
    reachability, selection and attention are derived inside the oracle.
    ``queries`` restricts the run to a subset of t.  Returns (sel int32 [n, K],
    out f32 [n, H, D], lse f32 [n, H])."""
    d = pf["dims"]
    T = int(pf["T"])
    qs = np.ascontiguousarray(np.arange(T) if queries is None else np.asarray(queries), np.int32)
    n = len(qs)
    H, D, K, HI, DI, W = d["n_heads"], d["head_dim"], d["index_topk"], d["index_heads"], d["index_dim"], d["window"]
    kvd = d["kv_dtype"]
    sel = np.full((n, K), -1, np.int32)
    if pf.get("sel_in") is not None:
        sel[:] = pf["sel_in"][qs]
    win_kv = pf["win_kv"]
    out = np.empty((n, H, D), np.float32)
    lse = np.empty((n, H), np.float32)
    rc = lib().csa2o_prefill_chunk(
        n, _ptr(qs), int(pf["pos0"]), int(pf["mode"]), int(pf["ratio"]), int(pf["pool_len"]),
        int(pf["win_pos0"]), int(win_kv.shape[0]), int(W), H, D, K, HI, DI, int(d["index_relu"]), kvd, float(scale),
        _ptr(_c(pf.get("cand_off"), np.int64)), _ptr(_c(pf.get("cand_idx"), np.int32)), _ptr(pf["q"]),
        _ptr(win_kv), _ptr(pf.get("win_scale")), _ptr(pf["comp_kv"]), _ptr(pf.get("comp_scale")),
        _ptr(_c(pf["idx_q"], np.float32)), _ptr(_c(pf.get("idx_w"), np.float32)),
        int(d.get("index_key_dtype", IDXK_F32)), _ptr(pf["idx_k"]), _ptr(pf.get("idx_k_scale")),
        _ptr(_c(sink, np.float32)), _ptr(sel), _ptr(out), _ptr(lse))
    _check(rc)
    return sel, out, lse
