"""Seeded synthetic workloads for the CSA2 attention step.

This module draws inputs and lays them out; it holds none of the attention's
arithmetic.  Both the HIP path (tests, benchmark) and the CPU oracle read the
arrays it returns.  The generator itself (counter-based SplitMix64 + Box-Muller,
nearest-even storage rounding, E4M3/UE8M0 quantisation of the fp8 tensors) is
specified in synth_c/csa2_synth.c.

Workloads follow the pages' setting (one 512-wide KV per position shared by 64
query heads of 512 dims, a 128-row sliding window, top-512 of the compressed
positions, 128-wide fp32 indexer): every value is i.i.d. N(0, 1) except the
query, which is N(0, 1) / sqrt(512) (the 1/sqrt(dim) factor folded into q).

A decode batch is a dict:
  dims        n_heads, head_dim, window, index_topk, index_dim, index_heads,
              index_relu, kv_dtype (0 bf16, 1 fp8 e4m3 + ue8m0/32), softmax_scale
  B           number of queries
  pos, mode, ratio, win_row0, win_len, pool_row0, pool_len   per-query metadata
  q           uint16 [B, H, D] (bf16 bits)
  win_kv      window rows [rows, D] (uint16 bf16, or uint8 e4m3) (+ win_scale [rows, D/32])
  comp_kv     compressed rows [rows, D] (same dtype)          (+ comp_scale)
  idx_q       float32 [B, H_I, D_I];  idx_w float32 [B, H_I] (weights=True) or None (unit)
  idx_k       float32 [rows, D_I], same row numbering as comp_kv
  sel_in      int32 [B, K] supplied selections (Reuse rows), -1 elsewhere, or None
  cand_off, cand_idx   Reindex lists (or None)
  max_pool_len
A prefill chunk is a dict with T, pos0, mode, ratio, win_pos0, pool_len, q, win_kv,
comp_kv, idx_q, idx_w, idx_k (one sequence): raw window row r holds position
win_pos0 + r.  Which rows each query reads is the method's business (the HIP
library and the oracle each derive it), not this module's.
"""
import ctypes as C
import math
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
# CSA2_SYNTH_LIB names another build of the same source (the sanitizer test's)
SYNTH_LIB = os.environ.get("CSA2_SYNTH_LIB") or os.path.join(PKG, "libcsa2_synth.so")

MODE_FULL, MODE_REINDEX, MODE_REUSE, MODE_WINDOW = 0, 1, 2, 3
KV_BF16, KV_FP8, KV_FP4 = 0, 1, 2
IDXK_F32, IDXK_MXFP4 = 0, 1

# streams: one per tensor kind
S_Q, S_WIN, S_POOL, S_IDXQ, S_IDXK, S_CTX, S_REUSE, S_CAND, S_IDXW = 1, 2, 3, 4, 5, 6, 7, 8, 9

_lib = None


def _L():
    global _lib
    if _lib is None:
        if not os.path.exists(SYNTH_LIB):
            from . import build
            build.build_synth()
        L = C.CDLL(SYNTH_LIB)
        u64, i64, dbl, P = C.c_uint64, C.c_int64, C.c_double, C.c_void_p
        L.synth_normal_bf16.argtypes = [u64, u64, u64, u64, dbl, P]
        L.synth_normal_f32.argtypes = [u64, u64, u64, u64, dbl, P]
        L.synth_normal_fp8.argtypes = [u64, u64, u64, u64, C.c_int, dbl, P, P]
        L.synth_normal_fp8.restype = C.c_int
        L.synth_uniform_int.argtypes = [u64, u64, u64, u64, i64, i64, P]
        L.synth_sample_distinct.argtypes = [u64, u64, i64, i64, P]
        L.synth_sample_distinct.restype = i64
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(C.c_void_p)


def normal_bf16(seed, stream, shape, start=0, scale=1.0):
    out = np.empty(shape, np.uint16)
    _L().synth_normal_bf16(seed, stream, start, out.size, scale, _p(out))
    return out


def normal_f32(seed, stream, shape, start=0, scale=1.0):
    out = np.empty(shape, np.float32)
    _L().synth_normal_f32(seed, stream, start, out.size, scale, _p(out))
    return out


def normal_fp8(seed, stream, rows, d, start_row=0, scale=1.0):
    codes = np.empty((rows, d), np.uint8)
    scales = np.empty((rows, d // 32), np.uint8)
    rc = _L().synth_normal_fp8(seed, stream, start_row, rows, d, scale, _p(codes), _p(scales))
    if rc != 0:
        raise ValueError("fp8 quantisation out of range")
    return codes, scales


def uniform_int(seed, stream, count, lo, hi, start=0):
    out = np.empty(count, np.int64)
    _L().synth_uniform_int(seed, stream, start, count, lo, hi, _p(out))
    return out


def sample_distinct(seed, stream, n, k):
    out = np.full(max(min(n, k), 1), -1, np.int32)
    got = _L().synth_sample_distinct(seed, stream, n, k, _p(out))
    return out[:max(got, 0)]


def bf16_bits_to_f32(a):
    """View bf16 bit patterns as float32 values (test helper)."""
    return (np.asarray(a, np.uint16).astype(np.uint32) << 16).view(np.float32)


def default_dims(kv_dtype=KV_BF16, index_heads=1, index_relu=0, index_topk=512, window=128):
    return dict(n_heads=64, head_dim=512, window=window, index_topk=index_topk, index_dim=128,
                index_heads=index_heads, index_relu=index_relu, kv_dtype=kv_dtype, softmax_scale=1.0)


def _kv_rows(seed, stream, rows, d, kv_dtype):
    if kv_dtype == KV_BF16:
        return normal_bf16(seed, stream, (rows, d)), None
    return normal_fp8(seed, stream, rows, d)


def decode_batch(seed, contexts, modes, ratios, dims=None, pool_cap=None, reuse_k=None, win_len=None,
                 weights=False):
    """General decode batch: query b sits at position contexts[b]-1 of its own
    sequence.  Full/Reuse queries get a pool of floor(context/ratio) rows (capped
    by pool_cap), window queries none.  Each query has min(window, context)
    window rows of its own.  weights=True draws per-head index weights
    ~ N(0, 1) (the indexer's per-token weights); otherwise they are None."""
    dims = dict(dims or default_dims())
    B = len(contexts)
    H, D, K = dims["n_heads"], dims["head_dim"], dims["index_topk"]
    HI, DI, W = dims["index_heads"], dims["index_dim"], dims["window"]
    ctx = np.asarray(contexts, np.int64)
    mode = np.asarray(modes, np.int32)
    ratio = np.asarray(ratios, np.int32)
    pos = ctx - 1
    pool_len = np.zeros(B, np.int32)
    for b in range(B):
        if mode[b] != MODE_WINDOW and ratio[b] > 0:
            pl = int(ctx[b] // ratio[b])
            pool_len[b] = pl if pool_cap is None else min(pl, pool_cap)
    pool_row0 = np.zeros(B, np.int64)
    pool_row0[1:] = np.cumsum(pool_len.astype(np.int64))[:-1]
    wl = np.minimum(ctx, W).astype(np.int32) if win_len is None else np.asarray(win_len, np.int32)
    win_row0 = np.zeros(B, np.int64)
    win_row0[1:] = np.cumsum(wl.astype(np.int64))[:-1]
    n_pool_rows = int(pool_len.sum())
    n_win_rows = int(wl.sum())
    kvd = dims["kv_dtype"]
    win_kv, win_scale = _kv_rows(seed, S_WIN, n_win_rows, D, kvd)
    comp_kv, comp_scale = _kv_rows(seed, S_POOL, n_pool_rows, D, kvd)
    inp = dict(
        name="decode", dims=dims, B=B, pos=pos, mode=mode, ratio=ratio,
        win_row0=win_row0, win_len=wl, pool_row0=pool_row0, pool_len=pool_len,
        q=normal_bf16(seed, S_Q, (B, H, D), scale=1.0 / math.sqrt(512.0)),
        win_kv=win_kv, win_scale=win_scale, comp_kv=comp_kv, comp_scale=comp_scale,
        idx_q=normal_f32(seed, S_IDXQ, (B, HI, DI)),
        idx_w=normal_f32(seed, S_IDXW, (B, HI)) if weights else None,
        idx_k=normal_f32(seed, S_IDXK, (n_pool_rows, DI)),
        sel_in=None, cand_off=None, cand_idx=None,
        max_pool_len=int(pool_len.max()) if B else 0,
    )
    if (mode == MODE_REUSE).any():
        sel = np.full((B, K), -1, np.int32)
        for b in np.nonzero(mode == MODE_REUSE)[0]:
            nv = min(int(pos[b] + 1) // int(ratio[b]), int(pool_len[b])) if ratio[b] > 0 else 0
            s = sample_distinct(seed, (S_REUSE << 32) + int(b), nv, reuse_k or K)
            sel[b, :len(s)] = s
        inp["sel_in"] = sel
    return inp


def add_reindex_lists(inp, seed, frac=0.25):
    """Give every Reindex query an ascending candidate list: a random subset of
    its pool rows (about ``frac`` of them, at least one), which may include rows
    the query cannot reach yet."""
    B = inp["B"]
    offs = np.zeros(B + 1, np.int64)
    parts = []
    for b in range(B):
        if inp["mode"][b] == MODE_REINDEX and inp["pool_len"][b] > 0:
            n = int(inp["pool_len"][b])
            s = sample_distinct(seed, (S_CAND << 32) + b, n, max(1, int(n * frac)))
        else:
            s = np.zeros(0, np.int32)
        parts.append(s)
        offs[b + 1] = offs[b] + len(s)
    inp["cand_off"] = offs
    inp["cand_idx"] = np.ascontiguousarray(np.concatenate(parts) if parts else np.zeros(0), np.int32)
    return inp


def prefill_chunk(seed, T, pos0, ratio, pool_len, dims=None, win_pos0=None, mode=MODE_FULL, weights=False):
    """One sequence: T queries at positions pos0 .. pos0+T-1.  The raw window rows
    cover positions win_pos0 .. pos0+T-1 (default: the W-1 positions before pos0
    as well, so every query sees a full window)."""
    dims = dict(dims or default_dims())
    H, D, HI, DI, W = dims["n_heads"], dims["head_dim"], dims["index_heads"], dims["index_dim"], dims["window"]
    if win_pos0 is None:
        win_pos0 = max(0, pos0 - W + 1)
    n_win = pos0 + T - win_pos0
    kvd = dims["kv_dtype"]
    win_kv, win_scale = _kv_rows(seed, S_WIN, n_win, D, kvd)
    comp_kv, comp_scale = _kv_rows(seed, S_POOL, pool_len, D, kvd)
    return dict(
        name="prefill", dims=dims, T=T, pos0=pos0, mode=mode, ratio=ratio, win_pos0=win_pos0,
        pool_len=pool_len,
        q=normal_bf16(seed, S_Q, (T, H, D), scale=1.0 / math.sqrt(512.0)),
        win_kv=win_kv, win_scale=win_scale, comp_kv=comp_kv, comp_scale=comp_scale,
        idx_q=normal_f32(seed, S_IDXQ, (T, HI, DI)),
        idx_w=normal_f32(seed, S_IDXW, (T, HI)) if weights else None,
        idx_k=normal_f32(seed, S_IDXK, (pool_len, DI)),
        sel_in=None, cand_off=None, cand_idx=None,
    )


# --- the five workloads -------------------------------------------------------

CONFIG_NAMES = ["tiny", "decode_full", "prefill", "decode_fp8_long", "mixed"]


def config(idx, index_heads=1):
    """Build workload ``idx`` (0..4) at its full size.  index_heads > 1 gives
    the workload the pages' indexer form instead of one plain-dot head:
    index_heads ReLU heads with per-head weights drawn N(0, 1)."""
    pages = index_heads > 1
    kw = dict(index_heads=index_heads, index_relu=1 if pages else 0)
    if idx == 0:  # one query, all 1,024 compressed rows reachable (pos 4095, ratio 4)
        return decode_batch(0, [4096], [MODE_FULL], [4], dims=default_dims(**kw), weights=pages)
    if idx == 1:  # 64 sequences at context 65,536, ratio 4 -> 16,384 candidates each
        return decode_batch(1, [65536] * 64, [MODE_FULL] * 64, [4] * 64, dims=default_dims(**kw), weights=pages)
    if idx == 2:  # 4,096 queries at 126,976 .. 131,071, ratio 8 -> pool of 16,384
        return prefill_chunk(2, 4096, 126976, 8, 16384, dims=default_dims(**kw), weights=pages)
    if idx == 3:  # 256 sequences at context 2^20, ratio 64, fp8 window and pool
        return decode_batch(3, [1 << 20] * 256, [MODE_FULL] * 256, [64] * 256,
                            dims=default_dims(kv_dtype=KV_FP8, **kw), weights=pages)
    if idx == 4:  # 128 queries, contexts U{1024..262144}; Full / Reuse / window-only by i mod 3
        ctx = uniform_int(4, S_CTX, 128, 1024, 262144)
        modes = [(MODE_FULL, MODE_REUSE, MODE_WINDOW)[i % 3] for i in range(128)]
        ratios = [0 if m == MODE_WINDOW else 4 for m in modes]
        return decode_batch(4, ctx, modes, ratios, dims=default_dims(**kw), weights=pages)
    raise ValueError(idx)
