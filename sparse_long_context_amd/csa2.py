"""Thin ctypes binding of libcsa2 (include/csa2.h).

Argument marshalling only: every step of the attention runs in the library's
HIP kernels.  Functions carry the C names; tensor arguments are torch device
tensors (or None for NULL), and the stream defaults to torch's current stream.
A non-OK status raises ``Csa2Error``.  The library must have been built
(``sparse_long_context_amd.build``); there is no fallback.
"""
import ctypes as C
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libcsa2.so")

CSA2_OK, CSA2_ERR_INVALID_ARG, CSA2_ERR_UNSUPPORTED, CSA2_ERR_WORKSPACE, CSA2_ERR_HIP, CSA2_ERR_PRECONDITION = range(6)
# bits of the device-side precondition word (CSA2_DEBUG_CHECK=1)
CSA2_PRE_MODE, CSA2_PRE_DESC, CSA2_PRE_LIST, CSA2_PRE_SEL, CSA2_PRE_KV_SCALE, CSA2_PRE_INDEX = 1, 2, 4, 8, 16, 32
MODE_FULL, MODE_REINDEX, MODE_REUSE, MODE_WINDOW = range(4)
KV_BF16, KV_FP8, KV_FP4 = 0, 1, 2
IDXK_F32, IDXK_MXFP4 = 0, 1


class Csa2Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


class Dims(C.Structure):
    _fields_ = [("n_heads", C.c_int32), ("head_dim", C.c_int32), ("window", C.c_int32),
                ("index_topk", C.c_int32), ("index_dim", C.c_int32), ("index_heads", C.c_int32),
                ("index_relu", C.c_int32), ("kv_dtype", C.c_int32), ("softmax_scale", C.c_float),
                ("index_key_dtype", C.c_int32)]

    @classmethod
    def from_dict(cls, d):
        return cls(**{k: d.get(k, 0) for k, _ in cls._fields_})


class Batch(C.Structure):
    _fields_ = [("pos", C.c_void_p), ("mode", C.c_void_p), ("compress_ratio", C.c_void_p),
                ("win_row0", C.c_void_p), ("win_len", C.c_void_p), ("pool_row0", C.c_void_p),
                ("pool_len", C.c_void_p), ("cand_off", C.c_void_p), ("cand_idx", C.c_void_p),
                ("max_candidates", C.c_int32)]


class PrefillDesc(C.Structure):
    _fields_ = [("pos0", C.c_int64), ("n_queries", C.c_int32), ("mode", C.c_int32),
                ("compress_ratio", C.c_int32), ("pool_len", C.c_int32), ("win_pos0", C.c_int64),
                ("cand_off", C.c_void_p), ("cand_idx", C.c_void_p), ("max_candidates", C.c_int32)]


class OutRope(C.Structure):
    """csa2_out_rope: the output de-rotation fused into the attention's writes."""
    _fields_ = [("rope_offset", C.c_int32), ("rope_dims", C.c_int32), ("inv_freq", C.c_void_p)]


def out_rope(rope_offset, rope_dims, inv_freq):
    """An OutRope over a device f64 tensor of rope_dims / 2 inverse frequencies."""
    return OutRope(int(rope_offset), int(rope_dims), _p(inv_freq))


def _rope(r):
    return None if r is None else C.byref(r)


_lib = None
EXPORTS = ["csa2_abi_version", "csa2_status_str", "csa2_last_hip_error", "csa2_last_precondition",
           "csa2_workspace_size",
           "csa2_index_scores", "csa2_topk", "csa2_attend", "csa2_decode", "csa2_prefill_workspace_size",
           "csa2_prefill", "csa2_quantize_fp4_kv", "csa2_quantize_mxfp4", "csa2_candidate_pool_workspace_size",
           "csa2_candidate_pool", "csa2_compress", "csa2_derotate", "csa2_decode_static",
           "csa2_prefill_index_scores", "csa2_compress_step"]
CSA2_STATIC_SCRATCH_BYTES = 64 << 20


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = C.CDLL(LIB_PATH)
        P, i32, i64, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_size_t
        L.csa2_abi_version.restype = C.c_int
        L.csa2_status_str.argtypes = [C.c_int]
        L.csa2_status_str.restype = C.c_char_p
        L.csa2_last_hip_error.restype = i32
        L.csa2_last_precondition.restype = C.c_uint32
        L.csa2_workspace_size.argtypes = [P, i32, i32, C.POINTER(sz)]
        L.csa2_index_scores.argtypes = [P, i32, P, P, P, P, P, P, i64, P]
        L.csa2_topk.argtypes = [P, i32, P, P, i64, P, P, sz, P]
        L.csa2_attend.argtypes = [P, i32, P, P, P, P, P, P, P, P, P, P, P, sz, P, P]
        L.csa2_decode.argtypes = [P, i32, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, sz, P, P]
        L.csa2_prefill_workspace_size.argtypes = [P, P, C.POINTER(sz)]
        L.csa2_prefill.argtypes = [P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, sz, P, P]
        L.csa2_quantize_fp4_kv.argtypes = [i64, i32, P, P, P, P]
        L.csa2_candidate_pool_workspace_size.argtypes = [i32, i32, i32, i32, C.POINTER(sz)]
        L.csa2_candidate_pool.argtypes = [i32, P, P, i64, i32, i32, P, P, P, sz, P]
        L.csa2_compress.argtypes = [i64, i32, i32, P, P, P, C.c_float, P, P]
        L.csa2_derotate.argtypes = [P, i32, P, i32, i32, P, P, P]
        L.csa2_quantize_mxfp4.argtypes = [i64, i32, P, P, P, P]
        L.csa2_decode_static.argtypes = [P, i32, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P]
        L.csa2_prefill_index_scores.argtypes = [P, P, P, P, P, P, P, i64, P, sz, P]
        L.csa2_compress_step.argtypes = [i32, i32, i32, P, P, P, P, P, P, C.c_float, P, P, P]
        for name in EXPORTS[4:]:
            getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


def status_str(s):
    return lib().csa2_status_str(int(s)).decode()


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ok(st, where):
    if st != CSA2_OK:
        raise Csa2Error(st, where)


def csa2_abi_version():
    return lib().csa2_abi_version()


def csa2_last_hip_error():
    return lib().csa2_last_hip_error()


def csa2_last_precondition():
    return lib().csa2_last_precondition()


def csa2_workspace_size(dims, B, max_candidates):
    out = C.c_size_t()
    _ok(lib().csa2_workspace_size(C.byref(dims), B, max_candidates, C.byref(out)), "csa2_workspace_size")
    return out.value


def csa2_index_scores(dims, B, batch, idx_q, idx_w, idx_k, scores, score_stride, stream=None, idx_k_scale=None):
    _ok(lib().csa2_index_scores(C.byref(dims), B, C.byref(batch), _p(idx_q), _p(idx_w), _p(idx_k),
                                _p(idx_k_scale), _p(scores), score_stride, _stream(stream)), "csa2_index_scores")


def csa2_topk(dims, B, batch, scores, score_stride, topk_idx, stream=None, workspace=None, workspace_bytes=0):
    _ok(lib().csa2_topk(C.byref(dims), B, C.byref(batch), _p(scores), score_stride, _p(topk_idx), _p(workspace),
                        workspace_bytes, _stream(stream)), "csa2_topk")


def csa2_attend(dims, B, batch, q, win_kv, win_scale, comp_kv, comp_scale, topk_idx, sink, out, lse,
                workspace, workspace_bytes, stream=None, rope=None):
    _ok(lib().csa2_attend(C.byref(dims), B, C.byref(batch), _p(q), _p(win_kv), _p(win_scale), _p(comp_kv),
                          _p(comp_scale), _p(topk_idx), _p(sink), _p(out), _p(lse), _p(workspace),
                          workspace_bytes, _rope(rope), _stream(stream)), "csa2_attend")


def csa2_decode(dims, B, batch, q, idx_q, idx_w, idx_k, win_kv, win_scale, comp_kv, comp_scale, topk_idx, sink,
                out, lse, workspace, workspace_bytes, stream=None, idx_k_scale=None, rope=None):
    _ok(lib().csa2_decode(C.byref(dims), B, C.byref(batch), _p(q), _p(idx_q), _p(idx_w), _p(idx_k),
                          _p(idx_k_scale), _p(win_kv),
                          _p(win_scale), _p(comp_kv), _p(comp_scale), _p(topk_idx), _p(sink), _p(out), _p(lse),
                          _p(workspace), workspace_bytes, _rope(rope), _stream(stream)), "csa2_decode")


def csa2_decode_static(dims, B, batch, q, idx_q, idx_w, idx_k, win_kv, win_scale, comp_kv, comp_scale, topk_idx,
                       sink, out, lse, stream=None, idx_k_scale=None, rope=None):
    _ok(lib().csa2_decode_static(C.byref(dims), B, C.byref(batch), _p(q), _p(idx_q), _p(idx_w), _p(idx_k),
                                 _p(idx_k_scale), _p(win_kv), _p(win_scale), _p(comp_kv), _p(comp_scale),
                                 _p(topk_idx), _p(sink), _p(out), _p(lse), _rope(rope), _stream(stream)),
        "csa2_decode_static")


def csa2_prefill_workspace_size(dims, desc):
    out = C.c_size_t()
    _ok(lib().csa2_prefill_workspace_size(C.byref(dims), C.byref(desc), C.byref(out)),
        "csa2_prefill_workspace_size")
    return out.value


def csa2_prefill_index_scores(dims, desc, idx_q, idx_w, idx_k, scores, score_stride, workspace, workspace_bytes,
                              stream=None, idx_k_scale=None):
    _ok(lib().csa2_prefill_index_scores(C.byref(dims), C.byref(desc), _p(idx_q), _p(idx_w), _p(idx_k),
                                        _p(idx_k_scale), _p(scores), score_stride, _p(workspace), workspace_bytes,
                                        _stream(stream)), "csa2_prefill_index_scores")


def csa2_prefill(dims, desc, q, idx_q, idx_w, idx_k, win_kv, win_scale, comp_kv, comp_scale, topk_idx, sink,
                 out, lse, workspace, workspace_bytes, stream=None, idx_k_scale=None, rope=None):
    _ok(lib().csa2_prefill(C.byref(dims), C.byref(desc), _p(q), _p(idx_q), _p(idx_w), _p(idx_k),
                           _p(idx_k_scale), _p(win_kv),
                           _p(win_scale), _p(comp_kv), _p(comp_scale), _p(topk_idx), _p(sink), _p(out), _p(lse),
                           _p(workspace), workspace_bytes, _rope(rope), _stream(stream)), "csa2_prefill")


def csa2_quantize_fp4_kv(n_rows, d, src, codes, scales, stream=None):
    _ok(lib().csa2_quantize_fp4_kv(n_rows, d, _p(src), _p(codes), _p(scales), _stream(stream)),
        "csa2_quantize_fp4_kv")


def csa2_quantize_mxfp4(n_rows, d, src, codes, scales, stream=None):
    _ok(lib().csa2_quantize_mxfp4(n_rows, d, _p(src), _p(codes), _p(scales), _stream(stream)),
        "csa2_quantize_mxfp4")


def csa2_candidate_pool_workspace_size(B, max_candidates, block_size, top_blocks):
    out = C.c_size_t()
    _ok(lib().csa2_candidate_pool_workspace_size(B, max_candidates, block_size, top_blocks, C.byref(out)),
        "csa2_candidate_pool_workspace_size")
    return out.value


def csa2_candidate_pool(B, batch, scores, score_stride, block_size, top_blocks, cand_off, cand_idx, workspace,
                        workspace_bytes, stream=None):
    _ok(lib().csa2_candidate_pool(B, C.byref(batch), _p(scores), score_stride, block_size, top_blocks, _p(cand_off),
                                  _p(cand_idx), _p(workspace), workspace_bytes, _stream(stream)), "csa2_candidate_pool")


def csa2_compress(n_groups, m, d, c, g, norm_w, eps, out, stream=None):
    _ok(lib().csa2_compress(n_groups, m, d, _p(c), _p(g), _p(norm_w), float(eps), _p(out), _stream(stream)),
        "csa2_compress")


def csa2_compress_step(B, m, d, pos, c_new, g_new, kv_state, score_state, norm_w, eps, out, emit_idx, stream=None):
    _ok(lib().csa2_compress_step(B, m, d, _p(pos), _p(c_new), _p(g_new), _p(kv_state), _p(score_state), _p(norm_w),
                                 float(eps), _p(out), _p(emit_idx), _stream(stream)), "csa2_compress_step")


def csa2_derotate(dims, B, pos, rope_offset, rope_dims, inv_freq, out, stream=None):
    _ok(lib().csa2_derotate(C.byref(dims), B, _p(pos), rope_offset, rope_dims, _p(inv_freq), _p(out),
                            _stream(stream)), "csa2_derotate")


# ---- device-resident workloads (torch used for memory only) -------------------

def _dev(a, device):
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:  # bf16 bit patterns travel as int16
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


class DecodeWorkload:
    """A decode batch (dict from ``synth``) copied to device memory, with its
    descriptor struct, output buffers and workspace."""

    def __init__(self, inp, device="cuda", sink=None):
        import torch
        self.inp = inp
        self.B = int(inp["B"])
        self.dims = Dims.from_dict(inp["dims"])
        d = lambda k: _dev(inp.get(k), device)  # noqa: E731
        self.pos, self.mode, self.ratio = d("pos"), d("mode"), d("ratio")
        self.win_row0, self.win_len, self.pool_row0, self.pool_len = d("win_row0"), d("win_len"), d("pool_row0"), d("pool_len")
        self.cand_off, self.cand_idx = d("cand_off"), d("cand_idx")
        self.q, self.win_kv, self.win_scale = d("q"), d("win_kv"), d("win_scale")
        self.comp_kv, self.comp_scale = d("comp_kv"), d("comp_scale")
        self.idx_q, self.idx_w, self.idx_k, self.idx_k_scale = d("idx_q"), d("idx_w"), d("idx_k"), d("idx_k_scale")
        self.sink = None if sink is None else _dev(np.asarray(sink, np.float32), device)
        K, H, D = inp["dims"]["index_topk"], inp["dims"]["n_heads"], inp["dims"]["head_dim"]
        if inp.get("cand_off") is not None:
            lens = np.diff(inp["cand_off"])
            self.max_cand = int(max(int(inp["max_pool_len"]), int(lens.max()) if len(lens) else 0))
        else:
            self.max_cand = int(inp["max_pool_len"])
        sel_in = inp.get("sel_in")
        self.topk = _dev(sel_in if sel_in is not None else np.full((self.B, K), -1, np.int32), device)
        self.out = torch.empty((self.B, H, D), dtype=torch.float32, device=device)
        self.lse = torch.empty((self.B, H), dtype=torch.float32, device=device)
        self.batch = Batch(_p(self.pos), _p(self.mode), _p(self.ratio), _p(self.win_row0), _p(self.win_len),
                           _p(self.pool_row0), _p(self.pool_len), _p(self.cand_off), _p(self.cand_idx),
                           self.max_cand)
        self.ws_bytes = csa2_workspace_size(self.dims, self.B, self.max_cand)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=device)

    def decode(self, stream=None, rope=None):
        csa2_decode(self.dims, self.B, self.batch, self.q, self.idx_q, self.idx_w, self.idx_k, self.win_kv,
                    self.win_scale, self.comp_kv, self.comp_scale, self.topk, self.sink, self.out, self.lse,
                    self.ws, self.ws_bytes, stream, idx_k_scale=self.idx_k_scale, rope=rope)


class PrefillWorkload:
    """A prefill chunk (dict from ``synth.prefill_chunk``) in device memory."""

    def __init__(self, pf, device="cuda", sink=None):
        import torch
        self.pf = pf
        self.T = int(pf["T"])
        self.dims = Dims.from_dict(pf["dims"])
        d = lambda k: _dev(pf.get(k), device)  # noqa: E731
        self.q, self.win_kv, self.win_scale = d("q"), d("win_kv"), d("win_scale")
        self.comp_kv, self.comp_scale = d("comp_kv"), d("comp_scale")
        self.idx_q, self.idx_w, self.idx_k, self.idx_k_scale = d("idx_q"), d("idx_w"), d("idx_k"), d("idx_k_scale")
        self.cand_off, self.cand_idx = d("cand_off"), d("cand_idx")
        self.sink = None if sink is None else _dev(np.asarray(sink, np.float32), device)
        K, H, D = pf["dims"]["index_topk"], pf["dims"]["n_heads"], pf["dims"]["head_dim"]
        max_cand = 0
        if pf.get("cand_off") is not None:
            max_cand = int(np.diff(pf["cand_off"]).max())
        self.desc = PrefillDesc(int(pf["pos0"]), self.T, int(pf["mode"]), int(pf["ratio"]), int(pf["pool_len"]),
                                int(pf["win_pos0"]), _p(self.cand_off), _p(self.cand_idx), max_cand)
        sel_in = pf.get("sel_in")
        self.topk = _dev(sel_in if sel_in is not None else np.full((self.T, K), -1, np.int32), device)
        self.out = torch.empty((self.T, H, D), dtype=torch.float32, device=device)
        self.lse = torch.empty((self.T, H), dtype=torch.float32, device=device)
        self.ws_bytes = csa2_prefill_workspace_size(self.dims, self.desc)
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=device)

    def index_scores(self, scores, stride, stream=None):
        csa2_prefill_index_scores(self.dims, self.desc, self.idx_q, self.idx_w, self.idx_k, scores, stride, self.ws,
                                  self.ws_bytes, stream, idx_k_scale=self.idx_k_scale)

    def prefill(self, stream=None, rope=None):
        csa2_prefill(self.dims, self.desc, self.q, self.idx_q, self.idx_w, self.idx_k, self.win_kv, self.win_scale,
                     self.comp_kv, self.comp_scale, self.topk, self.sink, self.out, self.lse, self.ws, self.ws_bytes,
                     stream, idx_k_scale=self.idx_k_scale, rope=rope)
