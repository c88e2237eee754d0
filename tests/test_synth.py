"""The seeded input generator: reproducible, slice-consistent, right shapes
and distributions.  (It holds no attention arithmetic.)"""
import numpy as np
import torch

from sparse_long_context_amd import synth


def test_counter_based_slices_agree():
    full = synth.normal_f32(5, 3, (1000,))
    part = synth.normal_f32(5, 3, (300,), start=400)
    assert np.array_equal(full[400:700], part)
    b_full = synth.normal_bf16(5, 3, (1000,))
    b_part = synth.normal_bf16(5, 3, (11,), start=7)
    assert np.array_equal(b_full[7:18], b_part)
    # different seeds / streams differ
    assert not np.array_equal(full, synth.normal_f32(6, 3, (1000,)))
    assert not np.array_equal(full, synth.normal_f32(5, 4, (1000,)))


def test_normal_moments():
    x = synth.normal_f32(1, 1, (1 << 20,)).astype(np.float64)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1) < 5e-3
    assert abs((x ** 4).mean() - 3) < 0.05


def test_bf16_is_rne_of_fp32():
    f = synth.normal_f32(2, 9, (4096,), scale=0.3)
    b = synth.normal_bf16(2, 9, (4096,), scale=0.3)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, ref)


def test_fp8_quantisation_properties():
    codes, scales = synth.normal_fp8(3, 2, 64, 512)
    x = synth.normal_f32(3, 2, (64, 512))
    val = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    sc = np.ldexp(1.0, scales.astype(np.int64) - 127).repeat(32, axis=1)
    deq = val * sc
    # scale is the smallest power of two covering the block max with 448
    amax = np.abs(x.reshape(64, 16, 32)).max(-1)
    s = np.ldexp(1.0, scales.astype(np.int64) - 127)
    assert (amax <= 448 * s).all() and (amax > 224 * s).all()
    # every code is the nearest e4m3 value: error at most half a step of its binade
    err = np.abs(deq - x)
    step = np.ldexp(1.0, np.floor(np.log2(np.maximum(np.abs(x) / sc, 2.0 ** -6))).astype(np.int64) - 3) * sc
    assert (err <= step / 2 + 1e-30).all()


def test_sample_distinct():
    s = synth.sample_distinct(4, 7, 10000, 512)
    assert len(s) == 512 and len(np.unique(s)) == 512 and (np.diff(s) > 0).all()
    assert s.min() >= 0 and s.max() < 10000
    assert np.array_equal(synth.sample_distinct(4, 7, 300, 512), np.arange(300))


def test_small_decode_batch_layout():
    inp = synth.decode_batch(0, [1000, 5000, 64], [0, 2, 3], [4, 4, 0],
                             dims=synth.default_dims())
    assert list(inp["pool_len"]) == [250, 1250, 0]
    assert list(inp["pool_row0"]) == [0, 250, 1500]
    assert list(inp["win_len"]) == [128, 128, 64]
    assert inp["comp_kv"].shape == (1500, 512) and inp["idx_k"].shape == (1500, 128)
    sel = inp["sel_in"][1]
    assert (sel[:512] >= 0).all() and (np.diff(sel) > 0).all() and sel.max() < 1250
