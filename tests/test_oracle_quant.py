"""Pins for oracle.quant: double-block NVFP4 and per-block FP8 quantizers.

Independent references: closed-form constructions whose codes and scales are
known (grid round trip with S = s = 1), invariants of the scale rules (the
inner block holding the outer maximum gets scale 448; no element needs
clipping; the RTN error bound of half a grid gap), the empty-block rule, and
unbiasedness of stochastic rounding over independent draws (TetraJet-v2
technical summary, section 2.A).
"""
import numpy as np
import pytest

from oracle import formats, philox, quant

GRID = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)


def codes_of(q):
    return quant.unpack_nibbles(q.codes)


def test_grid_round_trip_unit_scales():
    # outer max 2688 -> S = 1; a block whose max is 6 -> s = 1 -> d = 1: codes equal the grid values
    row = np.zeros(128, np.float32)
    row[0:16] = 2688.0
    vals = np.concatenate([GRID, -GRID[1:], [-0.0]]).astype(np.float32)  # 16 values incl. +-0
    row[16:32] = vals
    row[16] = 6.0  # keep the inner max at 6 (value 0 appears at position 17 instead)
    row[17] = 0.0
    q = quant.nvfp4_quantize_rows(row[None, :])
    assert q.s128[0, 0] == np.float32(1.0)
    assert q.s16[0, 1] == formats.e4m3_round_up(np.float32(1.0))
    got = formats.e2m1_decode(codes_of(q)[0, 16:32])
    np.testing.assert_array_equal(got, row[16:32].astype(np.float64))
    assert np.array_equal(np.signbit(got), np.signbit(row[16:32]))
    np.testing.assert_array_equal(quant.dequantize(q)[0, 16:32], row[16:32])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_outer_max_block_gets_scale_448(seed):
    r = np.random.default_rng(seed)
    y = (r.standard_normal((64, 384)) * np.exp(r.standard_normal((64, 1)) * 4)).astype(np.float32)
    q = quant.nvfp4_quantize_rows(y)
    a = np.abs(y).reshape(64, 3, 8, 16).max(-1)
    holder = a.argmax(-1)  # inner block holding each outer max
    s = q.s16.reshape(64, 3, 8)
    picked = np.take_along_axis(s, holder[..., None], axis=-1)[..., 0]
    assert np.all(picked == 0x7E)  # 448
    # and that block contains a code of magnitude 6 at the max position
    c = codes_of(q).reshape(64, 3, 8, 16)
    pos = np.abs(y).reshape(64, 3, 128).argmax(-1)
    cmax = np.take_along_axis(c.reshape(64, 3, 128), pos[..., None], axis=-1)[..., 0]
    assert np.all((cmax & 7) == 7)


def test_scaled_elements_never_need_clipping():
    r = np.random.default_rng(3)
    y = (r.standard_normal((256, 512)) * np.exp(r.standard_normal((256, 32)).repeat(16, 1) * 3)).astype(np.float32)
    q = quant.nvfp4_quantize_rows(y)
    s = formats.e4m3_decode(q.s16).astype(np.float32)
    d = (s * np.repeat(q.s128, 8, axis=1)).astype(np.float32)
    inv = (np.float32(1) / d).astype(np.float32)
    v = y * np.repeat(inv, 16, axis=1)
    assert np.abs(v).max() <= 6.0 * (1 + 4 * 2.0 ** -24)


def test_rtn_error_bound():
    r = np.random.default_rng(4)
    y = (r.standard_normal((128, 256)) * 3).astype(np.float32)
    q = quant.nvfp4_quantize_rows(y)
    xh = quant.dequantize(q).astype(np.float64)
    d = (formats.e4m3_decode(q.s16) * np.repeat(q.s128.astype(np.float64), 8, axis=1))
    d_e = np.repeat(d, 16, axis=1)
    v = np.abs(y.astype(np.float64)) / d_e
    half_gap = np.where(v < 2, 0.25, np.where(v < 4, 0.5, 1.0))
    assert np.all(np.abs(xh - y) <= half_gap * d_e * (1 + 1e-5) + 1e-30)


def test_empty_and_tiny_blocks():
    y = np.zeros((3, 256), np.float32)
    y[1, :] = -0.0
    y[2, :128] = np.float32(2.0 ** -101)  # below the empty-block threshold
    y[2, 128:] = 1.0
    q = quant.nvfp4_quantize_rows(y)
    c = codes_of(q)
    assert np.all(c[0] == 0) and np.all(c[1] == 8) and np.all(c[2, :128] == 0)
    assert np.all(q.s128[:2] == 0) and q.s128[2, 0] == 0 and q.s128[2, 1] > 0
    assert np.all(q.s16[:2] == 0) and np.all(q.s16[2, :8] == 0)
    f8 = quant.fp8_quantize_rows(y)
    assert np.all(f8.codes[0] == 0) and np.all(f8.codes[1] == 0x80) and np.all(f8.s128[:2] == 0)


def test_partial_outer_block():
    r = np.random.default_rng(5)
    y = r.standard_normal((4, 144)).astype(np.float32)  # one full block + a 16-element block
    q = quant.nvfp4_quantize_rows(y)
    assert q.s128.shape == (4, 2) and q.s16.shape == (4, 9)
    a_last = np.abs(y[:, 128:]).max(1)
    np.testing.assert_array_equal(q.s128[:, 1], (a_last / np.float32(2688)).astype(np.float32))
    assert np.all(q.s16[:, 8] == 0x7E)


def test_col_grouping_is_row_grouping_of_transpose():
    r = np.random.default_rng(6)
    x = r.standard_normal((96, 48)).astype(np.float32)
    qc = quant.quantize(x, grouping="col", rounding="sr", rht_mask=0x1357, seed=9, offset=4)
    from oracle import rht
    y = rht.rht_along_last(np.ascontiguousarray(x.T), 0x1357)
    u = philox.sr_draws_for_shape(y.shape, 9, 4)  # draws follow the output (grouped) layout
    qr = quant.nvfp4_quantize_rows(y, "sr", u)
    assert np.array_equal(qc.codes, qr.codes) and np.array_equal(qc.s16, qr.s16)
    assert np.array_equal(qc.s128, qr.s128) and (qc.rows, qc.L) == (48, 96)


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8"])
def test_sr_unbiased_over_offsets(fmt):
    r = np.random.default_rng(7)
    x = (r.standard_normal((16, 128)) * 2).astype(np.float32)
    n = 400
    acc = np.zeros(x.shape)
    for off in range(n):
        acc += quant.dequantize(quant.quantize(x, fmt=fmt, rounding="sr", seed=11, offset=off))
    mean = acc / n
    q0 = quant.quantize(x, fmt=fmt, rounding="rtn")
    # scales do not depend on the draws, so the per-element gap is fixed
    if fmt == "nvfp4":
        d = np.repeat(formats.e4m3_decode(q0.s16) * np.repeat(q0.s128.astype(np.float64), 8, 1), 16, 1)
        v = np.abs(x) / d
        gap = np.where(v < 2, 0.5, np.where(v < 4, 1.0, 2.0)) * d
    else:
        S8 = np.repeat(q0.s128.astype(np.float64), 128, 1)
        e = np.abs(x) / S8
        lo = formats.E4M3_POS[np.clip(np.searchsorted(formats.E4M3_POS, e, side="right") - 1, 0, 125)]
        hi = formats.E4M3_POS[np.clip(np.searchsorted(formats.E4M3_POS, e, side="right"), 0, 126)]
        gap = (hi - lo) * S8
    z = (mean - x) / (0.5 * gap / np.sqrt(n) + 1e-30)
    assert np.abs(z).max() < 6.0
    rtn_err = np.abs(quant.dequantize(q0) - x).mean()
    assert np.abs(mean - x).mean() < 0.25 * rtn_err


def test_fp8_unit_scale_round_trip():
    vals = formats.E4M3_POS[1:].astype(np.float32)  # 126 values ending in 448
    row = np.concatenate([vals, [0.0, -1.0]]).astype(np.float32)[None, :]  # 128 entries, max 448 -> S8 = 1
    q = quant.fp8_quantize_rows(row)
    assert q.s128[0, 0] == 1.0
    np.testing.assert_array_equal(quant.dequantize(q), row)


def test_dequantize_f64_matches_f32_within_one_rounding():
    r = np.random.default_rng(8)
    y = (r.standard_normal((32, 256)) * 10).astype(np.float32)
    q = quant.nvfp4_quantize_rows(y)
    d32 = quant.dequantize(q).astype(np.float64)
    d64 = quant.dequantize_f64(q)
    assert np.all(np.abs(d32 - d64) <= np.abs(d64) * 2.0 ** -24)


@pytest.mark.parametrize("rounding", ["rtn", "sr"])
def test_group_below_block_scale_range_encodes_zeros(rounding):
    """A group more than 2^149 below its outer block's scale (its amax / (6 S) underflows fp32):
    inner scale 0, codes the elements' signed zeros, dequantized values 0; the rest of the block
    is quantized as usual (the block maximum takes the largest inner scale)."""
    y = np.zeros((1, 128), np.float32)
    y[0, :16] = np.float32(3e37) * np.sign(np.arange(16) - 7.5).astype(np.float32)
    tiny = np.array([1e-39, -2e-39, 3e-40, -0.0, 0.0, 5e-39] + [1e-39] * 10, np.float32)
    y[0, 16:32] = tiny
    q = quant.quantize(y, rounding=rounding, seed=1, offset=0)
    assert (np.float32(1e-39) / (np.float32(6) * q.s128[0, 0])) == 0  # the ratio does underflow
    assert q.s16[0, 1] == 0 and q.s16[0, 0] == 0x7E
    c = codes_of(q)[0, 16:32]
    np.testing.assert_array_equal(c, np.where(np.signbit(tiny), 8, 0))
    d = quant.dequantize_f64(q)
    assert np.all(d[0, 16:32] == 0) and np.all(np.abs(d[0, :16]) > 1e37)
