"""Pins for the FP6 x FP4 variant's oracle: E2M3 elements (oracle.formats), the NVFP6 double block
(oracle.quant) and the backward with FP6 gradient operands (oracle.linear, grad_fmt="nvfp6").

Independent references: the E4M3FN grid (itself pinned against torch's float8_e4m3fn), np.rint on
the scaled value, closed forms of the double block, fp64 brute force, and statistics."""
import numpy as np
import pytest

from oracle import formats, gemm as ogemm, linear as olinear, quant

f32 = np.float32


def test_e2m3_grid_is_the_e4m3_values_on_an_eighth_step_up_to_7_5():
    """E2M3 magnitudes = the E4M3FN values of at most 7.5 that are multiples of 1/8 (so every FP6
    value has an E4M3 byte, the library's storage), 32 of them, largest 7.5."""
    e4 = formats.E4M3_POS
    ref = np.sort(e4[(e4 <= 7.5) & (np.floor(e4 * 8) == e4 * 8)])
    np.testing.assert_array_equal(formats.E2M3_MAG, ref)
    assert formats.E2M3_MAG.size == 32 and formats.E2M3_MAG[-1] == 7.5
    codes = np.arange(64, dtype=np.uint8)
    np.testing.assert_array_equal(formats.e4m3_decode(formats.e2m3_to_e4m3(codes)), formats.e2m3_decode(codes))
    # round trip of every grid value, both signs (-0 kept)
    for c in range(64):
        v = f32(formats.e2m3_decode(c))
        if c == 32:
            v = f32(-0.0)
        assert formats.e2m3_rtn(np.array([v]))[0] == c


@pytest.mark.parametrize("lo,hi", [(2.0 ** -6, 1.0), (1.0, 7.5)])
def test_e2m3_rtn_exhaustive_vs_rint(lo, hi):
    """Every 8th fp32 magnitude in [lo, hi] (both signs) against rint on the scaled value:
    below 1 the grid is k/8, above it 3 mantissa bits per binade; rint breaks ties to even."""
    a = np.arange(np.float32(lo).view(np.uint32), np.float32(hi).view(np.uint32) + 1, 8,
                  dtype=np.uint32).view(np.float32)
    a64 = a.astype(np.float64)
    e = np.floor(np.log2(np.maximum(a64, 1.0)))
    step = np.where(a64 < 1.0, 0.125, np.ldexp(1.0, (e - 3).astype(np.int64)))
    ref = np.rint(a64 / step) * step
    for sgn in (1, -1):
        got = formats.e2m3_decode(formats.e2m3_rtn((sgn * a).astype(np.float32)))
        np.testing.assert_array_equal(got, sgn * ref)


def test_e2m3_sr_up_probability_within_draw_resolution():
    u = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    grid = formats.E2M3_MAG
    vals = np.random.default_rng(4).uniform(0, 7.5, 40).astype(np.float32)
    for v in vals:
        out = formats.e2m3_decode(formats.e2m3_sr(np.full(65536, v), u))
        k = np.searchsorted(grid, float(v), side="right") - 1
        lo, hi = grid[k], grid[min(k + 1, 31)]
        assert set(np.unique(out)) <= {lo, hi}
        if hi == lo:
            continue
        p = (float(v) - lo) / (hi - lo)
        frac = np.count_nonzero(out == hi) / 65536.0
        assert p - 2.0 ** -16 < frac <= p


def test_nvfp6_double_block_closed_forms():
    """S = amax / 3360; the group holding the block maximum gets the inner scale 448 and encodes
    the maximum as +-7.5; every element's error is at most half a grid gap times d (RTN)."""
    rng = np.random.default_rng(1)
    y = (rng.standard_normal((64, 256)) * np.exp(rng.standard_normal((64, 1)))).astype(f32)
    q = quant.nvfp6_quantize_rows(y, "rtn")
    amax = np.abs(y).reshape(64, 2, 128).max(-1)
    np.testing.assert_array_equal(q.s128, (amax / f32(3360.0)).astype(f32))
    s_val = formats.e4m3_decode(q.s16)
    for r in range(64):
        for b in range(2):
            j = np.argmax(np.abs(y[r, b * 128:(b + 1) * 128])) // 16 + 8 * b
            assert s_val[r, j] == 448.0
            idx = b * 128 + np.argmax(np.abs(y[r, b * 128:(b + 1) * 128]))
            assert abs(formats.e4m3_decode(q.codes[r, idx])) == 7.5
    deq = quant.dequantize_f64(q)
    d = np.repeat(s_val, 16, axis=1) * np.repeat(q.s128.astype(np.float64), 128, axis=1)
    v = np.abs(y) / d
    gap = np.where(v < 1, 0.125, np.ldexp(1.0, np.floor(np.log2(np.maximum(v, 1))).astype(np.int64) - 3))
    assert np.all(np.abs(deq - y) <= 0.5 * gap * d * (1 + 1e-6) + 1e-30)


def test_fp6_product_brute_force():
    rng = np.random.default_rng(2)
    a = quant.quantize(rng.standard_normal((16, 48)).astype(f32), fmt="nvfp6", rounding="sr", seed=3, offset=1)
    b = quant.quantize(rng.standard_normal((24, 48)).astype(f32), fmt="nvfp4")
    A, B = quant.dequantize_f64(a), quant.dequantize_f64(b)
    ref = np.array([[sum(A[i, k] * B[j, k] for k in range(48)) for j in range(24)] for i in range(16)])
    np.testing.assert_allclose(ogemm.gemm_nt_f64(a, b), ref, rtol=1e-12, atol=1e-12)


def test_fp6_gradients_unbiased_and_closer_than_fp4():
    """With FP6 gradient operands the backward stays unbiased (mean over seeds -> the fp64 product of
    the quantized forward) and each draw lies closer to it than with FP4 gradients."""
    rng = np.random.default_rng(7)
    M, N, K = 64, 48, 64
    X = rng.standard_normal((M, K)).astype(f32)
    W = (rng.standard_normal((N, K)) * 0.05).astype(f32)
    dY = (rng.standard_normal((M, N)) * 0.01).astype(f32)
    fwd = olinear.linear_fwd(X, W)
    exact_dx = dY.astype(np.float64) @ quant.dequantize_f64(fwd["Wq"])
    exact_dw = dY.astype(np.float64).T @ quant.dequantize_f64(fwd["Xq"])
    err = {}
    for fmt in ("nvfp4", "nvfp6"):
        dx = [olinear.linear_bwd(dY, fwd, seed=s, offset=0, grad_fmt=fmt)["dX"] for s in range(64)]
        dw = [olinear.linear_bwd(dY, fwd, seed=s, offset=0, grad_fmt=fmt)["dW"] for s in range(64)]
        one = np.linalg.norm(dx[0] - exact_dx) / np.linalg.norm(exact_dx)
        mean = np.linalg.norm(np.mean(dx, 0) - exact_dx) / np.linalg.norm(exact_dx)
        mean_w = np.linalg.norm(np.mean(dw, 0) - exact_dw) / np.linalg.norm(exact_dw)
        assert mean < one / 4 and mean_w < 0.1  # averaging 64 draws shrinks the error ~8x
        err[fmt] = one
    assert err["nvfp6"] < 0.8 * err["nvfp4"]
