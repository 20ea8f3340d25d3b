"""GPU parity of the quantizers (bit-exact codes, E4M3 scales, FP32 scales vs the oracle).

Covers row (1x16) and column (16x1, transposed) grouping, RTN and Philox SR,
the 16-wide Hadamard transform, bf16 / fp32 / NVFP4 / FP8 inputs, NVFP4 and
FP8 outputs, channel gathers, ragged outer blocks, edge values, and the
8192x4096 quantizer-sweep tensor (sampled rows and columns).
"""
import numpy as np
import pytest
import torch

import synthetic
from oracle import philox, quant, rht

import _helpers as H

pytestmark = pytest.mark.gpu

tj2 = pytest.importorskip("bit_fully_quantized_amd")


def _x_bf16(shape, seed, std=1.0):
    bits = synthetic.normal_bf16(shape, std, seed)
    return bits, H.bf16_values(bits)


@pytest.mark.parametrize("shape", [(256, 512), (100, 400), (16, 16), (33, 2048)])
@pytest.mark.parametrize("rounding,use_rht", [("rtn", False), ("sr", False), ("sr", True)])
def test_row_bf16(shape, rounding, use_rht):
    bits, x = _x_bf16(shape, seed=shape[0] * 7 + shape[1])
    mask = philox.rht_signs(5, 17) if use_rht else None
    g = tj2.quantize(H.bf16_to_device(bits), grouping=tj2.GROUP_ROW, rounding=tj2.SR if rounding == "sr" else tj2.RTN,
                     rht=use_rht, signs=mask or 0, seed=5, offset=17)
    ref = quant.quantize(x, grouping="row", rounding=rounding, rht_mask=mask, seed=5, offset=17)
    H.assert_q_equal(g, ref, what=f"row {shape} {rounding} rht={use_rht}")
    H.assert_padding_zero(g)


@pytest.mark.parametrize("shape", [(512, 512), (48, 144)])
def test_row_f32_weights(shape):
    W = synthetic.normal_f32(shape, 0.02, seed=11)
    g = tj2.quantize(H.f32_to_device(W))
    H.assert_q_equal(g, quant.quantize(W), what="row f32")


@pytest.mark.parametrize("shape", [(256, 512), (400, 48), (128, 16), (2048, 96)])
@pytest.mark.parametrize("rounding,use_rht", [("rtn", False), ("sr", True)])
def test_col_bf16(shape, rounding, use_rht):
    bits, x = _x_bf16(shape, seed=3 + shape[0])
    mask = philox.rht_signs(9, 2) if use_rht else None
    g = tj2.quantize(H.bf16_to_device(bits), grouping=tj2.GROUP_COL, rounding=tj2.SR if rounding == "sr" else tj2.RTN,
                     rht=use_rht, signs=mask or 0, seed=9, offset=2)
    ref = quant.quantize(x, grouping="col", rounding=rounding, rht_mask=mask, seed=9, offset=2)
    assert (g.rows, g.len) == (shape[1], shape[0])
    H.assert_q_equal(g, ref, what=f"col {shape} {rounding}")
    H.assert_padding_zero(g)


@pytest.mark.parametrize("shape", [(256, 512), (144, 400)])
def test_col_from_nvfp4(shape):
    bits, x = _x_bf16(shape, seed=21)
    xq = tj2.quantize(H.bf16_to_device(bits))
    xq_ref = quant.quantize(x)
    H.assert_q_equal(xq, xq_ref, what="forward codes")
    mask = philox.rht_signs(1, 3)
    g = tj2.quantize(xq, grouping=tj2.GROUP_COL, rounding=tj2.SR, rht=True, signs=mask, seed=1, offset=3)
    ref = quant.quantize(quant.dequantize(xq_ref), grouping="col", rounding="sr", rht_mask=mask, seed=1, offset=3)
    H.assert_q_equal(g, ref, what="col from nvfp4")


def test_fp8_row_gather_and_col_from_fp8():
    bits, x = _x_bf16((256, 512), seed=31)
    outl = synthetic.outlier_columns(512, 0.125, seed=4)
    outl = np.sort(outl[:64])
    plan = tj2.OutlierPlan.from_indices(512, outl)
    xd = H.bf16_to_device(bits)
    g8 = tj2.quantize(xd, out_fmt=tj2.FP8, col_idx=plan.outliers)
    ref8 = quant.quantize(x[:, outl], fmt="fp8")
    H.assert_q_equal(g8, ref8, what="fp8 row gather")
    rest = np.setdiff1d(np.arange(512), outl)
    g4 = tj2.quantize(xd, col_idx=plan.rest)
    H.assert_q_equal(g4, quant.quantize(x[:, rest]), what="nvfp4 row gather")
    H.assert_padding_zero(g4)
    mask = philox.rht_signs(2, 5)
    gc = tj2.quantize(g8, grouping=tj2.GROUP_COL, rounding=tj2.SR, rht=True, signs=mask, seed=2, offset=5,
                      out_fmt=tj2.FP8)
    refc = quant.quantize(quant.dequantize(ref8), grouping="col", fmt="fp8", rounding="sr", rht_mask=mask,
                          seed=2, offset=5)
    H.assert_q_equal(gc, refc, what="fp8 col from fp8")


def test_edge_values():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    x[0, :] = 0.0
    x[1, :] = -0.0
    x[2, :128] = 2.0 ** -101          # empty outer block
    x[3, :] = 1e30
    x[3, 5] = -3e30
    x[4, :16] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0, -6.0]
    x[4, 16:32] = 6.0 * 448.0 / 16     # exact scale hits
    x[5, :] = np.float32(2.0 ** -130)  # fp32 subnormals
    x[5, 3] = 1.0
    x[6, ::2] = 0.0                    # half-zero groups
    x[7, :] = np.linspace(-1e-3, 1e3, 256, dtype=np.float32)
    xd = H.f32_to_device(x)
    for rounding, use_rht in [("rtn", False), ("sr", False), ("sr", True)]:
        for fmt in ["nvfp4", "fp8"]:
            mask = 0xB00F if use_rht else None
            g = tj2.quantize(xd, rounding=tj2.SR if rounding == "sr" else tj2.RTN, rht=use_rht, signs=mask or 0,
                             seed=77, offset=1, out_fmt=tj2.NVFP4 if fmt == "nvfp4" else tj2.FP8)
            ref = quant.quantize(x, fmt=fmt, rounding=rounding, rht_mask=mask, seed=77, offset=1)
            H.assert_q_equal(g, ref, what=f"edge {fmt} {rounding} {use_rht}")
    # bf16 subnormals through the column path
    bits = synthetic.f32_to_bf16_bits(x)
    g = tj2.quantize(H.bf16_to_device(bits), grouping=tj2.GROUP_COL, rounding=tj2.SR, seed=3, offset=3)
    H.assert_q_equal(g, quant.quantize(H.bf16_values(bits), grouping="col", rounding="sr", seed=3, offset=3),
                     what="edge col")


def test_quant_sweep_full_size_sampled():
    """8192x4096 bf16 N(0,1) with 1% of columns x64: full launches, sampled comparison."""
    R, C = synthetic.QUANT_SWEEP_SHAPE
    bits = synthetic.acts_with_outliers_bf16((R, C), 1.0, 0.01, 64.0, seed=synthetic.SEED_X)
    x = H.bf16_values(bits)
    xd = H.bf16_to_device(bits)
    rows = np.sort(np.random.default_rng(1).choice(R, 96, replace=False))
    cols = np.sort(np.random.default_rng(2).choice(C, 48, replace=False))
    cols = np.unique(np.concatenate([cols, [0, C - 1]]))
    mask = philox.rht_signs(0, 0)
    for rounding, use_rht in [("rtn", False), ("sr", False), ("sr", True)]:
        r = tj2.SR if rounding == "sr" else tj2.RTN
        g = tj2.quantize(xd, rounding=r, rht=use_rht, signs=mask if use_rht else 0, seed=0, offset=0)
        ref = H.oracle_rows(x[rows], rows, C, "nvfp4", rounding, 0, 0, mask if use_rht else None)
        H.assert_q_equal(g, ref, rows=rows, what=f"sweep row {rounding} {use_rht}")
        gc = tj2.quantize(xd, grouping=tj2.GROUP_COL, rounding=r, rht=use_rht, signs=mask if use_rht else 0,
                          seed=0, offset=2)
        refc = H.oracle_cols(x[:, cols], cols, C, "nvfp4", rounding, 0, 2, mask if use_rht else None)
        H.assert_q_equal(gc, refc, rows=cols, what=f"sweep col {rounding} {use_rht}")
    torch.cuda.synchronize()


def test_sr_unbiased_on_gpu():
    """Mean of dequantized SR outputs over offsets approaches the input (statistical)."""
    bits, x = _x_bf16((32, 256), seed=8)
    xd = H.bf16_to_device(bits)
    acc = np.zeros(x.shape)
    n = 256
    for off in range(n):
        g = tj2.quantize(xd, rounding=tj2.SR, seed=123, offset=off)
        acc += quant.dequantize(H.oracle_qtensor_from_gpu(g))
    err_sr = np.abs(acc / n - x).mean()
    err_rtn = np.abs(quant.dequantize(quant.quantize(x)) - x).mean()
    assert err_sr < 0.2 * err_rtn


def test_rtn_exhaustive_unit_step():
    """Every fp32 magnitude in [2^-8, 6], both signs, placed where the element step is exactly 1
    (outer max 2688 -> S = 1; every test group also holds a 6 -> s = 1): each code must equal
    round-to-nearest-even onto the E2M1 grid, computed independently with torch.round (half to even)."""
    lo = int(np.float32(2.0 ** -8).view(np.int32))
    hi = int(np.float32(6.0).view(np.int32))
    bits = torch.arange(lo, hi + 1, dtype=torch.int64, device="cuda").to(torch.int32)
    vals = bits.view(torch.float32)
    vals = torch.where(torch.arange(vals.numel(), device="cuda") % 2 == 0, vals, -vals)
    per_row = 7 * 15
    rows = (vals.numel() + per_row - 1) // per_row
    X = torch.zeros(rows, 128, dtype=torch.float32, device="cuda")
    X[:, 0] = 2688.0
    slots = torch.zeros(rows * per_row, dtype=torch.float32, device="cuda")
    slots[: vals.numel()] = vals
    body = X[:, 16:].view(rows, 7, 16)
    body[:, :, 0] = 6.0
    body[:, :, 1:] = slots.view(rows, 7, 15)
    q = tj2.quantize(X)
    assert torch.all(q.scale128[:, 0] == 1.0)
    assert torch.all(q.scale16[:, 1:8] == 0x38)  # E4M3 1.0
    c = q.codes[:, :64].view(rows, 64)
    nib = torch.stack([c & 15, c >> 4], dim=-1).view(rows, 128)[:, 16:].reshape(rows, 7, 16)[:, :, 1:].reshape(-1)
    nib = nib[: vals.numel()].to(torch.int64)
    a = vals.abs().double()
    step = torch.where(a < 2, 0.5, torch.where(a < 4, 1.0, 2.0))
    ref_mag = torch.clamp(torch.round(a / step) * step, max=6.0)
    grid = torch.tensor([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=torch.float64, device="cuda")
    ref_idx = torch.searchsorted(grid, ref_mag)
    ref = ref_idx | (torch.signbit(vals).to(torch.int64) << 3)
    bad = (nib != ref).sum().item()
    assert bad == 0, f"{bad} mismatches"


def test_fp8_rtn_exhaustive_unit_step():
    """Every fp32 magnitude in [2^-10, 448], both signs, quantized to FP8 where the element step is
    1 (outer max 448 -> S = 1): each code must equal round-to-nearest-even onto the E4M3 grid,
    computed independently with torch.round (half to even) on the grid step of each binade."""
    lo = int(np.float32(2.0 ** -10).view(np.int32))
    hi = int(np.float32(448.0).view(np.int32))
    bits = torch.arange(lo, hi + 1, dtype=torch.int64, device="cuda").to(torch.int32)
    vals = bits.view(torch.float32)
    vals = torch.where(torch.arange(vals.numel(), device="cuda") % 2 == 0, vals, -vals)
    per_row = 127
    rows = (vals.numel() + per_row - 1) // per_row
    X = torch.zeros(rows, 128, dtype=torch.float32, device="cuda")
    X[:, 0] = 448.0
    slots = torch.zeros(rows * per_row, dtype=torch.float32, device="cuda")
    slots[: vals.numel()] = vals
    X[:, 1:] = slots.view(rows, per_row)
    q = tj2.quantize(X, out_fmt=tj2.FP8)
    assert torch.all(q.scale128[:, 0] == 1.0)
    got = q.codes[:, 1:128].reshape(-1)[: vals.numel()].to(torch.int64)
    a = vals.abs().double()
    # grid step: 2^-9 below 2^-6 (subnormals), else 2^(e - 3) in the binade [2^e, 2^(e+1))
    e = torch.frexp(torch.clamp(a, min=2.0 ** -6)).exponent.double() - 1  # a in [2^e, 2^(e+1))
    step = torch.where(a < 2.0 ** -6, 2.0 ** -9, torch.exp2(e - 3))
    mag = torch.clamp(torch.round(a / step) * step, max=448.0)
    me = torch.frexp(torch.clamp(mag, min=2.0 ** -6)).exponent.double() - 1
    normal = mag >= 2.0 ** -6
    code = torch.where(normal, ((me + 7) * 8 + (mag / torch.exp2(me) - 1) * 8), mag / 2.0 ** -9).round().to(torch.int64)
    ref = code | (torch.signbit(vals).to(torch.int64) << 7)
    bad = (got != ref).sum().item()
    assert bad == 0, f"{bad} mismatches"
