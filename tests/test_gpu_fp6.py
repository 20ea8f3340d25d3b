"""GPU parity of the FP6 x FP4 variant (the mixed-precision strategy TetraJet-v2's technical summary
names as future work, section 5): NVFP6 quantizers (E2M3 elements in the double block) bit-exact against
the oracle, FP6 x FP4 products within the fp32-accumulation bound of the fp64 product of the oracle's
operands, and the FP6-gradient backward (nvfp6x4_linear_bwd) end to end, with and without an
outlier plan."""
import numpy as np
import pytest
import torch

import synthetic
from oracle import formats, gemm as ogemm, linear as olinear, philox, quant

import _helpers as H

pytestmark = pytest.mark.gpu

tj2 = pytest.importorskip("bit_fully_quantized_amd")


# row grouping at ragged row counts; column grouping (rows grouped by 16) at rows in multiples of 16
_NVFP6_CASES = [("row", 100, 400, "rtn", False), ("row", 33, 2048, "sr", False), ("row", 64, 256, "sr", True),
                ("row", 16, 16, "sr", True), ("row", 130, 144, "rtn", False),
                ("col", 112, 400, "rtn", False), ("col", 48, 2048, "sr", False), ("col", 64, 256, "sr", True),
                ("col", 16, 16, "sr", True), ("col", 144, 144, "rtn", False)]


@pytest.mark.parametrize("grouping,R,C,rounding,rht", _NVFP6_CASES)
def test_nvfp6_quantize(grouping, R, C, rounding, rht):
    bits = synthetic.normal_bf16((R, C), 1.0, R + C)
    x = H.bf16_values(bits)
    x[::5, ::7] *= 50.0  # heavy rows / columns
    bits = synthetic.f32_to_bf16_bits(x)
    x = H.bf16_values(bits)
    mask = philox.rht_signs(3, 7) if rht else None
    g = tj2.quantize(H.bf16_to_device(bits), grouping=tj2.GROUP_ROW if grouping == "row" else tj2.GROUP_COL,
                     rounding=tj2.SR if rounding == "sr" else tj2.RTN, rht=rht, signs=mask or 0, seed=3, offset=7,
                     out_fmt=tj2.NVFP6)
    ref = quant.quantize(x, grouping=grouping, fmt="nvfp6", rounding=rounding, rht_mask=mask, seed=3, offset=7)
    H.assert_q_equal(g, ref, what=f"nvfp6 {grouping} {rounding}")
    H.assert_padding_zero(g)


def test_nvfp6_rtn_exhaustive_unit_step():
    """Every fp32 magnitude in [2^-8, 7.5], both signs, placed where the element step is exactly 1
    (outer max 3360 -> S = 1; every test group also holds a 7.5 -> s = 1): each code must equal
    round-to-nearest-even onto the E2M3 grid, computed independently with torch.round (half to even)
    on the grid step (1/8 below 1, 2^(e-3) in binade e)."""
    lo = int(np.float32(2.0 ** -8).view(np.int32))
    hi = int(np.float32(7.5).view(np.int32))
    bits = torch.arange(lo, hi + 1, dtype=torch.int64, device="cuda").to(torch.int32)
    vals = bits.view(torch.float32)
    vals = torch.where(torch.arange(vals.numel(), device="cuda") % 2 == 0, vals, -vals)
    per_row = 7 * 15
    rows = (vals.numel() + per_row - 1) // per_row
    X = torch.zeros(rows, 128, dtype=torch.float32, device="cuda")
    X[:, 0] = 3360.0
    slots = torch.zeros(rows * per_row, dtype=torch.float32, device="cuda")
    slots[: vals.numel()] = vals
    body = X[:, 16:].view(rows, 7, 16)
    body[:, :, 0] = 7.5
    body[:, :, 1:] = slots.view(rows, 7, 15)
    q = tj2.quantize(X, out_fmt=tj2.NVFP6)
    assert torch.all(q.scale128[:, 0] == 1.0)
    assert torch.all(q.scale16[:, 1:8] == 0x38)  # E4M3 1.0
    codes = q.codes[:, 16:128].reshape(rows, 7, 16)[:, :, 1:].reshape(-1)[: vals.numel()].to(torch.int64)
    # the E4M3 bytes decode to the E2M3 values (sign bit 7, exponent bits 6..3 biased 7, mantissa 2..0)
    e = (codes >> 3) & 15
    m = (codes & 7).double()
    mag = torch.where(e == 0, m * 2.0 ** -9, torch.ldexp(1.0 + m / 8.0, (e - 7).clamp(min=-6)))
    got = torch.where((codes >> 7) == 1, -mag, mag)
    a = vals.abs().double()
    step = torch.where(a < 1, 0.125, torch.ldexp(torch.ones_like(a), torch.floor(torch.log2(a)).to(torch.int64) - 3))
    ref = torch.round(a / step) * step
    ref = torch.where(torch.signbit(vals), -ref, ref)
    bad = ((got != ref) | (torch.signbit(got) != torch.signbit(vals))).sum().item()
    assert bad == 0, f"{bad} mismatches"


@pytest.mark.parametrize("I,J,K", [(256, 384, 512), (200, 112, 400), (512, 256, 4096)])
def test_fp6_x_fp4_product(I, J, K):
    a_bits = synthetic.normal_bf16((I, K), 0.01, I + K)
    b = synthetic.normal_f32((J, K), 0.02, J)
    ga = tj2.quantize(H.bf16_to_device(a_bits), rounding=tj2.SR, seed=1, offset=2, out_fmt=tj2.NVFP6)
    gb = tj2.quantize(H.f32_to_device(b))
    ra = quant.quantize(H.bf16_values(a_bits), fmt="nvfp6", rounding="sr", seed=1, offset=2)
    rb = quant.quantize(b)
    H.assert_q_equal(ga, ra, what="A")
    H.assert_q_equal(gb, rb, what="B")
    ref = ogemm.gemm_nt_f64(ra, rb)
    c = tj2.gemm(ga, gb).cpu().numpy()
    assert H.rel_fro(c, ref) < 1e-5


@pytest.mark.parametrize("M,N,K,n_out", [(256, 512, 512, 0), (512, 256, 1024, 112), (144, 80, 400, 48)])
def test_fp6_backward(M, N, K, n_out):
    rng = np.random.default_rng(M + K)
    xb = synthetic.normal_bf16((M, K), 1.0, 11)
    W = synthetic.normal_f32((N, K), 0.02, 12)
    dyb = synthetic.normal_bf16((M, N), 0.01, 13)
    X, dY = H.bf16_values(xb), H.bf16_values(dyb)
    oplan = olinear.Plan.from_outliers(K, np.sort(rng.choice(K, n_out, replace=False))) if n_out else None
    gplan = tj2.OutlierPlan.from_indices(K, oplan.outliers) if n_out else None
    Y, saved = tj2.linear_fwd(H.bf16_to_device(xb), H.f32_to_device(W), N, plan=gplan, y_dtype=torch.float32)
    dX, dW, ops = tj2.linear_bwd(H.bf16_to_device(dyb), saved, K, seed=5, offset=40, plan=gplan,
                                 dx_dtype=torch.float32, keep_operands=True, grad_fmt=tj2.NVFP6)
    torch.cuda.synchronize()
    rf = olinear.linear_fwd(X, W, oplan)
    rb = olinear.linear_bwd(dY, rf, seed=5, offset=40, plan=oplan, grad_fmt="nvfp6")
    for name in ("dYq", "dYt", "Wt", "Xt") + (("W8t", "X8t") if n_out else ()):
        H.assert_q_equal(ops[name], rb[name], what=name)
    assert ops["dYq"].fmt == tj2.NVFP6 and ops["dYt"].fmt == tj2.NVFP6
    for name, got, ref in (("dX", dX, rb["dX"]), ("dW", dW, rb["dW"])):
        e = H.rel_fro(got.cpu().numpy(), ref)
        assert e < 1e-5, (name, e)
