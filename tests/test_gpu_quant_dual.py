"""GPU parity of the fused two-grouping quantizer of the output gradient (TetraJet-v2 technical
summary, sections 2.A and 2.C: dY enters dX grouped along N and dW grouped along M, each with its
own Hadamard signs and stochastic draws): one read of a bf16 tensor gives both operands, each
bit-exact against the oracle's row and column quantizers with the same signs and offsets."""
import numpy as np
import pytest

import synthetic
from oracle import philox, quant

import _helpers as H

pytestmark = pytest.mark.gpu

tj2 = pytest.importorskip("bit_fully_quantized_amd")


@pytest.mark.parametrize("M,N,rht,fmt", [(256, 384, True, "nvfp4"), (208, 400, True, "nvfp4"), (16, 16, True, "nvfp4"),
                                          (144, 2064, False, "nvfp4"), (1040, 128, True, "nvfp4"),
                                          (208, 272, True, "nvfp6")])
def test_quantize_dual_equals_oracle(M, N, rht, fmt):
    """Tiles of 128 x 128 with ragged last row and column tiles (rows and columns past the edge
    are the zero padding of both outputs' last outer blocks), with and without the transforms."""
    bits = synthetic.normal_bf16((M, N), 1.0, M + N)
    x = H.bf16_values(bits)
    x[::7, ::5] *= 40.0  # heavy rows and columns
    bits = synthetic.f32_to_bf16_bits(x)
    x = H.bf16_values(bits)
    seed, ro, co = 11, 20, 22
    f = tj2.NVFP4 if fmt == "nvfp4" else tj2.NVFP6
    rq, cq = tj2.quantize_dual(H.bf16_to_device(bits), rht=rht, seed=seed, row_offset=ro, col_offset=co, out_fmt=f)
    mr = philox.rht_signs(seed, ro) if rht else None
    mc = philox.rht_signs(seed, co) if rht else None
    ref_r = quant.quantize(x, grouping="row", fmt=fmt, rounding="sr", rht_mask=mr, seed=seed, offset=ro)
    ref_c = quant.quantize(x, grouping="col", fmt=fmt, rounding="sr", rht_mask=mc, seed=seed, offset=co)
    H.assert_q_equal(rq, ref_r, what=f"dual row {M}x{N}")
    H.assert_q_equal(cq, ref_c, what=f"dual col {M}x{N}")
    H.assert_padding_zero(rq)
    H.assert_padding_zero(cq)


def test_quantize_dual_equals_two_passes_at_size():
    """A 370M-style output gradient (16384 tokens x 3072): the fused pass equals the two separate
    library passes (row and column quantizers with the same signs and offsets) bit for bit."""
    import torch
    M, N = 16384, 3072
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    x = (torch.randn(M, N, generator=g, device="cuda") * 1e-3).to(torch.bfloat16)
    seed, ro, co = 77, 40, 42
    rq, cq = tj2.quantize_dual(x, rht=True, seed=seed, row_offset=ro, col_offset=co)
    r2 = tj2.quantize(x, grouping=tj2.GROUP_ROW, rounding=tj2.SR, rht=True, signs=philox.rht_signs(seed, ro), seed=seed,
                      offset=ro)
    c2 = tj2.quantize(x, grouping=tj2.GROUP_COL, rounding=tj2.SR, rht=True, signs=philox.rht_signs(seed, co), seed=seed,
                      offset=co)
    for a, b, what in [(rq, r2, "row"), (cq, c2, "col")]:
        assert torch.equal(a.codes, b.codes), what
        assert torch.equal(a.scale16, b.scale16), what
        assert torch.equal(a.scale128, b.scale128), what


def test_quantize_dual_extreme_magnitudes():
    """Outer blocks near the top of the fp32 range (group sums up to about 1.6e38, the largest the
    transform keeps finite) and of bf16 subnormals next to ordinary ones: the fused pass, which
    takes the transform's 1/4 into the group's reciprocal, equals the oracle bit for bit."""
    M, N = 256, 384
    x = H.bf16_values(synthetic.normal_bf16((M, N), 1.0, 91))
    x[:16] *= np.float32(2.5e36)
    x[16:32] *= np.float32(1e-39)
    x[:, 128:144] *= np.float32(1e-39)
    bits = synthetic.f32_to_bf16_bits(x)
    x = H.bf16_values(bits)
    assert np.isfinite(x).all() and np.abs(x).max() > 1e36 and (np.abs(x[16:32]) < 1.2e-38).all()
    seed, ro, co = 3, 6, 8
    rq, cq = tj2.quantize_dual(H.bf16_to_device(bits), rht=True, seed=seed, row_offset=ro, col_offset=co)
    ref_r = quant.quantize(x, grouping="row", rounding="sr", rht_mask=philox.rht_signs(seed, ro), seed=seed, offset=ro)
    ref_c = quant.quantize(x, grouping="col", rounding="sr", rht_mask=philox.rht_signs(seed, co), seed=seed, offset=co)
    H.assert_q_equal(rq, ref_r, what="dual row, extreme magnitudes")
    H.assert_q_equal(cq, ref_c, what="dual col, extreme magnitudes")
