"""nvfp4_gemm_noalloc (split-K partial sums in the library's static device scratch) through the C ABI,
against nvfp4_gemm with a caller workspace on the same operands: two calls in a row, the second on a
smaller product, both split over K; a product without a split; and the oracle's fp64 product."""
import ctypes

import numpy as np
import pytest
import torch

import synthetic
from oracle import gemm as ogemm, quant

import _helpers as H

pytestmark = pytest.mark.gpu

tj2 = pytest.importorskip("bit_fully_quantized_amd")


def _operands(I, J, K, seed):
    a_bits = synthetic.normal_bf16((I, K), 1.0, seed)
    b = synthetic.normal_f32((J, K), 0.02, seed + 1)
    ga = tj2.quantize(H.bf16_to_device(a_bits))
    gb = tj2.quantize(H.f32_to_device(b))
    ra = quant.quantize(H.bf16_values(a_bits))
    rb = quant.quantize(b)
    H.assert_q_equal(ga, ra, what="A")
    H.assert_q_equal(gb, rb, what="B")
    return ga, gb, ra, rb


def _noalloc(A, B, out, A2=None, B2=None, accumulate=False):
    L = tj2.lib()
    a, b = A.c(), B.c()
    a2 = ctypes.byref(A2.c()) if A2 is not None else None
    b2 = ctypes.byref(B2.c()) if B2 is not None else None
    st = L.nvfp4_gemm_noalloc(ctypes.byref(a), ctypes.byref(b), a2, b2, ctypes.c_void_p(out.data_ptr()),
                              tj2.F32 if out.dtype == torch.float32 else tj2.BF16, out.stride(0), None,
                              1 if accumulate else 0, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    tj2._lib.check("nvfp4_gemm_noalloc", st)
    return out


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_noalloc_matches_workspace_entry(dtype):
    print("nvfp4_gemm_noalloc: 256x128x8192 then 200x112x4096, split over K", flush=True)
    for I, J, K, seed in ((256, 128, 8192, 1), (200, 112, 4096, 2)):
        assert tj2.lib().nvfp4_gemm_workspace_size(I, J, K, 0) > 0  # the product splits over K
        ga, gb, ra, rb = _operands(I, J, K, seed)
        want = tj2.gemm(ga, gb, out_dtype=dtype, workspace=tj2.gemm_workspace(I, J, K))
        got = _noalloc(ga, gb, torch.full((I, J), 3.0, dtype=dtype, device="cuda"))
        torch.cuda.synchronize()
        assert torch.equal(got, want), (I, J, K)
        if dtype == torch.float32:
            assert H.rel_fro(got.cpu().numpy(), ogemm.gemm_nt_f64(ra, rb)) < 1e-5


def test_noalloc_unsplit_and_accumulate():
    I, J, K = 512, 384, 512  # four 128-element chunks: too short a reduction to split
    assert tj2.lib().nvfp4_gemm_workspace_size(I, J, K, 0) == 0
    ga, gb, ra, rb = _operands(I, J, K, 3)
    want = tj2.gemm(ga, gb)
    got = _noalloc(ga, gb, torch.empty(I, J, device="cuda"))
    assert torch.equal(got, want)
    # accumulate into fp32 through the split path (second small split product)
    I2, J2, K2 = 256, 128, 8192
    ga2, gb2, ra2, rb2 = _operands(I2, J2, K2, 4)
    base = torch.randn(I2, J2, device="cuda")
    want2 = tj2.gemm(ga2, gb2, out=base.clone(), accumulate=True, workspace=tj2.gemm_workspace(I2, J2, K2))
    got2 = _noalloc(ga2, gb2, base.clone(), accumulate=True)
    assert torch.equal(got2, want2)
