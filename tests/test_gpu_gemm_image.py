"""GPU parity of the image products: B decoded once into f16 chunk images (by a
decode pass, or written by the quantization that produces B: the backward's
column re-grouping, the forward's split quantization of the weights) and copied
into the product's LDS stages, used for products of at least 8 row tiles (2048
rows) when the workspace holds the image.

Each case checks the product against the oracle's fp64 product of the same
dequantized operands (relative Frobenius < 1e-5: fp32 accumulation of exact
f16 products), and, where the reduction is not split, bit for bit against the
product kernel that decodes B itself (same K order, same promotions)."""
import numpy as np
import pytest
import torch

import synthetic
from oracle import gemm as ogemm, linear as olinear, quant

import _helpers as H
from _linear_check import check_linear_sampled

pytestmark = pytest.mark.gpu

tj2 = pytest.importorskip("bit_fully_quantized_amd")


def _ops(I, J, K, seed, fmt_a="nvfp4", fmt_b="nvfp4"):
    a_bits = synthetic.normal_bf16((I, K), 1.0, seed)
    b = synthetic.normal_f32((J, K), 0.02, seed + 1)
    code = {"nvfp4": tj2.NVFP4, "fp8": tj2.FP8, "nvfp6": tj2.NVFP6}
    ga = tj2.quantize(H.bf16_to_device(a_bits), out_fmt=code[fmt_a])
    gb = tj2.quantize(H.f32_to_device(b), out_fmt=code[fmt_b])
    ra = quant.quantize(H.bf16_values(a_bits), fmt=fmt_a)
    rb = quant.quantize(b, fmt=fmt_b)
    H.assert_q_equal(ga, ra, what="A")
    H.assert_q_equal(gb, rb, what="B")
    return ga, gb, ra, rb


def _image_workspace(I, J, K):
    n = int(tj2.lib().nvfp4_gemm_workspace_size(I, J, K, 0))
    assert n > 0, "the image path applies to this shape"
    return torch.empty(n, dtype=torch.uint8, device="cuda")


@pytest.mark.parametrize("I,J,K", [(2100, 300, 880), (2048, 128, 128), (4096, 1040, 384), (2304, 16, 400)])
def test_image_product_bit_identical(I, J, K):
    """Ragged row, column and chunk tiles, one to seven chunks (no K split): the image product
    equals the direct product bit for bit, fp32 and bf16 outputs."""
    print(f"[image] plain {I}x{J}x{K}", flush=True)
    ga, gb, ra, rb = _ops(I, J, K, seed=I + J + K)
    ws = _image_workspace(I, J, K)
    for dtype in (torch.float32, torch.bfloat16):
        img = tj2.gemm(ga, gb, out_dtype=dtype, workspace=ws)
        direct = tj2.gemm(ga, gb, out_dtype=dtype, split_k=False)
        torch.cuda.synchronize()
        assert torch.equal(img, direct), dtype
    c = tj2.gemm(ga, gb, workspace=ws).cpu().numpy()
    assert H.rel_fro(c, ogemm.gemm_nt_f64(ra, rb)) < 1e-5


@pytest.mark.parametrize("I,J,K", [(2048, 200, 4096), (2304, 136, 8192)])
def test_image_product_split_k(I, J, K):
    """Few output tiles over a long reduction: the chunk ranges of the K splits read their
    images from the middle of the chunk sequence."""
    print(f"[image] split-K {I}x{J}x{K}", flush=True)
    ga, gb, ra, rb = _ops(I, J, K, seed=7 + K)
    c = tj2.gemm(ga, gb, workspace=_image_workspace(I, J, K)).cpu().numpy()
    assert H.rel_fro(c, ogemm.gemm_nt_f64(ra, rb)) < 1e-5


@pytest.mark.parametrize("fmt_a,fmt_b", [("nvfp4", "fp8"), ("fp8", "nvfp4"), ("nvfp6", "nvfp4")])
def test_image_product_formats(fmt_a, fmt_b):
    """FP8 B rows decoded into the image; FP8 and NVFP6 A operands against an image."""
    I, J, K = 2048, 256, 512
    print(f"[image] {fmt_a} x {fmt_b}", flush=True)
    ga, gb, ra, rb = _ops(I, J, K, seed=40, fmt_a=fmt_a, fmt_b=fmt_b)
    img = tj2.gemm(ga, gb, workspace=_image_workspace(I, J, K))
    direct = tj2.gemm(ga, gb, split_k=False)
    torch.cuda.synchronize()
    assert torch.equal(img, direct)
    assert H.rel_fro(img.cpu().numpy(), ogemm.gemm_nt_f64(ra, rb)) < 1e-5


def _two_segment_ops(I, J, K1, K2, seed):
    a_bits = synthetic.normal_bf16((I, K1 + K2), 1.0, seed)
    b = synthetic.normal_f32((J, K1 + K2), 0.02, seed + 1)
    a_f = H.bf16_values(a_bits)
    ga = tj2.quantize(H.bf16_to_device(np.ascontiguousarray(a_bits[:, :K1])))
    ga8 = tj2.quantize(H.bf16_to_device(np.ascontiguousarray(a_bits[:, K1:])), out_fmt=tj2.FP8)
    gb = tj2.quantize(H.f32_to_device(np.ascontiguousarray(b[:, :K1])))
    gb8 = tj2.quantize(H.f32_to_device(np.ascontiguousarray(b[:, K1:])), out_fmt=tj2.FP8)
    ra = quant.quantize(np.ascontiguousarray(a_f[:, :K1]))
    ra8 = quant.quantize(np.ascontiguousarray(a_f[:, K1:]), fmt="fp8")
    rb = quant.quantize(np.ascontiguousarray(b[:, :K1]))
    rb8 = quant.quantize(np.ascontiguousarray(b[:, K1:]), fmt="fp8")
    H.assert_q_equal(gb, rb, what="B")
    H.assert_q_equal(gb8, rb8, what="B8")
    ref = ogemm.gemm_nt_f64(ra, rb) + ogemm.gemm_nt_f64(ra8, rb8)
    return ga, gb, ga8, gb8, ref


# (rows, columns, NVFP4 length, FP8 length): fewer than 8 chunks or at least 256 output tiles, so
# one K split; NVFP4 chunk counts 2, 3, 5, 8 and 29 (both parities of the segment crossing), one to
# four FP8 chunks, ragged rows, columns and chunks
_TWO_SEG = [(2100, 200, 256, 16), (2304, 384, 384, 256), (2048, 256, 640, 112), (4096, 2048, 912, 112),
            (4096, 2048, 3680, 416)]


@pytest.mark.parametrize("I,J,K1,K2", _TWO_SEG)
def test_image_two_segment_product(I, J, K1, K2):
    """A two-segment product (NVFP4, then FP8) called on its own: both segments' B rows decoded into
    one image by one decode launch, the FP8 chunks inside the image kernel's pipelined loop.  Equal
    bit for bit to the direct two-segment product, and to the oracle."""
    print(f"[image] two segments {I}x{J}x({K1}+{K2})", flush=True)
    ga, gb, ga8, gb8, ref = _two_segment_ops(I, J, K1, K2, seed=90 + K1 + K2)
    ws = tj2.gemm_workspace(I, J, K1, K2)
    assert ws is not None and ws.numel() > 0, "room for the image"
    for dtype in (torch.float32, torch.bfloat16):
        img = tj2.gemm(ga, gb, ga8, gb8, out_dtype=dtype, workspace=ws)
        direct = tj2.gemm(ga, gb, ga8, gb8, out_dtype=dtype, split_k=False)
        torch.cuda.synchronize()
        assert torch.equal(img, direct), dtype
    c = tj2.gemm(ga, gb, ga8, gb8, workspace=ws).cpu().numpy()
    assert H.rel_fro(c, ref) < 1e-5


# (tokens, outputs, channels, outlier channels): at least 8 row tiles and one K split, so the
# forward's product runs from the image; NVFP4 chunk counts 2, 3, 5, 8 and 29 (both parities of the
# segment crossing), one to four FP8 chunks, ragged rows, columns and chunks
_FWD_IMG = [(2112, 208, 272, 16), (2048, 256, 400, 16), (2304, 384, 768, 144), (4096, 2048, 1024, 112),
            (4096, 2048, 4096, 416)]


@pytest.mark.parametrize("M,N,K,no", _FWD_IMG)
def test_forward_image_from_the_split_quantization(M, N, K, no):
    """The forward with an outlier plan: the weights' split quantization writes the product's B image
    (NVFP4 chunks, then FP8 chunks) and the two-segment image kernel runs the FP8 chunks inside its
    pipelined loop.  Y equals bit for bit the forward without room for the image (the direct
    two-segment product: same chunk order, same promotions); the weights' codes and sampled rows of
    Y match the oracle."""
    print(f"[image] forward {M}x{N}x{K} outliers={no}", flush=True)
    rng = np.random.default_rng(M + K)
    xb = synthetic.normal_bf16((M, K), 1.0, 100 + K)
    W = synthetic.normal_f32((N, K), 0.02, 101 + K)
    outl = np.sort(rng.choice(K, no, replace=False))
    plan = tj2.OutlierPlan.from_indices(K, outl)
    assert int(tj2.lib().nvfp4_linear_fwd_workspace_size(M, N, K, no)) > 0, "room for the image"
    X, Wd = H.bf16_to_device(xb), H.f32_to_device(W)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    Y32 = saved = None
    for dtype in (torch.float32, torch.bfloat16):
        Y, sv = tj2.linear_fwd(X, Wd, N, plan=plan, y_dtype=dtype)
        Yd, _ = tj2.linear_fwd(X, Wd, N, plan=plan, y_dtype=dtype, workspace=small)
        torch.cuda.synchronize()
        assert torch.equal(Y, Yd), dtype
        if dtype == torch.float32:
            Y32, saved = Y, sv
    rows = np.unique(np.concatenate([rng.choice(M, 64, replace=False), [0, M - 1]]))
    ref = olinear.linear_fwd(H.bf16_values(xb)[rows], W, olinear.Plan.from_outliers(K, outl))
    H.assert_q_equal(saved["Wq"], ref["Wq"], what="Wq")
    H.assert_q_equal(saved["W8"], ref["W8"], what="W8")
    assert H.rel_fro(Y32.cpu().numpy()[rows], ref["Y"]) < 1e-5


def _outlier_case(I, J, K, outl, seed):
    outl = np.asarray(outl, dtype=np.int64)
    rest = np.setdiff1d(np.arange(J), outl)
    a_bits = synthetic.normal_bf16((I, K), 1.0, seed)
    b = synthetic.normal_f32((J, K), 0.02, seed + 1)
    ga = tj2.quantize(H.bf16_to_device(a_bits))
    gb = tj2.quantize(H.f32_to_device(b[rest]))
    gb8 = tj2.quantize(H.f32_to_device(b[outl]), out_fmt=tj2.FP8)
    ra = quant.quantize(H.bf16_values(a_bits))
    rb = quant.quantize(np.ascontiguousarray(b[rest]))
    rb8 = quant.quantize(np.ascontiguousarray(b[outl]), fmt="fp8")
    H.assert_q_equal(gb, rb, what="B")
    H.assert_q_equal(gb8, rb8, what="B8")
    ref = np.zeros((I, J))
    ref[:, rest] = ogemm.gemm_nt_f64(ra, rb)
    ref[:, outl] = ogemm.gemm_nt_f64(ra, rb8)
    return ga, gb, gb8, tj2.OutlierPlan.from_indices(J, outl), ref


def _outlier_cases():
    rng = np.random.default_rng(23)
    return [
        ("random", 2304, 400, 896, np.sort(rng.choice(400, 48, replace=False))),
        ("tile-of-outliers", 2048, 384, 384, np.concatenate([np.arange(128), np.arange(368, 384)])),
        ("edges", 2100, 272, 128, np.concatenate([np.arange(8), np.arange(264, 272)])),
    ]


@pytest.mark.parametrize("name,I,J,K,outl", _outlier_cases(), ids=[c[0] for c in _outlier_cases()])
def test_image_outlier_cols(name, I, J, K, outl):
    """Outlier-column products: the image holds each output column's row (NVFP4 or FP8) in
    output order.  Equal bit for bit to the direct product, and to the oracle."""
    print(f"[image] outlier columns {name} {I}x{J}x{K}", flush=True)
    ga, gb, gb8, plan, ref = _outlier_case(I, J, K, outl, seed=50 + J)
    ws = _image_workspace(I, J, K)
    img = tj2.gemm_outlier_cols(ga, gb, gb8, plan, workspace=ws)
    # a workspace too small for the image: the direct product
    direct = tj2.gemm_outlier_cols(ga, gb, gb8, plan, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(img, direct)
    assert H.rel_fro(img.cpu().numpy(), ref) < 1e-5


def test_image_outlier_cols_split_k():
    I, J, K = 2048, 208, 8192
    print(f"[image] outlier columns split-K {I}x{J}x{K}", flush=True)
    outl = np.sort(np.random.default_rng(24).choice(J, 32, replace=False))
    ga, gb, gb8, plan, ref = _outlier_case(I, J, K, outl, seed=60)
    c = tj2.gemm_outlier_cols(ga, gb, gb8, plan, workspace=_image_workspace(I, J, K)).cpu().numpy()
    assert H.rel_fro(c, ref) < 1e-5


def test_backward_images_from_the_column_quantization():
    """The backward's dX and dW images written by the column re-grouping of W and X (with an
    outlier plan, so the FP8 rows land at their channels): dX and dW equal bit for bit those of
    the same backward without images (no K split at this shape), and sampled outputs match the
    oracle.  A second call with the re-grouped weights given decodes the dX image itself."""
    M, N, K = 2048, 2048, 4096
    rng = np.random.default_rng(5)
    xb = synthetic.normal_bf16((M, K), 1.0, 81)
    W = synthetic.normal_f32((N, K), 0.02, 82)
    dyb = synthetic.normal_bf16((M, N), 0.01, 83)
    plan_idx = np.sort(rng.choice(K, 128, replace=False))
    plan = tj2.OutlierPlan.from_indices(K, plan_idx)
    print(f"[image] backward M={M} N={N} K={K} outliers=128", flush=True)
    Y, saved = tj2.linear_fwd(H.bf16_to_device(xb), H.f32_to_device(W), N, plan=plan, y_dtype=torch.bfloat16)
    dY = H.bf16_to_device(dyb)
    ws = tj2.linear_bwd_workspace(M, N, K, len(plan_idx))
    dX, dW, ops = tj2.linear_bwd(dY, saved, K, seed=3, offset=16, plan=plan, dx_dtype=torch.bfloat16,
                                 keep_operands=True, workspace=ws)
    ops2 = tj2.bwd_operands(M, N, K, plan)
    small = torch.empty(16, dtype=torch.uint8, device="cuda")
    dX2, dW2, _ = tj2.linear_bwd(dY, saved, K, seed=3, offset=16, plan=plan, dx_dtype=torch.bfloat16,
                                 operands=ops2, workspace=small)
    # the re-grouped weights given (as the fused master pass provides them): dX decodes its image
    dX3, dW3, _ = tj2.linear_bwd(dY, saved, K, seed=3, offset=16, plan=plan, dx_dtype=torch.bfloat16,
                                 operands=ops, w_given=True, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(dX, dX2) and torch.equal(dW, dW2)
    assert torch.equal(dX, dX3) and torch.equal(dW, dW3)
    dX32, _, _ = tj2.linear_bwd(dY, saved, K, seed=3, offset=16, plan=plan, dx_dtype=torch.float32, workspace=ws)
    Y32, _ = tj2.linear_fwd(H.bf16_to_device(xb), H.f32_to_device(W), N, plan=plan, y_dtype=torch.float32)
    torch.cuda.synchronize()
    gpu = dict(saved=saved, ops=ops, Y=Y, dX=dX, dW=dW, Y32=Y32, dX32=dX32)
    err = check_linear_sampled(H.bf16_values(xb), W, H.bf16_values(dyb), plan_idx, 3, 16, gpu, rng, tag="image")
    print(f"[image] rel_fro dX {err['dX']:.2e} dW {err['dW']:.2e}", flush=True)


@pytest.mark.parametrize("I,J,K,img", [(4096, 1024, 1024, True), (2048, 1024, 1024, True), (2100, 300, 880, True),
                                       (1024, 640, 512, False), (1024, 1024, 16384, False)])
def test_bf16_output_is_rne_of_fp32_output(I, J, K, img):
    """A product's bf16 output is its fp32 output rounded to nearest even, bit for bit: the staged
    16-byte stores convert pairs with the hardware conversion, the ragged-tile element stores and
    the split-K reduction in software, and all of them must agree with torch's host rounding.
    Image products without and with a K split (the first two shapes), full and ragged tiles, a
    direct product, and a direct product split eight ways."""
    print(f"[image] bf16 rounding {I}x{J}x{K} image={img}", flush=True)
    ga, gb, _, _ = _ops(I, J, K, seed=3 * I + J)
    ws = _image_workspace(I, J, K) if img else tj2.gemm_workspace(I, J, K)
    c32 = tj2.gemm(ga, gb, workspace=ws)
    c16 = tj2.gemm(ga, gb, out_dtype=torch.bfloat16, workspace=ws)
    torch.cuda.synchronize()
    want = c32.cpu().to(torch.bfloat16)
    assert torch.equal(c16.cpu().view(torch.int16), want.view(torch.int16))
