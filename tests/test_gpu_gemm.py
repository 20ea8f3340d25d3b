"""GPU parity of the packed-operand products (relative Frobenius error <= 1e-3 vs
the oracle's fp64 product of the same dequantized operands, which are first
checked bit-exact against the oracle's own quantizers)."""
import numpy as np
import pytest
import torch

import synthetic
from oracle import gemm as ogemm, quant

import _helpers as H

pytestmark = pytest.mark.gpu

tj2 = pytest.importorskip("bit_fully_quantized_amd")


def _operands(I, J, K, seed, fmt_b="nvfp4", sr=False):
    a_bits = synthetic.normal_bf16((I, K), 1.0, seed)
    b = synthetic.normal_f32((J, K), 0.02, seed + 1)
    ga = tj2.quantize(H.bf16_to_device(a_bits), rounding=tj2.SR if sr else tj2.RTN, seed=seed, offset=0)
    gb = tj2.quantize(H.f32_to_device(b), out_fmt=tj2.FP8 if fmt_b == "fp8" else tj2.NVFP4)
    ra = quant.quantize(H.bf16_values(a_bits), rounding="sr" if sr else "rtn", seed=seed, offset=0)
    rb = quant.quantize(b, fmt=fmt_b)
    H.assert_q_equal(ga, ra, what="A")
    H.assert_q_equal(gb, rb, what="B")
    return ga, gb, ra, rb


@pytest.mark.parametrize("I,J,K", [(256, 512, 512), (208, 144, 400), (16, 16, 16), (128, 384, 1024),
                                   (300, 130, 272), (512, 256, 2048)])
def test_gemm_nvfp4(I, J, K):
    ga, gb, ra, rb = _operands(I, J, K, seed=I + J + K)
    c = tj2.gemm(ga, gb).cpu().numpy()
    ref = ogemm.gemm_nt_f64(ra, rb)
    assert H.rel_fro(c, ref) <= H.GEMM_TOL
    assert H.rel_fro(c, ref) < 1e-5  # fp32 accumulation of exact products


def test_gemm_mixed_fp8_segment_and_scatter():
    I, J, K = 192, 160, 256
    ga, gb8, ra, rb8 = _operands(I, J, K, seed=5, fmt_b="fp8", sr=True)
    c = tj2.gemm(ga, gb8).cpu().numpy()
    assert H.rel_fro(c, ogemm.gemm_nt_f64(ra, rb8)) < 1e-5
    # two segments (NVFP4 x NVFP4 + FP8 x FP8) into a column-scattered output
    ga2, gb2, ra2, rb2 = _operands(I, J, 112, seed=6)
    a8_bits = synthetic.normal_bf16((I, 112), 1.0, 60)
    b8_f = synthetic.normal_f32((J, 112), 0.02, 61)
    a8 = tj2.quantize(H.bf16_to_device(a8_bits), out_fmt=tj2.FP8)
    b8 = tj2.quantize(H.f32_to_device(b8_f), out_fmt=tj2.FP8)
    ra8 = quant.quantize(H.bf16_values(a8_bits), fmt="fp8")
    rb8b = quant.quantize(b8_f, fmt="fp8")
    H.assert_q_equal(a8, ra8, what="A8")
    H.assert_q_equal(b8, rb8b, what="B8")
    perm = np.random.default_rng(0).permutation(J + 32)[:J].astype(np.int32)
    out = torch.full((I, J + 32), 7.0, device="cuda")
    tj2.gemm(ga2, gb2, a8, b8, out=out, col_map=torch.from_numpy(perm).cuda())
    ref = ogemm.gemm_nt_f64(ra2, rb2) + ogemm.gemm_nt_f64(ra8, rb8b)
    got = out.cpu().numpy()
    assert H.rel_fro(got[:, perm], ref) < 1e-5
    untouched = np.setdiff1d(np.arange(J + 32), perm)
    assert np.all(got[:, untouched] == 7.0)
    # accumulate into fp32
    tj2.gemm(ga2, gb2, out=out, col_map=torch.from_numpy(perm).cuda(), accumulate=True)
    assert H.rel_fro(out.cpu().numpy()[:, perm], ref + ogemm.gemm_nt_f64(ra2, rb2)) < 1e-5


def test_gemm_bf16_output():
    ga, gb, ra, rb = _operands(256, 256, 512, seed=9)
    c = tj2.gemm(ga, gb, out_dtype=torch.bfloat16)
    assert H.bf16_ulp_ok(c, ogemm.gemm_nt_f64(ra, rb))


def test_gemm_heterogeneous_scales():
    """Rows / blocks whose outer scales differ by many binades: the per-128 promotion keeps them exact."""
    I, J, K = 128, 128, 512
    rng = np.random.default_rng(3)
    a = (rng.standard_normal((I, K)) * np.exp2(rng.integers(-40, 40, size=(I, K // 128))).repeat(128, 1)).astype(np.float32)
    b = (rng.standard_normal((J, K)) * np.exp2(rng.integers(-40, 40, size=(J, K // 128))).repeat(128, 1)).astype(np.float32)
    ga, gb = tj2.quantize(H.f32_to_device(a)), tj2.quantize(H.f32_to_device(b))
    ra, rb = quant.quantize(a), quant.quantize(b)
    H.assert_q_equal(ga, ra); H.assert_q_equal(gb, rb)
    c = tj2.gemm(ga, gb).cpu().numpy()
    assert H.rel_fro(c, ogemm.gemm_nt_f64(ra, rb)) < 1e-5


@pytest.mark.parametrize("I,J,ld,off", [(200, 300, 300, 0), (200, 256, 264, 8), (136, 256, 260, 2),
                                         (136, 256, 256, 1), (96, 128, 136, 4)])
def test_gemm_output_views(I, J, ld, off):
    """Outputs written into views of a wider buffer: ragged rows and columns, and leading dimensions and
    offsets that do (whole 16-byte row pieces) and do not (element stores) keep rows 16-byte aligned.
    Nothing outside the view changes; accumulation adds to what the view held."""
    ga, gb, ra, rb = _operands(I, J, 384, seed=I + J + ld + off)
    ref = ogemm.gemm_nt_f64(ra, rb)
    for dt in (torch.float32, torch.bfloat16):
        buf = torch.full((I * ld + off + 64,), 3.0, dtype=dt, device="cuda")
        out = buf[off:off + I * ld].view(I, ld)[:, :J]
        tj2.gemm(ga, gb, out=out, split_k=False)
        got = out.float().cpu().numpy()
        if dt == torch.float32:
            assert H.rel_fro(got, ref) < 1e-5
        else:
            assert H.bf16_ulp_ok(out, ref)
        rest = buf.float().cpu().numpy().copy()
        rest[off:off + I * ld].reshape(I, ld)[:, :J] = 3.0
        assert np.all(rest == 3.0), "write outside the output view"
    base = np.random.default_rng(off).standard_normal((I, ld)).astype(np.float32)
    buf = torch.zeros(I * ld + off + 64, dtype=torch.float32, device="cuda")
    view = buf[off:off + I * ld].view(I, ld)
    view.copy_(torch.from_numpy(base).cuda())
    tj2.gemm(ga, gb, out=view[:, :J], accumulate=True, split_k=False)
    got = view.cpu().numpy()
    assert H.rel_fro(got[:, :J] - base[:, :J], ref) < 1e-5
    np.testing.assert_array_equal(got[:, J:], base[:, J:])


@pytest.mark.parametrize("I,J,K1,K2,fmt2", [(256, 128, 880, 112, "fp8"), (200, 112, 4096, 4096, "nvfp4"),
                                             (256, 256, 3968, 1024, "fp8")])
def test_gemm_two_segments_split_k(I, J, K1, K2, fmt2):
    """A two-segment product (NVFP4 x NVFP4 + a second segment) over few output tiles: the K split
    runs over the chunks of both segments (a split boundary inside a segment, splits that lie in one
    segment), with the workspace sized by both reductions."""
    ga, gb, ra, rb = _operands(I, J, K1, seed=K1 + K2)
    a_bits = synthetic.normal_bf16((I, K2), 1.0, 70)
    b_f = synthetic.normal_f32((J, K2), 0.02, 71)
    f2 = tj2.FP8 if fmt2 == "fp8" else tj2.NVFP4
    a2 = tj2.quantize(H.bf16_to_device(a_bits), out_fmt=f2)
    b2 = tj2.quantize(H.f32_to_device(b_f), out_fmt=f2)
    ra2 = quant.quantize(H.bf16_values(a_bits), fmt=fmt2)
    rb2 = quant.quantize(b_f, fmt=fmt2)
    H.assert_q_equal(a2, ra2, what="A2")
    H.assert_q_equal(b2, rb2, what="B2")
    ws = tj2.gemm_workspace(I, J, K1, K2)
    assert ws is not None and ws.numel() >= tj2.lib().nvfp4_gemm_workspace_size(I, J, K1 + K2, 0)
    ref = ogemm.gemm_nt_f64(ra, rb) + ogemm.gemm_nt_f64(ra2, rb2)
    c = tj2.gemm(ga, gb, a2, b2, workspace=ws).cpu().numpy()
    assert H.rel_fro(c, ref) < 1e-5
    c1 = tj2.gemm(ga, gb, a2, b2, split_k=False).cpu().numpy()
    assert H.rel_fro(c1, ref) < 1e-5
    # a workspace too small for the split is refused, not silently ignored
    with pytest.raises(tj2.Tj2Error):
        tj2.gemm(ga, gb, a2, b2, workspace=ws[: ws.numel() - 256])


@pytest.mark.parametrize("I,J,K", [(256, 128, 8192), (200, 112, 4096), (16384 // 8, 112, 3072)])
def test_gemm_split_k(I, J, K):
    """Few output tiles and a long reduction: K is split over workgroups, partials reduced in order."""
    ga, gb, ra, rb = _operands(I, J, K, seed=I + K)
    ws = tj2.gemm_workspace(I, J, K)
    assert ws is not None and ws.numel() > 0
    ref = ogemm.gemm_nt_f64(ra, rb)
    c = tj2.gemm(ga, gb, workspace=ws).cpu().numpy()
    assert H.rel_fro(c, ref) < 1e-5
    c1 = tj2.gemm(ga, gb, split_k=False).cpu().numpy()
    assert H.rel_fro(c1, ref) < 1e-5
    # scattered bf16 output through the reduce pass
    perm = np.random.default_rng(1).permutation(J).astype(np.int32)
    cb = tj2.gemm(ga, gb, out_dtype=torch.bfloat16, col_map=torch.from_numpy(perm).cuda(), workspace=ws)
    assert H.bf16_ulp_ok(cb[:, perm], ref)


def _plan_cases():
    rng = np.random.default_rng(11)
    return [
        ("random", 256, 400, 256, np.sort(rng.choice(400, 48, replace=False))),
        ("tile-of-outliers", 300, 384, 384, np.concatenate([np.arange(128), np.arange(368, 384)])),
        ("strided", 128, 256, 512, np.arange(0, 256, 8)),
        ("edges", 64, 272, 128, np.concatenate([np.arange(8), np.arange(264, 272)])),
        ("split-k", 256, 208, 8192, np.sort(rng.choice(208, 32, replace=False))),
    ]


@pytest.mark.parametrize("name,I,J,K,outl", _plan_cases(), ids=[c[0] for c in _plan_cases()])
def test_gemm_outlier_cols(name, I, J, K, outl):
    """One product over all J output columns of a plan: NVFP4 rows for the non-outlier
    columns, FP8 rows for the outlier columns (backward dX / dW with OutControl)."""
    outl = np.asarray(outl, dtype=np.int64)
    rest = np.setdiff1d(np.arange(J), outl)
    a_bits = synthetic.normal_bf16((I, K), 1.0, 70 + I)
    b = synthetic.normal_f32((J, K), 0.02, 71 + J)
    ga = tj2.quantize(H.bf16_to_device(a_bits))
    gb = tj2.quantize(H.f32_to_device(b[rest]))
    gb8 = tj2.quantize(H.f32_to_device(b[outl]), out_fmt=tj2.FP8)
    ra = quant.quantize(H.bf16_values(a_bits))
    rb = quant.quantize(np.ascontiguousarray(b[rest]))
    rb8 = quant.quantize(np.ascontiguousarray(b[outl]), fmt="fp8")
    H.assert_q_equal(ga, ra, what="A")
    H.assert_q_equal(gb, rb, what="B")
    H.assert_q_equal(gb8, rb8, what="B8")
    ref = np.zeros((I, J))
    ref[:, rest] = ogemm.gemm_nt_f64(ra, rb)
    ref[:, outl] = ogemm.gemm_nt_f64(ra, rb8)
    plan = tj2.OutlierPlan.from_indices(J, outl)
    c = tj2.gemm_outlier_cols(ga, gb, gb8, plan).cpu().numpy()
    assert H.rel_fro(c, ref) < 1e-5
    cb = tj2.gemm_outlier_cols(ga, gb, gb8, plan, out_dtype=torch.bfloat16)
    assert H.bf16_ulp_ok(cb, ref)
    # accumulate into an fp32 output
    out = torch.from_numpy(c).cuda()
    tj2.gemm_outlier_cols(ga, gb, gb8, plan, out=out, accumulate=True)
    assert H.rel_fro(out.cpu().numpy(), 2 * ref) < 1e-5


def test_gemm_operand_codes_beyond_4gb():
    """An A operand whose packed codes exceed 4 GB (4096 rows x 2.1 M elements): rows past the 4 GB
    mark are addressed with 64-bit offsets.  Random packed operands (any byte is a pair of E2M1
    codes; E4M3 inner scales 2^-3..2^3; positive outer scales), seeded on the device; sampled
    outputs, including the last row, against the oracle's fp64 product of the same bytes."""
    I, J, K = 4096, 16, (1 << 21) + (1 << 14)
    nb = K // 128
    assert (I - 1) * nb * 64 >= (1 << 32)
    g = torch.Generator(device="cuda")
    g.manual_seed(7)

    def operand(rows):
        q = tj2.QTensor(tj2.NVFP4, rows, K)
        q.codes.random_(0, 256, generator=g)
        q.scale16.random_(0x20, 0x51, generator=g)
        q.scale128.copy_(torch.rand(q.scale128.shape, generator=g, device="cuda") * 0.5 + 0.5)
        return q

    def host(q, rows):
        idx = torch.tensor(rows, device="cuda")
        return quant.QTensor("nvfp4", q.codes[idx].cpu().numpy(), q.scale128[idx].cpu().numpy(),
                             q.scale16[idx].cpu().numpy(), len(rows), K)

    A, B = operand(I), operand(J)
    C = tj2.gemm(A, B, workspace=tj2.gemm_workspace(I, J, K)).cpu().numpy()
    rows, cols = [0, 2047, I - 1], [0, J - 1]
    ra, rb = host(A, rows), host(B, cols)
    del A, B
    torch.cuda.empty_cache()
    ref = ogemm.gemm_nt_f64(ra, rb)
    assert H.rel_fro(C[np.ix_(rows, cols)], ref) <= H.GEMM_TOL


@pytest.mark.parametrize("I,J,K", [(8192, 1280, 128), (8192, 1152, 384), (8400, 1040, 640)])
def test_gemm_many_tiles_short_reductions(I, J, K):
    """More 256x128 output tiles than compute units (several rounds of workgroups) over
    reductions of 1, 3 and 5 chunks (the prefetches of the first chunks run past the last
    one), with ragged last row and column tiles; fp32 and bf16 outputs."""
    ga, gb, ra, rb = _operands(I, J, K, seed=I + J + K)
    ref = ogemm.gemm_nt_f64(ra, rb)
    c = tj2.gemm(ga, gb).cpu().numpy()
    assert H.rel_fro(c, ref) < 1e-5
    cb = tj2.gemm(ga, gb, out_dtype=torch.bfloat16)
    assert H.bf16_ulp_ok(cb, ref)


def test_gemm_many_tiles_two_segments_and_outlier_cols():
    """Many output tiles through the two-segment product (NVFP4 chunks, then an FP8 chunk)
    and through the outlier-column product (NVFP4 and FP8 B rows in one tile)."""
    I, J, K1, K2 = 8192, 1152, 256, 112
    ga, gb, ra, rb = _operands(I, J, K1, seed=31)
    a8_bits = synthetic.normal_bf16((I, K2), 1.0, 32)
    b8_f = synthetic.normal_f32((J, K2), 0.02, 33)
    a8 = tj2.quantize(H.bf16_to_device(a8_bits), out_fmt=tj2.FP8)
    b8 = tj2.quantize(H.f32_to_device(b8_f), out_fmt=tj2.FP8)
    ra8 = quant.quantize(H.bf16_values(a8_bits), fmt="fp8")
    rb8 = quant.quantize(b8_f, fmt="fp8")
    ref = ogemm.gemm_nt_f64(ra, rb) + ogemm.gemm_nt_f64(ra8, rb8)
    cb = tj2.gemm(ga, gb, a8, b8, out_dtype=torch.bfloat16)
    assert H.bf16_ulp_ok(cb, ref)
    assert H.rel_fro(tj2.gemm(ga, gb, a8, b8).cpu().numpy(), ref) < 1e-5

    outl = np.sort(np.random.default_rng(34).choice(J, 96, replace=False))
    rest = np.setdiff1d(np.arange(J), outl)
    b = synthetic.normal_f32((J, K1), 0.02, 35)
    gb4 = tj2.quantize(H.f32_to_device(b[rest]))
    gb8 = tj2.quantize(H.f32_to_device(b[outl]), out_fmt=tj2.FP8)
    rb4 = quant.quantize(np.ascontiguousarray(b[rest]))
    rb8o = quant.quantize(np.ascontiguousarray(b[outl]), fmt="fp8")
    H.assert_q_equal(gb4, rb4, what="B")
    H.assert_q_equal(gb8, rb8o, what="B8")
    ref2 = np.zeros((I, J))
    ref2[:, rest] = ogemm.gemm_nt_f64(ra, rb4)
    ref2[:, outl] = ogemm.gemm_nt_f64(ra, rb8o)
    plan = tj2.OutlierPlan.from_indices(J, outl)
    cb2 = tj2.gemm_outlier_cols(ga, gb4, gb8, plan, out_dtype=torch.bfloat16)
    assert H.bf16_ulp_ok(cb2, ref2)


@pytest.mark.parametrize("I,J,K", [(1024, 1024, 16384), (3072, 1024, 16384)])
def test_split_k_reduction_paths(I, J, K):
    """The weight-gradient shapes whose K split is 8 (1024 x 1024) and 2 (3072 x 1024) over 16384
    tokens: the reduction's vector path (no column map) equals bit for bit its general path (the
    same product with an identity column map; both sum the partials in split order), for fp32, bf16
    and accumulating outputs; sampled rows match the oracle."""
    print(f"[gemm] split-K reduction {I}x{J}x{K}", flush=True)
    rng = np.random.default_rng(I + J)
    a_bits = synthetic.normal_bf16((I, K), 0.01, I)
    b = synthetic.normal_f32((J, K), 1.0, J + 1)
    ga = tj2.quantize(H.bf16_to_device(a_bits))
    gb = tj2.quantize(H.f32_to_device(b))
    ident = torch.arange(J, dtype=torch.int32, device="cuda")
    for dtype in (torch.float32, torch.bfloat16):
        vec = tj2.gemm(ga, gb, out_dtype=dtype)
        gen = tj2.gemm(ga, gb, out_dtype=dtype, col_map=ident)
        torch.cuda.synchronize()
        assert torch.equal(vec, gen), dtype
    base = torch.from_numpy(rng.standard_normal((I, J)).astype(np.float32)).cuda()
    acc_vec, acc_gen = base.clone(), base.clone()
    tj2.gemm(ga, gb, out=acc_vec, accumulate=True)
    tj2.gemm(ga, gb, out=acc_gen, col_map=ident, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(acc_vec, acc_gen)
    rows = np.unique(np.concatenate([rng.choice(I, 24, replace=False), [0, I - 1]]))
    ra = quant.quantize(np.ascontiguousarray(H.bf16_values(a_bits)[rows]))
    rb = quant.quantize(b)
    ref = ogemm.gemm_nt_f64(ra, rb)
    got = tj2.gemm(ga, gb).cpu().numpy()[rows]
    assert H.rel_fro(got, ref) < 1e-5
    assert H.rel_fro((acc_vec - base).cpu().numpy()[rows], ref) < 1e-5
