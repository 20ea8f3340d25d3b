"""C ABI checks that need no GPU: the library loads, exports every entry point
declared in include/tj2.h, and rejects bad arguments on the host (before any
device work) with the documented status codes."""
import ctypes
import os
import re

import pytest

from oracle import philox

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tj2.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    from bit_fully_quantized_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libtj2.so is not built (run __graft_entry__.build())")
    return _lib.lib()


def test_header_declares_entry_points():
    names = declared_functions()
    for n in ["nvfp4_quantize", "nvfp4_quantize_dual", "nvfp4_gemm", "nvfp4_gemm_outlier_cols", "nvfp4_linear_fwd", "nvfp4_linear_bwd", "osci_reset_step",
              "osci_reset_step_multi", "master_update_step", "master_update_step_multi", "tj2_channel_sumsq", "tj2_rht_signs", "tj2_last_error", "tj2_qtensor_bytes",
              "tj2_select_outliers", "tj2_channel_sumsq_workspace_size", "nvfp4_linear_fwd_workspace_size",
              "nvfp4_gemm_workspace_size", "nvfp4_linear_bwd_workspace_size"]:
        assert n in names


def test_exports_every_declared_symbol(L):
    from bit_fully_quantized_amd import _lib
    for n in declared_functions():
        assert hasattr(L, n), f"{n} not exported"
        assert n in _lib.SIGNATURES, f"{n} has no ctypes signature"


def test_version_and_rht_signs_match_oracle(L):
    assert b"gfx950" in L.tj2_version()
    for seed, off in [(0, 0), (0, 2), (1234, 8), (2 ** 63 + 5, 2 ** 40 + 3)]:
        assert L.tj2_rht_signs(seed, off) == philox.rht_signs(seed, off)


def test_qtensor_bytes(L):
    from bit_fully_quantized_amd import _lib
    c, s16, s128 = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    assert L.tj2_qtensor_bytes(_lib.NVFP4, 3, 144, ctypes.byref(c), ctypes.byref(s16), ctypes.byref(s128)) == 0
    assert (c.value, s16.value, s128.value) == (3 * 2 * 64, 3 * 2 * 8, 3 * 2 * 4)
    assert L.tj2_qtensor_bytes(_lib.FP8, 2, 128, ctypes.byref(c), ctypes.byref(s16), ctypes.byref(s128)) == 0
    assert (c.value, s16.value, s128.value) == (256, 0, 8)
    assert L.tj2_qtensor_bytes(_lib.NVFP4, 2, 100, None, None, None) == _lib.TJ2_ERR_SHAPE
    assert L.tj2_qtensor_bytes(7, 2, 128, None, None, None) == _lib.TJ2_ERR_ARG
    assert b"format" in L.tj2_last_error()


def fake_q(fmt, rows, length, base=0x10000):
    from bit_fully_quantized_amd import _lib
    return _lib.QTensorC(base, base + 0x1000 if fmt == _lib.NVFP4 else 0, base + 0x2000, rows, length, fmt, 0)


def test_quantize_argument_errors(L):
    from bit_fully_quantized_amd import _lib
    out = fake_q(_lib.NVFP4, 32, 64)
    q = lambda *a: L.nvfp4_quantize(*a)
    # bad grouping / rounding / null out / bad dtype
    assert q(0x1000, _lib.BF16, None, 32, 64, None, 0, 9, 0, 0, 0, 0, 0, ctypes.byref(out), None) == _lib.TJ2_ERR_ARG
    assert q(0x1000, _lib.BF16, None, 32, 64, None, 0, 0, 5, 0, 0, 0, 0, ctypes.byref(out), None) == _lib.TJ2_ERR_ARG
    assert q(0x1000, _lib.BF16, None, 32, 64, None, 0, 0, 0, 0, 0, 0, 0, None, None) == _lib.TJ2_ERR_ARG
    assert q(0x1000, 9, None, 32, 64, None, 0, 0, 0, 0, 0, 0, 0, ctypes.byref(out), None) == _lib.TJ2_ERR_ARG
    # misaligned input
    assert q(0x1002, _lib.BF16, None, 32, 64, None, 0, 0, 0, 0, 0, 0, 0, ctypes.byref(out), None) == _lib.TJ2_ERR_ALIGN
    # grouped length not a multiple of 16
    bad = fake_q(_lib.NVFP4, 32, 64)
    assert q(0x1000, _lib.BF16, None, 32, 40, None, 0, 0, 0, 0, 0, 0, 0, ctypes.byref(bad), None) == _lib.TJ2_ERR_SHAPE
    # output shape mismatch (column grouping transposes)
    assert q(0x1000, _lib.BF16, None, 32, 64, None, 0, 1, 0, 0, 0, 0, 0, ctypes.byref(out), None) == _lib.TJ2_ERR_SHAPE
    assert b"expected" in L.tj2_last_error()
    # gather with column grouping is unsupported
    assert q(0x1000, _lib.BF16, None, 32, 64, 0x3000, 16, 1, 0, 0, 0, 0, 0, ctypes.byref(out), None) == _lib.TJ2_ERR_UNSUPPORTED


def test_quantize_dual_argument_errors(L):
    from bit_fully_quantized_amd import _lib
    r, c = fake_q(_lib.NVFP4, 32, 64), fake_q(_lib.NVFP4, 64, 32, base=0x20000)
    q = lambda x, rows, cols, ro, co: L.nvfp4_quantize_dual(x, rows, cols, 1, 0, 0, 2, ro, co, None)
    assert q(0x1000, 32, 64, None, ctypes.byref(c)) == _lib.TJ2_ERR_ARG
    assert q(0x1002, 32, 64, ctypes.byref(r), ctypes.byref(c)) == _lib.TJ2_ERR_ALIGN
    assert q(0x1000, 32, 40, ctypes.byref(r), ctypes.byref(c)) == _lib.TJ2_ERR_SHAPE
    # col_out is [cols, rows]
    assert q(0x1000, 32, 64, ctypes.byref(r), ctypes.byref(r)) == _lib.TJ2_ERR_SHAPE
    # FP8 outputs, or mixed formats, are refused
    r8, c8 = fake_q(_lib.FP8, 32, 64), fake_q(_lib.FP8, 64, 32, base=0x20000)
    assert q(0x1000, 32, 64, ctypes.byref(r8), ctypes.byref(c8)) == _lib.TJ2_ERR_ARG
    c6 = fake_q(_lib.NVFP6, 64, 32, base=0x20000)
    assert q(0x1000, 32, 64, ctypes.byref(r), ctypes.byref(c6)) == _lib.TJ2_ERR_ARG


def test_gemm_and_linear_argument_errors(L):
    from bit_fully_quantized_amd import _lib
    A = fake_q(_lib.NVFP4, 64, 128)
    B = fake_q(_lib.NVFP4, 32, 96)
    assert L.nvfp4_gemm(ctypes.byref(A), ctypes.byref(B), None, None, 0x5000, _lib.F32, 32, None, 0, None, 0, None) == _lib.TJ2_ERR_SHAPE
    B = fake_q(_lib.NVFP4, 32, 128)
    assert L.nvfp4_gemm(ctypes.byref(A), ctypes.byref(B), ctypes.byref(A), None, 0x5000, _lib.F32, 32, None, 0, None, 0, None) == _lib.TJ2_ERR_ARG
    assert L.nvfp4_gemm(ctypes.byref(A), ctypes.byref(B), None, None, 0x5000, _lib.BF16, 32, None, 1, None, 0, None) == _lib.TJ2_ERR_UNSUPPORTED
    assert L.nvfp4_gemm(ctypes.byref(A), ctypes.byref(B), None, None, 0x5000, _lib.F32, 16, None, 0, None, 0, None) == _lib.TJ2_ERR_SHAPE
    # outlier-column product: plan / B8 consistency is checked on the host
    B8 = fake_q(_lib.FP8, 16, 128)
    plan = _lib.PlanC(0x7000, 0x8000, 16, 0)
    assert L.nvfp4_gemm_outlier_cols(ctypes.byref(A), ctypes.byref(B), ctypes.byref(B8), None, 0x5000, _lib.F32,
                                     48, 0, None, 0, None) == _lib.TJ2_ERR_ARG
    bad = _lib.PlanC(0x7000, 0x8000, 32, 0)
    assert L.nvfp4_gemm_outlier_cols(ctypes.byref(A), ctypes.byref(B), ctypes.byref(B8), ctypes.byref(bad), 0x5000,
                                     _lib.F32, 48, 0, None, 0, None) == _lib.TJ2_ERR_SHAPE
    assert L.nvfp4_gemm_outlier_cols(ctypes.byref(A), ctypes.byref(B), ctypes.byref(B8), ctypes.byref(plan), 0x5000,
                                     _lib.F32, 32, 0, None, 0, None) == _lib.TJ2_ERR_SHAPE
    assert L.nvfp4_gemm_outlier_cols(ctypes.byref(A), ctypes.byref(B8), ctypes.byref(B), ctypes.byref(plan), 0x5000,
                                     _lib.F32, 48, 0, None, 0, None) == _lib.TJ2_ERR_UNSUPPORTED
    Xq = fake_q(_lib.NVFP4, 64, 128)
    Wq = fake_q(_lib.NVFP4, 32, 128)
    # M not a multiple of 16
    assert L.nvfp4_linear_fwd(0x1000, 60, 128, 32, None, ctypes.byref(Wq), None, None, ctypes.byref(Xq), None,
                              0x9000, _lib.BF16, None, 0, None) == _lib.TJ2_ERR_SHAPE
    # plan with a bad outlier count
    plan = _lib.PlanC(0x7000, 0x8000, 8, 0)
    assert L.nvfp4_linear_fwd(0x1000, 64, 128, 32, None, ctypes.byref(Wq), None, ctypes.byref(plan),
                              ctypes.byref(Xq), None, 0x9000, _lib.BF16, None, 0, None) == _lib.TJ2_ERR_SHAPE
    # a workspace smaller than the forward's split asks for (a small M: few output tiles)
    need = L.nvfp4_linear_fwd_workspace_size(64, 32, 128 * 64, 0)
    assert need > 0 and L.nvfp4_linear_fwd_workspace_size(16384, 4096, 1024, 0) == 0
    Xb = fake_q(_lib.NVFP4, 64, 128 * 64)
    Wb = fake_q(_lib.NVFP4, 32, 128 * 64)
    assert L.nvfp4_linear_fwd(0x1000, 64, 128 * 64, 32, None, ctypes.byref(Wb), None, None, ctypes.byref(Xb), None,
                              0x9000, _lib.BF16, 0xB000, need - 1, None) == _lib.TJ2_ERR_ARG
    assert b"workspace" in L.tj2_last_error()
    # backward without workspace
    assert L.nvfp4_linear_bwd(0x1000, 64, 32, 128, ctypes.byref(Xq), None, ctypes.byref(Wq), None, None, 1, 0, 0,
                              0x9000, _lib.BF16, 0xA000, None, None, 0, None) == _lib.TJ2_ERR_ARG
    assert b"workspace" in L.tj2_last_error()
    assert L.nvfp4_linear_bwd_workspace_size(64, 32, 128, 0) > 0


def test_osci_argument_errors(L):
    from bit_fully_quantized_amd import _lib
    p = [0x1000 * (i + 1) for i in range(5)]
    assert L.osci_reset_step(*p, 16, 100, 1, ctypes.c_float(4.0), 1, None, None, None, None, None, None) == _lib.TJ2_ERR_SHAPE
    assert L.osci_reset_step(*p, 16, 128, 7, ctypes.c_float(4.0), 1, None, None, None, None, None, None) == _lib.TJ2_ERR_ARG
    assert L.osci_reset_step(*p, 16, 128, 1, ctypes.c_float(-1.0), 1, None, None, None, None, None, None) == _lib.TJ2_ERR_ARG
    assert L.osci_reset_step(None, *p[1:], 16, 128, 1, ctypes.c_float(4.0), 1, None, None, None, None, None, None) == _lib.TJ2_ERR_ARG
    assert L.tj2_channel_sumsq(0x1000, 64, 100, 0x2000, 0x3000, 1 << 20, None) == _lib.TJ2_ERR_SHAPE
    assert L.tj2_channel_sumsq(0x1000, 64, 128, 0x2000, None, 0, None) == _lib.TJ2_ERR_ARG
    need = L.tj2_channel_sumsq_workspace_size(1000, 128)
    assert need == 2 * 128 * 8  # two 512-row slabs of fp64 partial sums
    assert L.tj2_channel_sumsq(0x1000, 1000, 128, 0x2000, 0x3000, need - 8, None) == _lib.TJ2_ERR_ARG


def test_osci_multi_argument_errors(L):
    from bit_fully_quantized_amd import _lib
    def tensor(i, N=16, K=128, align=0):
        return _lib.OsciTensorC(*[0x1000 * (5 * i + j + 1) + align for j in range(5)], N, K, None)
    good = [tensor(i) for i in range(3)]
    arr = (_lib.OsciTensorC * 3)(*good)
    assert L.osci_reset_step_multi(None, 3, 1, ctypes.c_float(4.0), 1, None, None, None) == _lib.TJ2_ERR_ARG
    assert L.osci_reset_step_multi(arr, 0, 1, ctypes.c_float(4.0), 1, None, None, None) == _lib.TJ2_ERR_ARG
    assert L.osci_reset_step_multi(arr, 3, 7, ctypes.c_float(4.0), 1, None, None, None) == _lib.TJ2_ERR_ARG
    assert L.osci_reset_step_multi(arr, 3, 1, ctypes.c_float(-1.0), 1, None, None, None) == _lib.TJ2_ERR_ARG
    # one bad member (K not a multiple of 16, a misaligned array) rejects the whole call, named by index
    for bad, code in ((tensor(1, K=100), _lib.TJ2_ERR_SHAPE), (tensor(1, align=4), _lib.TJ2_ERR_ALIGN)):
        arr = (_lib.OsciTensorC * 3)(good[0], bad, good[2])
        assert L.osci_reset_step_multi(arr, 3, 1, ctypes.c_float(4.0), 1, None, None, None) == code
        assert b"tensors[1]" in L.tj2_last_error()


def test_master_multi_argument_errors(L):
    from bit_fully_quantized_amd import _lib
    def tensor(i, N=16, K=128, align=0):
        return _lib.MasterTensorC(*[0x1000 * (7 * i + j + 1) + align for j in range(7)], N, K, None)
    ap = _lib.AdamWC(1e-3, 0.9, 0.95, 1e-8, 0.1, 0.1, 0.05)
    good = [tensor(i) for i in range(3)]
    arr = (_lib.MasterTensorC * 3)(*good)
    assert L.master_update_step_multi(None, 3, ctypes.byref(ap), 1, ctypes.c_float(4.0), 1, None, None, None) == _lib.TJ2_ERR_ARG
    assert L.master_update_step_multi(arr, 0, ctypes.byref(ap), 1, ctypes.c_float(4.0), 1, None, None, None) == _lib.TJ2_ERR_ARG
    assert L.master_update_step_multi(arr, 3, None, 1, ctypes.c_float(4.0), 1, None, None, None) == _lib.TJ2_ERR_ARG
    assert L.master_update_step_multi(arr, 3, ctypes.byref(ap), 0, ctypes.c_float(4.0), 1, None, None, None) == _lib.TJ2_ERR_ARG
    for bad, code in ((tensor(2, K=100), _lib.TJ2_ERR_SHAPE), (tensor(2, align=4), _lib.TJ2_ERR_ALIGN)):
        arr = (_lib.MasterTensorC * 3)(good[0], good[1], bad)
        assert L.master_update_step_multi(arr, 3, ctypes.byref(ap), 1, ctypes.c_float(4.0), 1, None, None, None) == code
        assert b"tensors[2]" in L.tj2_last_error()


def test_master_update_argument_errors(L):
    from bit_fully_quantized_amd import _lib
    p = [0x1000 * (i + 1) for i in range(7)]
    ap = _lib.AdamWC(1e-3, 0.9, 0.95, 1e-8, 0.1, 0.1, 0.05)
    f4 = ctypes.c_float(4.0)
    assert L.master_update_step(*p, 16, 100, ctypes.byref(ap), _lib.OSCI_ACCUM, f4, 0, None, None, None, None, None, None, None) == _lib.TJ2_ERR_SHAPE
    assert L.master_update_step(*p, 16, 128, ctypes.byref(ap), _lib.OSCI_INIT, f4, 0, None, None, None, None, None, None, None) == _lib.TJ2_ERR_ARG
    assert L.master_update_step(*p, 16, 128, None, _lib.OSCI_ACCUM, f4, 0, None, None, None, None, None, None, None) == _lib.TJ2_ERR_ARG
    assert L.master_update_step(*p, 16, 128, ctypes.byref(ap), _lib.OSCI_ACCUM, ctypes.c_float(-1.0), 0, None, None, None, None, None,
                                None, None) == _lib.TJ2_ERR_ARG
    assert L.master_update_step(None, *p[1:], 16, 128, ctypes.byref(ap), _lib.OSCI_ACCUM, f4, 0, None, None, None, None, None,
                                None, None) == _lib.TJ2_ERR_ARG
    q = list(p)
    q[3] = 0x3008  # grad not 16-byte aligned
    assert L.master_update_step(*q, 16, 128, ctypes.byref(ap), _lib.OSCI_ACCUM, f4, 0, None, None, None, None, None, None, None) == _lib.TJ2_ERR_ALIGN


def test_diag_counter_alignment(L):
    # misaligned diagnostic counters are rejected on the host, before any launch
    from bit_fully_quantized_amd import _lib
    p = [0x1000 * (i + 1) for i in range(7)]
    ap = _lib.AdamWC(1e-3, 0.9, 0.95, 1e-8, 0.1, 0.1, 0.05)
    f4 = ctypes.c_float(4.0)
    d = _lib.OsciDiagC(0x5004, None)
    assert L.master_update_step(*p, 16, 128, ctypes.byref(ap), _lib.OSCI_ACCUM, f4, 0, None, None, None, None, None, ctypes.byref(d),
                                None) == _lib.TJ2_ERR_ALIGN
    assert b"8-byte" in L.tj2_last_error()
    d = _lib.OsciDiagC(None, 0x5002)
    assert L.osci_reset_step(*p[:5], 16, 128, _lib.OSCI_WINDOW_END, f4, 1, None, None, None, None, ctypes.byref(d),
                             None) == _lib.TJ2_ERR_ALIGN


def test_measurement_helpers_live_outside_the_product_library(L):
    # the benchmark's MFMA-only loop is in libtj2_measure.so, declared by include/tj2_measure.h
    from bit_fully_quantized_amd import _lib
    assert not hasattr(L, "tj2_mfma_peak_probe")
    M = _lib.measure_lib()
    assert M.tj2_mfma_peak_probe(16, 8, None, None) == 1
    assert M.tj2_mfma_peak_probe(0, 8, 0x1000, None) == 1
    assert M.tj2_mfma_peak_probe(16, 0, 0x1000, None) == 1
    text = open(os.path.join(ROOT, "include", "tj2_measure.h")).read()
    assert "tj2_mfma_peak_probe" in text
    # the access-pattern reference: argument checks only (they return before any launch)
    assert not hasattr(L, "tj2_stream_probe") and "tj2_stream_probe" in text
    five = (ctypes.c_void_p * 7)(*([0x10000] * 7))
    four = (ctypes.c_void_p * 6)(*([0x20000] * 6))
    assert M.tj2_stream_probe(None, 5, four, 4, 1024, None) == 1
    assert M.tj2_stream_probe(five, 6, four, 4, 1024, None) == 1  # only 5 / 4 and 7 / 6
    assert M.tj2_stream_probe(five, 7, four, 4, 1024, None) == 1
    assert M.tj2_stream_probe(five, 5, four, 4, 4, None) == 1  # n below 8
    bad = (ctypes.c_void_p * 7)(*([0x10004] + [0x10000] * 6))  # not 16-byte aligned
    assert M.tj2_stream_probe(bad, 5, four, 4, 1024, None) == 1


def _plan_from_library(L, scores, p):
    import numpy as np
    sc = np.ascontiguousarray(scores, dtype=np.float64)
    K = sc.size
    o = np.zeros(K, np.int32)
    r = np.zeros(K, np.int32)
    n = ctypes.c_int32(-1)
    st = L.tj2_select_outliers(sc.ctypes.data, K, ctypes.c_double(p), o.ctypes.data, r.ctypes.data, ctypes.byref(n))
    return st, o[: n.value], r[: K - n.value]


def test_select_outliers_matches_oracle(L):
    """tj2_select_outliers against the oracle's top-p selection (and its brute force pin): random
    scores, many exact ties, the lognormal channel gains of the 370M-style inputs."""
    import numpy as np
    from oracle import calib
    rng = np.random.default_rng(3)
    cases = [(rng.random(1024), 0.10), (np.floor(rng.random(4096) * 7.0), 0.10), (np.ones(128), 0.10),
             (np.exp(1.5 * rng.standard_normal(4096)) ** 2, 0.10), (rng.random(512), 0.03), (rng.random(96), 0.5)]
    for scores, p in cases:
        st, o, r = _plan_from_library(L, scores, p)
        assert st == 0
        want = calib.select_outliers(scores, p)
        np.testing.assert_array_equal(o, want)
        np.testing.assert_array_equal(np.sort(np.concatenate([o, r])), np.arange(scores.size))
        assert np.all(np.diff(r) > 0)


def test_select_outliers_errors(L):
    import numpy as np
    from bit_fully_quantized_amd import _lib
    assert _plan_from_library(L, np.ones(100), 0.1)[0] == _lib.TJ2_ERR_SHAPE  # K not a multiple of 16
    assert _plan_from_library(L, np.ones(128), 0.0)[0] == _lib.TJ2_ERR_ARG
    assert _plan_from_library(L, np.ones(128), 1.0)[0] == _lib.TJ2_ERR_ARG
    assert _plan_from_library(L, np.ones(16), 0.5)[0] == _lib.TJ2_ERR_SHAPE  # 16 of 16 channels: none left
    bad = np.ones(128)
    bad[5] = -1.0
    assert _plan_from_library(L, bad, 0.1)[0] == _lib.TJ2_ERR_ARG
    bad[5] = np.nan
    assert _plan_from_library(L, bad, 0.1)[0] == _lib.TJ2_ERR_ARG


def test_gemm_workspace_counts_both_segments(L):
    # a two-segment product splits over the chunks of both segments
    one = L.nvfp4_gemm_workspace_size(256, 128, 1024, 0)
    two = L.nvfp4_gemm_workspace_size(256, 128, 880, 112)
    assert two >= one > 0


def test_gemm_workspace_holds_the_b_image(L):
    # one-segment products of at least 8 row tiles (2048 rows) also take room for B decoded once:
    # per 128-column tile and 128-element chunk, 128 rows of 272 bytes, then the fp32 outer scales
    # [chunks][columns padded to 128]; the split-K partials come first (256-byte aligned)
    I, J, K = 2048, 3072, 16384
    part = 4 * I * J * 4  # four K splits of fp32 partial sums
    img = (J // 128) * (K // 128) * 128 * 272 + (K // 128) * J * 4
    assert L.nvfp4_gemm_workspace_size(I, J, K, 0) == part + img
    # 300 columns: 3 column tiles, scales padded to 384 columns
    assert L.nvfp4_gemm_workspace_size(16384, 300, 1024, 0) == 3 * 8 * 128 * 272 + 8 * 384 * 4
    # fewer row tiles (7): no image (7 chunks: no split either)
    assert L.nvfp4_gemm_workspace_size(1792, 300, 896, 0) == 0
    # a second K segment (the forward's FP8 outlier channels): its chunks follow the first's, when the
    # product runs unsplit (here fewer than 8 chunks); a split product, or one NVFP4 chunk: none
    assert L.nvfp4_gemm_workspace_size(16384, 300, 768, 128) == 3 * 7 * 128 * 272 + 7 * 384 * 4
    split_only = L.nvfp4_gemm_workspace_size(2048, 256, 3680, 416)  # 16 tiles over 33 chunks: a K split
    assert split_only > 0 and split_only % (2048 * 256 * 4) == 0  # whole fp32 partial sums, no image
    assert L.nvfp4_gemm_workspace_size(16384, 300, 128, 128) == 0


def test_forward_workspace_holds_the_b_image(L):
    # the forward with an outlier plan takes room for its product's B image, which the weights' split
    # quantization writes: W's NVFP4 chunks, then W8's FP8 chunks
    img = lambda J, nch: (J // 128) * nch * 128 * 272 + nch * J * 4  # noqa: E731
    assert L.nvfp4_linear_fwd_workspace_size(16384, 4096, 1024, 112) == img(4096, 9)
    assert L.nvfp4_linear_fwd_workspace_size(16384, 1024, 4096, 416) == img(1024, 33)
    # no plan, fewer than 8 row tiles, rows past the quantizer's 32 KB staging (K > 8192), or a
    # single NVFP4 chunk: no image
    assert L.nvfp4_linear_fwd_workspace_size(16384, 4096, 1024, 0) == 0
    assert L.nvfp4_linear_fwd_workspace_size(1792, 4096, 1024, 112) == 0
    assert L.nvfp4_linear_fwd_workspace_size(16384, 4096, 9216, 112) == 0
    assert L.nvfp4_linear_fwd_workspace_size(16384, 4096, 240, 112) == 0


def test_qtensor_block_count_limit(L):
    # operands are indexed by 128-element block in 32 bits; larger ones are rejected on the host
    from bit_fully_quantized_amd import _lib
    out = _lib.QTensorC(0x10000, 0x20000, 0x30000, 1 << 30, 1 << 30, _lib.NVFP4, 0)
    assert L.nvfp4_quantize(0x1000, _lib.BF16, None, 1 << 30, 1 << 30, None, 0, 0, 0, 0, 0, 0, 0, ctypes.byref(out),
                            None) == _lib.TJ2_ERR_SHAPE
    assert b"128-element blocks" in L.tj2_last_error()


def test_noalloc_refuses_products_beyond_its_scratch(L):
    # a 2048 x 3072 output over 16384 tokens splits 4 ways: 96 MiB of partial sums, more than the
    # library's 32 MiB scratch; refused on the host before any device work
    from bit_fully_quantized_amd import _lib
    A = fake_q(_lib.NVFP4, 2048, 16384)
    B = fake_q(_lib.NVFP4, 3072, 16384)
    assert L.nvfp4_gemm_workspace_size(2048, 3072, 16384, 0) >= 4 * 2048 * 3072 * 4
    assert L.nvfp4_gemm_noalloc(ctypes.byref(A), ctypes.byref(B), None, None, 0x9000, _lib.F32, 3072, None, 0,
                                None) == _lib.TJ2_ERR_SHAPE
    assert b"scratch" in L.tj2_last_error()
    assert L.nvfp4_gemm_noalloc(ctypes.byref(A), None, None, None, 0x9000, _lib.F32, 3072, None, 0,
                                None) == _lib.TJ2_ERR_ARG


def test_osci_plan_argument_errors(L):
    from bit_fully_quantized_amd import _lib
    p = [0x1000 * (i + 1) for i in range(5)]
    f4 = ctypes.c_float(4.0)
    plan = _lib.PlanC(0x7000, 0x8000, 16, 0)
    w8 = fake_q(_lib.FP8, 16, 16)
    # FP8 codes without a plan
    assert L.osci_reset_step(*p, 16, 128, 1, f4, 1, None, None, ctypes.byref(w8), None, None, None) == _lib.TJ2_ERR_ARG
    # with a plan the NVFP4 codes cover the K - n rest channels
    wq_full = fake_q(_lib.NVFP4, 16, 128)
    assert L.osci_reset_step(*p, 16, 128, 1, f4, 1, ctypes.byref(plan), ctypes.byref(wq_full), ctypes.byref(w8),
                             None, None, None) == _lib.TJ2_ERR_SHAPE
    # next-backward operands need the codes they are formed from
    q7 = [0x1000 * (i + 1) for i in range(7)]
    ap = _lib.AdamWC(1e-3, 0.9, 0.95, 1e-8, 0.1, 0.1, 0.05)
    wt = fake_q(_lib.NVFP4, 128, 16)
    nxt = _lib.NextBwdC(ctypes.pointer(wt), None, 0, 0, 1, 0)
    assert L.master_update_step(*q7, 16, 128, ctypes.byref(ap), _lib.OSCI_ACCUM, f4, 0, None, None, None,
                                ctypes.byref(nxt), None, None, None) == _lib.TJ2_ERR_ARG
    assert b"Wq_out" in L.tj2_last_error()
