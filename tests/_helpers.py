"""Shared helpers for the GPU parity tests (host <-> device marshalling, comparisons)."""
from __future__ import annotations

import numpy as np
import torch

import synthetic
from oracle import formats, philox, quant

GEMM_TOL = 1e-3  # relative Frobenius error bound of the products vs the fp64 reference


def bf16_to_device(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def f32_to_device(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()


def bf16_values(bits: np.ndarray) -> np.ndarray:
    return synthetic.bf16_bits_to_f32(bits)


def oracle_qtensor_from_gpu(q) -> quant.QTensor:
    """Oracle-side QTensor holding the GPU's (unpadded) bytes."""
    codes, s16, s128 = q.host()
    fmt = {2: "nvfp4", 3: "fp8", 4: "nvfp6"}[q.fmt]
    return quant.QTensor(fmt, codes.copy(), s128.copy(), None if s16 is None else s16.copy(), q.rows, q.len)


def assert_q_equal(gpu_q, ref: quant.QTensor, rows=None, what=""):
    """Bit-exact comparison of a GPU QTensor (optionally only `rows`) with an oracle QTensor."""
    codes, s16, s128 = gpu_q.host()
    sel = slice(None) if rows is None else rows
    np.testing.assert_array_equal(s128[sel].view(np.uint32), ref.s128.view(np.uint32), err_msg=f"{what}: scale128")
    if ref.fmt in ("nvfp4", "nvfp6"):
        np.testing.assert_array_equal(s16[sel], ref.s16, err_msg=f"{what}: scale16")
    np.testing.assert_array_equal(codes[sel], ref.codes, err_msg=f"{what}: codes")


def assert_padding_zero(gpu_q):
    nb = gpu_q.nb
    if gpu_q.len == nb * 128:
        return
    codes = gpu_q.codes.cpu().numpy()
    per = 64 if gpu_q.fmt == 2 else 128
    assert not codes[:, gpu_q.len * per // 128:].any(), "code padding not zero"
    if gpu_q.scale16 is not None:
        assert not gpu_q.scale16.cpu().numpy()[:, gpu_q.len // 16:].any(), "scale padding not zero"


def oracle_rows(y_rows: np.ndarray, row_ids, n_cols_total: int, fmt: str, rounding: str, seed: int, offset: int,
                rht_mask=None) -> quant.QTensor:
    """Oracle quantization of selected rows of a row-grouped quantizer input of width n_cols_total.

    Stochastic draws use each element's global row-major index, as the full call would.
    """
    from oracle import rht
    y = np.asarray(y_rows, dtype=np.float32)
    if rht_mask is not None:
        y = rht.rht_along_last(y, rht_mask)
    u16 = None
    if rounding == "sr":
        idx = (np.asarray(row_ids, dtype=np.uint64)[:, None] * np.uint64(n_cols_total)
               + np.arange(y.shape[1], dtype=np.uint64)[None, :])
        u16 = philox.sr_draws_u16(idx, seed, offset)
    if fmt == "nvfp4":
        return quant.nvfp4_quantize_rows(y, rounding, u16)
    if fmt == "nvfp6":
        return quant.nvfp6_quantize_rows(y, rounding, u16)
    return quant.fp8_quantize_rows(y, rounding, u16)


def oracle_cols(x_cols: np.ndarray, col_ids, n_cols_total: int, fmt: str, rounding: str, seed: int, offset: int,
                rht_mask=None) -> quant.QTensor:
    """Oracle column-grouped quantization of selected input columns (x_cols: [R, len(col_ids)]).

    Returns the transposed rows [len(col_ids), R]; draws use the output index c * R + r.
    """
    from oracle import rht
    y = np.ascontiguousarray(np.asarray(x_cols, dtype=np.float32).T)
    if rht_mask is not None:
        y = rht.rht_along_last(y, rht_mask)
    u16 = None
    if rounding == "sr":
        R = y.shape[1]
        idx = (np.asarray(col_ids, dtype=np.uint64)[:, None] * np.uint64(R)
               + np.arange(R, dtype=np.uint64)[None, :])
        u16 = philox.sr_draws_u16(idx, seed, offset)
    if fmt == "nvfp4":
        return quant.nvfp4_quantize_rows(y, rounding, u16)
    if fmt == "nvfp6":
        return quant.nvfp6_quantize_rows(y, rounding, u16)
    return quant.fp8_quantize_rows(y, rounding, u16)


def rel_fro(c, ref) -> float:
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(np.asarray(c, dtype=np.float64) - ref) / max(np.linalg.norm(ref), 1e-300))


def bf16_ulp_ok(c_bf16: torch.Tensor, ref: np.ndarray, fp32_tol: float = 1e-5) -> bool:
    """Each bf16 output is within one bf16 ulp (+ the fp32 accumulation slack) of the fp64 reference."""
    got = c_bf16.float().cpu().numpy().astype(np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    ulp = np.abs(ref) * 2.0 ** -7 + 1e-30
    scale = np.abs(ref).max()
    return bool(np.all(np.abs(got - ref) <= ulp + fp32_tol * scale))


def e2m1_decode(c):
    return formats.e2m1_decode(c)
