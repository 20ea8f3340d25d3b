"""ctypes declarations of libtj2.so (the C ABI in include/tj2.h).

The library is loaded from this package directory only; there is no fallback:
if it is missing, every call raises.  torch is imported first so the HIP
runtime it ships is the one the library binds to.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime before libtj2)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtj2.so")
MEASURE_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtj2_measure.so")

TJ2_OK, TJ2_ERR_ARG, TJ2_ERR_SHAPE, TJ2_ERR_ALIGN, TJ2_ERR_HIP, TJ2_ERR_UNSUPPORTED = range(6)
BF16, F32, NVFP4, FP8, NVFP6 = 0, 1, 2, 3, 4
GROUP_ROW, GROUP_COL = 0, 1
RTN, SR = 0, 1
OSCI_INIT, OSCI_ACCUM, OSCI_WINDOW_END = 0, 1, 2

STATUS_NAMES = {0: "TJ2_OK", 1: "TJ2_ERR_ARG", 2: "TJ2_ERR_SHAPE", 3: "TJ2_ERR_ALIGN", 4: "TJ2_ERR_HIP",
                5: "TJ2_ERR_UNSUPPORTED"}


class QTensorC(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scale16", ctypes.c_void_p), ("scale128", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("len", ctypes.c_int64), ("fmt", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class PlanC(ctypes.Structure):
    _fields_ = [("outliers", ctypes.c_void_p), ("rest", ctypes.c_void_p), ("n_outliers", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class BwdOperandsC(ctypes.Structure):
    _fields_ = [("dYq", QTensorC), ("dYt", QTensorC), ("Wt", QTensorC), ("Xt", QTensorC), ("W8t", QTensorC),
                ("X8t", QTensorC), ("w_given", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class Tj2Error(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed with {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None

P = ctypes.c_void_p
I32 = ctypes.c_int32
I64 = ctypes.c_int64
U32 = ctypes.c_uint32
U64 = ctypes.c_uint64
SZ = ctypes.c_size_t
QP = ctypes.POINTER(QTensorC)


class AdamWC(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float),
                ("bias_correction1", ctypes.c_float), ("bias_correction2", ctypes.c_float)]


class OsciDiagC(ctypes.Structure):
    _fields_ = [("flips", P), ("risk_hist", P)]


RISK_BINS = 32


PLANP = ctypes.POINTER(PlanC)


class NextBwdC(ctypes.Structure):
    _fields_ = [("Wt", QP), ("W8t", QP), ("seed", U64), ("offset", U64), ("rht", I32), ("reserved", I32)]


class OsciTensorC(ctypes.Structure):
    _fields_ = [("W", P), ("W_prev", P), ("Q_prev", P), ("dQ", P), ("dM", P), ("N", I64), ("K", I64), ("Wq_out", QP),
                ("plan", PLANP), ("W8_out", QP)]


class MasterTensorC(ctypes.Structure):
    _fields_ = [("W", P), ("m", P), ("v", P), ("grad", P), ("Q_prev", P), ("dQ", P), ("dM", P), ("N", I64), ("K", I64),
                ("Wq_out", QP), ("plan", PLANP), ("W8_out", QP), ("next", ctypes.POINTER(NextBwdC))]

SIGNATURES = {
    "tj2_last_error": (ctypes.c_char_p, []),
    "tj2_version": (ctypes.c_char_p, []),
    "tj2_qtensor_bytes": (I32, [I32, I64, I64, ctypes.POINTER(SZ), ctypes.POINTER(SZ), ctypes.POINTER(SZ)]),
    "tj2_rht_signs": (ctypes.c_uint16, [U64, U64]),
    "nvfp4_quantize": (I32, [P, I32, QP, I64, I64, P, I64, I32, I32, I32, U32, U64, U64, QP, P]),
    "nvfp4_quantize_dual": (I32, [P, I64, I64, I32, U64, U64, U64, QP, QP, P]),
    "nvfp4_gemm": (I32, [QP, QP, QP, QP, P, I32, I64, P, I32, P, SZ, P]),
    "nvfp4_gemm_workspace_size": (SZ, [I64, I64, I64, I64]),
    "nvfp4_gemm_noalloc": (I32, [QP, QP, QP, QP, P, I32, I64, P, I32, P]),
    "nvfp4_gemm_outlier_cols": (I32, [QP, QP, QP, ctypes.POINTER(PlanC), P, I32, I64, I32, P, SZ, P]),
    "nvfp4_linear_fwd": (I32, [P, I64, I64, I64, P, QP, QP, ctypes.POINTER(PlanC), QP, QP, P, I32, P, SZ, P]),
    "nvfp4_linear_fwd_workspace_size": (SZ, [I64, I64, I64, I32]),
    "nvfp4_linear_bwd": (I32, [P, I64, I64, I64, QP, QP, QP, QP, ctypes.POINTER(PlanC), I32, U64, U64, P, I32, P,
                               ctypes.POINTER(BwdOperandsC), P, SZ, P]),
    "nvfp4_linear_bwd_workspace_size": (SZ, [I64, I64, I64, I32]),
    "nvfp6x4_linear_bwd": (I32, [P, I64, I64, I64, QP, QP, QP, QP, ctypes.POINTER(PlanC), I32, U64, U64, P, I32, P,
                                 ctypes.POINTER(BwdOperandsC), P, SZ, P]),
    "nvfp6x4_linear_bwd_workspace_size": (SZ, [I64, I64, I64, I32]),
    "osci_reset_step": (I32, [P, P, P, P, P, I64, I64, I32, ctypes.c_float, I32, PLANP, QP, QP, P,
                              ctypes.POINTER(OsciDiagC), P]),
    "osci_reset_step_multi": (I32, [ctypes.POINTER(OsciTensorC), I32, I32, ctypes.c_float, I32, P,
                                    ctypes.POINTER(OsciDiagC), P]),
    "master_update_step_multi": (I32, [ctypes.POINTER(MasterTensorC), I32, ctypes.POINTER(AdamWC), I32,
                                       ctypes.c_float, I32, P, ctypes.POINTER(OsciDiagC), P]),
    "master_update_step": (I32, [P, P, P, P, P, P, P, I64, I64, ctypes.POINTER(AdamWC), I32, ctypes.c_float, I32,
                                 PLANP, QP, QP, ctypes.POINTER(NextBwdC), P, ctypes.POINTER(OsciDiagC), P]),
    "tj2_channel_sumsq_workspace_size": (SZ, [I64, I64]),
    "tj2_channel_sumsq": (I32, [P, I64, I64, P, P, SZ, P]),
    "tj2_select_outliers": (I32, [P, I64, ctypes.c_double, P, P, ctypes.POINTER(I32)]),
}


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m bit_fully_quantized_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


_mlib = None


def measure_lib():
    """The measurement helpers (libtj2_measure.so, include/tj2_measure.h): not part of the path."""
    global _mlib
    if _mlib is None:
        if not os.path.exists(MEASURE_LIB_PATH):
            raise RuntimeError(f"{MEASURE_LIB_PATH} is missing: build it with `python -m bit_fully_quantized_amd.build`")
        L = ctypes.CDLL(MEASURE_LIB_PATH)
        L.tj2_mfma_peak_probe.restype = I32
        L.tj2_mfma_peak_probe.argtypes = [I64, I32, P, P]
        L.tj2_decode_probe.restype = I32
        L.tj2_decode_probe.argtypes = [I32, I64, I32, P, P]
        L.tj2_stream_probe.restype = I32
        L.tj2_stream_probe.argtypes = [P, I32, P, I32, I64, P]
        _mlib = L
    return _mlib


def check(fn: str, status: int) -> None:
    if status != TJ2_OK:
        raise Tj2Error(fn, status, lib().tj2_last_error().decode())
