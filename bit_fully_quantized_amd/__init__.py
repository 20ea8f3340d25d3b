"""TetraJet-v2 NVFP4 linear layer on AMD MI355X: Python binding of libtj2.

Thin wrappers over the C ABI (include/tj2.h): they take torch tensors that
live on the GPU, pass their device pointers and the current HIP stream, and
check the returned status.  Every step of the path runs in the library's HIP
kernels; there is no Python or CPU implementation here.
"""
from __future__ import annotations

import ctypes
import math
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import (BF16, F32, FP8, GROUP_COL, GROUP_ROW, NVFP4, NVFP6, OSCI_ACCUM, OSCI_INIT, OSCI_WINDOW_END, RISK_BINS, RTN,
                   SR, Tj2Error, check, lib)

__all__ = ["QTensor", "OutlierPlan", "quantize", "gemm", "gemm_workspace", "linear_fwd", "linear_fwd_workspace",
           "linear_bwd", "linear_bwd_workspace", "osci_reset_step", "osci_reset_step_multi", "OsciBatch",
           "master_update_step", "master_update_step_multi", "MasterBatch", "NextBwd", "bwd_operands", "channel_sumsq",
           "select_outliers",
           "mfma_peak_probe", "rht_signs", "lib", "Tj2Error", "NVFP4", "FP8", "NVFP6", "BF16", "F32", "GROUP_ROW", "GROUP_COL",
           "RTN", "SR", "OSCI_INIT", "OSCI_ACCUM", "OSCI_WINDOW_END", "RISK_BINS"]


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _dense(t, name: str, dtypes, shape=None, optional: bool = False):
    """A tensor argument the library reads or writes whole: on the GPU, of one of `dtypes`,
    contiguous (the library assumes row-major rows of the logical width), of `shape` if given."""
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _matrix_out(t, name: str, dtypes, rows: int, cols: int):
    """An output matrix written with a leading dimension: rows x >= cols, unit column stride."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype not in dtypes or t.dim() != 2:
        raise ValueError(f"{name} must be a 2-D CUDA tensor of dtype {dtypes}")
    if t.stride(1) != 1 or t.shape[0] != rows or t.shape[1] < cols or (rows > 1 and t.stride(0) < cols):
        raise ValueError(f"{name} must be [{rows}, >= {cols}] with unit column stride")


_BF16 = (torch.bfloat16,)
_F32 = (torch.float32,)
_I32 = (torch.int32,)


class QTensor:
    """A quantized operand of `rows` x `len` elements grouped along `len` (device storage).

    codes    uint8 [rows, nb*64] (NVFP4) or [rows, nb*128] (FP8, NVFP6), nb = ceil(len/128)
    scale16  uint8 [rows, nb*8] E4M3 (NVFP4, NVFP6)
    scale128 float32 [rows, nb]
    """

    def __init__(self, fmt: int, rows: int, length: int, device="cuda"):
        if length % 16 or length <= 0 or rows <= 0:
            raise ValueError("len must be a positive multiple of 16 and rows positive")
        self.fmt, self.rows, self.len = fmt, rows, length
        nb = (length + 127) // 128
        self.nb = nb
        self.codes = torch.empty((rows, nb * (64 if fmt == NVFP4 else 128)), dtype=torch.uint8, device=device)
        self.scale16 = torch.empty((rows, nb * 8), dtype=torch.uint8, device=device) if fmt != FP8 else None
        self.scale128 = torch.empty((rows, nb), dtype=torch.float32, device=device)

    def c(self) -> _lib.QTensorC:
        return _lib.QTensorC(self.codes.data_ptr(), 0 if self.scale16 is None else self.scale16.data_ptr(),
                             self.scale128.data_ptr(), self.rows, self.len, self.fmt, 0)

    def clone(self) -> "QTensor":
        q = QTensor.__new__(QTensor)
        q.fmt, q.rows, q.len, q.nb = self.fmt, self.rows, self.len, self.nb
        q.codes, q.scale128 = self.codes.clone(), self.scale128.clone()
        q.scale16 = self.scale16.clone() if self.scale16 is not None else None
        return q

    # host views of the unpadded content (for tests)
    def host(self):
        codes = self.codes.cpu().numpy()
        if self.fmt == NVFP4:
            return (codes[:, : self.len // 2], self.scale16.cpu().numpy()[:, : self.len // 16],
                    self.scale128.cpu().numpy())
        if self.fmt == NVFP6:
            return codes[:, : self.len], self.scale16.cpu().numpy()[:, : self.len // 16], self.scale128.cpu().numpy()
        return codes[:, : self.len], None, self.scale128.cpu().numpy()


@dataclass
class OutlierPlan:
    outliers: torch.Tensor  # int32 device, ascending
    rest: torch.Tensor  # int32 device, ascending

    @staticmethod
    def from_indices(K: int, outliers, device="cuda") -> "OutlierPlan":
        o = sorted(int(i) for i in outliers)
        mask = [True] * K
        for i in o:
            mask[i] = False
        rest = [i for i in range(K) if mask[i]]
        return OutlierPlan(torch.tensor(o, dtype=torch.int32, device=device),
                           torch.tensor(rest, dtype=torch.int32, device=device))

    @property
    def n(self) -> int:
        return int(self.outliers.numel())

    def c(self) -> _lib.PlanC:
        return _lib.PlanC(self.outliers.data_ptr(), self.rest.data_ptr(), self.n, 0)


def rht_signs(seed: int, offset: int) -> int:
    return int(lib().tj2_rht_signs(seed, offset))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def quantize(x, *, grouping: int = GROUP_ROW, rounding: int = RTN, rht: bool = False, signs: int = 0,
             seed: int = 0, offset: int = 0, out_fmt: int = NVFP4, col_idx: torch.Tensor | None = None,
             out: QTensor | None = None) -> QTensor:
    """Quantize a dense bf16/fp32 tensor [rows, cols] or a QTensor (dequantized first)."""
    if isinstance(x, QTensor):
        rows, cols = x.rows, x.len
        xp, xd, xq = None, x.fmt, ctypes.byref(x.c())
    else:
        _dense(x, "x", (torch.bfloat16, torch.float32))
        if x.dim() != 2:
            raise ValueError("x must be 2-D")
        rows, cols = x.shape
        xp, xd, xq = x, _dtype_code(x), None
    _dense(col_idx, "col_idx", _I32, optional=True)
    n = int(col_idx.numel()) if col_idx is not None else cols
    if out is None:
        out = QTensor(out_fmt, rows, n) if grouping == GROUP_ROW else QTensor(out_fmt, cols, rows)
    oc = out.c()
    st = lib().nvfp4_quantize(_ptr(xp), xd, xq, rows, cols, _ptr(col_idx), n if col_idx is not None else 0,
                              grouping, rounding, 1 if rht else 0, signs, seed, offset, ctypes.byref(oc), _stream())
    check("nvfp4_quantize", st)
    return out


def quantize_dual(x: torch.Tensor, *, rht: bool = True, seed: int = 0, row_offset: int = 0, col_offset: int = 2,
                  out_fmt: int = NVFP4, row_out: QTensor | None = None,
                  col_out: QTensor | None = None) -> tuple[QTensor, QTensor]:
    """Both stochastic groupings of a bf16 tensor [rows, cols] from one read: along cols
    (signs and draws of row_offset) and along rows, stored transposed (col_offset)."""
    _dense(x, "x", (torch.bfloat16,))
    if x.dim() != 2:
        raise ValueError("x must be 2-D")
    rows, cols = x.shape
    if row_out is None:
        row_out = QTensor(out_fmt, rows, cols)
    if col_out is None:
        col_out = QTensor(out_fmt, cols, rows)
    rc, cc = row_out.c(), col_out.c()
    st = lib().nvfp4_quantize_dual(_ptr(x), rows, cols, 1 if rht else 0, seed, row_offset, col_offset,
                                   ctypes.byref(rc), ctypes.byref(cc), _stream())
    check("nvfp4_quantize_dual", st)
    return row_out, col_out


def gemm_workspace(I: int, J: int, K: int, K2: int = 0, device="cuda") -> torch.Tensor | None:
    """Split-K workspace of an I x J product over K (+ K2 for a second segment), or None."""
    n = int(lib().nvfp4_gemm_workspace_size(I, J, K, K2))
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def gemm(A: QTensor, B: QTensor, A2: QTensor | None = None, B2: QTensor | None = None, *,
         out: torch.Tensor | None = None, out_dtype=torch.float32, col_map: torch.Tensor | None = None,
         accumulate: bool = False, workspace: torch.Tensor | None = None, split_k: bool = True) -> torch.Tensor:
    """C = A B^T (+ A2 B2^T) on packed operands; C[i, col_map[j]] if col_map is given.

    With split_k (default) a workspace for K-split partial sums is allocated when the library asks
    for one (nvfp4_gemm_workspace_size); pass `workspace` to reuse a buffer."""
    if out is None:
        out = torch.empty((A.rows, B.rows), dtype=out_dtype, device=A.codes.device)
    _matrix_out(out, "out", (torch.float32, torch.bfloat16), A.rows, 1 if col_map is not None else B.rows)
    _dense(col_map, "col_map", _I32, optional=True)
    _dense(workspace, "workspace", (torch.uint8,), optional=True)
    if workspace is None and split_k:
        workspace = gemm_workspace(A.rows, B.rows, A.len, A2.len if A2 is not None else 0, device=A.codes.device)
    ac, bc = A.c(), B.c()
    a2 = ctypes.byref(A2.c()) if A2 is not None else None
    b2 = ctypes.byref(B2.c()) if B2 is not None else None
    st = lib().nvfp4_gemm(ctypes.byref(ac), ctypes.byref(bc), a2, b2, _ptr(out), _dtype_code(out), out.stride(0),
                          _ptr(col_map), 1 if accumulate else 0, _ptr(workspace),
                          0 if workspace is None else workspace.numel(), _stream())
    check("nvfp4_gemm", st)
    return out


def gemm_outlier_cols(A: QTensor, B: QTensor, B8: QTensor, plan: "OutlierPlan", *, out: torch.Tensor | None = None,
                      out_dtype=torch.float32, accumulate: bool = False,
                      workspace: torch.Tensor | None = None) -> torch.Tensor:
    """One product over all K output columns of a plan: C[:, rest[j]] = A B[j]^T, C[:, outliers[j]] = A B8[j]^T."""
    J = B.rows + B8.rows
    if out is None:
        out = torch.empty((A.rows, J), dtype=out_dtype, device=A.codes.device)
    _matrix_out(out, "out", (torch.float32, torch.bfloat16), A.rows, J)
    _dense(workspace, "workspace", (torch.uint8,), optional=True)
    if workspace is None:
        workspace = gemm_workspace(A.rows, J, A.len, device=A.codes.device)
    ac, bc, b8c, pc = A.c(), B.c(), B8.c(), plan.c()
    st = lib().nvfp4_gemm_outlier_cols(ctypes.byref(ac), ctypes.byref(bc), ctypes.byref(b8c), ctypes.byref(pc),
                                       _ptr(out), _dtype_code(out), out.stride(0), 1 if accumulate else 0,
                                       _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream())
    check("nvfp4_gemm_outlier_cols", st)
    return out


def linear_fwd_workspace(M: int, N: int, K: int, n_outliers: int = 0, device="cuda") -> torch.Tensor | None:
    n = int(lib().nvfp4_linear_fwd_workspace_size(M, N, K, n_outliers))
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def linear_fwd(X: torch.Tensor, W_master: torch.Tensor | None, N: int, *, Wq: QTensor | None = None,
               W8: QTensor | None = None, plan: OutlierPlan | None = None, y_dtype=torch.bfloat16,
               Y: torch.Tensor | None = None, Xq: QTensor | None = None, X8: QTensor | None = None,
               workspace: torch.Tensor | None = None):
    """Y = X W^T with NVFP4 operands; returns (Y, saved) with saved = dict(Xq, X8, Wq, W8).

    Output / saved buffers may be passed in (Y, Xq, X8, Wq, W8, workspace) to avoid allocations."""
    _dense(X, "X", _BF16)
    if X.dim() != 2:
        raise ValueError("X must be 2-D")
    M, K = X.shape
    _dense(W_master, "W_master", _F32, shape=(N, K), optional=True)
    if W_master is None and Wq is None:
        raise ValueError("W_master or Wq is required")
    K1 = K - (plan.n if plan else 0)
    if Xq is None:
        Xq = QTensor(NVFP4, M, K1)
    if plan and X8 is None:
        X8 = QTensor(FP8, M, plan.n)
    if Wq is None:
        Wq = QTensor(NVFP4, N, K1)
    if plan and W8 is None:
        W8 = QTensor(FP8, N, plan.n)
    if Y is None:
        Y = torch.empty((M, N), dtype=y_dtype, device=X.device)
    _dense(Y, "Y", (torch.bfloat16, torch.float32), shape=(M, N))
    if workspace is None:
        workspace = linear_fwd_workspace(M, N, K, plan.n if plan else 0, device=X.device)
    _dense(workspace, "workspace", (torch.uint8,), optional=True)
    pc = plan.c() if plan else None
    w8c = W8.c() if W8 is not None else None
    x8c = X8.c() if X8 is not None else None
    wqc, xqc = Wq.c(), Xq.c()
    st = lib().nvfp4_linear_fwd(_ptr(X), M, K, N, _ptr(W_master), ctypes.byref(wqc),
                                ctypes.byref(w8c) if w8c is not None else None,
                                ctypes.byref(pc) if pc is not None else None, ctypes.byref(xqc),
                                ctypes.byref(x8c) if x8c is not None else None, _ptr(Y), _dtype_code(Y),
                                _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream())
    check("nvfp4_linear_fwd", st)
    return Y, {"Xq": Xq, "X8": X8, "Wq": Wq, "W8": W8}


def linear_bwd_workspace(M: int, N: int, K: int, n_outliers: int = 0, device="cuda",
                         grad_fmt: int = NVFP4) -> torch.Tensor:
    f = lib().nvfp6x4_linear_bwd_workspace_size if grad_fmt == NVFP6 else lib().nvfp4_linear_bwd_workspace_size
    return torch.empty(int(f(M, N, K, n_outliers)), dtype=torch.uint8, device=device)


def bwd_operands(M: int, N: int, K: int, plan: OutlierPlan | None = None, device="cuda", grad_fmt: int = NVFP4) -> dict:
    """Buffers for the backward operands of one linear (tj2_bwd_operands): dYq, dYt (in grad_fmt), Wt, Xt
    (+ W8t, X8t)."""
    no = plan.n if plan else 0
    K1 = K - no
    ops = {"dYq": QTensor(grad_fmt, M, N, device), "dYt": QTensor(grad_fmt, N, M, device),
           "Wt": QTensor(NVFP4, K1, N, device), "Xt": QTensor(NVFP4, K1, M, device)}
    if plan:
        ops["W8t"] = QTensor(FP8, no, N, device)
        ops["X8t"] = QTensor(FP8, no, M, device)
    return ops


def linear_bwd(dY: torch.Tensor, saved: dict, K: int, *, seed: int, offset: int, rht: bool = True,
               plan: OutlierPlan | None = None, dx_dtype=torch.bfloat16, keep_operands: bool = False,
               operands: dict | None = None, w_given: bool = False, workspace: torch.Tensor | None = None,
               dX: torch.Tensor | None = None, dW: torch.Tensor | None = None, grad_fmt: int = NVFP4):
    """Returns (dX, dW, operands-or-None).  grad_fmt NVFP6: the FP6 x FP4 backward (nvfp6x4_linear_bwd),
    the two dY operands in NVFP6.

    operands: buffers from bwd_operands() to hold the backward operands (returned); keep_operands
    allocates them.  w_given: operands["Wt"] (and ["W8t"]) already hold this call's re-grouped
    weights (written by master_update_step's next-backward output) and are used as they are."""
    _dense(dY, "dY", _BF16)
    if dY.dim() != 2:
        raise ValueError("dY must be 2-D")
    M, N = dY.shape
    no = plan.n if plan else 0
    if dX is None:
        dX = torch.empty((M, K), dtype=dx_dtype, device=dY.device)
    if dW is None:
        dW = torch.empty((N, K), dtype=torch.float32, device=dY.device)
    _dense(dX, "dX", (torch.bfloat16, torch.float32), shape=(M, K))
    _dense(dW, "dW", _F32, shape=(N, K))
    _dense(workspace, "workspace", (torch.uint8,), optional=True)
    if w_given and operands is None:
        raise ValueError("w_given needs the operands holding Wt (and W8t)")
    if grad_fmt not in (NVFP4, NVFP6):
        raise ValueError("grad_fmt must be NVFP4 or NVFP6")
    ops = operands if operands is not None else (bwd_operands(M, N, K, plan, dY.device, grad_fmt) if keep_operands
                                                 else None)
    opsc = None
    if ops is not None:
        empty = _lib.QTensorC()
        opsc = _lib.BwdOperandsC(ops["dYq"].c(), ops["dYt"].c(), ops["Wt"].c(), ops["Xt"].c(),
                                 ops["W8t"].c() if plan else empty, ops["X8t"].c() if plan else empty,
                                 1 if w_given else 0, 0)
    if workspace is None:
        workspace = linear_bwd_workspace(M, N, K, no, dY.device, grad_fmt)
    pc = plan.c() if plan else None
    xqc, wqc = saved["Xq"].c(), saved["Wq"].c()
    x8c = saved["X8"].c() if saved.get("X8") is not None else None
    w8c = saved["W8"].c() if saved.get("W8") is not None else None
    fn = lib().nvfp6x4_linear_bwd if grad_fmt == NVFP6 else lib().nvfp4_linear_bwd
    st = fn(_ptr(dY), M, N, K, ctypes.byref(xqc), ctypes.byref(x8c) if x8c else None,
                                ctypes.byref(wqc), ctypes.byref(w8c) if w8c else None,
                                ctypes.byref(pc) if pc else None, 1 if rht else 0, seed, offset, _ptr(dX),
                                _dtype_code(dX), _ptr(dW), ctypes.byref(opsc) if opsc is not None else None,
                                _ptr(workspace), 0 if workspace is None else workspace.numel(), _stream())
    check("nvfp6x4_linear_bwd" if grad_fmt == NVFP6 else "nvfp4_linear_bwd", st)
    return dX, dW, ops


def _diag(flips: torch.Tensor | None, risk_hist: torch.Tensor | None):
    """Oscillation-diagnostic counters (device int64 / uint64; risk_hist holds RISK_BINS), or None."""
    if flips is None and risk_hist is None:
        return None
    for name, t, n in (("flips", flips, 1), ("risk_hist", risk_hist, RISK_BINS)):
        if t is not None and (not t.is_cuda or t.dtype not in (torch.int64, torch.uint64) or t.numel() < n
                              or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous device int64 tensor of at least {n} elements")
    return ctypes.byref(_lib.OsciDiagC(_ptr(flips), _ptr(risk_hist)))


def _qref(q):
    return ctypes.byref(q) if q is not None else None


def osci_reset_step(W, W_prev, Q_prev, dQ, dM, *, mode: int, tau: float = 4.0, reset_enabled: bool = False,
                    Wq_out: QTensor | None = None, reset_count: torch.Tensor | None = None,
                    flips: torch.Tensor | None = None, risk_hist: torch.Tensor | None = None,
                    plan: OutlierPlan | None = None, W8_out: QTensor | None = None) -> None:
    """OsciReset step; flips / risk_hist (optional device counters) receive the oscillation
    diagnostics: the number of elements whose quantized value changed, and at a window end the
    risk histogram (RISK_BINS bins, see include/tj2.h).  With an outlier plan, Q(w) quantizes the
    outlier channels to FP8 as the forward does; Wq_out is then [N, K - n] and W8_out [N, n]."""
    _dense(W, "W", _F32)
    N, K = W.shape
    for name, t in (("W_prev", W_prev), ("Q_prev", Q_prev), ("dQ", dQ), ("dM", dM)):
        _dense(t, name, _F32, shape=(N, K))
    _dense(reset_count, "reset_count", (torch.int64, torch.uint64), optional=True)
    wqc = Wq_out.c() if Wq_out is not None else None
    w8c = W8_out.c() if W8_out is not None else None
    pc = plan.c() if plan is not None else None
    st = lib().osci_reset_step(_ptr(W), _ptr(W_prev), _ptr(Q_prev), _ptr(dQ), _ptr(dM), N, K, mode,
                               ctypes.c_float(tau), 1 if reset_enabled else 0, _qref(pc), _qref(wqc), _qref(w8c),
                               _ptr(reset_count), _diag(flips, risk_hist), _stream())
    check("osci_reset_step", st)


class OsciBatch:
    """Descriptors of several OsciReset problems, built once: [(W, W_prev, Q_prev, dQ, dM, Wq_out or None
    [, plan, W8_out]), ...] (the tensors must stay alive and in place while the batch is used)."""

    def __init__(self, tensors):
        self.tensors = list(tensors)
        self._keep = []  # descriptors the array points to
        self.arr = (_lib.OsciTensorC * len(self.tensors))()
        for i, entry in enumerate(self.tensors):
            W, W_prev, Q_prev, dQ, dM, wq = entry[:6]
            plan, w8 = (entry[6], entry[7]) if len(entry) > 6 else (None, None)
            _dense(W, f"tensors[{i}].W", _F32)
            N, K = W.shape
            for name, t in (("W_prev", W_prev), ("Q_prev", Q_prev), ("dQ", dQ), ("dM", dM)):
                _dense(t, f"tensors[{i}].{name}", _F32, shape=(N, K))
            wqc = wq.c() if wq is not None else None
            w8c = w8.c() if w8 is not None else None
            pc = plan.c() if plan is not None else None
            self._keep += [wqc, w8c, pc]
            self.arr[i] = _lib.OsciTensorC(_ptr(W), _ptr(W_prev), _ptr(Q_prev), _ptr(dQ), _ptr(dM), N, K,
                                           ctypes.pointer(wqc) if wqc is not None else None,
                                           ctypes.pointer(pc) if pc is not None else None,
                                           ctypes.pointer(w8c) if w8c is not None else None)

    def __len__(self):
        return len(self.tensors)


def osci_reset_step_multi(tensors, *, mode: int, tau: float = 4.0, reset_enabled: bool = False,
                          reset_count: torch.Tensor | None = None, flips: torch.Tensor | None = None,
                          risk_hist: torch.Tensor | None = None) -> None:
    """osci_reset_step on several matrices at once (an OsciBatch, or the list it takes); the counters
    accumulate over all of them."""
    batch = tensors if isinstance(tensors, OsciBatch) else OsciBatch(tensors)
    st = lib().osci_reset_step_multi(batch.arr, len(batch), mode, ctypes.c_float(tau), 1 if reset_enabled else 0,
                                     _ptr(reset_count), _diag(flips, risk_hist), _stream())
    check("osci_reset_step_multi", st)


@dataclass
class NextBwd:
    """The next backward's re-grouped weight operands that a master pass forms (tj2_next_bwd):
    Wt [K1, N] NVFP4 and, with a plan, W8t [n, N] FP8, for nvfp4_linear_bwd at (seed, offset)."""
    Wt: QTensor
    W8t: QTensor | None
    seed: int
    offset: int
    rht: bool = True

    def c(self):
        self._wt = self.Wt.c()
        self._w8t = self.W8t.c() if self.W8t is not None else None
        return _lib.NextBwdC(ctypes.pointer(self._wt), ctypes.pointer(self._w8t) if self._w8t is not None else None,
                             self.seed, self.offset, 1 if self.rht else 0, 0)


def master_update_step(W, m, v, grad, Q_prev, dQ, dM, *, lr: float, bias_correction1: float,
                       bias_correction2: float, beta1: float = 0.9, beta2: float = 0.95, eps: float = 1e-8,
                       weight_decay: float = 0.1, mode: int = OSCI_ACCUM, tau: float = 4.0,
                       reset_enabled: bool = False, Wq_out: QTensor | None = None,
                       reset_count: torch.Tensor | None = None, flips: torch.Tensor | None = None,
                       risk_hist: torch.Tensor | None = None, plan: OutlierPlan | None = None,
                       W8_out: QTensor | None = None, next_bwd: NextBwd | None = None) -> None:
    """Fused master-weight pass: AdamW on W, then OsciReset (ACCUM / WINDOW_END) with the
    pre-update master as W_prev, then the forward codes (Wq_out, W8_out with a plan) and, with
    next_bwd, the next backward's re-grouped weights; diagnostics as osci_reset_step."""
    _dense(W, "W", _F32)
    N, K = W.shape
    for name, t in (("m", m), ("v", v), ("grad", grad), ("Q_prev", Q_prev), ("dQ", dQ), ("dM", dM)):
        _dense(t, name, _F32, shape=(N, K))
    _dense(reset_count, "reset_count", (torch.int64, torch.uint64), optional=True)
    ap = _lib.AdamWC(lr, beta1, beta2, eps, weight_decay, bias_correction1, bias_correction2)
    wqc = Wq_out.c() if Wq_out is not None else None
    w8c = W8_out.c() if W8_out is not None else None
    pc = plan.c() if plan is not None else None
    nx = next_bwd.c() if next_bwd is not None else None
    st = lib().master_update_step(_ptr(W), _ptr(m), _ptr(v), _ptr(grad), _ptr(Q_prev), _ptr(dQ), _ptr(dM), N, K,
                                  ctypes.byref(ap), mode, ctypes.c_float(tau), 1 if reset_enabled else 0, _qref(pc),
                                  _qref(wqc), _qref(w8c), _qref(nx), _ptr(reset_count), _diag(flips, risk_hist),
                                  _stream())
    check("master_update_step", st)


class MasterBatch:
    """Descriptors of several fused master-weight problems, built once:
    [(W, m, v, grad, Q_prev, dQ, dM, Wq_out or None [, plan, W8_out, NextBwd or None]), ...]
    (the tensors must stay alive and in place)."""

    def __init__(self, tensors):
        self.tensors = list(tensors)
        self._keep = []
        self.arr = (_lib.MasterTensorC * len(self.tensors))()
        for i, entry in enumerate(self.tensors):
            W, m, v, g, Q_prev, dQ, dM, wq = entry[:8]
            plan, w8, nxt = (entry[8], entry[9], entry[10]) if len(entry) > 8 else (None, None, None)
            _dense(W, f"tensors[{i}].W", _F32)
            N, K = W.shape
            for name, t in (("m", m), ("v", v), ("grad", g), ("Q_prev", Q_prev), ("dQ", dQ), ("dM", dM)):
                _dense(t, f"tensors[{i}].{name}", _F32, shape=(N, K))
            wqc = wq.c() if wq is not None else None
            w8c = w8.c() if w8 is not None else None
            pc = plan.c() if plan is not None else None
            nx = nxt.c() if nxt is not None else None
            self._keep += [wqc, w8c, pc, nx, nxt]
            self.arr[i] = _lib.MasterTensorC(_ptr(W), _ptr(m), _ptr(v), _ptr(g), _ptr(Q_prev), _ptr(dQ), _ptr(dM), N,
                                             K, ctypes.pointer(wqc) if wqc is not None else None,
                                             ctypes.pointer(pc) if pc is not None else None,
                                             ctypes.pointer(w8c) if w8c is not None else None,
                                             ctypes.pointer(nx) if nx is not None else None)

    def set_next_offsets(self, offsets):
        """Re-point the next-backward operands at new Philox offsets (one per matrix, in order)."""
        for i, off in enumerate(offsets):
            if self.arr[i].next:
                self.arr[i].next.contents.offset = off

    def __len__(self):
        return len(self.tensors)


def master_update_step_multi(tensors, *, lr: float, bias_correction1: float, bias_correction2: float,
                             beta1: float = 0.9, beta2: float = 0.95, eps: float = 1e-8, weight_decay: float = 0.1,
                             mode: int = OSCI_ACCUM, tau: float = 4.0, reset_enabled: bool = False,
                             reset_count: torch.Tensor | None = None, flips: torch.Tensor | None = None,
                             risk_hist: torch.Tensor | None = None) -> None:
    """master_update_step on several matrices at once (a MasterBatch, or the list it takes); the counters
    accumulate over all of them."""
    batch = tensors if isinstance(tensors, MasterBatch) else MasterBatch(tensors)
    ap = _lib.AdamWC(lr, beta1, beta2, eps, weight_decay, bias_correction1, bias_correction2)
    st = lib().master_update_step_multi(batch.arr, len(batch), ctypes.byref(ap), mode, ctypes.c_float(tau),
                                        1 if reset_enabled else 0, _ptr(reset_count), _diag(flips, risk_hist),
                                        _stream())
    check("master_update_step_multi", st)


def mfma_peak_probe(out: torch.Tensor, iters: int) -> float:
    """Measurement helper from libtj2_measure (not part of the path): an MFMA-only loop in
    out.numel() // 256 workgroups; returns the flops it performs (the caller times it on the
    current stream)."""
    wgs = out.numel() // 256
    if not out.is_cuda or out.dtype != torch.float32 or wgs < 1:
        raise ValueError("out must be a device float32 tensor of at least 256 elements")
    st = _lib.measure_lib().tj2_mfma_peak_probe(wgs, iters, _ptr(out), _stream())
    if st != 0:
        raise Tj2Error("tj2_mfma_peak_probe", st, "bad arguments or launch error")
    return float(wgs) * 4 * iters * 4 * 32768


def decode_probe(out: torch.Tensor, iters: int, packed_b: bool) -> float:
    """Measurement helper from libtj2_measure (not part of the path): the product's inner loop with B
    decoded once per workgroup into f16 LDS (packed_b False) or by every wave from packed LDS
    (packed_b True); out.numel() // 512 workgroups; returns the MFMA flops it performs."""
    wgs = out.numel() // 512
    if not out.is_cuda or out.dtype != torch.float32 or wgs < 1:
        raise ValueError("out must be a device float32 tensor of at least 512 elements")
    st = _lib.measure_lib().tj2_decode_probe(1 if packed_b else 0, wgs, iters, _ptr(out), _stream())
    if st != 0:
        raise Tj2Error("tj2_decode_probe", st, "bad arguments or launch error")
    return float(wgs) * 8 * iters * 32 * 32768


def stream_probe(src, dst) -> float:
    """Measurement helper from libtj2_measure (not part of the path): the OsciReset (5 reads, 4
    writes) or master-pass (7 reads, 6 writes) access pattern without arithmetic over equal-sized
    contiguous float32 device tensors; returns the bytes it moves."""
    n = src[0].numel()
    for t in list(src) + list(dst):
        if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != n:
            raise ValueError("stream_probe takes contiguous device float32 tensors of one size")
    sp = (ctypes.c_void_p * len(src))(*[t.data_ptr() for t in src])
    dp = (ctypes.c_void_p * len(dst))(*[t.data_ptr() for t in dst])
    st = _lib.measure_lib().tj2_stream_probe(sp, len(src), dp, len(dst), n, _stream())
    if st != 0:
        raise Tj2Error("tj2_stream_probe", st, "bad arguments or launch error")
    return 4.0 * (len(src) + len(dst)) * (n - n % 8)


def channel_sumsq(X: torch.Tensor, acc: torch.Tensor, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """acc[k] += sum_m X[m, k]^2 (fp64, fixed summation order); acc: device float64 [K]."""
    _dense(X, "X", _BF16)
    M, K = X.shape
    _dense(acc, "acc", (torch.float64,), shape=(K,))
    n = int(lib().tj2_channel_sumsq_workspace_size(M, K))
    if workspace is None:
        workspace = torch.empty(n, dtype=torch.uint8, device=X.device)
    _dense(workspace, "workspace", (torch.uint8,))
    check("tj2_channel_sumsq", lib().tj2_channel_sumsq(_ptr(X), M, K, _ptr(acc), _ptr(workspace), workspace.numel(),
                                                        _stream()))
    return acc


def select_outliers(scores, p: float, device="cuda") -> OutlierPlan:
    """Static outlier plan from host or device channel scores (fp64 [K]) by tj2_select_outliers:
    the ceil(p K / 16) * 16 largest scores, ties to the lower channel, both lists ascending."""
    sc = scores.detach().to("cpu", torch.float64).contiguous() if isinstance(scores, torch.Tensor) else \
        torch.as_tensor(scores, dtype=torch.float64).contiguous()
    K = int(sc.numel())
    outl = torch.empty(K, dtype=torch.int32)
    rest = torch.empty(K, dtype=torch.int32)
    n = ctypes.c_int32(0)
    check("tj2_select_outliers", lib().tj2_select_outliers(_ptr(sc), K, ctypes.c_double(p), _ptr(outl), _ptr(rest),
                                                            ctypes.byref(n)))
    n = n.value
    return OutlierPlan(outl[:n].to(device), rest[: K - n].contiguous().to(device))


def n_outliers(K: int, p: float) -> int:
    return int(math.ceil(p * K / 16.0)) * 16
