"""SmoothQuant W8A8 INT8 linear for AMD Instinct MI355X (gfx950).

A thin ctypes binding of libsqw8a8.so (C ABI in include/sq_w8a8.h).  Every
function here has the name of the C entry point it wraps and only marshals
arguments: tensors become device pointers, shapes and leading dimensions are
read off the tensors, and the current HIP stream is passed along.  All the
work runs in the library's gfx950 kernels; there is no fallback.  If the
library has not been built, every call raises.

PyTorch is used for device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libsqw8a8.so")

SQ_OK, SQ_ERR_NULL, SQ_ERR_SHAPE, SQ_ERR_DTYPE, SQ_ERR_ALPHA, SQ_ERR_UNSUPPORTED, \
    SQ_ERR_WORKSPACE, SQ_ERR_HIP = range(8)
SQ_F32, SQ_BF16, SQ_I8, SQ_I32 = range(4)
SQ_NORM_NONE, SQ_NORM_RMS = 0, 1
SQ_CALIB_ACCUMULATE = 1
SQ_CALIB_SKIP_ACT = 2

_lib = None


class SQError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


class _DebugOut(ctypes.Structure):
    _fields_ = [("xq", ctypes.c_void_p), ("x_scale", ctypes.c_void_p),
                ("row_rscale", ctypes.c_void_p), ("acc", ctypes.c_void_p)]


def lib() -> ctypes.CDLL:
    """The loaded libsqw8a8.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m w8a8_int8_gemm_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, F, U, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_uint, ctypes.c_int
        L.sq_calibrate.argtypes = [P, I, I64, I64, I64, I, P, F, P, I, I64, I64, F, U, P, P, P, P]
        L.sq_smooth_fold.argtypes = [P, I64, P, P, P, I, I64, I64, P, P]
        L.sq_quant_weight.argtypes = [P, I, I64, I64, I64, P, P, P, P]
        L.sq_quant_act.argtypes = [P, I, I64, I64, I64, I, P, F, P, P, P, P]
        L.sq_gemm_w8a8.argtypes = [P, P, I64, I64, P, P, I64, P, P, I, I64, P, P]
        L.sq_linear_workspace_bytes.argtypes = [I64, I64]
        L.sq_linear_workspace_bytes.restype = ctypes.c_size_t
        L.sq_w8a8_linear.argtypes = [P, I, I64, I64, I64, I, P, F, P, P, I64, P, P, I, I64, P,
                                     ctypes.c_size_t, ctypes.POINTER(_DebugOut), P]
        L.sq_w8a8_linear_noalloc.argtypes = [P, I, I64, I64, I64, I, P, F, P, P, I64, P, P, I,
                                             I64, ctypes.POINTER(_DebugOut), P]
        L.sq_act_static_scale.argtypes = [P, P, I64, P, P]
        L.sq_quant_act_static.argtypes = [P, I, I64, I64, I64, I, P, F, P, P, P, P, P]
        L.sq_w8a8_linear_static.argtypes = [P, I, I64, I64, I64, I, P, F, P, P, P, I64, P, P, I,
                                            I64, P, ctypes.c_size_t, ctypes.POINTER(_DebugOut), P]
        L.sq_quant_weight_fp8.argtypes = [P, I, I64, I64, I64, P, P, P, P]
        L.sq_quant_act_fp8.argtypes = [P, I, I64, I64, I64, I, P, F, P, P, P, P]
        L.sq_gemm_fp8.argtypes = [P, P, I64, I64, P, P, I64, P, P, I, I64, P, P]
        L.sq_w8a8_linear_fp8.argtypes = [P, I, I64, I64, I64, I, P, F, P, P, I64, P, P, I, I64,
                                         P, ctypes.c_size_t, ctypes.POINTER(_DebugOut), P]
        L.sq_act_static_scale_fp8.argtypes = [P, P, I64, P, P]
        L.sq_quant_act_static_fp8.argtypes = [P, I, I64, I64, I64, I, P, F, P, P, P, P, P]
        L.sq_w8a8_linear_static_fp8.argtypes = [P, I, I64, I64, I64, I, P, F, P, P, P, I64, P, P,
                                                I, I64, P, ctypes.c_size_t,
                                                ctypes.POINTER(_DebugOut), P]
        L.sq_calibrate_ln.argtypes = [P, I, I64, I64, I64, P, P, F, P, I, I64, I64, F,
                                      ctypes.c_uint, P, P, P, P]
        L.sq_smooth_fold_ln.argtypes = [P, I64, P, P, P, P, P]
        L.sq_quant_act_ln.argtypes = [P, I, I64, I64, I64, P, P, F, P, P, P, P, P]
        L.sq_w8a8_linear_ln.argtypes = [P, I, I64, I64, I64, P, P, F, P, P, I64, P, P, I, I64, P,
                                        ctypes.c_size_t, ctypes.POINTER(_DebugOut), P, P]
        L.sq_fold_prev_linear.argtypes = [P, I64, P, I, I64, I64, P, I64, P, P, P]
        L.sq_gptq_workspace_bytes.argtypes = [I64, I64, I64]
        L.sq_gptq_workspace_bytes.restype = ctypes.c_size_t
        L.sq_quant_weight_gptq.argtypes = [P, I, I64, I64, I, P, F, P, I, I64, I64, I64, P, F, P,
                                           P, P, P, ctypes.c_size_t, P]
        L.sq_status_string.argtypes = [I]
        L.sq_status_string.restype = ctypes.c_char_p
        L.sq_abi_version.restype = I
        for name in ("sq_calibrate", "sq_smooth_fold", "sq_quant_weight", "sq_quant_act",
                     "sq_gemm_w8a8", "sq_w8a8_linear", "sq_w8a8_linear_noalloc"):
            getattr(L, name).restype = I
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().sq_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != SQ_OK:
        raise SQError(status, where)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dtype(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return SQ_F32
    if t.dtype == torch.bfloat16:
        return SQ_BF16
    if t.dtype == torch.int8:
        return SQ_I8
    if t.dtype == torch.int32:
        return SQ_I32
    return -1


def _ld(t) -> int:
    """Leading dimension of a row-major 2-D tensor (unit inner stride required)."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError("expected a 2-D row-major tensor with unit inner stride")
    return t.stride(0)


# --- argument checks -----------------------------------------------------------
# The C side sees only pointers and sizes, so it cannot tell a host pointer or
# an undersized buffer from a good one; both would fault the GPU.  Every
# wrapper therefore checks, before the C call, that each tensor is on the GPU
# with the dtype the entry point takes and holds what the sizes read off the
# inputs (T, K, N) imply.

_FP = ("float32", "bfloat16")


def _dt(t) -> str:
    return str(t.dtype).replace("torch.", "")


def _need(t, name: str, dtypes, n: Optional[int] = None, *, required: bool = False) -> None:
    """t is None (unless required), or a GPU tensor of one of `dtypes`; with
    n given, also contiguous and holding at least n elements."""
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a tensor on the GPU")
    if _dt(t) not in dtypes:
        raise ValueError(f"{name} must be {' or '.join(dtypes)}, not {_dt(t)}")
    if n is not None:
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.numel() < n:
            raise ValueError(f"{name} holds {t.numel()} elements, {n} needed")


def _mat(t, name: str, dtypes, rows: Optional[int] = None, cols: Optional[int] = None):
    """A 2-D row-major GPU tensor (unit inner stride) of one of `dtypes` whose
    shape matches rows / cols where given; returns (rows, cols, ld)."""
    _need(t, name, dtypes, required=True)
    ld = _ld(t)
    r, c = t.shape
    if (rows is not None and r != rows) or (cols is not None and c != cols):
        want = f"[{'*' if rows is None else rows}, {'*' if cols is None else cols}]"
        raise ValueError(f"{name} is {list(t.shape)}, expected {want}")
    return r, c, ld


def _workspace_bytes(workspace) -> int:
    _need(workspace, "workspace", ("uint8", "int8"), 0)
    return 0 if workspace is None else workspace.numel() * workspace.element_size()


def _dbg(T: int, K: int, N: int, codes, dbg_xq, dbg_x_scale, dbg_row_rscale, dbg_acc, acc_dt):
    _need(dbg_xq, "dbg_xq", codes, T * K)
    _need(dbg_x_scale, "dbg_x_scale", ("float32",), T)
    _need(dbg_row_rscale, "dbg_row_rscale", ("float32",), T)
    _need(dbg_acc, "dbg_acc", acc_dt, T * N)
    if all(v is None for v in (dbg_xq, dbg_x_scale, dbg_row_rscale, dbg_acc)):
        return None
    return ctypes.byref(_DebugOut(_ptr(dbg_xq), _ptr(dbg_x_scale), _ptr(dbg_row_rscale),
                                  _ptr(dbg_acc)))


def _out(y, T: int, N: int, acc_out):
    """(dtype, ld) of the GEMM output y [T, N] (may be None when acc_out is given)."""
    if y is None:
        if acc_out is None:
            raise ValueError("y is required unless acc_out is given")
        return SQ_BF16, N
    _mat(y, "y", _FP, T, N)
    return _dtype(y), _ld(y)


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


# ---------------------------------------------------------------------------
# the C entry points
# ---------------------------------------------------------------------------

def sq_calibrate(x_cal, w, alpha: float, a, wmax=None, s=None, *, norm: bool = False, gamma=None,
                 eps: float = 1e-6, accumulate: bool = False, stream=None) -> None:
    """a[K] (running) activation absmax, wmax[K], s[K] -- see sq_calibrate in sq_w8a8.h.
    x_cal None: a[] is used as given (e.g. an alpha sweep over one calibration)."""
    _need(a, "a", ("float32",), required=True)
    K = a.shape[0]
    _need(a, "a", ("float32",), K)
    xt, xdt, xld = 0, SQ_BF16, K
    if x_cal is not None:
        xt, _, xld = _mat(x_cal, "x_cal", _FP, cols=K)
        xdt = _dtype(x_cal)
    N, wdt, wld = 0, SQ_BF16, 0
    if w is not None:
        _, N, wld = _mat(w, "w", _FP, rows=K)
        wdt = _dtype(w)
        _need(wmax, "wmax", ("float32",), K, required=True)
        _need(s, "s", ("float32",), K, required=True)
    _need(gamma, "gamma", ("float32",), K)
    flags = SQ_CALIB_ACCUMULATE if accumulate else 0
    if x_cal is None:
        flags |= SQ_CALIB_SKIP_ACT
    _check(lib().sq_calibrate(_ptr(x_cal), xdt, xt, K, xld, SQ_NORM_RMS if norm else SQ_NORM_NONE,
                              _ptr(gamma), eps, _ptr(w), wdt, N, wld, alpha, flags, _ptr(a),
                              _ptr(wmax), _ptr(s), _stream(stream)), "sq_calibrate")


def sq_smooth_fold(s, gamma=None, gamma_out=None, w=None, w_out=None, *, stream=None) -> None:
    """gamma_out = gamma / s, w_out = diag(s) W -- see sq_smooth_fold."""
    _need(s, "s", ("float32",), required=True)
    K = s.shape[0]
    _need(s, "s", ("float32",), K)
    _need(gamma, "gamma", ("float32",), K)
    _need(gamma_out, "gamma_out", ("float32",), K)
    N, wdt, wld = 0, SQ_BF16, 0
    if w is not None:
        _, N, wld = _mat(w, "w", _FP, rows=K)
        wdt = _dtype(w)
        _need(w_out, "w_out", ("float32",), K * N)
    _check(lib().sq_smooth_fold(_ptr(s), K, _ptr(gamma), _ptr(gamma_out), _ptr(w), wdt, N, wld,
                                _ptr(w_out), _stream(stream)), "sq_smooth_fold")


def sq_quant_weight(w, s, wq, w_scale, *, stream=None) -> None:
    """wq[N, K] int8 and w_scale[N] of diag(s) W (s may be None) -- see sq_quant_weight."""
    K, N, ld = _mat(w, "w", _FP)
    _need(s, "s", ("float32",), K)
    _need(wq, "wq", ("int8",), N * K, required=True)
    _need(w_scale, "w_scale", ("float32",), N, required=True)
    _check(lib().sq_quant_weight(_ptr(w), _dtype(w), K, N, ld, _ptr(s), _ptr(wq),
                                 _ptr(w_scale), _stream(stream)), "sq_quant_weight")


def sq_quant_act(x, gamma_f, xq, x_scale, *, norm: bool = False, eps: float = 1e-6,
                 row_rscale=None, stream=None) -> None:
    """xq[T, K] int8 and x_scale[T] of norm?(x) * gamma_f -- see sq_quant_act."""
    T, K, ld = _mat(x, "x", _FP)
    _need(gamma_f, "gamma_f", ("float32",), K)
    _need(xq, "xq", ("int8",), T * K, required=True)
    _need(x_scale, "x_scale", ("float32",), T, required=True)
    _need(row_rscale, "row_rscale", ("float32",), T)
    _check(lib().sq_quant_act(_ptr(x), _dtype(x), T, K, ld,
                              SQ_NORM_RMS if norm else SQ_NORM_NONE, _ptr(gamma_f), eps, _ptr(xq),
                              _ptr(x_scale), _ptr(row_rscale), _stream(stream)), "sq_quant_act")


def sq_gemm_w8a8(xq, x_scale, wq, w_scale, y=None, *, bias=None, acc_out=None, stream=None) -> None:
    """y = dequant(xq @ wq^T) + bias, or the int32 accumulators -- see sq_gemm_w8a8."""
    T, K, _ = _mat(xq, "xq", ("int8",))
    N, _, _ = _mat(wq, "wq", ("int8",), cols=K)
    _need(xq, "xq", ("int8",), T * K)
    _need(wq, "wq", ("int8",), N * K)
    _need(acc_out, "acc_out", ("int32",), T * N)
    _need(x_scale, "x_scale", ("float32",), T, required=acc_out is None)
    _need(w_scale, "w_scale", ("float32",), N, required=acc_out is None)
    _need(bias, "bias", ("float32",), N)
    ydt, yld = _out(y, T, N, acc_out)
    _check(lib().sq_gemm_w8a8(_ptr(xq), _ptr(x_scale), T, K, _ptr(wq), _ptr(w_scale), N,
                              _ptr(bias), _ptr(y), ydt, yld, _ptr(acc_out), _stream(stream)),
           "sq_gemm_w8a8")


def sq_linear_workspace_bytes(t: int, k: int) -> int:
    return int(lib().sq_linear_workspace_bytes(t, k))


def sq_w8a8_linear(x, gamma_f, wq, w_scale, y, workspace, *, norm: bool = False,
                   eps: float = 1e-6, bias=None, dbg_xq=None, dbg_x_scale=None,
                   dbg_row_rscale=None, dbg_acc=None, stream=None) -> None:
    """The online forward: sq_quant_act then sq_gemm_w8a8 -- see sq_w8a8_linear."""
    T, K, ld = _mat(x, "x", _FP)
    N, _, _ = _mat(wq, "wq", ("int8",), cols=K)
    _need(wq, "wq", ("int8",), N * K)
    _need(gamma_f, "gamma_f", ("float32",), K)
    _need(w_scale, "w_scale", ("float32",), N, required=dbg_acc is None)
    _need(bias, "bias", ("float32",), N)
    dbg = _dbg(T, K, N, ("int8",), dbg_xq, dbg_x_scale, dbg_row_rscale, dbg_acc, ("int32",))
    ydt, yld = _out(y, T, N, dbg_acc)
    ws_bytes = _workspace_bytes(workspace)
    _check(lib().sq_w8a8_linear(_ptr(x), _dtype(x), T, K, ld,
                                SQ_NORM_RMS if norm else SQ_NORM_NONE, _ptr(gamma_f), eps,
                                _ptr(wq), _ptr(w_scale), N, _ptr(bias), _ptr(y), ydt, yld,
                                _ptr(workspace), ws_bytes, dbg, _stream(stream)),
           "sq_w8a8_linear")


def sq_w8a8_linear_noalloc(x, gamma_f, wq, w_scale, y, *, norm: bool = False,
                           eps: float = 1e-6, bias=None, dbg_xq=None, dbg_x_scale=None,
                           dbg_row_rscale=None, dbg_acc=None, stream=None) -> None:
    """sq_w8a8_linear with the library's per-device scratch array in place of a
    workspace: no allocation (SQ_NOALLOC_SCRATCH_BYTES) -- see sq_w8a8_linear_noalloc."""
    T, K, ld = _mat(x, "x", _FP)
    N, _, _ = _mat(wq, "wq", ("int8",), cols=K)
    _need(wq, "wq", ("int8",), N * K)
    _need(gamma_f, "gamma_f", ("float32",), K)
    _need(w_scale, "w_scale", ("float32",), N, required=dbg_acc is None)
    _need(bias, "bias", ("float32",), N)
    dbg = _dbg(T, K, N, ("int8",), dbg_xq, dbg_x_scale, dbg_row_rscale, dbg_acc, ("int32",))
    ydt, yld = _out(y, T, N, dbg_acc)
    _check(lib().sq_w8a8_linear_noalloc(_ptr(x), _dtype(x), T, K, ld,
                                        SQ_NORM_RMS if norm else SQ_NORM_NONE, _ptr(gamma_f), eps,
                                        _ptr(wq), _ptr(w_scale), N, _ptr(bias), _ptr(y), ydt, yld,
                                        dbg, _stream(stream)),
           "sq_w8a8_linear_noalloc")


def sq_act_static_scale(a, gamma_f, x_scale_static, *, stream=None) -> None:
    """x_scale_static[0] = max_j(a[j] * |gamma_f[j]|) / 127 -- see sq_act_static_scale."""
    _need(a, "a", ("float32",), required=True)
    K = a.shape[0]
    _need(a, "a", ("float32",), K)
    _need(gamma_f, "gamma_f", ("float32",), K)
    _need(x_scale_static, "x_scale_static", ("float32",), 1, required=True)
    _check(lib().sq_act_static_scale(_ptr(a), _ptr(gamma_f), K, _ptr(x_scale_static),
                                     _stream(stream)), "sq_act_static_scale")


def sq_quant_act_static(x, gamma_f, x_scale_static, xq, x_scale, *, norm: bool = False,
                        eps: float = 1e-6, row_rscale=None, stream=None) -> None:
    """xq[T, K] int8 with one fixed step for every token -- see sq_quant_act_static."""
    T, K, ld = _mat(x, "x", _FP)
    _need(gamma_f, "gamma_f", ("float32",), K)
    _need(x_scale_static, "x_scale_static", ("float32",), 1, required=True)
    _need(xq, "xq", ("int8",), T * K, required=True)
    _need(x_scale, "x_scale", ("float32",), T, required=True)
    _need(row_rscale, "row_rscale", ("float32",), T)
    _check(lib().sq_quant_act_static(_ptr(x), _dtype(x), T, K, ld,
                                     SQ_NORM_RMS if norm else SQ_NORM_NONE, _ptr(gamma_f), eps,
                                     _ptr(x_scale_static), _ptr(xq), _ptr(x_scale),
                                     _ptr(row_rscale), _stream(stream)), "sq_quant_act_static")


def sq_w8a8_linear_static(x, gamma_f, x_scale_static, wq, w_scale, y, workspace, *,
                          norm: bool = False, eps: float = 1e-6, bias=None, dbg_xq=None,
                          dbg_x_scale=None, dbg_row_rscale=None, dbg_acc=None,
                          stream=None) -> None:
    """sq_w8a8_linear with the static step -- see sq_w8a8_linear_static."""
    T, K, ld = _mat(x, "x", _FP)
    N, _, _ = _mat(wq, "wq", ("int8",), cols=K)
    _need(wq, "wq", ("int8",), N * K)
    _need(gamma_f, "gamma_f", ("float32",), K)
    _need(x_scale_static, "x_scale_static", ("float32",), 1, required=True)
    _need(w_scale, "w_scale", ("float32",), N, required=dbg_acc is None)
    _need(bias, "bias", ("float32",), N)
    dbg = _dbg(T, K, N, ("int8",), dbg_xq, dbg_x_scale, dbg_row_rscale, dbg_acc, ("int32",))
    ydt, yld = _out(y, T, N, dbg_acc)
    ws_bytes = _workspace_bytes(workspace)
    _check(lib().sq_w8a8_linear_static(_ptr(x), _dtype(x), T, K, ld,
                                       SQ_NORM_RMS if norm else SQ_NORM_NONE, _ptr(gamma_f), eps,
                                       _ptr(x_scale_static), _ptr(wq), _ptr(w_scale), N,
                                       _ptr(bias), _ptr(y), ydt, yld, _ptr(workspace), ws_bytes,
                                       dbg, _stream(stream)),
           "sq_w8a8_linear_static")


def sq_quant_weight_fp8(w, s, wq, w_scale, *, stream=None) -> None:
    """wq[N, K] E4M3 bytes (uint8) and w_scale[N] of diag(s) W -- see sq_quant_weight_fp8."""
    K, N, ld = _mat(w, "w", _FP)
    _need(s, "s", ("float32",), K)
    _need(wq, "wq", ("uint8",), N * K, required=True)
    _need(w_scale, "w_scale", ("float32",), N, required=True)
    _check(lib().sq_quant_weight_fp8(_ptr(w), _dtype(w), K, N, ld, _ptr(s), _ptr(wq),
                                     _ptr(w_scale), _stream(stream)), "sq_quant_weight_fp8")


def sq_quant_act_fp8(x, gamma_f, xq, x_scale, *, norm: bool = False, eps: float = 1e-6,
                     row_rscale=None, stream=None) -> None:
    """xq[T, K] E4M3 bytes and x_scale[T] -- see sq_quant_act_fp8."""
    T, K, ld = _mat(x, "x", _FP)
    _need(gamma_f, "gamma_f", ("float32",), K)
    _need(xq, "xq", ("uint8",), T * K, required=True)
    _need(x_scale, "x_scale", ("float32",), T, required=True)
    _need(row_rscale, "row_rscale", ("float32",), T)
    _check(lib().sq_quant_act_fp8(_ptr(x), _dtype(x), T, K, ld,
                                  SQ_NORM_RMS if norm else SQ_NORM_NONE, _ptr(gamma_f), eps,
                                  _ptr(xq), _ptr(x_scale), _ptr(row_rscale), _stream(stream)),
           "sq_quant_act_fp8")


def sq_gemm_fp8(xq, x_scale, wq, w_scale, y=None, *, bias=None, acc_out=None, stream=None) -> None:
    """y = dequant(E4M3 product) + bias, or the fp32 accumulators -- see sq_gemm_fp8."""
    T, K, _ = _mat(xq, "xq", ("uint8",))
    N, _, _ = _mat(wq, "wq", ("uint8",), cols=K)
    _need(xq, "xq", ("uint8",), T * K)
    _need(wq, "wq", ("uint8",), N * K)
    _need(acc_out, "acc_out", ("float32",), T * N)
    _need(x_scale, "x_scale", ("float32",), T, required=acc_out is None)
    _need(w_scale, "w_scale", ("float32",), N, required=acc_out is None)
    _need(bias, "bias", ("float32",), N)
    ydt, yld = _out(y, T, N, acc_out)
    _check(lib().sq_gemm_fp8(_ptr(xq), _ptr(x_scale), T, K, _ptr(wq), _ptr(w_scale), N,
                             _ptr(bias), _ptr(y), ydt, yld, _ptr(acc_out), _stream(stream)),
           "sq_gemm_fp8")


def sq_w8a8_linear_fp8(x, gamma_f, wq, w_scale, y, workspace, *, norm: bool = False,
                       eps: float = 1e-6, bias=None, dbg_xq=None, dbg_x_scale=None,
                       dbg_row_rscale=None, dbg_acc=None, stream=None) -> None:
    """sq_quant_act_fp8 then sq_gemm_fp8 -- see sq_w8a8_linear_fp8."""
    T, K, ld = _mat(x, "x", _FP)
    N, _, _ = _mat(wq, "wq", ("uint8",), cols=K)
    _need(wq, "wq", ("uint8",), N * K)
    _need(gamma_f, "gamma_f", ("float32",), K)
    _need(w_scale, "w_scale", ("float32",), N, required=dbg_acc is None)
    _need(bias, "bias", ("float32",), N)
    dbg = _dbg(T, K, N, ("uint8",), dbg_xq, dbg_x_scale, dbg_row_rscale, dbg_acc,
               ("float32", "int32"))
    ydt, yld = _out(y, T, N, dbg_acc)
    ws_bytes = _workspace_bytes(workspace)
    _check(lib().sq_w8a8_linear_fp8(_ptr(x), _dtype(x), T, K, ld,
                                    SQ_NORM_RMS if norm else SQ_NORM_NONE, _ptr(gamma_f), eps,
                                    _ptr(wq), _ptr(w_scale), N, _ptr(bias), _ptr(y), ydt, yld,
                                    _ptr(workspace), ws_bytes, dbg, _stream(stream)),
           "sq_w8a8_linear_fp8")


def sq_abi_version() -> int:
    return int(lib().sq_abi_version())


def sq_act_static_scale_fp8(a, gamma_f, x_scale_static, *, stream=None) -> None:
    """x_scale_static[0] = max_j(a[j] * |gamma_f[j]|) / 448 -- see sq_act_static_scale_fp8."""
    _need(a, "a", ("float32",), required=True)
    K = a.shape[0]
    _need(a, "a", ("float32",), K)
    _need(gamma_f, "gamma_f", ("float32",), K)
    _need(x_scale_static, "x_scale_static", ("float32",), 1, required=True)
    _check(lib().sq_act_static_scale_fp8(_ptr(a), _ptr(gamma_f), K, _ptr(x_scale_static),
                                         _stream(stream)), "sq_act_static_scale_fp8")


def sq_quant_act_static_fp8(x, gamma_f, x_scale_static, xq, x_scale, *, norm: bool = False,
                            eps: float = 1e-6, row_rscale=None, stream=None) -> None:
    """xq[T, K] E4M3 bytes with one fixed step for every token -- see sq_quant_act_static_fp8."""
    T, K, ld = _mat(x, "x", _FP)
    _need(gamma_f, "gamma_f", ("float32",), K)
    _need(x_scale_static, "x_scale_static", ("float32",), 1, required=True)
    _need(xq, "xq", ("uint8",), T * K, required=True)
    _need(x_scale, "x_scale", ("float32",), T, required=True)
    _need(row_rscale, "row_rscale", ("float32",), T)
    _check(lib().sq_quant_act_static_fp8(_ptr(x), _dtype(x), T, K, ld,
                                         SQ_NORM_RMS if norm else SQ_NORM_NONE, _ptr(gamma_f),
                                         eps, _ptr(x_scale_static), _ptr(xq), _ptr(x_scale),
                                         _ptr(row_rscale), _stream(stream)),
           "sq_quant_act_static_fp8")


def sq_w8a8_linear_static_fp8(x, gamma_f, x_scale_static, wq, w_scale, y, workspace, *,
                              norm: bool = False, eps: float = 1e-6, bias=None, dbg_xq=None,
                              dbg_x_scale=None, dbg_row_rscale=None, dbg_acc=None,
                              stream=None) -> None:
    """sq_w8a8_linear_fp8 with the static step -- see sq_w8a8_linear_static_fp8."""
    T, K, ld = _mat(x, "x", _FP)
    N, _, _ = _mat(wq, "wq", ("uint8",), cols=K)
    _need(wq, "wq", ("uint8",), N * K)
    _need(gamma_f, "gamma_f", ("float32",), K)
    _need(x_scale_static, "x_scale_static", ("float32",), 1, required=True)
    _need(w_scale, "w_scale", ("float32",), N, required=dbg_acc is None)
    _need(bias, "bias", ("float32",), N)
    dbg = _dbg(T, K, N, ("uint8",), dbg_xq, dbg_x_scale, dbg_row_rscale, dbg_acc,
               ("float32", "int32"))
    ydt, yld = _out(y, T, N, dbg_acc)
    ws_bytes = _workspace_bytes(workspace)
    _check(lib().sq_w8a8_linear_static_fp8(_ptr(x), _dtype(x), T, K, ld,
                                           SQ_NORM_RMS if norm else SQ_NORM_NONE, _ptr(gamma_f),
                                           eps, _ptr(x_scale_static), _ptr(wq), _ptr(w_scale), N,
                                           _ptr(bias), _ptr(y), ydt, yld, _ptr(workspace),
                                           ws_bytes, dbg, _stream(stream)),
           "sq_w8a8_linear_static_fp8")


# --- LayerNorm form and the fold into the previous linear ---------------------

def sq_calibrate_ln(x_cal, w, alpha: float, a, wmax=None, s=None, *, gamma=None, beta=None,
                    eps: float = 1e-6, accumulate: bool = False, stream=None) -> None:
    """a[K] absmax of LN(x_cal) (x_cal None: a used as given), wmax[K], s[K] --
    see sq_calibrate_ln."""
    _need(a, "a", ("float32",), required=True)
    K = a.shape[0]
    _need(a, "a", ("float32",), K)
    xt, xdt, xld = 0, SQ_BF16, K
    if x_cal is not None:
        xt, _, xld = _mat(x_cal, "x_cal", _FP, cols=K)
        xdt = _dtype(x_cal)
    N, wdt, wld = 0, SQ_BF16, 0
    if w is not None:
        _, N, wld = _mat(w, "w", _FP, rows=K)
        wdt = _dtype(w)
        _need(wmax, "wmax", ("float32",), K, required=True)
        _need(s, "s", ("float32",), K, required=True)
    _need(gamma, "gamma", ("float32",), K)
    _need(beta, "beta", ("float32",), K)
    flags = SQ_CALIB_ACCUMULATE if accumulate else 0
    if x_cal is None:
        flags |= SQ_CALIB_SKIP_ACT
    _check(lib().sq_calibrate_ln(_ptr(x_cal), xdt, xt, K, xld, _ptr(gamma), _ptr(beta), eps,
                                 _ptr(w), wdt, N, wld, alpha, flags, _ptr(a), _ptr(wmax), _ptr(s),
                                 _stream(stream)), "sq_calibrate_ln")


def sq_smooth_fold_ln(s, gamma, beta, gamma_out, beta_out, *, stream=None) -> None:
    """gamma_out = gamma / s, beta_out = beta / s -- see sq_smooth_fold_ln."""
    _need(s, "s", ("float32",), required=True)
    K = s.shape[0]
    _need(s, "s", ("float32",), K)
    _need(gamma, "gamma", ("float32",), K)
    _need(beta, "beta", ("float32",), K)
    _need(gamma_out, "gamma_out", ("float32",), K, required=True)
    _need(beta_out, "beta_out", ("float32",), K, required=True)
    _check(lib().sq_smooth_fold_ln(_ptr(s), K, _ptr(gamma), _ptr(beta), _ptr(gamma_out),
                                   _ptr(beta_out), _stream(stream)), "sq_smooth_fold_ln")


def sq_quant_act_ln(x, gamma_f, beta_f, xq, x_scale, *, eps: float = 1e-6, row_mean=None,
                    row_rscale=None, stream=None) -> None:
    """Per-token INT8 of the smoothed LayerNorm output -- see sq_quant_act_ln."""
    T, K, ld = _mat(x, "x", _FP)
    _need(gamma_f, "gamma_f", ("float32",), K, required=True)
    _need(beta_f, "beta_f", ("float32",), K, required=True)
    _need(xq, "xq", ("int8",), T * K, required=True)
    _need(x_scale, "x_scale", ("float32",), T, required=True)
    _need(row_mean, "row_mean", ("float32",), T)
    _need(row_rscale, "row_rscale", ("float32",), T)
    _check(lib().sq_quant_act_ln(_ptr(x), _dtype(x), T, K, ld, _ptr(gamma_f), _ptr(beta_f),
                                 eps, _ptr(xq), _ptr(x_scale), _ptr(row_mean), _ptr(row_rscale),
                                 _stream(stream)), "sq_quant_act_ln")


def sq_w8a8_linear_ln(x, gamma_f, beta_f, wq, w_scale, y, workspace, *, eps: float = 1e-6,
                      bias=None, dbg_xq=None, dbg_x_scale=None, dbg_row_rscale=None,
                      dbg_acc=None, row_mean=None, stream=None) -> None:
    """sq_quant_act_ln then sq_gemm_w8a8 -- see sq_w8a8_linear_ln."""
    T, K, ld = _mat(x, "x", _FP)
    N, _, _ = _mat(wq, "wq", ("int8",), cols=K)
    _need(wq, "wq", ("int8",), N * K)
    _need(gamma_f, "gamma_f", ("float32",), K, required=True)
    _need(beta_f, "beta_f", ("float32",), K, required=True)
    _need(w_scale, "w_scale", ("float32",), N, required=dbg_acc is None)
    _need(bias, "bias", ("float32",), N)
    _need(row_mean, "row_mean", ("float32",), T)
    dbg = _dbg(T, K, N, ("int8",), dbg_xq, dbg_x_scale, dbg_row_rscale, dbg_acc, ("int32",))
    ydt, yld = _out(y, T, N, dbg_acc)
    ws_bytes = _workspace_bytes(workspace)
    _check(lib().sq_w8a8_linear_ln(_ptr(x), _dtype(x), T, K, ld, _ptr(gamma_f), _ptr(beta_f),
                                   eps, _ptr(wq), _ptr(w_scale), N, _ptr(bias), _ptr(y), ydt, yld,
                                   _ptr(workspace), ws_bytes, dbg, _ptr(row_mean),
                                   _stream(stream)), "sq_w8a8_linear_ln")


def sq_fold_prev_linear(s, w_prev, w_out, *, bias=None, bias_out=None, stream=None) -> None:
    """w_out = W_prev with column j divided by s_j (fp32), bias_out = bias / s --
    see sq_fold_prev_linear."""
    Kp, K, ld = _mat(w_prev, "w_prev", _FP)
    _need(s, "s", ("float32",), K, required=True)
    _, _, ldo = _mat(w_out, "w_out", ("float32",), Kp, K)
    _need(bias, "bias", ("float32",), K)
    _need(bias_out, "bias_out", ("float32",), K, required=bias is not None)
    _check(lib().sq_fold_prev_linear(_ptr(s), K, _ptr(w_prev), _dtype(w_prev), Kp, ld,
                                     _ptr(w_out), ldo, _ptr(bias), _ptr(bias_out),
                                     _stream(stream)), "sq_fold_prev_linear")


# --- GPTQ on the migrated weight ------------------------------------------------

def sq_gptq_workspace_bytes(t_cal: int, k: int, n: int) -> int:
    return int(lib().sq_gptq_workspace_bytes(t_cal, k, n))


def sq_quant_weight_gptq(x_cal, gamma_f, w, s, wq, w_scale, workspace, *, norm: bool = False,
                         eps: float = 1e-6, damp: float = 0.01, row_rscale=None,
                         stream=None) -> None:
    """wq[N, K] int8 by GPTQ rounding of diag(s) W with the Hessian of the
    calibration x^, w_scale[N] -- see sq_quant_weight_gptq."""
    T, K, xld = _mat(x_cal, "x_cal", _FP)
    _, N, wld = _mat(w, "w", _FP, rows=K)
    _need(gamma_f, "gamma_f", ("float32",), K)
    _need(s, "s", ("float32",), K)
    _need(wq, "wq", ("int8",), N * K, required=True)
    _need(w_scale, "w_scale", ("float32",), N, required=True)
    _need(row_rscale, "row_rscale", ("float32",), T)
    ws_bytes = _workspace_bytes(workspace)
    _check(lib().sq_quant_weight_gptq(_ptr(x_cal), _dtype(x_cal), T, xld,
                                      SQ_NORM_RMS if norm else SQ_NORM_NONE, _ptr(gamma_f), eps,
                                      _ptr(w), _dtype(w), K, N, wld, _ptr(s), damp, _ptr(wq),
                                      _ptr(w_scale), _ptr(row_rscale), _ptr(workspace), ws_bytes,
                                      _stream(stream)), "sq_quant_weight_gptq")
