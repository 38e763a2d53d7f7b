"""CPU oracle for the SmoothQuant W8A8 linear -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product path (``w8a8_int8_gemm_amd``) never
does, and this package never imports the product.

The arithmetic lives in ``sq_oracle.c`` (plain C loops, fp32 where the pages'
own code quantizes in fp32, fp64 for the RMSNorm mean and the smoothing
factor's powers).  This file is argument marshalling for it, plus the fp64
whole-layer reference and error metric used to measure quantization error
("SmoothQuant and W8A8", One layer, measured: ||XW - Q(X)Q(W)|| / ||XW||) and
the fake-quant cross-path of the pages' PyTorch class ("Taming the Outliers",
Implementation in PyTorch).

Every function here is pinned by tests/test_oracle_pins.py against values the
pages print, closed forms, brute force and library routines.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sq_oracle.c")
_LIB = os.environ.get("SQ_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (-O2, OpenMP, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-std=c11", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        F = ctypes.c_float
        _lib.oracle_rms_rscale.argtypes = [P, I, I64, I64, I64, F, P]
        _lib.oracle_act_absmax.argtypes = [P, I, I64, I64, I64, I, P, F, I, P]
        _lib.oracle_weight_absmax.argtypes = [P, I, I64, I64, I64, P]
        _lib.oracle_smooth_factor.argtypes = [P, P, I64, F, P]
        _lib.oracle_fold.argtypes = [P, I64, P, P, P, I, I64, I64, P]
        _lib.oracle_quant_weight.argtypes = [P, I64, I64, I64, P, P]
        _lib.oracle_quant_act.argtypes = [P, I, I64, I64, I64, I, P, F, P, P, P, P]
        _lib.oracle_static_scale.argtypes = [P, I, I64, I64, I64, I, F, P]
        _lib.oracle_static_scale.restype = F
        _lib.oracle_quant_act_static.argtypes = [P, I, I64, I64, I64, I, P, F, P, F, P, P, P]
        _lib.oracle_static_scale_fp8.argtypes = [P, I, I64, I64, I64, I, F, P]
        _lib.oracle_static_scale_fp8.restype = F
        _lib.oracle_quant_act_static_fp8.argtypes = [P, I, I64, I64, I64, I, P, F, P, F, P, P, P]
        _lib.oracle_ln_stats.argtypes = [P, I, I64, I64, I64, F, P, P]
        _lib.oracle_act_absmax_ln.argtypes = [P, I, I64, I64, I64, P, P, F, P]
        _lib.oracle_fold_ln.argtypes = [P, I64, P, P, P, P]
        _lib.oracle_quant_act_ln.argtypes = [P, I, I64, I64, I64, P, P, F, P, P, P, P, P, P]
        _lib.oracle_fold_prev.argtypes = [P, I64, P, I, I64, I64, P, P, P]
        _lib.oracle_smoothed_act.argtypes = [P, I, I64, I64, I64, I, P, F, P, P]
        _lib.oracle_e4m3_encode_array.argtypes = [P, I64, P]
        _lib.oracle_e4m3_decode_array.argtypes = [P, I64, P]
        _lib.oracle_quant_weight_fp8.argtypes = [P, I64, I64, I64, P, P]
        _lib.oracle_quant_act_fp8.argtypes = [P, I, I64, I64, I64, I, P, F, P, P, P, P]
        _lib.oracle_gemm_fp8.argtypes = [P, P, I64, I64, I64, P]
        _lib.oracle_int_gemm.argtypes = [P, P, I64, I64, I64, P]
        _lib.oracle_int_gemm.restype = I64
        _lib.oracle_epilogue.argtypes = [P, P, P, P, I64, I64, P]
        _lib.oracle_f32_to_bf16.argtypes = [P, I64, P]
        _lib.oracle_max_threads.restype = I
    return _lib


def max_threads() -> int:
    """Number of host threads the oracle's parallel loops use."""
    return int(_load().oracle_max_threads())


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _mat(x: np.ndarray):
    """(array, is_bf16) for an fp32 or bf16-bits (uint16) matrix, C-contiguous."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return x, 1
    if x.dtype != np.float32:
        raise TypeError(f"oracle expects float32 or bf16 bits (uint16), got {x.dtype}")
    return x, 0


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


# ---------------------------------------------------------------------------
# the steps
# ---------------------------------------------------------------------------

def rms_rscale(h: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    h, bf = _mat(h)
    T, K = h.shape
    r = np.empty(T, np.float32)
    _load().oracle_rms_rscale(_p(h), bf, T, K, K, float(eps), _p(r))
    return r


def act_absmax(x: np.ndarray, *, norm: bool = False, gamma=None, eps: float = 1e-6,
               a: Optional[np.ndarray] = None) -> np.ndarray:
    """Per-input-channel absmax over calibration tokens; ``a`` given -> running max."""
    x, bf = _mat(x)
    T, K = x.shape
    acc = a is not None
    out = np.array(a, dtype=np.float32, copy=True) if acc else np.empty(K, np.float32)
    g = _f32(gamma)
    _load().oracle_act_absmax(_p(x), bf, T, K, K, int(norm), _p(g), float(eps), int(acc), _p(out))
    return out


def weight_absmax(w: np.ndarray) -> np.ndarray:
    w, bf = _mat(w)
    K, N = w.shape
    out = np.empty(K, np.float32)
    _load().oracle_weight_absmax(_p(w), bf, K, N, N, _p(out))
    return out


def smooth_factor(a: np.ndarray, wmax: np.ndarray, alpha: float) -> np.ndarray:
    a = _f32(a)
    wmax = _f32(wmax)
    s = np.empty(a.shape[0], np.float32)
    _load().oracle_smooth_factor(_p(a), _p(wmax), a.shape[0], float(np.float32(alpha)), _p(s))
    return s


def fold(s: np.ndarray, gamma=None, w: Optional[np.ndarray] = None):
    """(gamma' = gamma/s, W^ = diag(s) W as fp32 or None)."""
    s = _f32(s)
    K = s.shape[0]
    g = _f32(gamma)
    gout = np.empty(K, np.float32)
    what = None
    wp, bf, N = None, 0, 0
    if w is not None:
        wp, bf = _mat(w)
        N = wp.shape[1]
        what = np.empty((K, N), np.float32)
    _load().oracle_fold(_p(s), K, _p(g), _p(gout), _p(wp), bf, N, N, _p(what))
    return gout, what


def quant_weight(w_hat: np.ndarray):
    """(qw [N,K] int8, w_scale [N] fp32) from the fp32 smoothed weight [K,N]."""
    w_hat = np.ascontiguousarray(w_hat, dtype=np.float32)
    K, N = w_hat.shape
    qw = np.empty((N, K), np.int8)
    ws = np.empty(N, np.float32)
    _load().oracle_quant_weight(_p(w_hat), K, N, N, _p(qw), _p(ws))
    return qw, ws


def quant_act(x: np.ndarray, gamma_f=None, *, norm: bool = False, r: Optional[np.ndarray] = None,
              eps: float = 1e-6):
    """(q [T,K] int8, x_scale [T] fp32, r [T] fp32 or None)."""
    x, bf = _mat(x)
    T, K = x.shape
    q = np.empty((T, K), np.int8)
    xs = np.empty(T, np.float32)
    rout = np.empty(T, np.float32) if norm else None
    _load().oracle_quant_act(_p(x), bf, T, K, K, int(norm), _p(_f32(r)), float(eps),
                             _p(_f32(gamma_f)), _p(q), _p(xs), _p(rout))
    return q, xs, rout


def static_scale(x_cal: np.ndarray, gamma_f=None, *, norm: bool = False, eps: float = 1e-6) -> np.float32:
    """Per-tensor activation step from the calibration tokens' maximum of x^."""
    x, bf = _mat(x_cal)
    T, K = x.shape
    return np.float32(_load().oracle_static_scale(_p(x), bf, T, K, K, int(norm), float(eps),
                                                  _p(_f32(gamma_f))))


def quant_act_static(x: np.ndarray, delta, gamma_f=None, *, norm: bool = False,
                     r: Optional[np.ndarray] = None, eps: float = 1e-6):
    """(q [T,K] int8, x_scale [T] fp32 = delta, r [T] fp32 or None) with a fixed step."""
    x, bf = _mat(x)
    T, K = x.shape
    q = np.empty((T, K), np.int8)
    xs = np.empty(T, np.float32)
    rout = np.empty(T, np.float32) if norm else None
    _load().oracle_quant_act_static(_p(x), bf, T, K, K, int(norm), _p(_f32(r)), float(eps),
                                    _p(_f32(gamma_f)), float(np.float32(delta)), _p(q), _p(xs),
                                    _p(rout))
    return q, xs, rout


# ---------------------------------------------------------------------------
# FP8 E4M3 variant
# ---------------------------------------------------------------------------

def e4m3_encode(v) -> np.ndarray:
    """Nearest E4M3 codes (uint8) of fp32 values, ties to even."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    out = np.empty(v.shape, np.uint8)
    _load().oracle_e4m3_encode_array(_p(v), v.size, _p(out))
    return out


def e4m3_decode(c) -> np.ndarray:
    c = np.ascontiguousarray(c, dtype=np.uint8)
    out = np.empty(c.shape, np.float32)
    _load().oracle_e4m3_decode_array(_p(c), c.size, _p(out))
    return out


def quant_weight_fp8(w_hat: np.ndarray):
    """(qw [N,K] E4M3 codes, w_scale [N]) with w_scale = amax / 448."""
    w_hat = np.ascontiguousarray(w_hat, dtype=np.float32)
    K, N = w_hat.shape
    qw = np.empty((N, K), np.uint8)
    ws = np.empty(N, np.float32)
    _load().oracle_quant_weight_fp8(_p(w_hat), K, N, N, _p(qw), _p(ws))
    return qw, ws


def quant_act_fp8(x: np.ndarray, gamma_f=None, *, norm: bool = False,
                  r: Optional[np.ndarray] = None, eps: float = 1e-6):
    """(q [T,K] E4M3 codes, x_scale [T] = amax_t / 448, r [T] or None)."""
    x, bf = _mat(x)
    T, K = x.shape
    q = np.empty((T, K), np.uint8)
    xs = np.empty(T, np.float32)
    rout = np.empty(T, np.float32) if norm else None
    _load().oracle_quant_act_fp8(_p(x), bf, T, K, K, int(norm), _p(_f32(r)), float(eps),
                                 _p(_f32(gamma_f)), _p(q), _p(xs), _p(rout))
    return q, xs, rout


def gemm_fp8(q: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """Exact sums of E4M3 products, fp64 [T,N]."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    qw = np.ascontiguousarray(qw, dtype=np.uint8)
    T, K = q.shape
    N = qw.shape[0]
    assert qw.shape[1] == K
    acc = np.empty((T, N), np.float64)
    _load().oracle_gemm_fp8(_p(q), _p(qw), T, K, N, _p(acc))
    return acc


def prepare_weight_fp8(w, s, gamma=None):
    """(gamma', qw [N,K] E4M3, w_scale [N]) -- fold then per-output-channel E4M3."""
    gp, what = fold(s, gamma, w)
    qw, ws = quant_weight_fp8(what)
    return gp, qw, ws


def static_scale_fp8(x_cal: np.ndarray, gamma_f=None, *, norm: bool = False,
                     eps: float = 1e-6) -> np.float32:
    """Per-tensor E4M3 activation step: the calibration tokens' maximum of |x^| / 448."""
    x, bf = _mat(x_cal)
    T, K = x.shape
    return np.float32(_load().oracle_static_scale_fp8(_p(x), bf, T, K, K, int(norm), float(eps),
                                                      _p(_f32(gamma_f))))


def quant_act_static_fp8(x: np.ndarray, delta, gamma_f=None, *, norm: bool = False,
                         r: Optional[np.ndarray] = None, eps: float = 1e-6):
    """(q [T,K] E4M3 codes, x_scale [T] = delta, r [T] or None): quotients clip to +-448."""
    x, bf = _mat(x)
    T, K = x.shape
    q = np.empty((T, K), np.uint8)
    xs = np.empty(T, np.float32)
    rout = np.empty(T, np.float32) if norm else None
    _load().oracle_quant_act_static_fp8(_p(x), bf, T, K, K, int(norm), _p(_f32(r)), float(eps),
                                        _p(_f32(gamma_f)), float(np.float32(delta)), _p(q),
                                        _p(xs), _p(rout))
    return q, xs, rout


def linear_static_fp8(x, delta, gamma_f, qw, w_scale, bias=None, *, norm=False, r=None,
                      eps=1e-6, out_bf16=True):
    """E4M3 forward with one static activation step for every token."""
    q, xs, rr = quant_act_static_fp8(x, delta, gamma_f, norm=norm, r=r, eps=eps)
    acc = gemm_fp8(q, qw)
    y = epilogue_f32acc(acc.astype(np.float32), xs, w_scale, bias)
    return dict(q=q, x_scale=xs, r=rr, acc=acc, y32=y, y=to_bf16(y) if out_bf16 else y)


def linear_fp8(x, gamma_f, qw, w_scale, bias=None, *, norm=False, r=None, eps=1e-6,
               out_bf16=True):
    """E4M3 forward: quantize activations per token, exact product sums (fp64,
    rounded once to fp32 for the epilogue), epilogue as for INT8."""
    q, xs, rr = quant_act_fp8(x, gamma_f, norm=norm, r=r, eps=eps)
    acc = gemm_fp8(q, qw)
    y = epilogue_f32acc(acc.astype(np.float32), xs, w_scale, bias)
    return dict(q=q, x_scale=xs, r=rr, acc=acc, y32=y, y=to_bf16(y) if out_bf16 else y)


def epilogue_f32acc(acc: np.ndarray, x_scale, w_scale, bias=None) -> np.ndarray:
    """y = fp32(fp32(x_scale[t] * w_scale[n]) * acc[t,n]) + bias[n] for fp32 acc."""
    acc = np.asarray(acc, np.float32)
    sc = (np.asarray(x_scale, np.float32)[:, None] * np.asarray(w_scale, np.float32)[None, :])
    y = (sc.astype(np.float32) * acc).astype(np.float32)
    if bias is not None:
        y = (y + np.asarray(bias, np.float32)[None, :]).astype(np.float32)
    return y


def int_gemm(q: np.ndarray, qw: np.ndarray) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int8)
    qw = np.ascontiguousarray(qw, dtype=np.int8)
    T, K = q.shape
    N = qw.shape[0]
    assert qw.shape[1] == K
    acc = np.empty((T, N), np.int32)
    ov = _load().oracle_int_gemm(_p(q), _p(qw), T, K, N, _p(acc))
    if ov:
        raise OverflowError(f"{ov} int32 accumulator overflows")
    return acc


def epilogue(acc: np.ndarray, x_scale, w_scale, bias=None) -> np.ndarray:
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    T, N = acc.shape
    y = np.empty((T, N), np.float32)
    _load().oracle_epilogue(_p(acc), _p(_f32(x_scale)), _p(_f32(w_scale)), _p(_f32(bias)), T, N, _p(y))
    return y


def to_bf16(y: np.ndarray) -> np.ndarray:
    y = np.ascontiguousarray(y, dtype=np.float32)
    out = np.empty(y.shape, np.uint16)
    _load().oracle_f32_to_bf16(_p(y), y.size, _p(out))
    return out


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------

def calibrate(x_cal, w, alpha, *, norm=False, gamma=None, eps=1e-6):
    """(a, wmax, s) -- the offline calibration phase."""
    a = act_absmax(x_cal, norm=norm, gamma=gamma, eps=eps)
    wm = weight_absmax(w)
    return a, wm, smooth_factor(a, wm, alpha)


def prepare_weight(w, s, gamma=None):
    """(gamma', qw [N,K], w_scale [N]) -- fold then per-output-channel quant."""
    gp, what = fold(s, gamma, w)
    qw, ws = quant_weight(what)
    return gp, qw, ws


def linear(x, gamma_f, qw, w_scale, bias=None, *, norm=False, r=None, eps=1e-6, out_bf16=True):
    """The online forward: quantize activations, integer GEMM, epilogue."""
    q, xs, rr = quant_act(x, gamma_f, norm=norm, r=r, eps=eps)
    acc = int_gemm(q, qw)
    y = epilogue(acc, xs, w_scale, bias)
    return dict(q=q, x_scale=xs, r=rr, acc=acc, y32=y, y=to_bf16(y) if out_bf16 else y)


def linear_static(x, delta, gamma_f, qw, w_scale, bias=None, *, norm=False, r=None, eps=1e-6,
                  out_bf16=True):
    """The online forward with one static activation step for every token."""
    q, xs, rr = quant_act_static(x, delta, gamma_f, norm=norm, r=r, eps=eps)
    acc = int_gemm(q, qw)
    y = epilogue(acc, xs, w_scale, bias)
    return dict(q=q, x_scale=xs, r=rr, acc=acc, y32=y, y=to_bf16(y) if out_bf16 else y)


# ---------------------------------------------------------------------------
# GPTQ on the migrated weights
# ---------------------------------------------------------------------------

def smoothed_act(x: np.ndarray, gamma_f=None, *, norm: bool = False,
                 r: Optional[np.ndarray] = None, eps: float = 1e-6) -> np.ndarray:
    """x^ [T,K] fp32 exactly as the activation quantizer forms it."""
    x, bf = _mat(x)
    T, K = x.shape
    out = np.empty((T, K), np.float32)
    _load().oracle_smoothed_act(_p(x), bf, T, K, K, int(norm), _p(_f32(r)), float(eps),
                                _p(_f32(gamma_f)), _p(out))
    return out


def gptq(w_hat: np.ndarray, xhat: np.ndarray, *, damp: float = 0.01, return_quotients=False,
         columns: Optional[np.ndarray] = None):
    """GPTQ error-compensating rounding of the migrated weight ("06 --
    SmoothQuant", section 10: SmoothQuant migration first, then GPTQ on the
    migrated weights).  The pages name the step only; this follows the
    published GPTQ algorithm, unblocked, in fp64:
      H = X^T X over the calibration tokens' x^ (any positive scale: the codes
          do not depend on it); a dead input (H_jj = 0) gets H_jj = 1 and its
          weight row zeroed; H += damp * mean(diag H) * I;
      U = the upper Cholesky factor of H^-1 (H^-1 = U^T U);
      the per-output-channel step of the plain quantizer, w_scale[n] =
          fp32(max_j |W^[j,n]| / 127), fixed;
      for each input channel j in order: q_j = clamp(rne(W[j,:] / w_scale),
          +-127) (0 where w_scale is 0), e = (W[j,:] - w_scale * q_j) / U_jj,
          and every later row k takes W[k,:] -= U_jk * e.
    damp is taken as an fp32 value (the library's argument type).
    w_hat [K,N] fp32, xhat [T,K] fp32.  Returns (qw [N,K] int8, w_scale [N]),
    plus the quotients W[j,n] / w_scale[n] the rounding saw [K,N] when asked.
    Output channels never interact, so ``columns`` (indices) computes only
    those channels; the results are then [len(columns), ...] in that order.
    The two halves are gptq_factor (H and U) and gptq_round (the row loop)."""
    W = np.asarray(w_hat, np.float32)
    if columns is not None:
        W = np.ascontiguousarray(W[:, np.asarray(columns)])
    U, dead = gptq_factor(xhat, damp=damp)
    return gptq_round(W, U, dead, return_quotients=return_quotients)


def gptq_factor(xhat: np.ndarray, *, damp: float = 0.01):
    """(U [K,K] fp64, dead [K] bool): the damped Hessian's inverse factor of
    gptq.  H = X^T X of the fp32 x^ in fp64; a dead input gets H_jj = 1;
    H += fp32(damp) * mean(diag H) * I; U = the upper Cholesky factor of H^-1."""
    damp = float(np.float32(damp))
    X = np.asarray(xhat, np.float32).astype(np.float64)
    K = X.shape[1]
    H = X.T @ X
    dead = np.diag(H) == 0
    H[dead, dead] = 1.0
    H[np.diag_indices(K)] += damp * np.mean(np.diag(H))
    U = np.linalg.cholesky(np.linalg.inv(H)).T
    return U, dead


def gptq_round(w_hat: np.ndarray, U: np.ndarray, dead: np.ndarray, *, return_quotients=False,
               force_codes: Optional[np.ndarray] = None,
               force_rows: Optional[np.ndarray] = None):
    """The row loop of gptq on w_hat [K,N] fp32 with gptq_factor's (U, dead).
    force_codes [N,K] int8 with force_rows [N]: in output channel n the rows
    j < force_rows[n] take the code force_codes[n, j] instead of their own
    rounding (the error they leave still reaches the later rows).  That
    continues the algorithm from a given set of earlier decisions, e.g. the
    other side of a quotient that sits on a rounding boundary."""
    W = np.array(w_hat, np.float32)
    K, N = W.shape
    ws = (np.abs(W).max(axis=0) / np.float32(127)).astype(np.float32)
    W = W.astype(np.float64)
    W[dead, :] = 0.0
    d = ws.astype(np.float64)
    live = d > 0
    Q = np.zeros((K, N), np.int8)
    quot = np.zeros((K, N)) if return_quotients else None
    forced = None
    if force_codes is not None:
        fc = np.asarray(force_codes, np.int8)
        fr = np.asarray(force_rows, np.int64)
        assert fc.shape == (N, K) and fr.shape == (N,)
        forced = (fc, fr)
    for j in range(K):
        q = np.zeros(N)
        if quot is not None:
            quot[j, live] = W[j, live] / d[live]
        q[live] = np.clip(np.rint(W[j, live] / d[live]), -127, 127)
        if forced is not None:
            take = j < forced[1]
            q[take] = forced[0][take, j]
        Q[j] = q.astype(np.int8)
        e = (W[j] - d * q) / U[j, j]
        W[j + 1:] -= np.outer(U[j, j + 1:], e)
    if quot is not None:
        return np.ascontiguousarray(Q.T), ws, quot
    return np.ascontiguousarray(Q.T), ws


# ---------------------------------------------------------------------------
# LayerNorm form and the fold into the previous linear
# ---------------------------------------------------------------------------

def ln_stats(h: np.ndarray, eps: float = 1e-6):
    """(mean [T], r [T]) fp32: LayerNorm row mean and 1/sqrt(var + eps)."""
    h, bf = _mat(h)
    T, K = h.shape
    m, r = np.empty(T, np.float32), np.empty(T, np.float32)
    _load().oracle_ln_stats(_p(h), bf, T, K, K, float(eps), _p(m), _p(r))
    return m, r


def act_absmax_ln(h: np.ndarray, gamma=None, beta=None, eps: float = 1e-6) -> np.ndarray:
    """Per-channel absmax of LN(h) with the norm's own gamma and beta."""
    h, bf = _mat(h)
    T, K = h.shape
    a = np.empty(K, np.float32)
    _load().oracle_act_absmax_ln(_p(h), bf, T, K, K, _p(_f32(gamma)), _p(_f32(beta)),
                                 float(eps), _p(a))
    return a


def fold_ln(s: np.ndarray, gamma=None, beta=None):
    """(gamma' = gamma/s, beta' = beta/s)."""
    s = _f32(s)
    K = s.shape[0]
    gout, bout = np.empty(K, np.float32), np.empty(K, np.float32)
    _load().oracle_fold_ln(_p(s), K, _p(_f32(gamma)), _p(_f32(beta)), _p(gout), _p(bout))
    return gout, bout


def quant_act_ln(h: np.ndarray, gamma_f=None, beta_f=None, *, mean=None, r=None,
                 eps: float = 1e-6):
    """(q [T,K] int8, x_scale [T], mean [T], r [T]) of the smoothed LayerNorm output."""
    h, bf = _mat(h)
    T, K = h.shape
    q = np.empty((T, K), np.int8)
    xs = np.empty(T, np.float32)
    mo, ro = np.empty(T, np.float32), np.empty(T, np.float32)
    _load().oracle_quant_act_ln(_p(h), bf, T, K, K, _p(_f32(mean)), _p(_f32(r)), float(eps),
                                _p(_f32(gamma_f)), _p(_f32(beta_f)), _p(q), _p(xs), _p(mo),
                                _p(ro))
    return q, xs, mo, ro


def linear_ln(h, gamma_f, beta_f, qw, w_scale, bias=None, *, mean=None, r=None, eps=1e-6,
              out_bf16=True):
    """The online forward behind a smoothed LayerNorm."""
    q, xs, mo, ro = quant_act_ln(h, gamma_f, beta_f, mean=mean, r=r, eps=eps)
    acc = int_gemm(q, qw)
    y = epilogue(acc, xs, w_scale, bias)
    return dict(q=q, x_scale=xs, mean=mo, r=ro, acc=acc, y32=y, y=to_bf16(y) if out_bf16 else y)


def fold_prev(s: np.ndarray, w_prev: np.ndarray, bias=None):
    """(W_prev [K_prev, K] with column j divided by s_j as fp32, bias / s or None)."""
    s = _f32(s)
    K = s.shape[0]
    wp, bf = _mat(w_prev)
    K_prev = wp.shape[0]
    assert wp.shape[1] == K
    wout = np.empty((K_prev, K), np.float32)
    bout = None if bias is None else np.empty(K, np.float32)
    _load().oracle_fold_prev(_p(s), K, _p(wp), bf, K_prev, K, _p(wout), _p(_f32(bias)), _p(bout))
    return wout, bout


def reference_ln_fp64(h, w, bias=None, *, gamma=None, beta=None, eps=1e-6) -> np.ndarray:
    """Unsmoothed, unquantized LayerNorm -> linear in fp64."""
    hf = (h.astype(np.uint32) << 16).view(np.float32) if h.dtype == np.uint16 else h
    wf = (w.astype(np.uint32) << 16).view(np.float32) if w.dtype == np.uint16 else w
    X = hf.astype(np.float64)
    mu = X.mean(axis=1, keepdims=True)
    var = ((X - mu) ** 2).mean(axis=1, keepdims=True)
    X = (X - mu) / np.sqrt(var + float(np.float32(eps)))
    if gamma is not None:
        X = X * np.asarray(gamma, np.float64)[None, :]
    if beta is not None:
        X = X + np.asarray(beta, np.float64)[None, :]
    Y = X @ wf.astype(np.float64)
    if bias is not None:
        Y = Y + np.asarray(bias, np.float64)[None, :]
    return Y


def reference_fp64(x, w, bias=None, *, norm=False, gamma=None, eps=1e-6) -> np.ndarray:
    """Unsmoothed, unquantized layer in fp64: Y = norm?(X) @ W + b."""
    xf = (x.astype(np.uint32) << 16).view(np.float32) if x.dtype == np.uint16 else x
    wf = (w.astype(np.uint32) << 16).view(np.float32) if w.dtype == np.uint16 else w
    X = xf.astype(np.float64)
    if norm:
        ms = (X * X).mean(axis=1, keepdims=True)
        X = X / np.sqrt(ms + float(np.float32(eps)))
        if gamma is not None:
            X = X * np.asarray(gamma, np.float64)[None, :]
    Y = X @ wf.astype(np.float64)
    if bias is not None:
        Y = Y + np.asarray(bias, np.float64)[None, :]
    return Y


def rel_error(y_ref: np.ndarray, y) -> float:
    """||Y_ref - y||_F / ||Y_ref||_F in fp64 (y may be bf16 bits)."""
    yf = (y.astype(np.uint32) << 16).view(np.float32) if y.dtype == np.uint16 else y
    d = y_ref - yf.astype(np.float64)
    return float(np.sqrt((d * d).sum()) / np.sqrt((y_ref * y_ref).sum()))


def fake_quant_fp64(q, x_scale, qw, w_scale) -> np.ndarray:
    """(q * Delta_t) @ (qw * Delta_n)^T in fp64 -- the dequantize-then-multiply
    simulation of the pages' PyTorch class, before bias."""
    A = q.astype(np.float64) * np.asarray(x_scale, np.float64)[:, None]
    B = qw.astype(np.float64) * np.asarray(w_scale, np.float64)[:, None]
    return A @ B.T
