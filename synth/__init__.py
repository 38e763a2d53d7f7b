"""Seeded synthetic inputs for the SmoothQuant W8A8 linear.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no absmax, no smoothing factor, no quantizer).  Both the
CPU oracle's tests and the GPU path take their inputs from here, so the two
sides always see the same bytes.

Shapes and value laws stand in for the workloads the pages describe:
  * outlier-laden activations -- a few input channels carry values tens of
    times larger than the rest, consistently across tokens ("Taming the
    Outliers", The Problem and the evaluation script's generator; "SmoothQuant
    and W8A8", Why activations are the hard part: absmax 17.5 against a median
    channel under 0.68 on a 4096-wide query projection);
  * well-behaved Gaussian weights ("06 -- SmoothQuant", section 1);
  * RMSNorm in front of the fused q/k/v and gate/up projections ("SmoothQuant
    and W8A8", The trick).

Generation recipe (numpy PCG64):
  * each workload has a base seed; ``SeedSequence(seed).spawn(8)`` gives the
    substreams [0] outlier channels, [1] outlier magnitudes and gamma,
    [2] calibration activations, [3] evaluation activations, [4] weights,
    [5] bias;
  * activations are drawn block by block (a fixed number of rows per block,
    each block with its own child seed), so a draw does not depend on the
    number of threads used;
  * values are drawn in fp32 and cast to bf16 with round-to-nearest-even; the
    bf16 bit patterns are the canonical input for both sides.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

# ---------------------------------------------------------------------------
# bf16 bit helpers (input encoding only)
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round to nearest, ties to even.

    Inputs are finite by construction; NaN/Inf are not expected here."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit pattern (uint16) -> fp32 (exact widening)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ---------------------------------------------------------------------------
# Workload descriptions
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    T: int            # evaluation tokens (rows of X)
    K: int            # input channels
    N: int            # output channels
    Tc: int           # calibration tokens (rows of X_cal)
    sigma_x: float    # base activation std
    n_outliers: int
    outlier_mult: float          # fixed multiplier (0 -> drawn, see outlier_range)
    outlier_range: tuple = (0.0, 0.0)   # U(lo, hi) target calibration absmax
    fixed_outliers: tuple = ()          # explicit outlier channel list
    sigma_w: float = 0.02
    alpha: float = 0.5
    norm: bool = False                  # RMSNorm in front of the linear
    gamma_range: tuple = (1.0, 1.0)
    io_dtype: str = "bf16"              # activations/weights in, output out
    bias_sigma: float = 0.05
    alphas: tuple = ()                  # alpha sweep (reported)
    layernorm: bool = False             # LayerNorm (gamma and beta) instead of RMSNorm
    beta_sigma: float = 0.0             # LayerNorm beta ~ N(0, beta_sigma^2)
    row_shift: float = 0.0              # per-token offset ~ N(0, row_shift^2) (LN removes it)

    def with_sizes(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # tiny smoothed linear, fp32 in/out
    "tiny": Workload("tiny", 101, T=64, K=256, N=256, Tc=128, sigma_x=1.0,
                     n_outliers=4, outlier_mult=40.0, fixed_outliers=(3, 77, 150, 201),
                     sigma_w=0.02, alpha=0.5, io_dtype="f32"),
    # 4096-wide query projection, prefill of 8192 tokens (the headline case)
    "qproj_prefill": Workload("qproj_prefill", 102, T=8192, K=4096, N=4096, Tc=8192,
                              sigma_x=0.25, n_outliers=8, outlier_mult=0.0,
                              outlier_range=(10.0, 17.5), sigma_w=0.015, alpha=0.5,
                              alphas=(0.1, 0.25, 0.5, 0.75, 1.0)),
    # RMSNorm -> fused QKV (GQA 4096 + 1024 + 1024)
    "rmsnorm_qkv": Workload("rmsnorm_qkv", 103, T=2048, K=4096, N=6144, Tc=128 * 512,
                            sigma_x=1.0, n_outliers=16, outlier_mult=50.0,
                            sigma_w=0.02, alpha=0.85, norm=True, gamma_range=(0.5, 1.5)),
    # MLP gate|up after the post-attention norm (norm already folded upstream)
    "gate_up": Workload("gate_up", 104, T=4096, K=4096, N=28672, Tc=8192,
                        sigma_x=0.3, n_outliers=12, outlier_mult=30.0,
                        sigma_w=0.02, alpha=0.5),
    # LayerNorm -> fused QKV: the LayerNorm form of the smoothed norm (its
    # gamma and beta both take 1/s); tokens carry an offset the norm removes
    "layernorm_qkv": Workload("layernorm_qkv", 106, T=2048, K=4096, N=6144, Tc=16384,
                              sigma_x=1.0, n_outliers=16, outlier_mult=50.0,
                              sigma_w=0.02, alpha=0.85, norm=True, gamma_range=(0.5, 1.5),
                              layernorm=True, beta_sigma=0.1, row_shift=2.0),
    # decode-shaped GEMM plus a large calibration pass
    "decode": Workload("decode", 105, T=16, K=8192, N=8192, Tc=128 * 2048,
                       sigma_x=1.0, n_outliers=24, outlier_mult=60.0,
                       sigma_w=0.01, alpha=0.5),
}

_BLOCK_ELEMS = 1 << 22   # elements per independently seeded block of activations


def _streams(seed: int):
    return np.random.SeedSequence(seed).spawn(8)


def outlier_channels(w: Workload) -> np.ndarray:
    if w.fixed_outliers:
        return np.array(w.fixed_outliers, dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64(_streams(w.seed)[0]))
    return np.sort(rng.permutation(w.K)[: w.n_outliers]).astype(np.int64)


def _gaussian_rows(ss: np.random.SeedSequence, rows: int, cols: int, sigma: float,
                   threads: Optional[int] = None) -> np.ndarray:
    """[rows, cols] fp32 ~ N(0, sigma^2), drawn in independently seeded row blocks."""
    rpb = max(1, _BLOCK_ELEMS // cols)
    nblk = (rows + rpb - 1) // rpb
    children = ss.spawn(nblk)
    out = np.empty((rows, cols), dtype=np.float32)

    def fill(b):
        r0 = b * rpb
        r1 = min(rows, r0 + rpb)
        g = np.random.Generator(np.random.PCG64(children[b]))
        g.standard_normal(out=out[r0:r1], dtype=np.float32)
        if sigma != 1.0:
            out[r0:r1] *= np.float32(sigma)

    if threads is None:
        threads = min(16, os.cpu_count() or 1)
    if nblk == 1 or threads <= 1:
        for b in range(nblk):
            fill(b)
    else:
        with _cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(nblk)))
    return out


@dataclass
class Inputs:
    wl: Workload
    x_cal: Optional[np.ndarray]   # [Tc, K] (bf16 bits uint16, or fp32)
    x: Optional[np.ndarray]       # [T, K]
    w: np.ndarray                 # [K, N] row-major (input channel j = row j)
    gamma: Optional[np.ndarray]   # [K] fp32 (RMSNorm weight) or None
    bias: np.ndarray              # [N] fp32
    outliers: np.ndarray
    meta: dict = field(default_factory=dict)
    beta: Optional[np.ndarray] = None   # [K] fp32 LayerNorm bias, or None

    @property
    def io_bf16(self) -> bool:
        return self.wl.io_dtype == "bf16"

    def as_f32(self, a: np.ndarray) -> np.ndarray:
        return bf16_bits_to_f32(a) if a.dtype == np.uint16 else a


def make_inputs(w: Workload, *, calib: bool = True, evaluation: bool = True,
                threads: Optional[int] = None) -> Inputs:
    st = _streams(w.seed)
    outl = outlier_channels(w)
    rng1 = np.random.Generator(np.random.PCG64(st[1]))
    if w.outlier_mult > 0:
        mults = None
        target = None
    else:
        target = rng1.uniform(w.outlier_range[0], w.outlier_range[1], size=len(outl)).astype(np.float32)
        mults = None
    gamma = None
    if w.norm:
        gamma = rng1.uniform(w.gamma_range[0], w.gamma_range[1], size=w.K).astype(np.float32)

    beta = None
    if w.layernorm:
        beta = np.random.Generator(np.random.PCG64(st[6])).normal(
            0.0, w.beta_sigma, size=w.K).astype(np.float32)
    shift_rng = np.random.Generator(np.random.PCG64(st[7]))

    def shifted(a):
        if w.row_shift > 0 and a is not None:
            a += shift_rng.normal(0.0, w.row_shift, size=(a.shape[0], 1)).astype(np.float32)
        return a

    x_cal = None
    if calib or target is not None:
        x_cal = _gaussian_rows(st[2], w.Tc, w.K, w.sigma_x, threads)
    if target is not None:
        # scale each outlier channel so that its calibration absmax is the drawn target
        base = np.abs(x_cal[:, outl]).max(axis=0)
        mults = (target / base).astype(np.float32)
    else:
        mults = np.full(len(outl), w.outlier_mult, dtype=np.float32)
    if x_cal is not None:
        x_cal[:, outl] *= mults
        shifted(x_cal)
    x = None
    if evaluation:
        x = _gaussian_rows(st[3], w.T, w.K, w.sigma_x, threads)
        x[:, outl] *= mults
        shifted(x)
    wt = _gaussian_rows(st[4], w.K, w.N, w.sigma_w, threads)
    bias = np.random.Generator(np.random.PCG64(st[5])).normal(0.0, w.bias_sigma, size=w.N).astype(np.float32)

    if w.io_dtype == "bf16":
        x_cal = f32_to_bf16_bits(x_cal) if (x_cal is not None and calib) else None
        x = f32_to_bf16_bits(x) if x is not None else None
        wt = f32_to_bf16_bits(wt)
    elif not calib:
        x_cal = None
    return Inputs(w, x_cal, x, wt, gamma, bias, outl,
                  meta={"outlier_mult": mults.tolist()}, beta=beta)
