"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times.  The oracle recomputes sampled outputs one token (or one
channel) at a time: the calibration maxima over all tokens, the quantized
weight in full, and every output of a sample of tokens including the first
and last tile.  Same bar as test_gpu_parity: bit-exact when fed the GPU's
scales."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
import synth  # noqa: E402
import w8a8_int8_gemm_amd as sq  # noqa: E402
from _gpu_util import (DEV, f32, gpu_calibrate, gpu_linear, gpu_prepare_weight, say,  # noqa: E402
                       to_dev, to_np)


def _ulps(a, b):
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    return np.abs(a.view(np.int32).astype(np.int64) - b.view(np.int32).astype(np.int64))


def _sample_rows(T, n, seed):
    rng = np.random.default_rng(seed)
    rows = {0, 1, T - 1, T - 2, min(255, T - 1), min(256, T - 1)}
    rows |= set(rng.choice(T, size=min(n, T), replace=False).tolist())
    return np.array(sorted(rows))


def _check_layer(name, sample=48, calib_cols=None):
    wl = synth.WORKLOADS[name]
    say(f"full-size {name}: T={wl.T} K={wl.K} N={wl.N} Tc={wl.Tc} norm={wl.norm}")
    inp = synth.make_inputs(wl)
    g = None if inp.gamma is None else to_dev(inp.gamma)
    xc = to_dev(inp.x_cal)
    w = to_dev(inp.w)
    a, wm, s = gpu_calibrate(xc, w, wl.alpha, norm=wl.norm, gamma=g)
    gp, wq, wsc = gpu_prepare_weight(w, s, g)
    y, dbg = gpu_linear(to_dev(inp.x), gp, wq, wsc, to_dev(inp.bias), norm=wl.norm)
    torch.cuda.synchronize()
    del xc
    # calibration: every channel (or a sample of channels for the largest pass)
    cols = np.arange(wl.K) if calib_cols is None else calib_cols
    xcal = inp.x_cal if calib_cols is None else np.ascontiguousarray(inp.x_cal[:, cols])
    gam = None if inp.gamma is None else inp.gamma[cols]
    if wl.norm:
        # the RMS factor needs whole rows; with every column present this is direct
        assert calib_cols is None
    a_ref = oracle.act_absmax(xcal, norm=wl.norm, gamma=gam)
    d = _ulps(to_np(a)[cols], a_ref)
    if wl.norm:
        assert d.max() <= 1 and (d == 0).mean() > 0.99
    else:
        assert d.max() == 0
    wm_ref = oracle.weight_absmax(inp.w)
    np.testing.assert_array_equal(to_np(wm), wm_ref)
    s_ref = oracle.smooth_factor(to_np(a), wm_ref, wl.alpha)
    assert _ulps(to_np(s), s_ref).max() <= 1
    # weight fold + quant in full, fed the GPU's s
    s_h = to_np(s)
    gp_ref, qw_ref, ws_ref = oracle.prepare_weight(inp.w, s_h, inp.gamma)
    np.testing.assert_array_equal(to_np(gp), gp_ref)
    np.testing.assert_array_equal(to_np(wsc), ws_ref)
    np.testing.assert_array_equal(to_np(wq), qw_ref)
    # forward: sampled tokens, every output channel
    rows = _sample_rows(wl.T, sample, wl.seed)
    r_gpu = to_np(dbg["dbg_row_rscale"])[rows] if wl.norm else None
    fed = oracle.linear(inp.x[rows], gp_ref, qw_ref, ws_ref, inp.bias, norm=wl.norm, r=r_gpu)
    np.testing.assert_array_equal(to_np(dbg["dbg_xq"])[rows], fed["q"])
    np.testing.assert_array_equal(to_np(dbg["dbg_x_scale"])[rows], fed["x_scale"])
    np.testing.assert_array_equal(to_np(y)[rows], fed["y"])
    if wl.norm:
        r_own = oracle.rms_rscale(inp.x[rows])
        assert _ulps(r_gpu, r_own).max() <= 1


def test_qproj_prefill_full():
    _check_layer("qproj_prefill")


def test_rmsnorm_qkv_full():
    _check_layer("rmsnorm_qkv")


def test_gate_up_full():
    _check_layer("gate_up", sample=24)


def test_decode_full():
    # 4 GiB of calibration activations: the oracle checks 64 sampled channels,
    # including every outlier channel
    wl = synth.WORKLOADS["decode"]
    cols = np.unique(np.concatenate([synth.outlier_channels(wl), np.arange(0, wl.K, 211),
                                     [wl.K - 1]]))[:96]
    _check_layer("decode", sample=16, calib_cols=cols)
