"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values the
pages print (tests/golden/), closed forms, brute force on tiny inputs, an
independent high-precision evaluation, or a library routine for a step that
reduces to one.  None of these needs a GPU.
"""
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


def _codes_for(values, amax):
    """Quantize a one-token row whose absmax is ``amax`` through the oracle."""
    row = np.array([amax] + list(values), dtype=np.float32)[None, :]
    q, xs, _ = oracle.quant_act(row, np.ones(row.shape[1], np.float32))
    return q[0, 1:], float(xs[0])


# ---------------------------------------------------------------------------
# worked values printed on the pages
# ---------------------------------------------------------------------------

def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line)
    return rows


def _weight_codes_for(values, amax):
    """Quantize a one-output-channel weight column whose absmax is ``amax``."""
    col = np.array([amax] + list(values), dtype=np.float32)[:, None]
    qw, ws = oracle.quant_weight(col)
    return qw[0, 1:], float(ws[0])


@pytest.mark.parametrize("path", ["activation", "weight"])
def test_quantizer_worked_values(path):
    rows = _golden_rows("quantizer_worked.txt")
    assert len(rows) >= 9
    fn = _codes_for if path == "activation" else _weight_codes_for
    for r in rows:
        amax, value, delta_printed, tol, code = r.split()
        q, d = fn([float(value)], float(amax))
        assert abs(d - float(delta_printed)) <= float(tol), r
        assert int(q[0]) == int(code), (r, int(q[0]))


def test_smoothing_worked_values():
    for r in _golden_rows("smoothing_worked.txt"):
        _, rest = r.split(None, 1)
        vec, s, ch, expect = [p.strip() for p in rest.split(";")]
        x = np.array([float(v) for v in vec.split()], np.float32)
        s = np.array([float(v) for v in s.split()], np.float32)
        ch = int(ch)
        gp, _ = oracle.fold(s)
        # activations are divided by s: x * (1/s)
        smoothed = F32(x[ch] * gp[ch])
        assert abs(abs(float(smoothed)) - float(expect)) < 2e-6, r
        # the matching weight row is multiplied by s, the other rows untouched
        w = np.arange(len(x) * 3, dtype=np.float32).reshape(len(x), 3) + 1
        _, what = oracle.fold(s, None, w)
        np.testing.assert_array_equal(what[ch], w[ch] * s[ch])
        for j in range(len(x)):
            if s[j] == 1:
                np.testing.assert_array_equal(what[j], w[j])


# ---------------------------------------------------------------------------
# closed forms of the smoothing factor ("06 -- SmoothQuant" section 3;
# "SmoothQuant and W8A8", The trick; "SmoothQuant: Weight-Only vs W8A8",
# Migration Strength)
# ---------------------------------------------------------------------------

def _tiny():
    return synth.make_inputs(synth.WORKLOADS["tiny"])


def test_alpha_one_every_channel_peaks_at_one():
    inp = _tiny()
    a, wm, s = oracle.calibrate(inp.x_cal, inp.w, 1.0)
    np.testing.assert_array_equal(s, np.maximum(a, F32(1e-5)))
    # dividing form (the pages' x / s): the peak is exactly 1 for every channel
    xc = inp.as_f32(inp.x_cal)
    peaks = np.abs(xc / s[None, :]).max(axis=0)
    np.testing.assert_array_equal(peaks, np.ones_like(peaks))
    # folded form x * fp32(1/s): within one rounding of 1
    gp, _ = oracle.fold(s)
    peaks_f = np.abs(xc * gp[None, :]).max(axis=0)
    assert np.all(np.abs(peaks_f - 1) <= 2 ** -23)


def test_alpha_zero_is_inverse_weight_max():
    inp = _tiny()
    a, wm, s = oracle.calibrate(inp.x_cal, inp.w, 0.0)
    # s_j = 1 / max|W_j| (not "no smoothing")
    np.testing.assert_array_equal(s, F32(1.0) / wm)
    assert not np.allclose(s, 1.0)


def test_weight_absmax_indexes_input_rows():
    w = np.zeros((5, 7), np.float32)
    w[2, 6] = -3.0   # input channel 2
    w[4, 0] = 0.5
    wm = oracle.weight_absmax(w)
    np.testing.assert_array_equal(wm, np.array([0, 0, 3.0, 0, 0.5], np.float32))


def test_smoothing_factor_matches_high_precision():
    """s_j against an independent 40-digit evaluation of a^alpha / w^(1-alpha)."""
    getcontext().prec = 40
    rng = np.random.default_rng(7)
    a = (rng.uniform(0.01, 200.0, 300)).astype(np.float32)
    w = (rng.uniform(0.001, 0.5, 300)).astype(np.float32)
    for alpha in (0.1, 0.25, 0.5, 0.75, 0.85, 1.0):
        s = oracle.smooth_factor(a, w, alpha)
        al = Decimal(float(F32(alpha)))
        for j in range(len(a)):
            A = Decimal(float(a[j]))
            W = Decimal(float(w[j]))
            exact = (al * A.ln()).exp() / ((Decimal(1) - al) * W.ln()).exp()
            ref = F32(float(exact))
            # exact equality unless the value sits on an fp32 rounding boundary
            if s[j] != ref:
                assert abs(float(s[j]) - float(exact)) <= 0.5000001 * np.spacing(s[j]), (alpha, j)


def test_smoothing_factor_guards():
    a = np.array([0.0, 5.0, 3.0], np.float32)
    w = np.array([0.2, 0.0, 1e12], np.float32)
    s = oracle.smooth_factor(a, w, 0.5)
    assert s[0] == F32(1e-5)            # dead channel: clamp at 1e-5
    assert s[1] == 1.0                  # all-zero weight row: s = 1
    assert s[2] == F32(1e-5)            # tiny quotient clamps too


# ---------------------------------------------------------------------------
# the invariance Y = (X diag(s)^-1)(diag(s) W)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("alpha", [0.1, 0.5, 0.85, 1.0])
def test_invariance_fp64_and_folded(alpha):
    inp = _tiny()
    _, _, s = oracle.calibrate(inp.x_cal, inp.w, alpha)
    X = inp.as_f32(inp.x).astype(np.float64)
    W = inp.as_f32(inp.w).astype(np.float64)
    Y = X @ W
    sd = s.astype(np.float64)
    Y2 = (X / sd[None, :]) @ (sd[:, None] * W)
    assert np.linalg.norm(Y2 - Y) / np.linalg.norm(Y) < 1e-12
    # the oracle's folded fp32 tensors: gamma' = 1/s on X, W^ = diag(s) W
    gp, what = oracle.fold(s, None, inp.w)
    Y3 = (X * gp.astype(np.float64)[None, :]) @ what.astype(np.float64)
    assert np.linalg.norm(Y3 - Y) / np.linalg.norm(Y) < 1e-5


def test_fold_into_norm_weight():
    rng = np.random.default_rng(3)
    s = rng.uniform(0.1, 30, 64).astype(np.float32)
    g = rng.uniform(0.5, 1.5, 64).astype(np.float32)
    gp, _ = oracle.fold(s, g)
    np.testing.assert_array_equal(gp, g / s)


# ---------------------------------------------------------------------------
# quantizer: brute force and invariants ("Taming the Outliers", the
# quantization equation; "SmoothQuant: Weight-Only vs W8A8", Step Size)
# ---------------------------------------------------------------------------

def _nearest_code_bruteforce(v, d):
    """Search all 255 codes for the one nearest v (exact in fp64), ties to even."""
    best, berr = None, None
    for c in range(-127, 128):
        e = abs(float(v) - c * float(d))
        if best is None or e < berr or (e == berr and c % 2 == 0):
            best, berr = c, e
    return best, berr


def test_bruteforce_8x8x8_whole_layer():
    rng = np.random.default_rng(11)
    T = K = N = 8
    x = rng.standard_normal((T, K)).astype(np.float32)
    x[:, 2] *= 30
    w = (rng.standard_normal((K, N)) * 0.1).astype(np.float32)
    xc = rng.standard_normal((16, K)).astype(np.float32)
    xc[:, 2] *= 30
    a, wm, s = oracle.calibrate(xc, w, 0.5)
    gp, qw, ws = oracle.prepare_weight(w, s)
    _, what = oracle.fold(s, None, w)
    out = oracle.linear(x, gp, qw, ws, None, out_bf16=False)
    q, xs = out["q"], out["x_scale"]
    # activation codes: nearest code on the grid, unless the fp32 quotient sits
    # on a half-integer boundary (not the case for this draw; checked)
    for t in range(T):
        for k in range(K):
            xh = F32(x[t, k] * gp[k])
            c, _ = _nearest_code_bruteforce(xh, xs[t])
            qq = float(xh) / float(xs[t])
            assert abs(abs(qq - math.floor(qq)) - 0.5) > 1e-4
            assert q[t, k] == c
    for n in range(N):
        for k in range(K):
            c, _ = _nearest_code_bruteforce(what[k, n], ws[n])
            assert qw[n, k] == c
    # integer GEMM: plain triple loop in Python integers
    for t in range(T):
        for n in range(N):
            assert out["acc"][t, n] == sum(int(q[t, k]) * int(qw[n, k]) for k in range(K))
    # absmax against Python max
    for j in range(K):
        assert a[j] == max(abs(float(v)) for v in xc[:, j])
        assert wm[j] == max(abs(float(v)) for v in w[j, :])


def test_quantizer_ties_to_even_and_range():
    # amax 127 -> Delta = 1 exactly, so quotients are the values themselves
    vals = [2.5, 3.5, -2.5, -0.5, 0.5, 1.5, 126.5, -126.5, 0.49999997]
    q, d = _codes_for(vals, 127.0)
    assert d == 1.0
    assert list(q) == [2, 4, -2, 0, 0, 2, 126, -126, 0]
    # the largest magnitude maps to exactly +-127 and -128 never appears
    rng = np.random.default_rng(5)
    x = rng.standard_normal((50, 300)).astype(np.float32) * rng.uniform(0.01, 100, (50, 1)).astype(np.float32)
    q, xs, _ = oracle.quant_act(x, np.ones(300, np.float32))
    assert q.min() >= -127 and q.max() <= 127
    np.testing.assert_array_equal(np.abs(q).max(axis=1), np.full(50, 127))


def test_quantizer_half_step_bound_and_power_of_two_scaling():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((40, 512)) * rng.uniform(0.1, 10, (40, 1))).astype(np.float32)
    x[:, 17] *= 25
    q, xs, _ = oracle.quant_act(x, np.ones(512, np.float32))
    err = np.abs(x.astype(np.float64) - q.astype(np.float64) * xs[:, None].astype(np.float64))
    bound = xs[:, None].astype(np.float64) * (0.5 + 2.0 ** -17)
    assert np.all(err <= bound)
    for k in (-3, 1, 6):
        q2, xs2, _ = oracle.quant_act((x * F32(2.0 ** k)).astype(np.float32), np.ones(512, np.float32))
        np.testing.assert_array_equal(q2, q)
        np.testing.assert_array_equal(xs2, xs * F32(2.0 ** k))


def test_weight_quant_half_step_bound():
    rng = np.random.default_rng(10)
    what = (rng.standard_normal((300, 40)) * rng.uniform(0.01, 3, (1, 40))).astype(np.float32)
    what[17] *= 20
    qw, ws = oracle.quant_weight(what)
    err = np.abs(what.T.astype(np.float64) - qw.astype(np.float64) * ws[:, None].astype(np.float64))
    assert np.all(err <= ws[:, None].astype(np.float64) * (0.5 + 2.0 ** -17))
    np.testing.assert_array_equal(np.abs(qw).max(axis=1), np.full(40, 127))


def test_zero_rows_and_columns():
    x = np.zeros((3, 64), np.float32)
    x[1, 5] = 2.0
    q, xs, _ = oracle.quant_act(x, np.ones(64, np.float32))
    assert xs[0] == 0 and xs[2] == 0 and np.all(q[0] == 0) and np.all(q[2] == 0)
    assert q[1, 5] == 127
    what = np.zeros((64, 4), np.float32)
    what[3, 1] = -0.5
    qw, ws = oracle.quant_weight(what)
    assert ws[0] == 0 and np.all(qw[0] == 0) and qw[1, 3] == -127
    acc = oracle.int_gemm(q, qw)
    y = oracle.epilogue(acc, xs, ws, np.array([1, 2, 3, 4], np.float32))
    np.testing.assert_array_equal(y[0], [1, 2, 3, 4])


# ---------------------------------------------------------------------------
# RMSNorm reciprocal scale (norm named in "SmoothQuant and W8A8", The trick)
# ---------------------------------------------------------------------------

def test_rms_rscale_closed_forms():
    eps = 1e-6
    h = np.full((1, 256), 3.0, np.float32)
    r = oracle.rms_rscale(h, eps)
    assert r[0] == F32(1.0 / math.sqrt(9.0 + float(F32(eps))))
    h = np.tile(np.array([1.0, -1.0], np.float32), (2, 64))
    h[1] *= 4
    r = oracle.rms_rscale(h, eps)
    assert r[0] == F32(1.0 / math.sqrt(1.0 + float(F32(eps))))
    assert r[1] == F32(1.0 / math.sqrt(16.0 + float(F32(eps))))
    # bf16 input is widened exactly
    hb = synth.f32_to_bf16_bits(h)
    np.testing.assert_array_equal(oracle.rms_rscale(hb, eps), r)


def test_rms_rscale_against_fsum():
    rng = np.random.default_rng(2)
    h = rng.standard_normal((20, 1000)).astype(np.float32)
    h[:, 7] *= 50
    r = oracle.rms_rscale(h, 1e-6)
    for t in range(20):
        ms = math.fsum(float(v) * float(v) for v in h[t]) / 1000
        ref = F32(1.0 / math.sqrt(ms + float(F32(1e-6))))
        assert abs(float(r[t]) - float(ref)) <= float(np.spacing(ref))


def test_norm_mode_activation_order():
    """x^ = fp32(fp32(h * r) * gamma') in norm mode, for quant and calibration."""
    rng = np.random.default_rng(4)
    h = rng.standard_normal((6, 128)).astype(np.float32)
    g = rng.uniform(0.5, 1.5, 128).astype(np.float32)
    r = oracle.rms_rscale(h)
    q, xs, rr = oracle.quant_act(h, g, norm=True)
    np.testing.assert_array_equal(rr, r)
    xh = ((h * r[:, None]).astype(np.float32) * g[None, :]).astype(np.float32)
    q2, xs2, _ = oracle.quant_act(xh, None)
    np.testing.assert_array_equal(q, q2)
    np.testing.assert_array_equal(xs, xs2)
    a = oracle.act_absmax(h, norm=True, gamma=g)
    np.testing.assert_array_equal(a, np.abs(xh).max(axis=0))


def test_calibration_running_max():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((100, 64)).astype(np.float32)
    a1 = oracle.act_absmax(x[:40])
    a2 = oracle.act_absmax(x[40:], a=a1)
    np.testing.assert_array_equal(a2, np.abs(x).max(axis=0))


# ---------------------------------------------------------------------------
# integer GEMM and epilogue
# ---------------------------------------------------------------------------

def test_int_gemm_matches_numpy_int64():
    rng = np.random.default_rng(12)
    q = rng.integers(-127, 128, (37, 320), dtype=np.int8)
    qw = rng.integers(-127, 128, (53, 320), dtype=np.int8)
    acc = oracle.int_gemm(q, qw)
    ref = q.astype(np.int64) @ qw.astype(np.int64).T
    np.testing.assert_array_equal(acc, ref)


def test_int_gemm_extreme_fits_int32():
    K = 8192
    q = np.full((2, K), 127, np.int8)
    q[1] = -127
    qw = np.full((3, K), 127, np.int8)
    acc = oracle.int_gemm(q, qw)
    assert acc[0, 0] == 127 * 127 * K and acc[1, 2] == -127 * 127 * K


def test_epilogue_equals_fake_quant_and_bound():
    inp = _tiny()
    _, _, s = oracle.calibrate(inp.x_cal, inp.w, 0.5)
    gp, qw, ws = oracle.prepare_weight(inp.w, s)
    out = oracle.linear(inp.x, gp, qw, ws, inp.bias, out_bf16=False)
    y_sim = oracle.fake_quant_fp64(out["q"], out["x_scale"], qw, ws) + inp.bias[None, :].astype(np.float64)
    y = out["y32"].astype(np.float64)
    tol = 4 * 2.0 ** -24 * (np.abs(y_sim) + np.abs(inp.bias)[None, :]) + 1e-30
    assert np.all(np.abs(y - y_sim) <= tol)
    # a-priori quantization error bound against the exact smoothed product
    X = inp.as_f32(inp.x)
    xh = (X * gp[None, :]).astype(np.float64)
    _, what = oracle.fold(s, None, inp.w)
    Wh = what.astype(np.float64)
    exact = xh @ Wh + inp.bias[None, :]
    xsd = out["x_scale"].astype(np.float64)[:, None]
    wsd = ws.astype(np.float64)[None, :]
    bound = (np.abs(xh).sum(1, keepdims=True) * wsd / 2 + xsd * np.abs(Wh).sum(0, keepdims=True) / 2
             + X.shape[1] * xsd * wsd / 4) * (1 + 1e-5) + 1e-6 * np.abs(exact)
    assert np.all(np.abs(y - exact) <= bound)


def test_bf16_rounding_of_output():
    y = np.array([1.0, 1.00390625, 1.01171875, -2.5, 3.0e-3, 1.0 + 2 ** -8 + 2 ** -20], np.float32)
    b = oracle.to_bf16(y)
    back = synth.bf16_bits_to_f32(b)
    # ties to even at 1 + 2^-8 (-> 1.0) and 1 + 3*2^-8 (-> 1 + 2^-6); above the tie rounds up
    assert back[0] == 1.0 and back[1] == 1.0 and back[2] == F32(1.015625)
    assert back[3] == -2.5 and back[5] == F32(1.0078125)
    assert abs(back[4] - 3.0e-3) <= 3.0e-3 * 2 ** -8


# ---------------------------------------------------------------------------
# qualitative claims: smoothing cuts INT8 error on outlier data
# ("SmoothQuant and W8A8", One layer, measured; "Taming the Outliers",
#  evaluation script)
# ---------------------------------------------------------------------------

def _layer_error(inp, alpha):
    X, W = inp.x, inp.w
    if alpha is None:       # unsmoothed point: s = 1
        s = np.ones(inp.wl.K, np.float32)
    else:
        _, _, s = oracle.calibrate(inp.x_cal, W, alpha)
    gp, qw, ws = oracle.prepare_weight(W, s)
    out = oracle.linear(X, gp, qw, ws, None, out_bf16=False)
    ref = oracle.reference_fp64(X, W)
    return oracle.rel_error(ref, out["y32"])


def test_smoothing_reduces_error_tiny():
    inp = _tiny()
    e0 = _layer_error(inp, None)
    e5 = _layer_error(inp, 0.5)
    assert e5 < e0 / 2, (e0, e5)


def test_evaluation_script_shape():
    """128 -> 64 linear, 100 calibration and 10 test samples, 5% of the
    channels multiplied by 50, alpha 0.5: smoothed error below unsmoothed."""
    rng = np.random.default_rng(0)
    xc = rng.standard_normal((100, 128)).astype(np.float32)
    xt = rng.standard_normal((10, 128)).astype(np.float32)
    idx = rng.permutation(128)[: int(128 * 0.05)]
    xc[:, idx] *= 50
    xt[:, idx] *= 50
    W = rng.standard_normal((128, 64)).astype(np.float32)
    ref = oracle.reference_fp64(xt, W)
    errs = []
    for s in (np.ones(128, np.float32), oracle.calibrate(xc, W, 0.5)[2]):
        gp, qw, ws = oracle.prepare_weight(W, s)
        errs.append(oracle.rel_error(ref, oracle.linear(xt, gp, qw, ws, out_bf16=False)["y32"]))
    assert errs[1] < errs[0], errs


# ---------------------------------------------------------------------------
# static per-tensor activation step ("SmoothQuant and W8A8", One layer,
# measured: one scale per tensor from the calibration tokens' maximum; Gotchas:
# what the calibration never saw is clipped)
# ---------------------------------------------------------------------------

def test_static_scale_worked_values():
    # a calibration set whose largest |x| is amax gives the pages' step, and
    # the worked value maps to the printed code through the static path
    for r in _golden_rows("quantizer_worked.txt"):
        amax, value, delta_printed, tol, code = r.split()
        cal = np.array([[float(amax), 0.1], [-0.5 * float(amax), 0.0]], np.float32)
        d = oracle.static_scale(cal)
        assert abs(float(d) - float(delta_printed)) <= float(tol), r
        q, xs, _ = oracle.quant_act_static(np.array([[float(value), 0.0]], np.float32), d)
        assert int(q[0, 0]) == int(code), r
        assert xs[0] == d


def test_static_equals_dynamic_on_the_calibration_maximum():
    # a token that holds the calibration maximum has the same step, hence the
    # same codes, under the static and the per-token quantizer
    rng = np.random.default_rng(21)
    x = rng.standard_normal((64, 256)).astype(np.float32)
    x[:, 9] *= 40
    g = rng.uniform(0.5, 1.5, 256).astype(np.float32)
    d = oracle.static_scale(x, g)
    t = int(np.argmax(np.abs(x * g).max(axis=1)))
    qs, _, _ = oracle.quant_act_static(x[t:t + 1], d, g)
    qd, xd, _ = oracle.quant_act(x[t:t + 1], g)
    assert xd[0] == d
    np.testing.assert_array_equal(qs, qd)


def test_static_quant_clips_past_the_calibrated_maximum():
    rng = np.random.default_rng(22)
    cal = rng.standard_normal((32, 16)).astype(np.float32)
    d = oracle.static_scale(cal)
    x = (rng.standard_normal((8, 16)) * 3).astype(np.float32)   # well past the calibration range
    q, _, _ = oracle.quant_act_static(x, d)
    assert np.abs(q).max() == 127
    for t in range(8):
        for k in range(16):
            qq = float(x[t, k]) / float(d)
            assert abs(abs(qq - math.floor(qq)) - 0.5) > 1e-4
            c, _ = _nearest_code_bruteforce(x[t, k], d)   # searches -127..127 only
            assert q[t, k] == c, (t, k, qq)


def test_static_scale_norm_mode_by_channel_maxima():
    # max over tokens and channels of |fp32(fp32(h r_t) g_k)| equals
    # max_k fp32(max_t |fp32(h r_t)| * |g_k|): rounding is monotone and sign
    # symmetric, the route the GPU takes from the channel maxima
    rng = np.random.default_rng(23)
    h = rng.standard_normal((96, 320)).astype(np.float32)
    h[:, 5] *= 30
    g = rng.uniform(-1.5, 1.5, 320).astype(np.float32)
    d = oracle.static_scale(h, g, norm=True)
    m = oracle.act_absmax(h, norm=True, gamma=None)
    via = F32(np.max((m * np.abs(g)).astype(np.float32)) / F32(127.0))
    assert d == via
    # and with no norm the same identity on the raw absmax
    d0 = oracle.static_scale(h, g)
    a0 = oracle.act_absmax(h)
    assert d0 == F32(np.max((a0 * np.abs(g)).astype(np.float32)) / F32(127.0))


def test_static_zero_step_gives_zero_codes():
    x = np.zeros((3, 64), np.float32)
    d = oracle.static_scale(x)
    assert d == 0.0
    q, xs, _ = oracle.quant_act_static(np.ones((2, 64), np.float32), d)
    assert not q.any() and not xs.any()


# ---------------------------------------------------------------------------
# FP8 E4M3 variant ("SmoothQuant and W8A8", One layer, measured: weights per
# output channel and activations per token in FP8 E4M3)
# ---------------------------------------------------------------------------

def _e4m3_table():
    """Every finite E4M3 value from the format's definition: bias 7, 3 mantissa
    bits, exponent field 0 subnormal, 0x7F/0xFF NaN."""
    vals = {}
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            continue
        v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
        vals[c] = -v if s else v
    return vals


def test_e4m3_decode_definition_and_round_trip():
    tab = _e4m3_table()
    codes = np.array(sorted(tab), np.uint8)
    dec = oracle.e4m3_decode(codes)
    np.testing.assert_array_equal(dec, np.array([tab[c] for c in codes], np.float32))
    assert np.isnan(oracle.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()
    assert tab[0x38] == 1.0 and tab[0x7E] == 448.0 and tab[0x01] == 2.0 ** -9 and tab[0x08] == 2.0 ** -6
    # encoding a finite value reproduces its code (+0 and -0 keep their sign)
    np.testing.assert_array_equal(oracle.e4m3_encode(dec), codes)


def test_e4m3_encode_is_nearest_ties_to_even():
    tab = _e4m3_table()
    pos = sorted((v, c) for c, v in tab.items() if c < 0x80)
    rng = np.random.default_rng(31)
    v = np.concatenate([rng.uniform(0, 448, 3000), np.exp(rng.uniform(np.log(1e-4), np.log(448), 3000)),
                        # exact midpoints between neighbours: ties
                        [(a[0] + b[0]) / 2 for a, b in zip(pos, pos[1:])]]).astype(np.float32)
    v = np.concatenate([v, -v])
    got = oracle.e4m3_encode(v)
    for x, c in zip(v, got):
        a = abs(float(x))
        best = min(pos, key=lambda p: (abs(p[0] - a), p[1] & 1))   # nearest, then even mantissa
        assert (int(c) & 0x7F) == best[1], (x, hex(c), best)
        assert (int(c) >> 7) == (1 if x < 0 else 0)


def test_e4m3_relative_precision_over_the_pages_range():
    # with a token maximum of 17.5 the step is 17.5/448: every value from 0.68
    # to 17.5 keeps a relative error of at most half an E4M3 mantissa step
    # (1/16); INT8 at the same maximum rounds 0.68 to 5 steps of 0.138
    x = np.linspace(0.68, 17.5, 2001).astype(np.float32)
    row = np.concatenate([[17.5], x]).astype(np.float32)[None, :]
    q, xs, _ = oracle.quant_act_fp8(row, np.ones(row.shape[1], np.float32))
    assert xs[0] == F32(17.5) / F32(448.0)
    back = oracle.e4m3_decode(q[0, 1:]).astype(np.float64) * float(xs[0])
    rel = np.abs(back - x) / x
    assert rel.max() <= 1 / 16 + 1e-6
    qi, xi, _ = oracle.quant_act(row, np.ones(row.shape[1], np.float32))
    assert qi[0, 1] == 5 and abs(float(qi[0, 1]) * float(xi[0]) - 0.68) / 0.68 > 0.01


def test_fp8_quantizers_map_the_maximum_to_448():
    rng = np.random.default_rng(32)
    x = (rng.standard_normal((20, 256)) * rng.uniform(0.1, 30, (20, 1))).astype(np.float32)
    q, xs, _ = oracle.quant_act_fp8(x)
    np.testing.assert_array_equal(xs, (np.abs(x).max(axis=1) / F32(448.0)).astype(np.float32))
    assert (np.abs(oracle.e4m3_decode(q)).max(axis=1) == 448.0).all()
    w = (rng.standard_normal((300, 24)) * rng.uniform(0.01, 2, (1, 24))).astype(np.float32)
    qw, ws = oracle.quant_weight_fp8(w)
    np.testing.assert_array_equal(ws, (np.abs(w).max(axis=0) / F32(448.0)).astype(np.float32))
    np.testing.assert_array_equal(qw, oracle.e4m3_encode((w / ws[None, :]).astype(np.float32)).T)
    # codes are the nearest E4M3 of the fp32 quotient, as in the INT8 quantizer
    np.testing.assert_array_equal(q, oracle.e4m3_encode((x / xs[:, None]).astype(np.float32)))


def test_gemm_fp8_matches_numpy_fp64():
    rng = np.random.default_rng(33)
    q = rng.integers(0, 256, (12, 320)).astype(np.uint8)
    qw = rng.integers(0, 256, (9, 320)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x10          # no NaN codes
    qw[(qw & 0x7F) == 0x7F] = 0x20
    acc = oracle.gemm_fp8(q, qw)
    ref = oracle.e4m3_decode(q).astype(np.float64) @ oracle.e4m3_decode(qw).astype(np.float64).T
    np.testing.assert_array_equal(acc, ref)


# static per-tensor E4M3 step ("SmoothQuant and W8A8", One layer, measured:
# one static scale per tensor from the calibration tokens' maximum, in INT8
# and in FP8 E4M3; Gotchas: values past the calibrated maximum are clipped)

def test_static_fp8_equals_dynamic_fp8_on_the_calibration_maximum():
    rng = np.random.default_rng(34)
    x = rng.standard_normal((48, 320)).astype(np.float32)
    x[:, 17] *= 25
    g = rng.uniform(0.5, 1.5, 320).astype(np.float32)
    d = oracle.static_scale_fp8(x, g)
    t = int(np.argmax(np.abs(x * g).max(axis=1)))
    qs, xs, _ = oracle.quant_act_static_fp8(x[t:t + 1], d, g)
    qd, xd, _ = oracle.quant_act_fp8(x[t:t + 1], g)
    assert xd[0] == d and xs[0] == d
    np.testing.assert_array_equal(qs, qd)
    # and the same maximum gives the INT8 static step over 127 instead of 448
    assert oracle.static_scale(x, g) * F32(127.0) == pytest.approx(float(d) * 448.0, rel=1e-6)


def test_static_fp8_clips_past_the_calibrated_maximum():
    tab = _e4m3_table()
    pos = sorted((v, c) for c, v in tab.items() if c < 0x80)
    rng = np.random.default_rng(35)
    cal = rng.standard_normal((32, 16)).astype(np.float32)
    d = oracle.static_scale_fp8(cal)
    x = (rng.standard_normal((8, 16)) * 3).astype(np.float32)    # well past the calibration range
    q, _, _ = oracle.quant_act_static_fp8(x, d)
    assert (q & 0x7F).max() == 0x7E                               # 448 reached, never NaN
    for t in range(8):
        for k in range(16):
            a = abs(float(np.float32(x[t, k]) / d))
            best = 0x7E if a >= 448 else min(pos, key=lambda p: (abs(p[0] - a), p[1] & 1))[1]
            assert (int(q[t, k]) & 0x7F) == best, (t, k, a)
            assert (int(q[t, k]) >> 7) == (1 if x[t, k] < 0 else 0)


def test_static_fp8_zero_step_gives_zero_codes():
    d = oracle.static_scale_fp8(np.zeros((3, 64), np.float32))
    assert d == 0.0
    q, xs, _ = oracle.quant_act_static_fp8(np.ones((2, 64), np.float32), d)
    assert not q.any() and not xs.any()


# LayerNorm form of the smoothed norm ("SmoothQuant: Weight-Only vs W8A8",
# Integration with Transformers: S^-1 folds into gamma and beta) and the fold
# into the previous linear's output columns ("06 -- SmoothQuant", section 7)

def _ln_rows(seed, T=24, K=320, shift=3.0):
    rng = np.random.default_rng(seed)
    h = (rng.standard_normal((T, K)) + shift * rng.standard_normal((T, 1))).astype(np.float32)
    h[:, 11] *= 20
    return h


def test_ln_stats_against_exact_sums():
    h = _ln_rows(40)
    m, r = oracle.ln_stats(h, eps=1e-5)
    for t in range(h.shape[0]):
        row = [float(v) for v in h[t]]
        mu = math.fsum(row) / len(row)                       # correctly rounded sum
        var = math.fsum((v - mu) ** 2 for v in row) / len(row)
        assert abs(float(m[t]) - mu) <= abs(mu) * 2 ** -23 + 1e-12
        rr = 1.0 / math.sqrt(var + float(F32(1e-5)))
        assert abs(float(r[t]) - rr) <= rr * 2 ** -23


def test_ln_absmax_against_torch_layer_norm():
    torch = pytest.importorskip("torch")
    h = _ln_rows(41)
    rng = np.random.default_rng(42)
    g = rng.uniform(0.5, 1.5, h.shape[1]).astype(np.float32)
    b = rng.uniform(-0.3, 0.3, h.shape[1]).astype(np.float32)
    a = oracle.act_absmax_ln(h, g, b, eps=1e-5)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(h.astype(np.float64)), (h.shape[1],),
                                         torch.from_numpy(g.astype(np.float64)),
                                         torch.from_numpy(b.astype(np.float64)),
                                         eps=float(F32(1e-5))).abs().max(dim=0).values.numpy()
    np.testing.assert_allclose(a, ref, rtol=4 * 2 ** -23, atol=1e-6)


def test_ln_fold_invariance_and_alpha_one():
    h = _ln_rows(43)
    K = h.shape[1]
    rng = np.random.default_rng(44)
    g = rng.uniform(0.5, 1.5, K).astype(np.float32)
    b = rng.uniform(-0.3, 0.3, K).astype(np.float32)
    w = (rng.standard_normal((K, 48)) * 0.02).astype(np.float32)
    a = oracle.act_absmax_ln(h, g, b)
    s = oracle.smooth_factor(a, oracle.weight_absmax(w), 0.5)
    gp, bp = oracle.fold_ln(s, g, b)
    _, what = oracle.fold(s, None, w)
    # (LN(h) * gamma/s + beta/s) diag(s) W = (LN(h) * gamma + beta) W, fp64 with the fp32 tensors
    n = (h - h.mean(1, keepdims=True)) / np.sqrt(h.astype(np.float64).var(1, keepdims=True) + 1e-6)
    lhs = (n * gp.astype(np.float64) + bp.astype(np.float64)) @ what.astype(np.float64)
    rhs = (n * g.astype(np.float64) + b.astype(np.float64)) @ w.astype(np.float64)
    assert np.abs(lhs - rhs).max() <= 1e-5 * np.abs(rhs).max()
    # alpha = 1: s = a, every smoothed channel then peaks at 1 (up to the roundings)
    s1 = oracle.smooth_factor(a, oracle.weight_absmax(w), 1.0)
    np.testing.assert_array_equal(s1, a)
    g1, b1 = oracle.fold_ln(s1, g, b)
    np.testing.assert_allclose(oracle.act_absmax_ln(h, g1, b1), 1.0, rtol=4 * 2 ** -23)


def test_quant_act_ln_reduces_to_rms_on_zero_mean_rows():
    # rows built of +-v pairs have an exactly zero mean: LayerNorm with beta = 0
    # is then the RMSNorm form, whose quantizer is pinned above
    rng = np.random.default_rng(45)
    half = rng.standard_normal((16, 160)).astype(np.float32)
    half[:, 3] *= 25
    h = np.empty((16, 320), np.float32)
    h[:, 0::2], h[:, 1::2] = half, -half
    g = rng.uniform(0.5, 1.5, 320).astype(np.float32)
    q, xs, m, r = oracle.quant_act_ln(h, g, None)
    assert not m.any()
    qr, xr, rr = oracle.quant_act(h, g, norm=True)
    np.testing.assert_array_equal(r, rr)
    np.testing.assert_array_equal(xs, xr)
    np.testing.assert_array_equal(q, qr)


def test_quant_act_ln_half_step_bound():
    torch = pytest.importorskip("torch")
    h = _ln_rows(46)
    rng = np.random.default_rng(47)
    g = rng.uniform(0.2, 1.5, h.shape[1]).astype(np.float32)
    b = rng.uniform(-0.5, 0.5, h.shape[1]).astype(np.float32)
    q, xs, _, _ = oracle.quant_act_ln(h, g, b)
    ln = torch.nn.functional.layer_norm(torch.from_numpy(h.astype(np.float64)), (h.shape[1],),
                                        torch.from_numpy(g.astype(np.float64)),
                                        torch.from_numpy(b.astype(np.float64)),
                                        eps=float(F32(1e-6))).numpy()
    np.testing.assert_allclose(xs, np.abs(ln).max(1) / 127, rtol=8 * 2 ** -23)
    err = np.abs(ln - q.astype(np.float64) * xs[:, None].astype(np.float64))
    assert np.all(err <= xs[:, None] * (0.5 + 1e-4))
    assert np.abs(q).max() == 127 and q.min() >= -127


def test_fold_prev_invariance_and_exact_powers_of_two():
    rng = np.random.default_rng(48)
    Kp, K, N, T = 96, 128, 40, 12
    x = rng.standard_normal((T, Kp))
    wp = (rng.standard_normal((Kp, K)) * 0.05).astype(np.float32)
    bp = rng.standard_normal(K).astype(np.float32)
    w = (rng.standard_normal((K, N)) * 0.02).astype(np.float32)
    s = rng.uniform(0.05, 20, K).astype(np.float32)
    wpf, bpf = oracle.fold_prev(s, wp, bp)
    _, what = oracle.fold(s, None, w)
    lhs = (x @ wpf.astype(np.float64) + bpf.astype(np.float64)) @ what.astype(np.float64)
    rhs = (x @ wp.astype(np.float64) + bp.astype(np.float64)) @ w.astype(np.float64)
    assert np.abs(lhs - rhs).max() <= 1e-5 * np.abs(rhs).max()
    s2 = np.exp2(rng.integers(-6, 7, K)).astype(np.float32)
    wq2, bq2 = oracle.fold_prev(s2, wp, bp)
    np.testing.assert_array_equal(wq2.astype(np.float64) * s2[None, :], wp.astype(np.float64))
    np.testing.assert_array_equal(bq2.astype(np.float64) * s2, bp.astype(np.float64))


# GPTQ on the migrated weights ("06 -- SmoothQuant", section 10 names the
# step; the algorithm is the published GPTQ, restated in oracle.gptq)

def _rtn(w_hat):
    return oracle.quant_weight(w_hat)


def test_gptq_with_uncorrelated_inputs_is_round_to_nearest():
    # every calibration token lights one channel: H is diagonal (damping
    # keeps it so), U is diagonal and no error reaches another row
    rng = np.random.default_rng(60)
    K, N = 40, 24
    x = np.zeros((4 * K, K), np.float32)
    for t in range(4 * K):
        x[t, t % K] = rng.uniform(0.5, 3.0)
    w = (rng.standard_normal((K, N)) * 0.05).astype(np.float32)
    q, ws = oracle.gptq(w, x)
    q0, ws0 = _rtn(w)
    np.testing.assert_array_equal(ws, ws0)
    np.testing.assert_array_equal(q, q0)


def test_gptq_two_inputs_closed_form():
    # K = 2: with row 0 rounded, the row-1 weight minimizing the output error
    # (w - w')^T H (w - w') is w1 + (H01 / H11) (w0 - Delta q0)
    rng = np.random.default_rng(61)
    for trial in range(20):
        x = rng.standard_normal((50, 2)).astype(np.float32)
        x[:, 1] += rng.uniform(-2, 2) * x[:, 0]
        w = (rng.standard_normal((2, 12)) * 0.05).astype(np.float32)
        q, ws = oracle.gptq(w, x, damp=0.01)
        X = x.astype(np.float64)
        H = X.T @ X
        H += 0.01 * np.mean(np.diag(H)) * np.eye(2)
        d = ws.astype(np.float64)
        q0 = np.clip(np.rint(w[0].astype(np.float64) / d), -127, 127)
        w1 = w[1].astype(np.float64) + H[0, 1] / H[1, 1] * (w[0] - d * q0)
        np.testing.assert_array_equal(q[:, 0], q0.astype(np.int8))
        np.testing.assert_array_equal(q[:, 1], np.clip(np.rint(w1 / d), -127, 127).astype(np.int8))


def test_gptq_matches_the_explicit_inverse_formulation():
    # the same greedy rounding written with the explicit inverse Hessian of the
    # remaining inputs (optimal brain surgeon updates, the inverse shrunk by
    # Gaussian elimination after each input) instead of a Cholesky factor
    rng = np.random.default_rng(62)
    K, N, T = 24, 10, 200
    x = (rng.standard_normal((T, K)) @ rng.standard_normal((K, K))).astype(np.float32)
    w = (rng.standard_normal((K, N)) * 0.05).astype(np.float32)
    q, ws = oracle.gptq(w, x)
    X = x.astype(np.float64)
    H = X.T @ X
    H += 0.01 * np.mean(np.diag(H)) * np.eye(K)
    Hi = np.linalg.inv(H)
    W = w.astype(np.float64)
    d = ws.astype(np.float64)
    for j in range(K):
        qj = np.clip(np.rint(W[j] / d), -127, 127)
        assert np.array_equal(q[:, j], qj.astype(np.int8)), j
        err = (W[j] - d * qj) / Hi[j, j]
        W -= np.outer(Hi[:, j], err)             # rows already done change too but are never read
        Hi = Hi - np.outer(Hi[:, j], Hi[j, :]) / Hi[j, j]


def test_gptq_lowers_the_layer_error_on_correlated_inputs():
    rng = np.random.default_rng(63)
    K, N, T = 96, 48, 600
    mix = np.eye(K) + rng.standard_normal((K, K)) / np.sqrt(K)
    x = (rng.standard_normal((T, K)) @ mix).astype(np.float32)
    w = (rng.standard_normal((K, N)) * 0.05).astype(np.float32)
    q, ws = oracle.gptq(w, x)
    q0, _ = _rtn(w)
    X = x.astype(np.float64)

    def err(codes):
        return np.linalg.norm(X @ (w.astype(np.float64) - (codes.T * ws[None, :].astype(np.float64))))

    assert err(q) < 0.85 * err(q0)


def test_gptq_dead_inputs_and_zero_columns():
    rng = np.random.default_rng(64)
    K, N = 16, 8
    x = rng.standard_normal((40, K)).astype(np.float32)
    x[:, 5] = 0.0                                   # an input channel calibration never saw
    w = (rng.standard_normal((K, N)) * 0.05).astype(np.float32)
    w[:, 3] = 0.0                                   # an output channel with no weight
    q, ws = oracle.gptq(w, x)
    assert not q[:, 5].any() and not q[3].any() and ws[3] == 0


def test_gptq_output_channels_are_independent():
    # the rounding of one output channel never reads another's weights: the
    # same codes come out of the full weight and of any subset of its columns
    rng = np.random.default_rng(65)
    x = (rng.standard_normal((120, 48)) @ rng.standard_normal((48, 48))).astype(np.float32)
    w = (rng.standard_normal((48, 30)) * 0.05).astype(np.float32)
    q, ws = oracle.gptq(w, x)
    cols = np.array([29, 0, 11, 12])
    qc, wc = oracle.gptq(w, x, columns=cols)
    np.testing.assert_array_equal(qc, q[cols])
    np.testing.assert_array_equal(wc, ws[cols])
