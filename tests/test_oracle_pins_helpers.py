"""Pins of the oracle's helper functions that the GPU tests use as checkers.

Each helper is checked by a function ``_pin_*`` against something other than
the helper itself: the pinned C epilogue, hand-worked fp32 roundings, an
fsum/fp64 evaluation written out element by element, and torch's own
LayerNorm / RMSNorm.  Each ``_pin_*`` is then run once more on copies of the
helper with a plausible mistake planted (a multiply order swapped, r_t
omitted, beta dropped, ...) and must reject every one of them.

Sources: the dequantization epilogue Y = scale_x * scale_w * Y_int32 ("06 --
SmoothQuant", section 7; "Taming the Outliers", System Architecture step I6);
the smoothed activation x^ = (h * r_t) * gamma' the quantizer and GPTQ's
Hessian read ("SmoothQuant and W8A8", The trick; "06 -- SmoothQuant",
section 10); the LayerNorm reference of the per-layer error ("SmoothQuant:
Weight-Only vs W8A8", Integration with Transformers; "SmoothQuant and W8A8",
One layer, measured).
"""
import math

import numpy as np
import pytest

import oracle

F32 = np.float32


def _f(v):
    """A Python float rounded to fp32 (numpy rounds to nearest even)."""
    return float(F32(v))


# ---------------------------------------------------------------------------
# epilogue_f32acc: y = fp32(fp32(xs[t] * ws[n]) * acc[t,n]) + b[n]
# ---------------------------------------------------------------------------

def _pin_epilogue_f32acc(fn):
    rng = np.random.default_rng(7)
    T, N = 37, 29
    # integer accumulators below 2^24 are exact in fp32, so the fp32-accumulator
    # form must equal the pinned int32 epilogue bit for bit
    acc = rng.integers(-(1 << 24) + 1, 1 << 24, size=(T, N)).astype(np.int32)
    acc[0, :4] = [0, 1, -1, (1 << 24) - 1]
    xs = (rng.uniform(0.5, 2.0, T) * 2.0 ** rng.integers(-12, -4, T)).astype(F32)
    ws = (rng.uniform(0.5, 2.0, N) * 2.0 ** rng.integers(-12, -4, N)).astype(F32)
    b = rng.normal(0, 0.05, N).astype(F32)
    for bias in (None, b):
        want = oracle.epilogue(acc, xs, ws, bias)
        got = fn(acc.astype(F32), xs, ws, bias)
        assert got.dtype == F32 and got.shape == (T, N)
        np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
    # hand-worked rounding: xs = ws = 1 + 2^-23, acc = 3.
    #   fp32(xs * ws) = 1 + 2^-22 (the 2^-46 term is lost), times 3 is
    #   3 + 3 * 2^-22, exact in fp32 (ulp 2^-22 at 3).  Multiplying ws * acc
    #   first would give fp32(3 + 1.5 * 2^-22) = 3 + 2^-21 (tie to even), then
    #   times xs 3 + 2^-20: the order is visible.
    e = 1.0 + 2.0 ** -23
    y = fn(np.array([[3.0]], F32), np.array([e], F32), np.array([e], F32), None)
    assert float(y[0, 0]) == 3.0 + 3 * 2.0 ** -22
    # bias added after the product, in fp32: 0.375 + 2^-30 rounds back to 0.375
    y = fn(np.array([[3.0]], F32), np.array([0.5], F32), np.array([0.25], F32),
           np.array([2.0 ** -30], F32))
    assert float(y[0, 0]) == 0.375
    # and a bias that is kept: 0.375 + 1.0 = 1.375 exactly
    y = fn(np.array([[3.0]], F32), np.array([0.5], F32), np.array([0.25], F32),
           np.array([1.0], F32))
    assert float(y[0, 0]) == 1.375
    # zero accumulators give the bias exactly
    y = fn(np.zeros((2, 3), F32), np.ones(2, F32), np.ones(3, F32), b[:3])
    np.testing.assert_array_equal(y, np.broadcast_to(b[:3], (2, 3)))


def test_epilogue_f32acc_pins():
    _pin_epilogue_f32acc(oracle.epilogue_f32acc)


def _epi_order_swapped(acc, xs, ws, bias=None):   # xs * fp32(ws * acc)
    acc = np.asarray(acc, F32)
    y = (np.asarray(xs, F32)[:, None] * (np.asarray(ws, F32)[None, :] * acc).astype(F32)).astype(F32)
    return y if bias is None else (y + np.asarray(bias, F32)[None, :]).astype(F32)


def _epi_fp64(acc, xs, ws, bias=None):            # one rounding at the end
    y = (np.asarray(xs, np.float64)[:, None] * np.asarray(ws, np.float64)[None, :]
         * np.asarray(acc, np.float64))
    if bias is not None:
        y = y + np.asarray(bias, np.float64)[None, :]
    return y.astype(F32)


def _epi_bias_dropped(acc, xs, ws, bias=None):
    return oracle.epilogue_f32acc(acc, xs, ws, None)


def _epi_transposed_scales(acc, xs, ws, bias=None):
    acc = np.asarray(acc, F32)
    T, N = acc.shape
    xs2 = np.resize(np.asarray(ws, F32), T)
    ws2 = np.resize(np.asarray(xs, F32), N)
    return oracle.epilogue_f32acc(acc, xs2, ws2, bias)


@pytest.mark.parametrize("mutant", [_epi_order_swapped, _epi_fp64, _epi_bias_dropped,
                                    _epi_transposed_scales])
def test_epilogue_f32acc_pins_reject_planted_mistakes(mutant):
    with pytest.raises(AssertionError):
        _pin_epilogue_f32acc(mutant)


# ---------------------------------------------------------------------------
# smoothed_act: x^ = fp32(x * gamma') or fp32(fp32(h * r_t) * gamma')
# ---------------------------------------------------------------------------

def _rows(seed, T=19, K=192):
    rng = np.random.default_rng(seed)
    h = (rng.standard_normal((T, K)) * rng.uniform(0.2, 3.0, (T, 1))).astype(F32)
    h[:, 5] *= 30.0
    h[3] = 0.0                      # a zero row: r_t = 1/sqrt(eps)
    g = rng.uniform(0.05, 2.0, K).astype(F32)
    return h, g


def _fsum_r(h, eps):
    """r_t = fp32(1 / sqrt(mean_k h^2 + fp32(eps))) from a correctly rounded sum."""
    K = h.shape[1]
    out = []
    for row in h:
        ms = math.fsum(float(v) * float(v) for v in row) / K
        out.append(_f(1.0 / math.sqrt(ms + _f(eps))))
    return np.array(out, F32)


def _pin_smoothed_act(fn):
    eps = 1e-6
    h, g = _rows(11)
    T, K = h.shape
    # plain mode, element by element in Python floats rounded to fp32
    got = fn(h, g)
    assert got.dtype == F32 and got.shape == (T, K)
    for t in (0, 1, 7, T - 1):
        for k in range(K):
            assert float(got[t, k]) == _f(float(h[t, k]) * float(g[k]))
    # norm mode with the factor given: fp32(fp32(h * r_t) * gamma')
    r = _fsum_r(h, eps)
    got = fn(h, g, norm=True, r=r)
    for t in range(T):
        for k in range(0, K, 3):
            assert float(got[t, k]) == _f(_f(float(h[t, k]) * float(r[t])) * float(g[k]))
    # norm mode computing r_t itself: the same values, r_t within one fp32 ulp
    # of the fsum evaluation (fp64 sums in another order)
    own = fn(h, g, norm=True)
    for t in range(T):
        if not np.array_equal(own[t], got[t]):
            rt = float(r[t])
            alt = [rt * (1 + 2.0 ** -23), rt * (1 - 2.0 ** -24)]
            assert any(np.array_equal(own[t], np.array(
                [_f(_f(float(h[t, k]) * _f(a)) * float(g[k])) for k in range(K)], F32))
                for a in alt)
    # the column maxima are the pinned calibration absmax of the same activation
    np.testing.assert_array_equal(np.abs(fn(h, g, norm=True)).max(0),
                                  oracle.act_absmax(h, norm=True, gamma=g))
    np.testing.assert_array_equal(np.abs(fn(h, np.ones(K, F32))).max(0), oracle.act_absmax(h))
    # and the row maxima / 127 are the pinned per-token steps
    _, xs, _ = oracle.quant_act(h, g, norm=True, r=r)
    np.testing.assert_array_equal((np.abs(got).max(1) / F32(127)).astype(F32), xs)
    # gamma' = NULL means ones
    np.testing.assert_array_equal(fn(h, None), h)


def test_smoothed_act_pins():
    _pin_smoothed_act(oracle.smoothed_act)


def _sa_r_omitted(x, gamma_f=None, *, norm=False, r=None, eps=1e-6):
    return oracle.smoothed_act(x, gamma_f)


def _sa_gamma_first(x, gamma_f=None, *, norm=False, r=None, eps=1e-6):
    if not norm:
        return oracle.smoothed_act(x, gamma_f)
    rr = _fsum_r(x, eps) if r is None else np.asarray(r, F32)
    g = np.ones(x.shape[1], F32) if gamma_f is None else np.asarray(gamma_f, F32)
    return ((x * g[None, :]).astype(F32) * rr[:, None]).astype(F32)


def _sa_one_rounding(x, gamma_f=None, *, norm=False, r=None, eps=1e-6):
    if not norm:
        return oracle.smoothed_act(x, gamma_f)
    rr = _fsum_r(x, eps) if r is None else np.asarray(r, F32)
    g = np.ones(x.shape[1], F32) if gamma_f is None else np.asarray(gamma_f, F32)
    return (x.astype(np.float64) * rr[:, None].astype(np.float64) * g[None, :]).astype(F32)


def _sa_rms_without_mean(x, gamma_f=None, *, norm=False, r=None, eps=1e-6):
    if not norm or r is not None:
        return oracle.smoothed_act(x, gamma_f, norm=norm, r=r, eps=eps)
    ss = (x.astype(np.float64) ** 2).sum(1)      # sum, not mean
    rr = (1.0 / np.sqrt(ss + float(F32(eps)))).astype(F32)
    return oracle.smoothed_act(x, gamma_f, norm=True, r=rr)


@pytest.mark.parametrize("mutant", [_sa_r_omitted, _sa_gamma_first, _sa_one_rounding,
                                    _sa_rms_without_mean])
def test_smoothed_act_pins_reject_planted_mistakes(mutant):
    with pytest.raises(AssertionError):
        _pin_smoothed_act(mutant)


# ---------------------------------------------------------------------------
# reference_ln_fp64 / reference_fp64 / rel_error: the fp64 layer references
# ---------------------------------------------------------------------------

def _ln_inputs(seed=21, T=23, K=96, N=40):
    rng = np.random.default_rng(seed)
    h = (rng.standard_normal((T, K)) + 3.0 * rng.standard_normal((T, 1))).astype(F32)
    h[:, 7] *= 25.0
    w = (rng.standard_normal((K, N)) * 0.05).astype(F32)
    g = rng.uniform(0.5, 1.5, K).astype(F32)
    be = rng.normal(0, 0.3, K).astype(F32)
    b = rng.normal(0, 0.05, N).astype(F32)
    return h, w, g, be, b


def _pin_reference_ln(fn):
    torch = pytest.importorskip("torch")
    h, w, g, be, b = _ln_inputs()
    eps = 1e-6
    t64 = lambda a: torch.from_numpy(np.asarray(a, np.float64))  # noqa: E731
    for gam, bet, bias in ((g, be, b), (None, None, None), (g, None, b), (None, be, None)):
        ln = torch.nn.functional.layer_norm(t64(h), (h.shape[1],),
                                            None if gam is None else t64(gam),
                                            None if bet is None else t64(bet), eps=_f(eps))
        want = ln @ t64(w)
        if bias is not None:
            want = want + t64(bias)
        got = fn(h, w, bias, gamma=gam, beta=bet, eps=eps)
        np.testing.assert_allclose(got, want.numpy(), rtol=1e-11, atol=1e-12)
    # bf16 inputs are widened exactly (the bits shifted into the high half)
    hb = (h.view(np.uint32) >> 16).astype(np.uint16)
    hw = (hb.astype(np.uint32) << 16).view(F32)
    np.testing.assert_allclose(fn(hb, w, gamma=g, beta=be), fn(hw, w, gamma=g, beta=be),
                               rtol=0, atol=0)


def test_reference_ln_fp64_pins():
    _pin_reference_ln(oracle.reference_ln_fp64)


def _ln_beta_dropped(h, w, bias=None, *, gamma=None, beta=None, eps=1e-6):
    return oracle.reference_ln_fp64(h, w, bias, gamma=gamma, beta=None, eps=eps)


def _ln_as_rms(h, w, bias=None, *, gamma=None, beta=None, eps=1e-6):
    X = h.astype(np.float64)
    X = X / np.sqrt((X * X).mean(1, keepdims=True) + _f(eps))
    if gamma is not None:
        X = X * gamma.astype(np.float64)
    if beta is not None:
        X = X + beta.astype(np.float64)
    Y = X @ w.astype(np.float64)
    return Y if bias is None else Y + bias.astype(np.float64)


def _ln_gamma_on_beta(h, w, bias=None, *, gamma=None, beta=None, eps=1e-6):
    X = h.astype(np.float64)
    X = (X - X.mean(1, keepdims=True)) / np.sqrt(X.var(1, keepdims=True) + _f(eps))
    g = 1.0 if gamma is None else gamma.astype(np.float64)
    bb = 0.0 if beta is None else beta.astype(np.float64)
    Y = ((X + bb) * g) @ w.astype(np.float64)
    return Y if bias is None else Y + bias.astype(np.float64)


def _ln_no_eps(h, w, bias=None, *, gamma=None, beta=None, eps=1e-6):
    return oracle.reference_ln_fp64(h, w, bias, gamma=gamma, beta=beta, eps=0.0)


def _ln_bias_dropped(h, w, bias=None, *, gamma=None, beta=None, eps=1e-6):
    return oracle.reference_ln_fp64(h, w, None, gamma=gamma, beta=beta, eps=eps)


@pytest.mark.parametrize("mutant", [_ln_beta_dropped, _ln_as_rms, _ln_gamma_on_beta, _ln_no_eps,
                                    _ln_bias_dropped])
def test_reference_ln_fp64_pins_reject_planted_mistakes(mutant):
    with pytest.raises(AssertionError):
        _pin_reference_ln(mutant)


def _pin_reference_rms(fn):
    torch = pytest.importorskip("torch")
    h, w, g, _, b = _ln_inputs(22)
    eps = 1e-6
    t64 = lambda a: torch.from_numpy(np.asarray(a, np.float64))  # noqa: E731
    rms = torch.nn.functional.rms_norm(t64(h), (h.shape[1],), t64(g), eps=_f(eps))
    np.testing.assert_allclose(fn(h, w, b, norm=True, gamma=g, eps=eps),
                               (rms @ t64(w) + t64(b)).numpy(), rtol=1e-11, atol=1e-12)
    # plain mode on a tiny case against fsum dot products
    x, ww = h[:3, :8], w[:8, :5]
    got = fn(x, ww)
    for t in range(3):
        for n in range(5):
            want = math.fsum(float(x[t, k]) * float(ww[k, n]) for k in range(8))
            assert abs(got[t, n] - want) <= 1e-12 * (1 + abs(want))


def test_reference_fp64_pins():
    _pin_reference_rms(oracle.reference_fp64)


def _rms_gamma_dropped(x, w, bias=None, *, norm=False, gamma=None, eps=1e-6):
    return oracle.reference_fp64(x, w, bias, norm=norm, gamma=None, eps=eps)


def _rms_with_mean(x, w, bias=None, *, norm=False, gamma=None, eps=1e-6):
    if not norm:
        return oracle.reference_fp64(x, w, bias)
    return oracle.reference_ln_fp64(x, w, bias, gamma=gamma, eps=eps)


@pytest.mark.parametrize("mutant", [_rms_gamma_dropped, _rms_with_mean])
def test_reference_fp64_pins_reject_planted_mistakes(mutant):
    with pytest.raises(AssertionError):
        _pin_reference_rms(mutant)


def test_rel_error_is_the_frobenius_ratio():
    ref = np.array([[3.0, 0.0], [0.0, 4.0]])
    y = np.array([[3.0, 0.0], [0.0, 0.0]], F32)
    assert oracle.rel_error(ref, y) == 0.8          # ||(0,0,0,4)|| / ||(3,0,0,4)|| = 4/5
    # bf16 bits are widened: 0x4040 is 3.0, 0x4080 is 4.0
    yb = np.array([[0x4040, 0], [0, 0x4080]], np.uint16)
    assert oracle.rel_error(ref, yb) == 0.0
