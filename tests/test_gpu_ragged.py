"""GPU parity at any output width N >= 1 and at wide norm-mode calibration.

The pages' only interface is a linear of arbitrary in/out sizes ("Taming the
Outliers", Implementation in PyTorch: SmoothQuantLinear(in_features,
out_features, alpha)), so every call that reads the weight takes any N, with
the ragged end of each row masked.  The weight is placed in a row-padded
buffer whose padding holds 3e38: a kernel that read past column N would raise
a weight maximum or a step far from the oracle's.

Also: norm-mode calibration of rows wider than 8192 (the RMSNorm and LayerNorm
forms, "SmoothQuant and W8A8", The trick; "SmoothQuant: Weight-Only vs W8A8",
Integration with Transformers), checked against the oracle; and the binding's
argument checks, which must refuse before anything is launched.

Bar: weight maxima, folded weights, steps, codes, accumulators and outputs
bit-exact when the oracle is fed the GPU's smoothing factor (and RMS factors);
calibration maxima in norm mode within one fp32 ulp (they inherit the row's
fp64 statistics, summed in another order).
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
import synth  # noqa: E402
import w8a8_int8_gemm_amd as sq  # noqa: E402
from _gptq_check import check_gptq_codes  # noqa: E402
from _gpu_util import DEV, f32, say, to_dev, to_np  # noqa: E402

F32 = np.float32
POISON_BF16 = 0x7F61   # about 3e38
POISON_F32 = np.float32(3e38)


def _ulps(a, b):
    a = np.asarray(a, F32).view(np.int32).astype(np.int64)
    b = np.asarray(b, F32).view(np.int32).astype(np.int64)
    return np.abs(a - b)


def _padded(w: np.ndarray):
    """A device copy of W [K, N] in rows padded to a 16-byte multiple, the
    padding poisoned; returns the [K, N] view."""
    K, N = w.shape
    if w.dtype == np.uint16:
        ld = (N + 7) // 8 * 8
        buf = np.full((K, ld), POISON_BF16, np.uint16)
    else:
        ld = (N + 3) // 4 * 4
        buf = np.full((K, ld), POISON_F32, F32)
    buf[:, :N] = w
    return to_dev(buf)[:, :N]


def _linear(x, gp, wq, wsc, bias, *, norm, out_dtype):
    """sq_w8a8_linear into rows padded to a 16-byte multiple (the ABI's rule
    for leading dimensions); the padding must come back untouched."""
    T, K = x.shape
    N = wq.shape[0]
    per = 8 if out_dtype == torch.bfloat16 else 4
    ybuf = torch.full((T, (N + per - 1) // per * per), 5.0, dtype=out_dtype, device=DEV)
    work = torch.empty(sq.sq_linear_workspace_bytes(T, K), dtype=torch.uint8, device=DEV)
    dbg = dict(dbg_xq=torch.empty((T, K), dtype=torch.int8, device=DEV), dbg_x_scale=f32(T),
               dbg_row_rscale=f32(T) if norm else None)
    sq.sq_w8a8_linear(x, gp, wq, wsc, ybuf[:, :N], work, norm=norm, bias=bias, **dbg)
    return ybuf, dbg


RAGGED = [
    # (workload, sizes, weight dtype): which weight-quantization path runs
    ("qproj_prefill", dict(T=300, Tc=500, K=512, N=77), "bf16"),       # strip kernel
    ("qproj_prefill", dict(T=96, Tc=200, K=256, N=1), "bf16"),         # strip kernel, one column
    ("rmsnorm_qkv", dict(T=257, Tc=300, K=1024, N=1001), "bf16"),      # norm mode, strip kernel
    ("qproj_prefill", dict(T=130, Tc=256, K=4608, N=1001), "bf16"),    # three-launch path (K > 4096)
    ("tiny", dict(N=77), "f32"),                                        # fp32 weight, fp32 out
    ("gate_up", dict(T=70, Tc=128, K=256, N=3), "f32"),
]


@pytest.mark.parametrize("name,sizes,wdt", RAGGED)
def test_ragged_n_end_to_end(name, sizes, wdt):
    wl = synth.WORKLOADS[name].with_sizes(**sizes)
    say(f"ragged N {name} {sizes} w {wdt}")
    inp = synth.make_inputs(wl)
    K, N, T = wl.K, wl.N, wl.T
    w_np = inp.w if wdt == "bf16" or inp.w.dtype == F32 else synth.bf16_bits_to_f32(inp.w)
    w = _padded(w_np)
    g = None if inp.gamma is None else to_dev(inp.gamma)
    a, wm, s = f32(K), f32(K), f32(K)
    sq.sq_calibrate(to_dev(inp.x_cal), w, wl.alpha, a, wm, s, norm=wl.norm, gamma=g)
    gp, w_hat = f32(K), f32(K * N)
    sq.sq_smooth_fold(s, g, gp, w, w_hat)
    wq, wsc = torch.empty((N, K), dtype=torch.int8, device=DEV), f32(N)
    sq.sq_quant_weight(w, s, wq, wsc)
    wq8, wsc8 = torch.empty((N, K), dtype=torch.uint8, device=DEV), f32(N)
    sq.sq_quant_weight_fp8(w, s, wq8, wsc8)
    out_dt = torch.bfloat16 if wl.io_dtype == "bf16" else torch.float32
    ybuf, dbg = _linear(to_dev(inp.x), gp, wq, wsc, to_dev(inp.bias), norm=wl.norm,
                        out_dtype=out_dt)
    torch.cuda.synchronize()
    yb = to_np(ybuf)
    y = yb[:, :N]
    fill = np.uint16(0x40A0) if out_dt == torch.bfloat16 else F32(5.0)   # 5.0
    assert (yb[:, N:] == fill).all()                                      # padding untouched
    np.testing.assert_array_equal(to_np(wm), oracle.weight_absmax(w_np))
    a_ref = oracle.act_absmax(inp.x_cal, norm=wl.norm, gamma=inp.gamma)
    if wl.norm:
        assert _ulps(to_np(a), a_ref).max() <= 1
    else:
        np.testing.assert_array_equal(to_np(a), a_ref)
    s_h = to_np(s)
    assert _ulps(s_h, oracle.smooth_factor(to_np(a), to_np(wm), wl.alpha)).max() <= 1
    gp_ref, what_ref = oracle.fold(s_h, inp.gamma, w_np)
    np.testing.assert_array_equal(to_np(gp), gp_ref)
    np.testing.assert_array_equal(to_np(w_hat).reshape(K, N), what_ref)
    qw_ref, ws_ref = oracle.quant_weight(what_ref)
    np.testing.assert_array_equal(to_np(wsc), ws_ref)
    np.testing.assert_array_equal(to_np(wq), qw_ref)
    qw8_ref, ws8_ref = oracle.quant_weight_fp8(what_ref)
    np.testing.assert_array_equal(to_np(wsc8), ws8_ref)
    np.testing.assert_array_equal(to_np(wq8), qw8_ref)
    r = to_np(dbg["dbg_row_rscale"]) if wl.norm else None
    fed = oracle.linear(inp.x, gp_ref, qw_ref, ws_ref, inp.bias, norm=wl.norm, r=r,
                        out_bf16=wl.io_dtype == "bf16")
    np.testing.assert_array_equal(to_np(dbg["dbg_xq"]), fed["q"])
    np.testing.assert_array_equal(y, fed["y"])


def test_ragged_n_gptq():
    rng = np.random.default_rng(90)
    Tc, K, N = 200, 256, 77
    x = rng.standard_normal((Tc, K)).astype(F32)
    x[:, 1:] += 0.5 * x[:, :-1]
    w = (rng.standard_normal((K, N)) * 0.05).astype(F32)
    say(f"ragged N gptq K={K} N={N}")
    wq, wsc = torch.empty((N, K), dtype=torch.int8, device=DEV), f32(N)
    work = torch.empty(sq.sq_gptq_workspace_bytes(Tc, K, N), dtype=torch.uint8, device=DEV)
    sq.sq_quant_weight_gptq(to_dev(x), None, _padded(w), None, wq, wsc, work)
    torch.cuda.synchronize()
    U, dead = oracle.gptq_factor(oracle.smoothed_act(x))
    _, ws_ref = oracle.gptq_round(w, U, dead)
    np.testing.assert_array_equal(to_np(wsc), ws_ref)
    check_gptq_codes(to_np(wq), w, U, dead)


@pytest.mark.parametrize("K,dt", [(12288, "bf16"), (8256, "f32"), (20480, "bf16")])
def test_wide_norm_calibration(K, dt):
    wl = synth.WORKLOADS["rmsnorm_qkv"].with_sizes(Tc=301, K=K, N=40, io_dtype=dt)
    say(f"wide rms calibration K={K} {dt}")
    inp = synth.make_inputs(wl, evaluation=False)
    a = f32(K)
    sq.sq_calibrate(to_dev(inp.x_cal), None, wl.alpha, a, norm=True, gamma=to_dev(inp.gamma))
    a2 = f32(K)
    sq.sq_calibrate(to_dev(inp.x_cal[:150]), None, wl.alpha, a2, norm=True,
                    gamma=to_dev(inp.gamma))
    sq.sq_calibrate(to_dev(inp.x_cal[150:]), None, wl.alpha, a2, norm=True,
                    gamma=to_dev(inp.gamma), accumulate=True)
    torch.cuda.synchronize()
    a_ref = oracle.act_absmax(inp.x_cal, norm=True, gamma=inp.gamma)
    d = _ulps(to_np(a), a_ref)
    assert d.max() <= 1 and (d == 0).mean() > 0.99
    np.testing.assert_array_equal(to_np(a2), to_np(a))


@pytest.mark.parametrize("K,dt", [(12288, "bf16"), (9216, "f32")])
def test_wide_layernorm_calibration(K, dt):
    wl = synth.WORKLOADS["layernorm_qkv"].with_sizes(T=8, K=K, N=40, Tc=203, io_dtype=dt)
    say(f"wide ln calibration K={K} {dt}")
    inp = synth.make_inputs(wl, evaluation=False)
    a = f32(K)
    sq.sq_calibrate_ln(to_dev(inp.x_cal), None, wl.alpha, a, gamma=to_dev(inp.gamma),
                       beta=to_dev(inp.beta))
    torch.cuda.synchronize()
    a_ref = oracle.act_absmax_ln(inp.x_cal, inp.gamma, inp.beta)
    np.testing.assert_allclose(to_np(a), a_ref, rtol=2.0 ** -20, atol=0)


def test_wide_norm_end_to_end():
    wl = synth.WORKLOADS["rmsnorm_qkv"].with_sizes(T=65, Tc=130, K=12288, N=264)
    say(f"wide norm end to end K={wl.K}")
    inp = synth.make_inputs(wl)
    K = wl.K
    g, w = to_dev(inp.gamma), to_dev(inp.w)
    a, wm, s = f32(K), f32(K), f32(K)
    sq.sq_calibrate(to_dev(inp.x_cal), w, wl.alpha, a, wm, s, norm=True, gamma=g)
    gp = f32(K)
    sq.sq_smooth_fold(s, g, gp)
    wq, wsc = torch.empty((wl.N, K), dtype=torch.int8, device=DEV), f32(wl.N)
    sq.sq_quant_weight(w, s, wq, wsc)
    ybuf, dbg = _linear(to_dev(inp.x), gp, wq, wsc, to_dev(inp.bias), norm=True,
                        out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    gp_ref, qw_ref, ws_ref = oracle.prepare_weight(inp.w, to_np(s), inp.gamma)
    np.testing.assert_array_equal(to_np(wq), qw_ref)
    fed = oracle.linear(inp.x, gp_ref, qw_ref, ws_ref, inp.bias, norm=True,
                        r=to_np(dbg["dbg_row_rscale"]))
    np.testing.assert_array_equal(to_np(ybuf)[:, :wl.N], fed["y"])


def test_binding_refuses_bad_tensors_before_launch():
    """A host tensor, a wrong dtype or an undersized output is a ValueError
    raised before the C call: the output buffer keeps its sentinel."""
    say("binding argument checks")
    T, K, N = 64, 128, 40
    xq = torch.zeros((T, K), dtype=torch.int8, device=DEV)
    wq = torch.zeros((N, K), dtype=torch.int8, device=DEV)
    xs, ws = f32(T, 1.0), f32(N, 1.0)
    y = torch.full((T, N), 7.0, dtype=torch.bfloat16, device=DEV)
    bad = [
        dict(xq=xq.cpu()),                                     # host tensor
        dict(wq=wq.to(torch.int16)),                           # dtype
        dict(wq=wq[:, :64]),                                   # K mismatch
        dict(x_scale=f32(T - 1)),                              # too few scales
        dict(w_scale=f32(N - 1)),
        dict(y=torch.empty((T - 1, N), dtype=torch.bfloat16, device=DEV)),
        dict(y=torch.empty((T, N), dtype=torch.float16, device=DEV)),
        dict(bias=f32(N - 1)),
    ]
    for kw in bad:
        args = dict(xq=xq, x_scale=xs, wq=wq, w_scale=ws, y=y)
        args.update(kw)
        with pytest.raises(ValueError):
            sq.sq_gemm_w8a8(args["xq"], args["x_scale"], args["wq"], args["w_scale"], args["y"],
                            bias=kw.get("bias"))
    x = torch.zeros((T, K), dtype=torch.bfloat16, device=DEV)
    work = torch.empty(sq.sq_linear_workspace_bytes(T, K), dtype=torch.uint8, device=DEV)
    with pytest.raises(ValueError):
        sq.sq_w8a8_linear(x, None, wq, ws, y, work, dbg_xq=torch.empty((T, K - 8),
                                                                         dtype=torch.int8,
                                                                         device=DEV))
    with pytest.raises(ValueError):
        sq.sq_quant_act(x, f32(K - 64), torch.empty((T, K), dtype=torch.int8, device=DEV), xs)
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())


def test_deep_subnormal_steps():
    """Tokens (and weight columns) whose maximum is so small that the step is a
    deep subnormal, rounded far from max / 127 (or / 448): quotients then pass
    127.5 (448) and must clamp as the definition does, in both formats."""
    say("deep subnormal steps")
    K = 256
    rng = np.random.default_rng(91)
    rows = []
    for amax in (2e-43, 7e-42, 3e-40, 1e-38):
        r = (rng.uniform(-1.0, 1.0, K) * amax).astype(F32)
        r[0] = F32(amax)
        r[1] = F32(-amax)
        rows.append(r)
    x = np.stack(rows)
    T = x.shape[0]
    xq, xs = torch.empty((T, K), dtype=torch.int8, device=DEV), f32(T)
    sq.sq_quant_act(to_dev(x), None, xq, xs)
    xq8, xs8 = torch.empty((T, K), dtype=torch.uint8, device=DEV), f32(T)
    sq.sq_quant_act_fp8(to_dev(x), None, xq8, xs8)
    w = np.ascontiguousarray(x.T)                         # the same values as weight columns
    wq, wsc = torch.empty((T, K), dtype=torch.int8, device=DEV), f32(T)
    sq.sq_quant_weight(_padded(w), None, wq, wsc)
    wq8, wsc8 = torch.empty((T, K), dtype=torch.uint8, device=DEV), f32(T)
    sq.sq_quant_weight_fp8(_padded(w), None, wq8, wsc8)
    torch.cuda.synchronize()
    q_ref, xs_ref, _ = oracle.quant_act(x, None)
    assert np.abs(x[0] / xs_ref[0]).max() > 127.5          # the case that needs the clamp
    np.testing.assert_array_equal(to_np(xs), xs_ref)
    np.testing.assert_array_equal(to_np(xq), q_ref)
    q8_ref, xs8_ref, _ = oracle.quant_act_fp8(x)
    np.testing.assert_array_equal(to_np(xs8), xs8_ref)
    np.testing.assert_array_equal(to_np(xq8), q8_ref)
    qw_ref, ws_ref = oracle.quant_weight(w)
    np.testing.assert_array_equal(to_np(wsc), ws_ref)
    np.testing.assert_array_equal(to_np(wq), qw_ref)
    qw8_ref, ws8_ref = oracle.quant_weight_fp8(w)
    np.testing.assert_array_equal(to_np(wsc8), ws8_ref)
    np.testing.assert_array_equal(to_np(wq8), qw8_ref)
