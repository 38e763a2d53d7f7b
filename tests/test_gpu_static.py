"""GPU parity of the static per-tensor activation step (one scale for every
token, from the calibration tokens' maximum) against the CPU oracle.

The same bar as test_gpu_parity: the step bit-exact (a maximum and one
division, order-free), codes and int32 accumulators bit-exact when both sides
are fed the same step (and RMSNorm factors), bf16 outputs bit-exact when fed
the same scales.  Covers clipping past the calibrated maximum, a zero step,
norm mode, the K > 8192 path and ragged shapes.
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
from _gpu_util import DEV, f32, gpu_prepare_weight, say, to_dev, to_np  # noqa: E402


def _check_step(d_gpu, d_ref, norm):
    """Bit-exact without a norm (a maximum and one division).  In norm mode the
    step inherits the RMSNorm factor of the maximal token, which both sides
    round from an fp64 sum taken in different orders: within one fp32 ulp."""
    a = np.array([d_gpu], np.float32).view(np.int32).astype(np.int64)
    b = np.array([d_ref], np.float32).view(np.int32).astype(np.int64)
    assert abs(int(a[0] - b[0])) <= (1 if norm else 0), (d_gpu, d_ref)


def _gpu_static_scale(xc, gp, *, norm, gamma=None):
    """The GPU route: channel absmax (norm mode: of h * r_t, gamma = NULL),
    then max_j a_j * |gamma'_j| / 127."""
    K = xc.shape[1]
    a = f32(K)
    sq.sq_calibrate(xc, None, 0.5, a, norm=norm, gamma=None)
    d = f32(1)
    sq.sq_act_static_scale(a, gp, d)
    return d


@pytest.mark.parametrize("T,K,norm,dt", [(64, 512, False, "bf16"), (200, 4096, False, "bf16"),
                                         (37, 1344, True, "bf16"), (96, 320, False, "f32"),
                                         (24, 8192, True, "bf16"), (8, 16384, False, "bf16")])
def test_static_step_and_codes(T, K, norm, dt):
    wl = synth.WORKLOADS["rmsnorm_qkv" if norm else "qproj_prefill"].with_sizes(
        T=T, Tc=2 * T, K=K, N=64)
    if dt == "f32":
        wl = wl.with_sizes(io_dtype="f32")
    say(f"static step T={T} K={K} norm={norm} {dt}")
    inp = synth.make_inputs(wl)
    rng = np.random.default_rng(T + K)
    gp_h = rng.uniform(0.3, 2.0, K).astype(np.float32)
    gp = to_dev(gp_h)
    d = _gpu_static_scale(to_dev(inp.x_cal), gp, norm=norm)
    d_ref = oracle.static_scale(inp.x_cal, gp_h, norm=norm)
    _check_step(to_np(d)[0], d_ref, norm)
    d_ref = to_np(d)[0]   # both sides quantize with the same step from here on
    # evaluation tokens, some of them past the calibrated range
    x = to_dev(inp.x)
    xq = torch.empty((T, K), dtype=torch.int8, device=DEV)
    xs, rr = f32(T), f32(T)
    sq.sq_quant_act_static(x, gp, d, xq, xs, norm=norm, row_rscale=rr if norm else None)
    torch.cuda.synchronize()
    r_gpu = to_np(rr) if norm else None
    q_ref, xs_ref, _ = oracle.quant_act_static(inp.x, d_ref, gp_h, norm=norm, r=r_gpu)
    np.testing.assert_array_equal(to_np(xq), q_ref)
    np.testing.assert_array_equal(to_np(xs), xs_ref)


def test_static_clipping_and_zero_step():
    say("static clipping and zero step")
    rng = np.random.default_rng(3)
    K, T = 1024, 40
    x = (rng.standard_normal((T, K)) * 4).astype(np.float32)
    x[:, 7] *= 50                                       # far past the step's range
    xd = to_dev(x)
    for delta in (np.float32(0.01), np.float32(1e-3), np.float32(0.0), np.float32(1e-40)):
        d = to_dev(np.array([delta], np.float32))
        xq = torch.empty((T, K), dtype=torch.int8, device=DEV)
        xs = f32(T)
        sq.sq_quant_act_static(xd, None, d, xq, xs)
        torch.cuda.synchronize()
        q_ref, xs_ref, _ = oracle.quant_act_static(x, delta)
        np.testing.assert_array_equal(to_np(xq), q_ref)
        np.testing.assert_array_equal(to_np(xs), xs_ref)
        if delta > 0:
            assert np.abs(to_np(xq)).max() == 127


@pytest.mark.parametrize("name,sizes", [("qproj_prefill", dict(T=300, Tc=512, K=1024, N=640)),
                                        ("rmsnorm_qkv", dict(T=130, Tc=256, K=2048, N=384))])
def test_static_linear_end_to_end(name, sizes):
    wl = synth.WORKLOADS[name].with_sizes(**sizes)
    say(f"static linear {name} {sizes}")
    inp = synth.make_inputs(wl)
    T, K, N = wl.T, wl.K, wl.N
    g = None if inp.gamma is None else to_dev(inp.gamma)
    xc, w = to_dev(inp.x_cal), to_dev(inp.w)
    a, wm, s = f32(K), f32(K), f32(K)
    sq.sq_calibrate(xc, w, wl.alpha, a, wm, s, norm=wl.norm, gamma=g)
    gp, wq, wsc = gpu_prepare_weight(w, s, g)
    d = _gpu_static_scale(xc, gp, norm=wl.norm)
    y = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
    work = torch.empty(sq.sq_linear_workspace_bytes(T, K), dtype=torch.uint8, device=DEV)
    dbg_xq = torch.empty((T, K), dtype=torch.int8, device=DEV)
    rr = f32(T)
    sq.sq_w8a8_linear_static(to_dev(inp.x), gp, d, wq, wsc, y, work, norm=wl.norm,
                             bias=to_dev(inp.bias), dbg_xq=dbg_xq,
                             dbg_row_rscale=rr if wl.norm else None)
    torch.cuda.synchronize()
    gp_h = to_np(gp)
    d_ref = oracle.static_scale(inp.x_cal, gp_h, norm=wl.norm)
    _check_step(to_np(d)[0], d_ref, wl.norm)
    d_ref = to_np(d)[0]
    _, qw_ref, ws_ref = oracle.prepare_weight(inp.w, to_np(s), inp.gamma)
    out = oracle.linear_static(inp.x, d_ref, gp_h, qw_ref, ws_ref, inp.bias, norm=wl.norm,
                               r=to_np(rr) if wl.norm else None)
    np.testing.assert_array_equal(to_np(dbg_xq), out["q"])
    np.testing.assert_array_equal(to_np(y), out["y"])
    # the static step is never finer than the per-token ones: error is reported, not gated
    ref = oracle.reference_fp64(inp.x, inp.w, inp.bias, norm=wl.norm, gamma=inp.gamma)
    err = oracle.rel_error(ref, to_np(y))
    say(f"  static-step layer error {err:.4%}")
    assert err < 0.2


@pytest.mark.parametrize("T,K,norm,dt", [(5, 12288, False, "bf16"), (4, 9216, True, "f32")])
def test_static_codes_without_gamma_on_wide_rows(T, K, norm, dt):
    """A fixed step, gamma_f = NULL, rows of 8200-16384 values (the
    workgroup-per-token register kernel): INT8 and FP8 codes bit-exact,
    quotients past the step's range clipped."""
    rng = np.random.default_rng(5 * T + K)
    x = rng.standard_normal((T, K)).astype(np.float32)
    x[:, rng.permutation(K)[:5]] *= 40
    xin = synth.f32_to_bf16_bits(x) if dt == "bf16" else x
    delta = np.float32(0.05)   # many quotients past 127 (and past 448 for FP8)
    say(f"static without gamma T={T} K={K} norm={norm} {dt}")
    d = torch.tensor([delta], dtype=torch.float32, device=DEV)
    xq = torch.empty((T, K), dtype=torch.int8, device=DEV)
    xs, rr = f32(T), f32(T)
    sq.sq_quant_act_static(to_dev(xin), None, d, xq, xs, norm=norm,
                           row_rscale=rr if norm else None)
    xq8 = torch.empty((T, K), dtype=torch.uint8, device=DEV)
    xs8, rr8 = f32(T), f32(T)
    sq.sq_quant_act_static_fp8(to_dev(xin), None, d, xq8, xs8, norm=norm,
                               row_rscale=rr8 if norm else None)
    torch.cuda.synchronize()
    r_gpu = to_np(rr) if norm else None
    q_ref, xs_ref, _ = oracle.quant_act_static(xin, delta, None, norm=norm, r=r_gpu)
    np.testing.assert_array_equal(to_np(xq), q_ref)
    np.testing.assert_array_equal(to_np(xs), xs_ref)
    q8_ref, xs8_ref, _ = oracle.quant_act_static_fp8(xin, delta, None, norm=norm,
                                                     r=to_np(rr8) if norm else None)
    np.testing.assert_array_equal(to_np(xq8), q8_ref)
    np.testing.assert_array_equal(to_np(xs8), xs8_ref)
