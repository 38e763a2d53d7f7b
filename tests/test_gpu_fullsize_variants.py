"""Full-size GPU parity of the variants in the launch configurations the
benchmark times: the FP8 E4M3 path and the static per-tensor step on the
headline q-projection (8192 x 4096 x 4096), the LayerNorm form on its
2048 x 4096 x 6144 workload, and GPTQ on the headline weight with its 8192
calibration tokens.  The oracle recomputes the calibration over every token,
the quantized weight in full, and the outputs of sampled tokens (GPTQ:
sampled output channels, which never interact).  Same bars as the reduced-
size tests."""
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
from _gpu_util import DEV, f32, fp8_acc_bound, gpu_calibrate, say, to_dev, to_np  # noqa: E402


def _rows(T, n, seed):
    rng = np.random.default_rng(seed)
    rows = {0, 1, T - 1, T - 2, min(255, T - 1), min(256, T - 1)}
    rows |= set(rng.choice(T, size=min(n, T), replace=False).tolist())
    return np.array(sorted(rows))


def _ulps(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(a - b)


def _headline():
    wl = synth.WORKLOADS["qproj_prefill"]
    inp = synth.make_inputs(wl)
    xc, x, w = to_dev(inp.x_cal), to_dev(inp.x), to_dev(inp.w)
    a, wm, s = gpu_calibrate(xc, w, wl.alpha)
    gp = f32(wl.K)
    sq.sq_smooth_fold(s, None, gp)
    return wl, inp, xc, x, w, a, s, gp


def test_fp8_headline_full():
    wl, inp, xc, x, w, a, s, gp = _headline()
    T, K, N = wl.T, wl.K, wl.N
    say(f"full-size fp8 T={T} K={K} N={N}")
    wq, wsc = torch.empty((N, K), dtype=torch.uint8, device=DEV), f32(N)
    sq.sq_quant_weight_fp8(w, s, wq, wsc)
    y = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
    work = torch.empty(sq.sq_linear_workspace_bytes(T, K), dtype=torch.uint8, device=DEV)
    xq, xs = torch.empty((T, K), dtype=torch.uint8, device=DEV), f32(T)
    sq.sq_w8a8_linear_fp8(x, gp, wq, wsc, y, work, bias=to_dev(inp.bias), dbg_xq=xq, dbg_x_scale=xs)
    acc = torch.empty((T, N), dtype=torch.float32, device=DEV)
    sq.sq_gemm_fp8(xq, xs, wq, wsc, None, acc_out=acc)
    torch.cuda.synchronize()
    _, what = oracle.fold(to_np(s), None, inp.w)
    qw_ref, ws_ref = oracle.quant_weight_fp8(what)
    np.testing.assert_array_equal(to_np(wsc), ws_ref)
    np.testing.assert_array_equal(to_np(wq), qw_ref)
    rows = _rows(T, 24, 11)
    q_ref, xs_ref, _ = oracle.quant_act_fp8(inp.x[rows], to_np(gp))
    np.testing.assert_array_equal(to_np(xq)[rows], q_ref)
    np.testing.assert_array_equal(to_np(xs)[rows], xs_ref)
    acc_r = to_np(acc)[rows].astype(np.float64)
    err = np.abs(acc_r - oracle.gemm_fp8(q_ref, qw_ref))
    assert np.all(err <= fp8_acc_bound(q_ref, qw_ref))
    y_fed = oracle.to_bf16(oracle.epilogue_f32acc(to_np(acc)[rows], xs_ref, ws_ref, inp.bias))
    np.testing.assert_array_equal(to_np(y)[rows], y_fed)


def test_static_step_headline_full():
    wl, inp, xc, x, w, a, s, gp = _headline()
    T, K, N = wl.T, wl.K, wl.N
    say(f"full-size static step T={T} K={K} N={N}")
    wq, wsc = torch.empty((N, K), dtype=torch.int8, device=DEV), f32(N)
    sq.sq_quant_weight(w, s, wq, wsc)
    d = f32(1)
    sq.sq_act_static_scale(a, gp, d)
    y = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
    work = torch.empty(sq.sq_linear_workspace_bytes(T, K), dtype=torch.uint8, device=DEV)
    xq = torch.empty((T, K), dtype=torch.int8, device=DEV)
    sq.sq_w8a8_linear_static(x, gp, d, wq, wsc, y, work, bias=to_dev(inp.bias), dbg_xq=xq)
    torch.cuda.synchronize()
    d_ref = oracle.static_scale(inp.x_cal, to_np(gp))
    assert to_np(d)[0] == d_ref
    _, qw_ref, ws_ref = oracle.prepare_weight(inp.w, to_np(s))
    np.testing.assert_array_equal(to_np(wq), qw_ref)
    rows = _rows(T, 24, 12)
    out = oracle.linear_static(inp.x[rows], d_ref, to_np(gp), qw_ref, ws_ref, inp.bias)
    np.testing.assert_array_equal(to_np(xq)[rows], out["q"])
    np.testing.assert_array_equal(to_np(y)[rows], out["y"])


def test_layernorm_qkv_full():
    wl = synth.WORKLOADS["layernorm_qkv"]
    T, K, N = wl.T, wl.K, wl.N
    say(f"full-size layernorm T={T} K={K} N={N} Tc={wl.Tc}")
    inp = synth.make_inputs(wl)
    g, b, w = to_dev(inp.gamma), to_dev(inp.beta), to_dev(inp.w)
    a, wm, s = f32(K), f32(K), f32(K)
    sq.sq_calibrate_ln(to_dev(inp.x_cal), w, wl.alpha, a, wm, s, gamma=g, beta=b)
    gp, bp = f32(K), f32(K)
    sq.sq_smooth_fold_ln(s, g, b, gp, bp)
    wq, wsc = torch.empty((N, K), dtype=torch.int8, device=DEV), f32(N)
    sq.sq_quant_weight(w, s, wq, wsc)
    y = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
    work = torch.empty(sq.sq_linear_workspace_bytes(T, K), dtype=torch.uint8, device=DEV)
    xq, m, r = torch.empty((T, K), dtype=torch.int8, device=DEV), f32(T), f32(T)
    sq.sq_w8a8_linear_ln(to_dev(inp.x), gp, bp, wq, wsc, y, work, bias=to_dev(inp.bias),
                         dbg_xq=xq, dbg_row_rscale=r, row_mean=m)
    torch.cuda.synchronize()
    np.testing.assert_allclose(to_np(a), oracle.act_absmax_ln(inp.x_cal, inp.gamma, inp.beta),
                               rtol=2.0 ** -20, atol=0)
    assert _ulps(to_np(s), oracle.smooth_factor(to_np(a), to_np(wm), wl.alpha)).max() <= 1
    g_ref, b_ref = oracle.fold_ln(to_np(s), inp.gamma, inp.beta)
    np.testing.assert_array_equal(to_np(gp), g_ref)
    np.testing.assert_array_equal(to_np(bp), b_ref)
    _, qw_ref, ws_ref = oracle.prepare_weight(inp.w, to_np(s))
    np.testing.assert_array_equal(to_np(wq), qw_ref)
    rows = _rows(T, 32, 13)
    m_ref, r_ref = oracle.ln_stats(inp.x[rows])
    assert _ulps(to_np(m)[rows], m_ref).max() <= 1 and _ulps(to_np(r)[rows], r_ref).max() <= 1
    out = oracle.linear_ln(inp.x[rows], g_ref, b_ref, qw_ref, ws_ref, inp.bias,
                           mean=to_np(m)[rows], r=to_np(r)[rows])
    np.testing.assert_array_equal(to_np(xq)[rows], out["q"])
    np.testing.assert_array_equal(to_np(y)[rows], out["y"])


def test_gptq_headline_full():
    wl, inp, xc, x, w, a, s, gp = _headline()
    Tc, K, N = wl.Tc, wl.K, wl.N
    say(f"full-size gptq K={K} N={N} Tc={Tc}")
    wq, wsc = torch.empty((N, K), dtype=torch.int8, device=DEV), f32(N)
    work = torch.empty(sq.sq_gptq_workspace_bytes(Tc, K, N), dtype=torch.uint8, device=DEV)
    sq.sq_quant_weight_gptq(xc, gp, w, s, wq, wsc, work)
    torch.cuda.synchronize()
    del work
    xhat = oracle.smoothed_act(inp.x_cal, to_np(gp))
    _, what = oracle.fold(to_np(s), None, inp.w)
    cols = np.unique(np.concatenate([[0, 1, N - 1], np.random.default_rng(14).choice(N, 9)]))
    U, dead = oracle.gptq_factor(xhat)
    w_cols = np.ascontiguousarray(what[:, cols])
    _, ws_ref = oracle.gptq_round(w_cols, U, dead)
    np.testing.assert_array_equal(to_np(wsc)[cols], ws_ref)
    parted = check_gptq_codes(to_np(wq)[cols], w_cols, U, dead)
    say(f"  partings at near-ties over {len(cols)} sampled channels: {parted}")
