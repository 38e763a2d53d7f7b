"""GPU parity of the whole-block pieces against the CPU oracle: the LayerNorm
form of the smoothed norm (gamma and beta both take 1/s), the fold of 1/s into
the previous linear's output columns, and a decoder layer's four linears
wired the way the pages map them (norm -> fused q|k|v and norm -> fused
gate|up smoothed; output and down projections plain per-token W8A8).

Bar: LayerNorm statistics within one fp32 ulp of the oracle's (fp64 sums in
another order), and everything downstream bit-exact when the oracle is fed
the GPU's statistics; folds bit-exact; every linear's codes and bf16 outputs
bit-exact against the oracle on the same inputs; layer errors no worse than
the oracle's.
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
from _gpu_util import (DEV, f32, gpu_calibrate, gpu_linear, gpu_prepare_weight, say,  # noqa: E402
                       to_dev, to_np)


def _ulps(a, b):
    a = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    b = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(a - b)


def _ln_inputs(T, K, N, Tc, dt="bf16", seed_shift=0):
    wl = synth.WORKLOADS["layernorm_qkv"].with_sizes(T=T, K=K, N=N, Tc=Tc,
                                                     seed=106 + seed_shift, io_dtype=dt)
    return wl, synth.make_inputs(wl)


@pytest.mark.parametrize("T,K,dt", [(37, 512, "bf16"), (64, 4096, "bf16"), (20, 1344, "f32"),
                                    (9, 8192, "bf16"), (5, 16384, "bf16"), (11, 12352, "bf16"),
                                    (6, 9216, "f32"), (3, 20480, "bf16"), (300, 3072, "bf16"),
                                    (40, 2112, "f32"), (9, 2048, "bf16")])
def test_quant_act_ln(T, K, dt):
    wl, inp = _ln_inputs(T, K, 64, 16, dt)
    say(f"ln quant T={T} K={K} {dt}")
    rng = np.random.default_rng(K + T)
    gp = rng.uniform(0.2, 2.0, K).astype(np.float32)
    bp = rng.normal(0, 0.2, K).astype(np.float32)
    xq = torch.empty((T, K), dtype=torch.int8, device=DEV)
    xs, m, r = f32(T), f32(T), f32(T)
    sq.sq_quant_act_ln(to_dev(inp.x), to_dev(gp), to_dev(bp), xq, xs, row_mean=m, row_rscale=r)
    torch.cuda.synchronize()
    m_ref, r_ref = oracle.ln_stats(inp.x)
    assert _ulps(to_np(m), m_ref).max() <= 1 and _ulps(to_np(r), r_ref).max() <= 1
    q_ref, xs_ref, _, _ = oracle.quant_act_ln(inp.x, gp, bp, mean=to_np(m), r=to_np(r))
    np.testing.assert_array_equal(to_np(xs), xs_ref)
    np.testing.assert_array_equal(to_np(xq), q_ref)


def _hard_ln_rows(K, dt, seed):
    """Rows that stress one-pass statistics: a large offset against a small
    spread, an extreme first element (the shift) over a near-zero mean, a
    constant row, tiny and huge magnitudes, and exact +-1 alternation."""
    rng = np.random.default_rng(seed)
    rows = [
        1000.0 + rng.normal(0, 1, K),                    # mean / spread ~ 500 in bf16
        np.r_[3000.0, rng.normal(0, 1, K - 1)],          # the shift is a 3000-sigma outlier
        np.r_[-rng.normal(0, 1, K - 1), 1e4][::-1],      # the shift is -1e4, the rest N(0,1)
        np.full(K, 2.5),                                 # constant: var = 0 exactly
        rng.normal(0, 1e-20, K),                         # tiny
        rng.normal(0, 1e15, K) + 3e16,                   # huge with an offset
        np.tile([1.0, -1.0], K // 2),                    # mean exactly 0
        rng.standard_cauchy(K).clip(-1e6, 1e6),          # heavy tails
    ]
    h = np.stack(rows).astype(np.float32)
    return synth.f32_to_bf16_bits(h) if dt == "bf16" else h


@pytest.mark.parametrize("K,dt", [(512, "bf16"), (4096, "bf16"), (4096, "f32"), (12352, "bf16"),
                                  (20480, "bf16"), (9216, "f32")])
def test_ln_statistics_hard_rows(K, dt):
    """The GPU takes the LayerNorm mean and variance in one pass of fp64 sums
    shifted by the row's first element; on rows built to break such sums the
    statistics stay within one fp32 ulp of the oracle's two-pass definition
    (quantizer kernels of every width), the codes and steps are bit-exact
    given the GPU's statistics, and the calibration maxima follow (narrow and
    wide calibration kernels)."""
    h = _hard_ln_rows(K, dt, K)
    T = h.shape[0]
    say(f"ln hard rows K={K} {dt}")
    eps = 1e-5
    gp = np.ones(K, np.float32)
    bp = np.zeros(K, np.float32)
    xq = torch.empty((T, K), dtype=torch.int8, device=DEV)
    xs, m, r = f32(T), f32(T), f32(T)
    sq.sq_quant_act_ln(to_dev(h), to_dev(gp), to_dev(bp), xq, xs, eps=eps, row_mean=m,
                       row_rscale=r)
    a = f32(K)
    sq.sq_calibrate_ln(to_dev(h), None, 0.5, a, eps=eps)
    torch.cuda.synchronize()
    m_ref, r_ref = oracle.ln_stats(h, eps=eps)
    assert _ulps(to_np(m), m_ref).max() <= 1, (to_np(m), m_ref)
    assert _ulps(to_np(r), r_ref).max() <= 1, (to_np(r), r_ref)
    q_ref, xs_ref, _, _ = oracle.quant_act_ln(h, gp, bp, eps=eps, mean=to_np(m), r=to_np(r))
    np.testing.assert_array_equal(to_np(xs), xs_ref)
    np.testing.assert_array_equal(to_np(xq), q_ref)
    a_ref = oracle.act_absmax_ln(h, eps=eps)
    np.testing.assert_allclose(to_np(a), a_ref, rtol=2.0 ** -20, atol=0)


@pytest.mark.parametrize("K,dt", [(512, "bf16"), (4096, "bf16"), (1344, "f32"), (8192, "bf16"),
                                  (4096, "f32"), (8192, "f32")])
def test_calibrate_and_fold_ln(K, dt):
    wl, inp = _ln_inputs(8, K, 96, 300, dt)
    say(f"ln calibrate K={K} {dt}")
    g, b = to_dev(inp.gamma), to_dev(inp.beta)
    a, wm, s = f32(K), f32(K), f32(K)
    sq.sq_calibrate_ln(to_dev(inp.x_cal), to_dev(inp.w), wl.alpha, a, wm, s, gamma=g, beta=b)
    gp, bp = f32(K), f32(K)
    sq.sq_smooth_fold_ln(s, g, b, gp, bp)
    torch.cuda.synchronize()
    a_ref = oracle.act_absmax_ln(inp.x_cal, inp.gamma, inp.beta)
    # the maxima inherit the rows' statistics (one fp32 ulp apart at most)
    np.testing.assert_allclose(to_np(a), a_ref, rtol=2.0 ** -20, atol=0)
    np.testing.assert_array_equal(to_np(wm), oracle.weight_absmax(inp.w))
    s_ref = oracle.smooth_factor(to_np(a), to_np(wm), wl.alpha)
    assert _ulps(to_np(s), s_ref).max() <= 1
    g_ref, b_ref = oracle.fold_ln(to_np(s), inp.gamma, inp.beta)
    np.testing.assert_array_equal(to_np(gp), g_ref)
    np.testing.assert_array_equal(to_np(bp), b_ref)


@pytest.mark.parametrize("sizes", [dict(T=300, K=1024, N=640, Tc=512),
                                   dict(T=130, K=4096, N=384, Tc=256)])
def test_linear_ln_end_to_end(sizes):
    wl, inp = _ln_inputs(**sizes)
    T, K, N = wl.T, wl.K, wl.N
    say(f"ln linear {sizes}")
    g, b, w = to_dev(inp.gamma), to_dev(inp.beta), to_dev(inp.w)
    a, wm, s = f32(K), f32(K), f32(K)
    sq.sq_calibrate_ln(to_dev(inp.x_cal), w, wl.alpha, a, wm, s, gamma=g, beta=b)
    gp, bp = f32(K), f32(K)
    sq.sq_smooth_fold_ln(s, g, b, gp, bp)
    wq = torch.empty((N, K), dtype=torch.int8, device=DEV)
    wsc = f32(N)
    sq.sq_quant_weight(w, s, wq, wsc)
    y = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
    work = torch.empty(sq.sq_linear_workspace_bytes(T, K), dtype=torch.uint8, device=DEV)
    dbg_xq = torch.empty((T, K), dtype=torch.int8, device=DEV)
    m, r = f32(T), f32(T)
    sq.sq_w8a8_linear_ln(to_dev(inp.x), gp, bp, wq, wsc, y, work, bias=to_dev(inp.bias),
                         dbg_xq=dbg_xq, dbg_row_rscale=r, row_mean=m)
    torch.cuda.synchronize()
    _, qw_ref, ws_ref = oracle.prepare_weight(inp.w, to_np(s))
    np.testing.assert_array_equal(to_np(wq), qw_ref)
    out = oracle.linear_ln(inp.x, to_np(gp), to_np(bp), qw_ref, ws_ref, inp.bias,
                           mean=to_np(m), r=to_np(r))
    np.testing.assert_array_equal(to_np(dbg_xq), out["q"])
    np.testing.assert_array_equal(to_np(y), out["y"])
    ref = oracle.reference_ln_fp64(inp.x, inp.w, inp.bias, gamma=inp.gamma, beta=inp.beta)
    e_gpu, e_ref = oracle.rel_error(ref, to_np(y)), oracle.rel_error(ref, out["y"])
    # the same layer without smoothing, for the record
    _, qw0, ws0 = oracle.prepare_weight(inp.w, np.ones(K, np.float32))
    e_raw = oracle.rel_error(ref, oracle.linear_ln(inp.x, inp.gamma, inp.beta, qw0, ws0,
                                                   inp.bias)["y"])
    say(f"  LayerNorm layer error {e_gpu:.4%} (oracle {e_ref:.4%}, unsmoothed {e_raw:.4%})")
    assert e_gpu <= e_ref * 1.01 + 1e-6


@pytest.mark.parametrize("dt,ldw_pad,ldo_pad", [("bf16", 0, 0), ("f32", 64, 4), ("bf16", 8, 12)])
def test_fold_prev_linear(dt, ldw_pad, ldo_pad):
    say(f"fold prev {dt} pads {ldw_pad} {ldo_pad}")
    rng = np.random.default_rng(5 + ldw_pad)
    Kp, K = 200, 1344
    wp = (rng.standard_normal((Kp, K + ldw_pad)) * 0.05).astype(np.float32)
    if dt == "bf16":
        wp = synth.f32_to_bf16_bits(wp)
    s = rng.uniform(0.05, 30, K).astype(np.float32)
    bias = rng.standard_normal(K).astype(np.float32)
    w_in = to_dev(wp)[:, :K]
    w_out = torch.empty((Kp, K + ldo_pad), dtype=torch.float32, device=DEV)[:, :K]
    b_out = f32(K)
    sq.sq_fold_prev_linear(to_dev(s), w_in, w_out, bias=to_dev(bias), bias_out=b_out)
    torch.cuda.synchronize()
    w_ref, b_ref = oracle.fold_prev(s, np.ascontiguousarray(wp[:, :K]), bias)
    np.testing.assert_array_equal(to_np(w_out), w_ref)
    np.testing.assert_array_equal(to_np(b_out), b_ref)


def _silu_mul(gu, inter):
    """The MLP's activation, fp32 on the host (not part of the smoothed path):
    silu(gate) * up from the fused gate|up output."""
    v = synth.bf16_bits_to_f32(gu).astype(np.float32)
    g, u = v[:, :inter], v[:, inter:]
    return (g / (np.float32(1) + np.exp(-g)) * u).astype(np.float32)


def test_decoder_layer_mapping():
    """One decoder layer's linears: RMSNorm -> q|k|v (GQA) and RMSNorm -> gate|up
    smoothed; o_proj and down_proj plain per-token W8A8.  Then down_proj
    smoothed as well, its 1/s folded into up's output columns (the mapping the
    pages attribute to AWQ): every output bit-exact against the oracle, and
    the errors of both MLP variants against the fp64 layer."""
    say("decoder layer mapping")
    T, H, KV, I = 96, 512, 128, 1024
    rng = np.random.default_rng(77)

    def w_(k, n, sigma=0.02):
        return synth.f32_to_bf16_bits((rng.standard_normal((k, n)) * sigma).astype(np.float32))

    def act(t, k, n_out, mult):
        x = rng.standard_normal((t, k)).astype(np.float32)
        x[:, rng.permutation(k)[:n_out]] *= mult
        return synth.f32_to_bf16_bits(x)

    h1, h1c = act(T, H, 8, 40), act(256, H, 8, 40)
    w_qkv, g1 = w_(H, H + 2 * KV), rng.uniform(0.5, 1.5, H).astype(np.float32)
    attn = act(T, H, 4, 10)                       # stands in for the attention output
    w_o = w_(H, H)
    h2, h2c = act(T, H, 6, 30), act(256, H, 6, 30)
    w_gu, g2 = w_(H, 2 * I), rng.uniform(0.5, 1.5, H).astype(np.float32)
    w_d = w_(I, H)
    errs = {}

    def smoothed(x, xc, w, g, alpha):
        """calibrate, fold into the norm, quantize; the linear behind the norm"""
        _, _, s = gpu_calibrate(to_dev(xc), to_dev(w), alpha, norm=True, gamma=to_dev(g))
        gp, wq, wsc = gpu_prepare_weight(to_dev(w), s, to_dev(g))
        y, kw = gpu_linear(to_dev(x), gp, wq, wsc, norm=True)
        torch.cuda.synchronize()
        _, qw_ref, ws_ref = oracle.prepare_weight(w, to_np(s), g)
        out = oracle.linear(x, to_np(gp), qw_ref, ws_ref, norm=True,
                            r=to_np(kw["dbg_row_rscale"]))
        np.testing.assert_array_equal(to_np(y), out["y"])
        return to_np(y)

    def plain(x, w, s=None):
        """per-token W8A8 with no norm; s folds into the weight rows only (the
        activation arrives already divided by s)"""
        K, N = w.shape
        wq = torch.empty((N, K), dtype=torch.int8, device=DEV)
        wsc = f32(N)
        sq.sq_quant_weight(to_dev(w), None if s is None else to_dev(s), wq, wsc)
        y, _ = gpu_linear(to_dev(x), None, wq, wsc)
        torch.cuda.synchronize()
        _, qw_ref, ws_ref = oracle.prepare_weight(w, np.ones(K, np.float32) if s is None else s)
        np.testing.assert_array_equal(to_np(y), oracle.linear(x, None, qw_ref, ws_ref)["y"])
        return to_np(y)

    def rms64(h, g):
        x = synth.bf16_bits_to_f32(h).astype(np.float64)
        return x / np.sqrt((x * x).mean(1, keepdims=True) + float(np.float32(1e-6))) * g

    qkv = smoothed(h1, h1c, w_qkv, g1, 0.5)
    errs["qkv"] = oracle.rel_error(oracle.reference_fp64(h1, w_qkv, norm=True, gamma=g1), qkv)
    y_o = plain(attn, w_o)
    errs["o_proj"] = oracle.rel_error(oracle.reference_fp64(attn, w_o), y_o)

    # MLP in fp64, the reference for both variants
    gu64 = rms64(h2, g2) @ synth.bf16_bits_to_f32(w_gu).astype(np.float64)
    a64 = gu64[:, :I] / (1 + np.exp(-gu64[:, :I])) * gu64[:, I:]
    ref_d = a64 @ synth.bf16_bits_to_f32(w_d).astype(np.float64)

    # (1) down_proj plain
    gu = smoothed(h2, h2c, w_gu, g2, 0.5)
    errs["gate_up"] = oracle.rel_error(rms64(h2, g2) @ synth.bf16_bits_to_f32(w_gu).astype(np.float64), gu)
    y_d = plain(_silu_mul(gu, I), w_d)
    errs["down"] = oracle.rel_error(ref_d, y_d)

    # (2) down_proj smoothed: s_d from the MLP activations of a calibration
    # batch, 1/s_d folded into up's output columns (then gate|up calibrated on
    # the folded weight), diag(s_d) folded into down's rows
    a_cal = _silu_mul(smoothed(h2c, h2c, w_gu, g2, 0.5), I)
    s_d = oracle.smooth_factor(np.abs(a_cal).max(0).astype(np.float32),
                               oracle.weight_absmax(w_d), 0.5)
    gu_f = torch.empty((H, 2 * I), dtype=torch.float32, device=DEV)
    gu_f[:, :I] = to_dev(w_gu)[:, :I].float()
    sq.sq_fold_prev_linear(to_dev(s_d), to_dev(w_gu)[:, I:], gu_f[:, I:])
    torch.cuda.synchronize()
    up_ref, _ = oracle.fold_prev(s_d, np.ascontiguousarray(w_gu[:, I:]))
    np.testing.assert_array_equal(to_np(gu_f[:, I:]), up_ref)
    gu2 = smoothed(h2, h2c, to_np(gu_f), g2, 0.5)
    y_d2 = plain(_silu_mul(gu2, I), w_d, s=s_d)
    errs["down_smoothed"] = oracle.rel_error(ref_d, y_d2)
    say("  " + ", ".join(f"{k} {v:.3%}" for k, v in errs.items()))

    # the same norm -> linear pairs unsmoothed, for the record
    def unsmoothed(x, w, g):
        _, qw0, ws0 = oracle.prepare_weight(w, np.ones(w.shape[0], np.float32))
        y0 = oracle.linear(x, g, qw0, ws0, norm=True)["y"]
        return oracle.rel_error(oracle.reference_fp64(x, w, norm=True, gamma=g), y0)

    e0_qkv, e0_gu = unsmoothed(h1, w_qkv, g1), unsmoothed(h2, w_gu, g2)
    say(f"  unsmoothed: qkv {e0_qkv:.3%}, gate_up {e0_gu:.3%}")
    # reported, not gated beyond sanity: how much smoothing helps depends on
    # alpha and on the outliers (the pages' own sweep)
    assert max(errs.values()) < 0.15
