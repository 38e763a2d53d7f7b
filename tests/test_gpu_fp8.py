"""GPU parity of the FP8 E4M3 variant against the CPU oracle.

Bar: weight and activation codes and their steps bit-exact (both sides take
the nearest E4M3 value of the same correctly rounded fp32 quotient, ties to
even); the GEMM's fp32 accumulators within the bound of the FP8 matrix
instruction's own arithmetic (below) of the exact (fp64) sums, and bit-exact
where no product loses bits in it; the epilogue bit-exact when fed the GPU's
accumulators; end-to-end bf16 outputs within 2e-3 relative (1e-2 absolute
floor) of the oracle, widened by the scaled accumulator bound.

The accumulator bound.  v_mfma_f32_32x32x64_f8f6f4 adds its products in
groups of 8 consecutive k: every product of a group is aligned to the group's
largest product and cut (toward zero) below 2^-13 of it, the group sums are
then added in fp32.  So each of the 7 other products of a group loses less
than 2^-12 * max_g |a_k b_k| (2^-12, not 2^-13: room for the carry of the
significand product), and the K/8 + 1 fp32 roundings add at most
(K/8 + 1) * 2^-24 * sum_k |a_k b_k|.  Measured on the chip with single
products placed against one another (same group: bits below 2^-13 of the
larger one gone; other group or other K step: kept to fp32).
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
from _gpu_util import DEV, f32, gpu_calibrate, say, to_dev, to_np  # noqa: E402

F32 = np.float32


def _u8(shape):
    return torch.empty(shape, dtype=torch.uint8, device=DEV)


@pytest.mark.parametrize("K,N", [(256, 64), (1344, 200), (4096, 520)])
def test_quant_weight_fp8(K, N):
    wl = synth.WORKLOADS["qproj_prefill"].with_sizes(T=8, Tc=64, K=K, N=N)
    say(f"fp8 weight K={K} N={N}")
    inp = synth.make_inputs(wl)
    w = to_dev(inp.w)
    _, _, s = gpu_calibrate(to_dev(inp.x_cal), w, wl.alpha)
    wq, wsc = _u8((N, K)), f32(N)
    sq.sq_quant_weight_fp8(w, s, wq, wsc)
    torch.cuda.synchronize()
    _, what = oracle.fold(to_np(s), None, inp.w)
    qw_ref, ws_ref = oracle.quant_weight_fp8(what)
    np.testing.assert_array_equal(to_np(wsc), ws_ref)
    np.testing.assert_array_equal(to_np(wq), qw_ref)


def test_quant_weight_fp8_zero_column():
    say("fp8 weight zero column")
    rng = np.random.default_rng(41)
    w = (rng.standard_normal((128, 64)) * 0.02).astype(np.float32)
    w[:, 5] = 0.0
    wq, wsc = _u8((64, 128)), f32(64)
    sq.sq_quant_weight_fp8(to_dev(w), None, wq, wsc)
    torch.cuda.synchronize()
    qw_ref, ws_ref = oracle.quant_weight_fp8(w)
    np.testing.assert_array_equal(to_np(wsc), ws_ref)
    np.testing.assert_array_equal(to_np(wq), qw_ref)
    assert ws_ref[5] == 0 and not qw_ref[5].any()


@pytest.mark.parametrize("T,K,norm,dt", [(64, 512, False, "bf16"), (37, 4096, False, "bf16"),
                                         (29, 1344, True, "bf16"), (16, 8192, True, "bf16"),
                                         (40, 320, False, "f32"), (6, 16384, False, "bf16")])
def test_quant_act_fp8(T, K, norm, dt):
    wl = synth.WORKLOADS["rmsnorm_qkv" if norm else "qproj_prefill"].with_sizes(
        T=T, Tc=T, K=K, N=64)
    if dt == "f32":
        wl = wl.with_sizes(io_dtype="f32")
    say(f"fp8 act T={T} K={K} norm={norm} {dt}")
    inp = synth.make_inputs(wl)
    g = np.random.default_rng(T).uniform(0.3, 2.0, K).astype(np.float32)
    xq, xs, rr = _u8((T, K)), f32(T), f32(T)
    sq.sq_quant_act_fp8(to_dev(inp.x), to_dev(g), xq, xs, norm=norm, row_rscale=rr if norm else None)
    torch.cuda.synchronize()
    q_ref, xs_ref, _ = oracle.quant_act_fp8(inp.x, g, norm=norm, r=to_np(rr) if norm else None)
    np.testing.assert_array_equal(to_np(xs), xs_ref)
    np.testing.assert_array_equal(to_np(xq), q_ref)


@pytest.mark.parametrize("T,K,dt,norm", [(6, 14336, "bf16", False), (3, 12288, "f32", True)])
def test_quant_act_fp8_without_gamma(T, K, dt, norm):
    """FP8 codes of rows that take the workgroup-per-token register kernel."""
    rng = np.random.default_rng(3 * T + K)
    x = rng.standard_normal((T, K)).astype(np.float32)
    x[:, rng.permutation(K)[:5]] *= 40
    xin = synth.f32_to_bf16_bits(x) if dt == "bf16" else x
    say(f"fp8 act without gamma T={T} K={K} {dt} norm={norm}")
    xq, xs, rr = _u8((T, K)), f32(T), f32(T)
    sq.sq_quant_act_fp8(to_dev(xin), None, xq, xs, norm=norm, row_rscale=rr if norm else None)
    torch.cuda.synchronize()
    q_ref, xs_ref, _ = oracle.quant_act_fp8(xin, None, norm=norm, r=to_np(rr) if norm else None)
    np.testing.assert_array_equal(to_np(xs), xs_ref)
    np.testing.assert_array_equal(to_np(xq), q_ref)


def test_quant_act_fp8_ties_subnormals_and_zero_rows():
    say("fp8 act ties")
    tab = np.array([v for c, v in sorted({c: float(oracle.e4m3_decode(np.array([c], np.uint8))[0])
                                          for c in range(0x7F)}.items())], np.float64)
    mids = ((tab[:-1] + tab[1:]) / 2).astype(np.float32)            # exact midpoints: ties
    K = 512
    rows = []
    r0 = np.zeros(K, np.float32)
    r0[0] = 448.0                                                   # step exactly 1
    r0[1:1 + len(mids)] = mids[: K - 1]
    rows.append(r0)
    r1 = -r0                                                        # negative ties
    rows.append(r1)
    r2 = np.zeros(K, np.float32)                                    # all-zero token
    rows.append(r2)
    r3 = np.zeros(K, np.float32)
    r3[0] = 448.0
    r3[1:40] = np.float32(2.0 ** -12) * np.arange(1, 40)            # deep subnormal quotients
    r3[40] = -0.0
    rows.append(r3)
    # step 1: one fp32 ulp either side of every midpoint; step 3 (1/3 is
    # inexact in fp32): three times every midpoint, exactly (ties) and one ulp
    # below -- quotients the quantizer's product by the reciprocal cannot
    # place on its own
    for scale in (1.0, 3.0):
        for toward in (np.inf, -np.inf):
            r = np.zeros(K, np.float32)
            r[0] = np.float32(448.0 * scale)
            m = (mids[: K - 1] * np.float32(scale)).astype(np.float32)
            r[1:1 + len(m)] = m if (scale != 1.0 and toward == np.inf) else \
                np.nextafter(m, np.float32(toward))
            rows.append(r)
    x = np.stack(rows).astype(np.float32)
    xq, xs = _u8(x.shape), f32(x.shape[0])
    sq.sq_quant_act_fp8(to_dev(x), None, xq, xs)
    torch.cuda.synchronize()
    q_ref, xs_ref, _ = oracle.quant_act_fp8(x)
    np.testing.assert_array_equal(to_np(xs), xs_ref)
    np.testing.assert_array_equal(to_np(xq), q_ref)


def _acc_bound(q, qw):
    """Bound on |GPU accumulator - exact sum| per output (module docstring)."""
    a = np.abs(oracle.e4m3_decode(q).astype(np.float64))
    b = np.abs(oracle.e4m3_decode(qw).astype(np.float64))
    K = a.shape[1]
    gmax = np.zeros((a.shape[0], b.shape[0]))
    for g in range(0, K, 8):
        m = np.zeros_like(gmax)
        for k in range(g, min(g + 8, K)):
            np.maximum(m, np.multiply.outer(a[:, k], b[:, k]), out=m)
        gmax += m
    return 7 * 2.0 ** -12 * gmax + (K // 8 + 1) * 2.0 ** -24 * (a @ b.T)


def _rand_codes(rng, shape, span):
    """E4M3 codes of values spread over `span` binades (no NaN codes)."""
    v = (rng.standard_normal(shape) * np.exp2(rng.uniform(-span, 0, shape)) * 200).astype(np.float32)
    return oracle.e4m3_encode(np.clip(v, -448, 448))


@pytest.mark.parametrize("T,N,K,span", [(256, 256, 512, 6), (300, 520, 1344, 6), (64, 96, 4096, 12),
                                        (520, 600, 2048, 3), (8, 40, 320, 6)])
def test_gemm_fp8_accumulators(T, N, K, span):
    say(f"fp8 gemm T={T} N={N} K={K} span={span}")
    rng = np.random.default_rng(T * 7 + N)
    q = _rand_codes(rng, (T, K), span)
    qw = _rand_codes(rng, (N, K), span)
    acc = torch.empty((T, N), dtype=torch.float32, device=DEV)
    sq.sq_gemm_fp8(to_dev(q), f32(T, 1.0), to_dev(qw), f32(N, 1.0), None, acc_out=acc)
    torch.cuda.synchronize()
    exact = oracle.gemm_fp8(q, qw)
    bound = _acc_bound(q, qw)
    err = np.abs(to_np(acc).astype(np.float64) - exact)
    assert np.all(err <= bound), float((err / bound).max())


def test_gemm_fp8_group_arithmetic():
    """The premises of the bound: products in one group of 8 k lose the bits
    below 2^-13 of the group's largest; other groups and K steps keep fp32."""
    say("fp8 gemm group arithmetic")
    K = 128
    rows, want = [], []
    for j, v, kept in ((1, 2.0 ** -5, True), (7, 2.0 ** -6, False), (7, -(2.0 ** -6), False),
                       (8, 2.0 ** -9, True), (40, -(2.0 ** -9), True), (72, 2.0 ** -9, True)):
        x = np.zeros(K, np.float32)
        x[0], x[j] = 256.0, v
        rows.append(x)
        want.append(256.0 + v if kept else 256.0)
    X = np.stack(rows)
    W = np.ones((1, K), np.float32)
    q, qw = oracle.e4m3_encode(X), oracle.e4m3_encode(W)
    assert np.array_equal(oracle.e4m3_decode(q), X)
    acc = torch.empty((len(rows), 1), dtype=torch.float32, device=DEV)
    sq.sq_gemm_fp8(to_dev(q), f32(len(rows), 1.0), to_dev(qw), f32(1, 1.0), None, acc_out=acc)
    torch.cuda.synchronize()
    got = to_np(acc)[:, 0].astype(np.float64)
    np.testing.assert_array_equal(got, np.array(want))
    assert np.all(np.abs(got - oracle.gemm_fp8(q, qw)[:, 0]) <= _acc_bound(q, qw)[:, 0])


@pytest.mark.parametrize("T,N,K", [(200, 136, 4096), (1500, 4096, 128), (1800, 6104, 64),
                                   (4200, 4100, 192), (7179, 3091, 128),   # several tiles per
                                   (4625, 4999, 128)])                     # workgroup
def test_gemm_fp8_exact_when_every_partial_sum_is_representable(T, N, K):
    say(f"fp8 gemm exact small integers T={T} N={N} K={K}")
    rng = np.random.default_rng(42 + T)
    vals = np.array([-4, -3, -2, -1, 0, 1, 2, 3, 4], np.float32)
    q = oracle.e4m3_encode(rng.choice(vals, (T, K)))
    qw = oracle.e4m3_encode(rng.choice(vals, (N, K)))
    acc = torch.empty((T, N), dtype=torch.float32, device=DEV)
    sq.sq_gemm_fp8(to_dev(q), f32(T, 1.0), to_dev(qw), f32(N, 1.0), None, acc_out=acc)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(acc), oracle.gemm_fp8(q, qw).astype(np.float32))


@pytest.mark.parametrize("name,sizes", [("qproj_prefill", dict(T=300, Tc=512, K=1024, N=640)),
                                        ("rmsnorm_qkv", dict(T=130, Tc=256, K=2048, N=384)),
                                        ("decode", dict(T=16, Tc=256, K=2048, N=512))])
def test_linear_fp8_end_to_end(name, sizes):
    wl = synth.WORKLOADS[name].with_sizes(**sizes)
    say(f"fp8 linear {name} {sizes}")
    inp = synth.make_inputs(wl)
    T, K, N = wl.T, wl.K, wl.N
    g = None if inp.gamma is None else to_dev(inp.gamma)
    w = to_dev(inp.w)
    _, _, s = gpu_calibrate(to_dev(inp.x_cal), w, wl.alpha, norm=wl.norm, gamma=g)
    gp = f32(K)
    sq.sq_smooth_fold(s, g, gp)
    wq, wsc = _u8((N, K)), f32(N)
    sq.sq_quant_weight_fp8(w, s, wq, wsc)
    y = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
    work = torch.empty(sq.sq_linear_workspace_bytes(T, K), dtype=torch.uint8, device=DEV)
    dbg_xq, dbg_xs = _u8((T, K)), f32(T)
    rr = f32(T)
    bias = to_dev(inp.bias)
    sq.sq_w8a8_linear_fp8(to_dev(inp.x), gp, wq, wsc, y, work, norm=wl.norm, bias=bias,
                          dbg_xq=dbg_xq, dbg_x_scale=dbg_xs,
                          dbg_row_rscale=rr if wl.norm else None)
    acc = torch.empty((T, N), dtype=torch.float32, device=DEV)
    sq.sq_gemm_fp8(dbg_xq, dbg_xs, wq, wsc, None, acc_out=acc)
    torch.cuda.synchronize()
    gp_h, s_h = to_np(gp), to_np(s)
    _, qw_ref, ws_ref = oracle.prepare_weight_fp8(inp.w, s_h, inp.gamma)
    np.testing.assert_array_equal(to_np(wq), qw_ref)
    np.testing.assert_array_equal(to_np(wsc), ws_ref)
    out = oracle.linear_fp8(inp.x, gp_h, qw_ref, ws_ref, inp.bias, norm=wl.norm,
                            r=to_np(rr) if wl.norm else None)
    np.testing.assert_array_equal(to_np(dbg_xq), out["q"])
    np.testing.assert_array_equal(to_np(dbg_xs), out["x_scale"])
    # epilogue fed the GPU's own accumulators: bit-exact
    y_fed = oracle.to_bf16(oracle.epilogue_f32acc(to_np(acc), out["x_scale"], ws_ref, inp.bias))
    np.testing.assert_array_equal(to_np(y), y_fed)
    # against the oracle's exact-sum path
    yo = synth.bf16_bits_to_f32(out["y"])
    yg = synth.bf16_bits_to_f32(to_np(y))
    # the accumulators may differ by the bound; the fp32 outputs then by the
    # scaled bound, and after rounding to bf16 by up to one more bf16 ulp
    slack = np.abs(out["x_scale"][:, None] * ws_ref[None, :]) * _acc_bound(out["q"], qw_ref)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(yo), 2.0 ** -126))) - 7)
    tol = np.maximum(2e-3 * np.abs(yo), 1e-2) + slack + ulp
    diff = np.abs(yg - yo)
    i = np.unravel_index(np.argmax(diff - tol), diff.shape)
    assert np.all(diff <= tol), (i, float(yg[i]), float(yo[i]), float(slack[i]), float(tol[i]))
    ref = oracle.reference_fp64(inp.x, inp.w, inp.bias, norm=wl.norm, gamma=inp.gamma)
    e_gpu, e_ref = oracle.rel_error(ref, to_np(y)), oracle.rel_error(ref, out["y"])
    say(f"  fp8 layer error gpu {e_gpu:.4%} oracle {e_ref:.4%}")
    assert e_gpu <= e_ref * 1.01 + 1e-6


# --- static per-tensor E4M3 step -------------------------------------------

def _check_step(d_gpu, d_ref, norm):
    """Bit-exact without a norm; in norm mode within one fp32 ulp (the RMSNorm
    factor of the maximal token comes from fp64 sums in different orders)."""
    a = int(np.array([d_gpu], np.float32).view(np.int32)[0])
    b = int(np.array([d_ref], np.float32).view(np.int32)[0])
    assert abs(a - b) <= (1 if norm else 0), (d_gpu, d_ref)


def _gpu_static_scale_fp8(xc, gp, *, norm):
    a = f32(xc.shape[1])
    sq.sq_calibrate(xc, None, 0.5, a, norm=norm, gamma=None)
    d = f32(1)
    sq.sq_act_static_scale_fp8(a, gp, d)
    return d


@pytest.mark.parametrize("T,K,norm,dt", [(64, 512, False, "bf16"), (37, 1344, True, "bf16"),
                                         (96, 320, False, "f32"), (8, 16384, False, "bf16"),
                                         (24, 8192, True, "bf16")])
def test_static_fp8_step_and_codes(T, K, norm, dt):
    wl = synth.WORKLOADS["rmsnorm_qkv" if norm else "qproj_prefill"].with_sizes(
        T=T, Tc=2 * T, K=K, N=64)
    if dt == "f32":
        wl = wl.with_sizes(io_dtype="f32")
    say(f"fp8 static step T={T} K={K} norm={norm} {dt}")
    inp = synth.make_inputs(wl)
    rng = np.random.default_rng(T + K + 1)
    gp_h = rng.uniform(0.3, 2.0, K).astype(np.float32)
    gp = to_dev(gp_h)
    d = _gpu_static_scale_fp8(to_dev(inp.x_cal), gp, norm=norm)
    _check_step(to_np(d)[0], oracle.static_scale_fp8(inp.x_cal, gp_h, norm=norm), norm)
    d_ref = to_np(d)[0]
    xq, xs, rr = _u8((T, K)), f32(T), f32(T)
    sq.sq_quant_act_static_fp8(to_dev(inp.x), gp, d, xq, xs, norm=norm,
                               row_rscale=rr if norm else None)
    torch.cuda.synchronize()
    q_ref, xs_ref, _ = oracle.quant_act_static_fp8(inp.x, d_ref, gp_h, norm=norm,
                                                   r=to_np(rr) if norm else None)
    np.testing.assert_array_equal(to_np(xq), q_ref)
    np.testing.assert_array_equal(to_np(xs), xs_ref)


def test_static_fp8_clipping_and_zero_step():
    say("fp8 static clipping and zero step")
    rng = np.random.default_rng(4)
    K, T = 1024, 40
    x = (rng.standard_normal((T, K)) * 4).astype(np.float32)
    x[:, 7] *= 50                                       # far past the step's range
    x[3] = 0.0
    xd = to_dev(x)
    for delta in (np.float32(0.05), np.float32(1e-3), np.float32(0.0), np.float32(1e-40)):
        d = to_dev(np.array([delta], np.float32))
        xq, xs = _u8((T, K)), f32(T)
        sq.sq_quant_act_static_fp8(xd, None, d, xq, xs)
        torch.cuda.synchronize()
        q_ref, xs_ref, _ = oracle.quant_act_static_fp8(x, delta)
        np.testing.assert_array_equal(to_np(xq), q_ref)
        np.testing.assert_array_equal(to_np(xs), xs_ref)
        if delta > 0:
            assert (to_np(xq) & 0x7F).max() == 0x7E     # clipped to 448, never NaN


@pytest.mark.parametrize("name,sizes", [("qproj_prefill", dict(T=300, Tc=512, K=1024, N=640)),
                                        ("rmsnorm_qkv", dict(T=130, Tc=256, K=2048, N=384))])
def test_static_fp8_linear_end_to_end(name, sizes):
    wl = synth.WORKLOADS[name].with_sizes(**sizes)
    say(f"fp8 static linear {name} {sizes}")
    inp = synth.make_inputs(wl)
    T, K, N = wl.T, wl.K, wl.N
    g = None if inp.gamma is None else to_dev(inp.gamma)
    xc, w = to_dev(inp.x_cal), to_dev(inp.w)
    _, _, s = gpu_calibrate(xc, w, wl.alpha, norm=wl.norm, gamma=g)
    gp = f32(K)
    sq.sq_smooth_fold(s, g, gp)
    wq, wsc = _u8((N, K)), f32(N)
    sq.sq_quant_weight_fp8(w, s, wq, wsc)
    d = _gpu_static_scale_fp8(xc, gp, norm=wl.norm)
    y = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
    work = torch.empty(sq.sq_linear_workspace_bytes(T, K), dtype=torch.uint8, device=DEV)
    dbg_xq, dbg_xs, rr = _u8((T, K)), f32(T), f32(T)
    bias = to_dev(inp.bias)
    sq.sq_w8a8_linear_static_fp8(to_dev(inp.x), gp, d, wq, wsc, y, work, norm=wl.norm, bias=bias,
                                 dbg_xq=dbg_xq, dbg_x_scale=dbg_xs,
                                 dbg_row_rscale=rr if wl.norm else None)
    acc = torch.empty((T, N), dtype=torch.float32, device=DEV)
    sq.sq_gemm_fp8(dbg_xq, dbg_xs, wq, wsc, None, acc_out=acc)
    torch.cuda.synchronize()
    gp_h, s_h = to_np(gp), to_np(s)
    _check_step(to_np(d)[0], oracle.static_scale_fp8(inp.x_cal, gp_h, norm=wl.norm), wl.norm)
    d_ref = to_np(d)[0]
    _, qw_ref, ws_ref = oracle.prepare_weight_fp8(inp.w, s_h, inp.gamma)
    np.testing.assert_array_equal(to_np(wq), qw_ref)
    out = oracle.linear_static_fp8(inp.x, d_ref, gp_h, qw_ref, ws_ref, inp.bias, norm=wl.norm,
                                   r=to_np(rr) if wl.norm else None)
    np.testing.assert_array_equal(to_np(dbg_xq), out["q"])
    np.testing.assert_array_equal(to_np(dbg_xs), out["x_scale"])
    y_fed = oracle.to_bf16(oracle.epilogue_f32acc(to_np(acc), out["x_scale"], ws_ref, inp.bias))
    np.testing.assert_array_equal(to_np(y), y_fed)
    yo = synth.bf16_bits_to_f32(out["y"])
    yg = synth.bf16_bits_to_f32(to_np(y))
    slack = np.abs(out["x_scale"][:, None] * ws_ref[None, :]) * _acc_bound(out["q"], qw_ref)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(yo), 2.0 ** -126))) - 7)
    assert np.all(np.abs(yg - yo) <= np.maximum(2e-3 * np.abs(yo), 1e-2) + slack + ulp)
    ref = oracle.reference_fp64(inp.x, inp.w, inp.bias, norm=wl.norm, gamma=inp.gamma)
    say(f"  fp8 static-step layer error {oracle.rel_error(ref, to_np(y)):.4%}")
