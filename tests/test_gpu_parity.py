"""GPU parity: every kernel behind the C ABI against the CPU oracle, element by
element, on the same seeded inputs.

The bar: codes, int32 accumulators, absmax values and scales bit-exact when
both sides are fed the same fp32 scales (and RMSNorm factors); the smoothing
factor and the RMSNorm factor within one fp32 ulp of the oracle (both round an
fp64 value whose last bits depend on the library's pow and on summation
order); end-to-end bf16 outputs within 2e-3 relative (1e-2 absolute floor)
of an independent oracle run, and a quantization error no worse than the
oracle's.  Shapes span several tiles, ragged tails and the edge cases.
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

F32 = np.float32


def _ulps(a, b):
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    return np.abs(a.view(np.int32).astype(np.int64) - b.view(np.int32).astype(np.int64))


def _wl(name, **sizes):
    return synth.WORKLOADS[name].with_sizes(**sizes) if sizes else synth.WORKLOADS[name]


# ---------------------------------------------------------------------------
# (a) calibration
# ---------------------------------------------------------------------------

CALIB_CASES = [
    ("tiny", {}),
    ("qproj_prefill", dict(Tc=1001, K=512, N=776)),
    ("gate_up", dict(Tc=333, K=1024, N=1032)),
]


@pytest.mark.parametrize("name,sizes", CALIB_CASES)
def test_calibrate_no_norm(name, sizes):
    wl = _wl(name, **sizes)
    say(f"calibrate no-norm {name} Tc={wl.Tc} K={wl.K} N={wl.N}")
    inp = synth.make_inputs(wl, evaluation=False)
    a, wm, s = gpu_calibrate(to_dev(inp.x_cal), to_dev(inp.w), wl.alpha)
    torch.cuda.synchronize()
    a_ref = oracle.act_absmax(inp.x_cal)
    wm_ref = oracle.weight_absmax(inp.w)
    np.testing.assert_array_equal(to_np(a), a_ref)
    np.testing.assert_array_equal(to_np(wm), wm_ref)
    s_ref = oracle.smooth_factor(a_ref, wm_ref, wl.alpha)
    d = _ulps(to_np(s), s_ref)
    assert d.max() <= 1 and (d == 0).mean() > 0.999, d.max()


def test_calibrate_accumulate_and_alpha_sweep():
    wl = _wl("qproj_prefill", Tc=900, K=256, N=264)
    inp = synth.make_inputs(wl, evaluation=False)
    say("calibrate accumulate + alpha sweep")
    x = to_dev(inp.x_cal)
    w = to_dev(inp.w)
    K = wl.K
    a = f32(K)
    sq.sq_calibrate(x[:400], None, 0.5, a)
    sq.sq_calibrate(x[400:], None, 0.5, a, accumulate=True)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(a), oracle.act_absmax(inp.x_cal))
    wm_ref = oracle.weight_absmax(inp.w)
    for alpha in (0.0, 0.1, 0.25, 0.5, 0.75, 1.0):
        wm, s = f32(K), f32(K)
        sq.sq_calibrate(None, w, alpha, a, wm, s)   # reuse a[]
        torch.cuda.synchronize()
        s_ref = oracle.smooth_factor(to_np(a), wm_ref, alpha)
        assert _ulps(to_np(s), s_ref).max() <= 1, alpha
        if alpha == 1.0:
            np.testing.assert_array_equal(to_np(s), np.maximum(to_np(a), F32(1e-5)))
        if alpha == 0.0:
            np.testing.assert_array_equal(to_np(s), F32(1) / wm_ref)


@pytest.mark.parametrize("K", [320, 4096, 8192])
def test_calibrate_norm(K):
    wl = _wl("rmsnorm_qkv", Tc=517, K=K, N=64)
    say(f"calibrate rmsnorm K={K}")
    inp = synth.make_inputs(wl, evaluation=False)
    g = to_dev(inp.gamma)
    a = f32(K)
    sq.sq_calibrate(to_dev(inp.x_cal), None, wl.alpha, a, norm=True, gamma=g)
    torch.cuda.synchronize()
    a_ref = oracle.act_absmax(inp.x_cal, norm=True, gamma=inp.gamma)
    d = _ulps(to_np(a), a_ref)
    # both sides round the same fp64 RMS factor; its last bit may differ
    assert d.max() <= 1 and (d == 0).mean() > 0.99


def test_calibrate_zero_rows_and_columns():
    K, N = 128, 64
    x = np.zeros((50, K), np.float32)
    x[7, 3] = -2.0
    w = np.zeros((K, N), np.float32)
    w[3, 5] = 0.5
    say("calibrate zero rows/columns")
    a, wm, s = gpu_calibrate(to_dev(x), to_dev(w), 0.5)
    torch.cuda.synchronize()
    a_ref, wm_ref, s_ref = oracle.calibrate(x, w, 0.5)
    np.testing.assert_array_equal(to_np(a), a_ref)
    np.testing.assert_array_equal(to_np(wm), wm_ref)
    np.testing.assert_array_equal(to_np(s), s_ref)   # s = 1 for zero rows of W
    assert to_np(s)[0] == 1.0


# ---------------------------------------------------------------------------
# (b) fold and weight quantization
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,sizes", [("tiny", {}), ("rmsnorm_qkv", dict(Tc=64, K=704, N=520))])
def test_fold_and_quant_weight(name, sizes):
    wl = _wl(name, **sizes)
    say(f"fold + quant weight {name} K={wl.K} N={wl.N}")
    inp = synth.make_inputs(wl, evaluation=False)
    w = to_dev(inp.w)
    _, _, s = gpu_calibrate(to_dev(inp.x_cal), w, wl.alpha, norm=wl.norm,
                            gamma=None if inp.gamma is None else to_dev(inp.gamma))
    g = None if inp.gamma is None else to_dev(inp.gamma)
    gp, wq, wsc = gpu_prepare_weight(w, s, g)
    w_out = torch.empty((wl.K, wl.N), dtype=torch.float32, device=DEV)
    sq.sq_smooth_fold(s, None, None, w, w_out)
    torch.cuda.synchronize()
    s_h = to_np(s)
    gp_ref, what_ref = oracle.fold(s_h, inp.gamma, inp.w)
    np.testing.assert_array_equal(to_np(gp), gp_ref)
    np.testing.assert_array_equal(to_np(w_out), what_ref)
    qw_ref, ws_ref = oracle.quant_weight(what_ref)
    np.testing.assert_array_equal(to_np(wsc), ws_ref)
    np.testing.assert_array_equal(to_np(wq), qw_ref)
    # unfused: quantize the materialised fp32 W^ with s = NULL
    wq2 = torch.empty_like(wq)
    ws2 = f32(wl.N)
    sq.sq_quant_weight(w_out, None, wq2, ws2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(wq2), qw_ref)
    np.testing.assert_array_equal(to_np(ws2), ws_ref)


def test_quant_weight_zero_column():
    w = np.random.default_rng(1).standard_normal((128, 16)).astype(np.float32)
    w[:, 3] = 0
    say("quant weight zero column")
    wq = torch.empty((16, 128), dtype=torch.int8, device=DEV)
    wsc = f32(16)
    sq.sq_quant_weight(to_dev(w), None, wq, wsc)
    torch.cuda.synchronize()
    qw_ref, ws_ref = oracle.quant_weight(w)
    np.testing.assert_array_equal(to_np(wq), qw_ref)
    np.testing.assert_array_equal(to_np(wsc), ws_ref)
    assert ws_ref[3] == 0


# ---------------------------------------------------------------------------
# (c) fused RMSNorm -> smooth -> per-token quant
# ---------------------------------------------------------------------------

# K past 8192: a workgroup per token, the row in registers up to 16384 (whole
# and ragged chunk counts), three passes over the row beyond; up to 4096 tokens
# of 4096-16384 values also take a workgroup per token (both sides of that
# bound at 4096 / 4097 tokens)
QACT_CASES = [(37, 256, "f32"), (300, 4096, "bf16"), (129, 8192, "bf16"), (3, 320, "bf16"),
              (5, 16384, "bf16"), (64, 1024, "f32"), (11, 14336, "bf16"), (4, 8256, "bf16"),
              (7, 10304, "f32"), (3, 24576, "bf16"), (256, 4096, "bf16"), (1000, 4096, "bf16"),
              (200, 4096, "f32"), (16, 12288, "bf16"), (4096, 4096, "bf16"), (4097, 4096, "bf16")]


@pytest.mark.parametrize("norm", [False, True])
@pytest.mark.parametrize("T,K,dt", QACT_CASES)
def test_quant_act(T, K, dt, norm):
    rng = np.random.default_rng(T * 7 + K)
    x = rng.standard_normal((T, K)).astype(np.float32)
    x[:, rng.permutation(K)[:5]] *= 40
    if T > 2:
        x[1] = 0.0                                   # a zero token
        x[2, :] = np.float32(0.5) * np.arange(K) % 5  # exact half-steps (ties)
        x[2, 0] = 127.0 if not norm else x[2, 0]
    xin = synth.f32_to_bf16_bits(x) if dt == "bf16" else x
    g = rng.uniform(0.01, 3.0, K).astype(np.float32)
    say(f"quant act T={T} K={K} {dt} norm={norm}")
    xq = torch.empty((T, K), dtype=torch.int8, device=DEV)
    xs = f32(T)
    rr = f32(T) if norm else None
    sq.sq_quant_act(to_dev(xin), to_dev(g), xq, xs, norm=norm, row_rscale=rr)
    torch.cuda.synchronize()
    r_gpu = to_np(rr) if norm else None
    q_ref, xs_ref, r_ref = oracle.quant_act(xin, g, norm=norm, r=r_gpu)
    np.testing.assert_array_equal(to_np(xs), xs_ref)
    np.testing.assert_array_equal(to_np(xq), q_ref)
    if norm:
        r_own = oracle.rms_rscale(xin)
        assert _ulps(r_gpu, r_own).max() <= 1


@pytest.mark.parametrize("T,K,dt,norm", [(6, 14336, "bf16", False), (3, 4096, "bf16", False),
                                         (5, 16384, "bf16", True), (4, 12288, "f32", False),
                                         (3, 9216, "f32", True), (2, 16384, "f32", False),
                                         (3, 8256, "bf16", False)])
def test_quant_act_without_gamma(T, K, dt, norm):
    """gamma_f = NULL (an unsmoothed linear): the factor 1 on both sides.  Rows
    of 8200-16384 values take the workgroup-per-token register kernel."""
    rng = np.random.default_rng(T + K)
    x = rng.standard_normal((T, K)).astype(np.float32)
    x[:, rng.permutation(K)[:5]] *= 40
    if T > 2:
        x[1] = 0.0                                   # a zero token
    xin = synth.f32_to_bf16_bits(x) if dt == "bf16" else x
    say(f"quant act without gamma T={T} K={K} {dt} norm={norm}")
    xq = torch.empty((T, K), dtype=torch.int8, device=DEV)
    xs = f32(T)
    rr = f32(T) if norm else None
    sq.sq_quant_act(to_dev(xin), None, xq, xs, norm=norm, row_rscale=rr)
    torch.cuda.synchronize()
    r_gpu = to_np(rr) if norm else None
    q_ref, xs_ref, _ = oracle.quant_act(xin, np.ones(K, np.float32), norm=norm, r=r_gpu)
    np.testing.assert_array_equal(to_np(xs), xs_ref)
    np.testing.assert_array_equal(to_np(xq), q_ref)
    if norm:
        assert _ulps(r_gpu, oracle.rms_rscale(xin)).max() <= 1


def test_quant_act_ties_and_fallback():
    """Rows whose quotients sit exactly on half-integers take the division path."""
    K = 512
    x = np.zeros((4, K), np.float32)
    x[:, 0] = 127.0                                   # Delta = 1 exactly
    x[0, 1:] = (np.arange(1, K) % 255 - 127) + 0.5    # every value a tie
    x[1, 1:] = (np.arange(1, K) % 255 - 127) + 0.5 + 1e-5
    x[2, 1:] = np.linspace(-126.9, 126.9, K - 1)
    x[3, 0] = 1e-38                                   # Delta subnormal
    x[3, 1:4] = [5e-39, -3e-39, 1e-39]
    say("quant act ties")
    xq = torch.empty((4, K), dtype=torch.int8, device=DEV)
    xs = f32(4)
    sq.sq_quant_act(to_dev(x), None, xq, xs)
    torch.cuda.synchronize()
    q_ref, xs_ref, _ = oracle.quant_act(x, None)
    np.testing.assert_array_equal(to_np(xs), xs_ref)
    np.testing.assert_array_equal(to_np(xq), q_ref)


# ---------------------------------------------------------------------------
# (d) INT8 GEMM and epilogue
# ---------------------------------------------------------------------------

GEMM_SHAPES = [(300, 520, 704), (256, 256, 4096), (513, 1000, 128), (1, 520, 704), (16, 520, 704),
               (17, 264, 640), (33, 96, 192), (64, 1024, 1024), (65, 8, 64), (1000, 40, 64),
               (384, 2056, 512),
               # 128 x 256 tiles (ragged T), then 128 x 384 tiles (one round of
               # them fills the GPU where 256 x 256 tiles would not): ragged T
               # and N, 64- and 128-byte stages, and whole tiles
               (1500, 4096, 256), (1800, 6104, 128), (1500, 6000, 192), (1536, 6144, 128),
               # ragged N on the tile kernels: 128 x 128 tiles with 64- and
               # 128-byte stages, 128 x 256 and 256 x 256 tiles
               (300, 77, 704), (257, 1003, 128), (129, 4, 64), (2100, 3001, 256),
               (4096, 3001, 128),
               # more tiles than workgroups (each workgroup walks several tiles;
               # the last round partial), ragged T and N: 374 tiles of 256 x 192,
               # 380 of 256 x 256, 510 of 128 x 256, 506 of 128 x 384, 493 of
               # 256 x 192; then one round: 242 tiles of 128 x 384, 195 of
               # 256 x 192
               (4200, 4100, 192), (4625, 4999, 64), (6402, 2312, 192), (2827, 8068, 64),
               (7179, 3091, 128), (1290, 8068, 128), (1044, 7427, 128)]


@pytest.mark.parametrize("T,N,K", GEMM_SHAPES)
def test_gemm_accumulators(T, N, K):
    rng = np.random.default_rng(T + 3 * N + 7 * K)
    q = rng.integers(-127, 128, (T, K), dtype=np.int8)
    qw = rng.integers(-127, 128, (N, K), dtype=np.int8)
    say(f"gemm acc T={T} N={N} K={K}")
    acc = torch.empty((T, N), dtype=torch.int32, device=DEV)
    sq.sq_gemm_w8a8(to_dev(q), None, to_dev(qw), None, None, acc_out=acc)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(acc), oracle.int_gemm(q, qw))


def test_gemm_two_launches_in_flight_on_two_streams():
    """Two persistent GEMM launches, each with as many workgroups as the device
    holds, queued on two streams at once: the workgroups of the second wait
    for free compute units (no workgroup waits for another), and both results
    equal the oracle."""
    shapes = [(4200, 4100, 192), (7179, 3091, 128)]
    rng = np.random.default_rng(11)
    ops = []
    for T, N, K in shapes:
        q = rng.integers(-127, 128, (T, K), dtype=np.int8)
        qw = rng.integers(-127, 128, (N, K), dtype=np.int8)
        ops.append((q, qw, torch.empty((T, N), dtype=torch.int32, device=DEV)))
    say("gemm two streams")
    dq = [(to_dev(q), to_dev(qw)) for q, qw, _ in ops]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for (xq, wq), (_, _, acc), st in zip(dq, ops, streams):
            sq.sq_gemm_w8a8(xq, None, wq, None, None, acc_out=acc, stream=st)
    torch.cuda.synchronize()
    for q, qw, acc in ops:
        np.testing.assert_array_equal(to_np(acc), oracle.int_gemm(q, qw))


@pytest.mark.parametrize("T,N,K", [(2, 8, 65536), (65, 16, 65536)])
def test_gemm_extreme_accumulators(T, N, K):
    q = np.full((T, K), 127, np.int8)
    q[1::2] = -127
    qw = np.full((N, K), 127, np.int8)
    qw[::3, ::2] = -127
    say(f"gemm extreme T={T} N={N} K={K}")
    acc = torch.empty((T, N), dtype=torch.int32, device=DEV)
    sq.sq_gemm_w8a8(to_dev(q), None, to_dev(qw), None, None, acc_out=acc)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(acc), oracle.int_gemm(q, qw))


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("with_bias", [False, True])
@pytest.mark.parametrize("T,N,K", [(300, 520, 704), (16, 264, 512), (40, 77, 128), (512, 512, 256),
                                   (300, 77, 768), (257, 1003, 128), (129, 4, 64),
                                   (2100, 3001, 256), (1500, 6000, 192), (4200, 4100, 128),
                                   (7179, 3091, 64), (6402, 2312, 128), (4625, 4999, 64)])
def test_gemm_epilogue(T, N, K, out, with_bias):
    rng = np.random.default_rng(T * N + K)
    q = rng.integers(-127, 128, (T, K), dtype=np.int8)
    qw = rng.integers(-127, 128, (N, K), dtype=np.int8)
    xs = rng.uniform(1e-4, 0.5, T).astype(np.float32)
    xs[0] = 0.0
    wsc = rng.uniform(1e-5, 0.01, N).astype(np.float32)
    bias = rng.normal(0, 0.1, N).astype(np.float32) if with_bias else None
    ld = N + 24 if out == "bf16" else N + 12   # padded rows, still 16-byte multiples
    if out == "bf16":
        ld = (ld + 7) // 8 * 8
    else:
        ld = (ld + 3) // 4 * 4
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    say(f"gemm epilogue T={T} N={N} K={K} {out} bias={with_bias}")
    ybuf = torch.zeros((T, ld), dtype=dt, device=DEV)
    y = ybuf[:, :N]
    sq.sq_gemm_w8a8(to_dev(q), to_dev(xs), to_dev(qw), to_dev(wsc), y,
                    bias=None if bias is None else to_dev(bias))
    torch.cuda.synchronize()
    y_ref = oracle.epilogue(oracle.int_gemm(q, qw), xs, wsc, bias)
    yb = to_np(ybuf)
    if out == "bf16":
        np.testing.assert_array_equal(yb[:, :N], oracle.to_bf16(y_ref))
    else:
        np.testing.assert_array_equal(yb[:, :N], y_ref)
    assert np.all(yb[:, N:] == 0)   # the padding is not written


# ---------------------------------------------------------------------------
# (a)-(d) end to end
# ---------------------------------------------------------------------------

E2E_CASES = [
    ("tiny", {}),
    ("qproj_prefill", dict(T=300, Tc=1024, K=1024, N=776)),
    ("rmsnorm_qkv", dict(T=257, Tc=600, K=1024, N=1544)),
    ("gate_up", dict(T=130, Tc=512, K=512, N=2048)),
    ("decode", dict(T=16, Tc=700, K=2048, N=1024)),
]


@pytest.mark.parametrize("name,sizes", E2E_CASES)
def test_end_to_end(name, sizes):
    wl = _wl(name, **sizes)
    say(f"end to end {name} T={wl.T} K={wl.K} N={wl.N} Tc={wl.Tc}")
    inp = synth.make_inputs(wl)
    g = None if inp.gamma is None else to_dev(inp.gamma)
    w = to_dev(inp.w)
    _, _, s = gpu_calibrate(to_dev(inp.x_cal), w, wl.alpha, norm=wl.norm, gamma=g)
    gp, wq, wsc = gpu_prepare_weight(w, s, g)
    out_dt = torch.bfloat16 if wl.io_dtype == "bf16" else torch.float32
    y, dbg = gpu_linear(to_dev(inp.x), gp, wq, wsc, to_dev(inp.bias), norm=wl.norm,
                        out_dtype=out_dt)
    torch.cuda.synchronize()
    yg = to_np(y)
    # 1. fed the GPU's s (and r): every intermediate and the output bit-exact
    s_h = to_np(s)
    gp_ref, qw_ref, ws_ref = oracle.prepare_weight(inp.w, s_h, inp.gamma)
    np.testing.assert_array_equal(to_np(gp), gp_ref)
    np.testing.assert_array_equal(to_np(wq), qw_ref)
    np.testing.assert_array_equal(to_np(wsc), ws_ref)
    r_gpu = to_np(dbg["dbg_row_rscale"]) if wl.norm else None
    fed = oracle.linear(inp.x, gp_ref, qw_ref, ws_ref, inp.bias, norm=wl.norm, r=r_gpu,
                        out_bf16=wl.io_dtype == "bf16")
    np.testing.assert_array_equal(to_np(dbg["dbg_xq"]), fed["q"])
    np.testing.assert_array_equal(to_np(dbg["dbg_x_scale"]), fed["x_scale"])
    np.testing.assert_array_equal(yg, fed["y"])
    # 2. independent oracle run: outputs within 2e-3 relative, 1e-2 absolute floor
    _, _, s_ref = oracle.calibrate(inp.x_cal, inp.w, wl.alpha, norm=wl.norm, gamma=inp.gamma)
    gp2, qw2, ws2 = oracle.prepare_weight(inp.w, s_ref, inp.gamma)
    own = oracle.linear(inp.x, gp2, qw2, ws2, inp.bias, norm=wl.norm,
                        out_bf16=wl.io_dtype == "bf16")
    yo = synth.bf16_bits_to_f32(own["y"]) if wl.io_dtype == "bf16" else own["y"]
    yf = synth.bf16_bits_to_f32(yg) if wl.io_dtype == "bf16" else yg
    tol = np.maximum(2e-3 * np.abs(yo), 1e-2)
    assert np.all(np.abs(yf - yo) <= tol)
    # 3. quantization error against the fp64 unsmoothed layer: no worse than the oracle's
    ref = oracle.reference_fp64(inp.x, inp.w, inp.bias, norm=wl.norm, gamma=inp.gamma)
    e_gpu = oracle.rel_error(ref, yg)
    e_ora = oracle.rel_error(ref, own["y"])
    say(f"  rel error gpu {e_gpu:.5f} oracle {e_ora:.5f}")
    assert e_gpu <= e_ora * (1 + 1e-6) + 1e-12
