"""GPU parity of the two weight-quantization paths behind sq_quant_weight and
sq_quant_weight_fp8, bit for bit against the oracle's fold and quantization:

  * the one-launch strip kernel (bf16 weight; every K <= 2048, and K <= 4096
    when the strips fill at most two rounds of the compute units, the last
    at least 90%): 512- and 1024-thread strips with one or two register
    groups of rows, half-empty last strips, a partial second half of K,
    strip counts that are and are not a multiple of the XCD count;
  * the three-launch path (fp32 weights, K > 4096, and K in (2048, 4096]
    with too few or too many strips).

Also the cases the strip kernel's rounding by the reciprocal must hand to the
IEEE division: quotients on and within a few ulps of half-integers, an
all-zero column (zero step) and a step whose reciprocal overflows.
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
from _gpu_util import DEV, f32, say, to_dev, to_np  # noqa: E402

F32 = np.float32

# (K, N) on a 256-CU part: strip kernel for (4096, 4096), (4096, 8192),
# (3072, 3688) and every K <= 2048; three-launch path for the rest
SHAPES = [(4096, 4096), (4096, 8192), (3072, 3688), (4096, 264), (3072, 24), (2048, 1032),
          (1088, 72), (1024, 128), (704, 520), (64, 8), (8192, 136)]


def _weight(K, N, seed):
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((K, N)).astype(F32) * F32(0.02)
    w[rng.permutation(K)[:3]] *= 25                    # outlier input channels
    w[:, rng.permutation(N)[:2]] *= 8                  # and output channels
    s = np.exp(rng.normal(0.0, 1.0, K)).astype(F32)   # smoothing factors around 1
    return synth.f32_to_bf16_bits(w), s


def _quant(w_dev, s_dev, K, N, fp8=False):
    wq = torch.empty((N, K), dtype=torch.uint8 if fp8 else torch.int8, device=DEV)
    ws = f32(N)
    (sq.sq_quant_weight_fp8 if fp8 else sq.sq_quant_weight)(w_dev, s_dev, wq, ws)
    torch.cuda.synchronize()
    return to_np(wq), to_np(ws)


@pytest.mark.parametrize("K,N", SHAPES)
def test_quant_weight_bf16_paths(K, N):
    w, s = _weight(K, N, K * 31 + N)
    say(f"quant weight bf16 K={K} N={N}")
    wd, sd = to_dev(w), to_dev(s)
    _, what = oracle.fold(s, None, w)
    qw_ref, ws_ref = oracle.quant_weight(what)
    qw, ws = _quant(wd, sd, K, N)
    np.testing.assert_array_equal(ws, ws_ref)
    np.testing.assert_array_equal(qw, qw_ref)
    # unfused: s = NULL quantizes W itself
    qw_ref2, ws_ref2 = oracle.quant_weight(synth.bf16_bits_to_f32(w))
    qw2, ws2 = _quant(wd, None, K, N)
    np.testing.assert_array_equal(ws2, ws_ref2)
    np.testing.assert_array_equal(qw2, qw_ref2)


@pytest.mark.parametrize("K,N", [(4096, 4096), (3072, 3688), (4096, 264), (1088, 72), (704, 520),
                                 (8192, 136)])
def test_quant_weight_fp8_bf16_paths(K, N):
    w, s = _weight(K, N, K * 17 + N)
    say(f"quant weight fp8 bf16 K={K} N={N}")
    _, what = oracle.fold(s, None, w)
    qw_ref, ws_ref = oracle.quant_weight_fp8(what)
    qw, ws = _quant(to_dev(w), to_dev(s), K, N, fp8=True)
    np.testing.assert_array_equal(ws, ws_ref)
    np.testing.assert_array_equal(qw, qw_ref)


def test_quant_weight_fp32_path():
    K, N = 512, 40
    rng = np.random.default_rng(5)
    w = rng.standard_normal((K, N)).astype(F32)
    s = np.exp(rng.normal(0.0, 1.0, K)).astype(F32)
    say("quant weight fp32")
    _, what = oracle.fold(s, None, w)
    qw_ref, ws_ref = oracle.quant_weight(what)
    qw, ws = _quant(to_dev(w), to_dev(s), K, N)
    np.testing.assert_array_equal(ws, ws_ref)
    np.testing.assert_array_equal(qw, qw_ref)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_quant_weight_near_ties_and_degenerate_steps(dt):
    """Columns whose step is 3 or 1.5 exactly (row 0 sets the maximum: W = 1
    or 0.5 times s_0 = 381), with every other W^ = +-s_j and s_j within three
    ulps of (m + 1/2) * 3: the quotients sit on or next to half-integers, where
    rounding by fp32(1/3) and by the correctly rounded quotient can part.
    Plus an all-zero column and a column whose step is so small that its
    reciprocal overflows.  The same values as a bf16 weight (the strip kernel
    at this size) and as an fp32 one (the three-launch path)."""
    K, N = 1024, 64
    rng = np.random.default_rng(11)
    m = rng.integers(0, 127, K).astype(np.float64)
    base = ((m + 0.5) * 3.0).astype(F32)
    nud = rng.integers(-3, 4, K)
    s = base.copy()
    for j in range(K):
        for _ in range(abs(int(nud[j]))):
            s[j] = np.nextafter(s[j], F32(np.inf) if nud[j] > 0 else F32(0), dtype=F32)
    s[0] = F32(381.0)
    w = np.where(rng.random((K, N)) < 0.5, F32(1.0), F32(-1.0)).astype(F32)
    w[0, :] = 1.0
    w[:, 1::2] *= F32(0.5)                         # step 1.5 on the odd columns
    w[:, 5] = 0.0                                  # zero step
    w[:, 6] = 0.0
    w[0, 6] = F32(2.0 ** -133)                     # bf16 subnormal: step 2^-133 * 381 / 127
    s_col6 = np.float64(2.0 ** -133) * 381.0 / 127.0
    assert 1.0 / s_col6 > np.finfo(F32).max        # its reciprocal overflows in fp32
    wb = synth.f32_to_bf16_bits(w)
    assert np.array_equal(synth.bf16_bits_to_f32(wb), w)   # all exact in bf16
    _, what = oracle.fold(s, None, wb)
    qw_ref, ws_ref = oracle.quant_weight(what)
    assert ws_ref[0] == 3.0 and ws_ref[1] == 1.5 and ws_ref[5] == 0.0
    # near-tie count: quotients within 2^-15 of a half-integer (ties included)
    quot = (what / np.where(ws_ref == 0, 1, ws_ref)[None, :]).astype(F32)
    near = np.abs(np.abs(quot - np.rint(quot)) - 0.5) < 2.0 ** -15
    assert near.sum() > K * N // 4
    say(f"quant weight near ties {dt}")
    qw, ws = _quant(to_dev(wb if dt == "bf16" else w), to_dev(s), K, N)
    np.testing.assert_array_equal(ws, ws_ref)
    np.testing.assert_array_equal(qw, qw_ref)
    assert (qw[5] == 0).all()
