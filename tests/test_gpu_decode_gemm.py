"""The decode GEMM (T <= 64), bit for bit against the oracle: int32
accumulators and the bf16 / fp32 epilogue.  Every kernel shape the launcher
picks on a 256-CU part: 16-channel workgroups of 8 waves (up to 4 tokens, or
K > 4096 with fewer than 256 * 32 channels) and 32-channel workgroups of 4
waves, with 1, 2, 3 and 4 token blocks; per-wave stage counts from 0 (waves
past the last k-step) through the two-stage loop and each of its 1-, 2- and
3-stage tails; N ragged against the channel blocks."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import oracle  # noqa: E402
import w8a8_int8_gemm_amd as sq  # noqa: E402
from _gpu_util import DEV, say, to_dev, to_np  # noqa: E402

# (T, N, K)
ACC_SHAPES = [(1, 8, 64), (4, 300, 14336), (3, 264, 3072), (5, 77, 1088), (16, 520, 704),
              (16, 4096, 8192), (16, 8192, 4160), (16, 136, 4160), (7, 1000, 2048),
              (16, 16, 5120), (16, 8192, 1088), (9, 8200, 2048), (20, 33, 14336),
              (32, 1000, 4160), (40, 77, 1088), (48, 40, 64), (64, 300, 576), (64, 64, 8192)]


def _ops(T, N, K, seed):
    rng = np.random.default_rng(seed)
    q = rng.integers(-127, 128, (T, K), dtype=np.int8)
    qw = rng.integers(-127, 128, (N, K), dtype=np.int8)
    return rng, q, qw


@pytest.mark.parametrize("T,N,K", ACC_SHAPES)
def test_decode_accumulators(T, N, K):
    _, q, qw = _ops(T, N, K, T * 7 + N * 3 + K)
    say(f"decode gemm acc T={T} N={N} K={K}")
    acc = torch.empty((T, N), dtype=torch.int32, device=DEV)
    sq.sq_gemm_w8a8(to_dev(q), None, to_dev(qw), None, None, acc_out=acc)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(acc), oracle.int_gemm(q, qw))


def test_decode_extreme_accumulators():
    """|acc| at its largest: K = 8192 products of 127 * 127, both signs."""
    T, N, K = 16, 48, 8192
    q = np.full((T, K), 127, np.int8)
    q[1::2] = -127
    qw = np.full((N, K), 127, np.int8)
    qw[::3, ::2] = -127
    say("decode gemm extreme")
    acc = torch.empty((T, N), dtype=torch.int32, device=DEV)
    sq.sq_gemm_w8a8(to_dev(q), None, to_dev(qw), None, None, acc_out=acc)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(acc), oracle.int_gemm(q, qw))


@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("T,N,K", [(16, 520, 3072), (1, 77, 1088), (9, 4096, 4096),
                                   (12, 8192, 1024)])
def test_decode_epilogue(T, N, K, out):
    rng, q, qw = _ops(T, N, K, T + N + K)
    xs = rng.uniform(1e-4, 0.5, T).astype(np.float32)
    xs[0] = 0.0
    wsc = rng.uniform(1e-5, 0.01, N).astype(np.float32)
    bias = rng.normal(0, 0.1, N).astype(np.float32)
    step = 8 if out == "bf16" else 4
    ld = (N + 24 + step - 1) // step * step      # padded rows, 16-byte multiples
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    say(f"decode gemm epilogue T={T} N={N} K={K} {out}")
    ybuf = torch.zeros((T, ld), dtype=dt, device=DEV)
    sq.sq_gemm_w8a8(to_dev(q), to_dev(xs), to_dev(qw), to_dev(wsc), ybuf[:, :N], bias=to_dev(bias))
    torch.cuda.synchronize()
    y_ref = oracle.epilogue(oracle.int_gemm(q, qw), xs, wsc, bias)
    yb = to_np(ybuf)
    if out == "bf16":
        np.testing.assert_array_equal(yb[:, :N], oracle.to_bf16(y_ref))
    else:
        np.testing.assert_array_equal(yb[:, :N], y_ref)
    assert np.all(yb[:, N:] == 0)   # the padding is not written
