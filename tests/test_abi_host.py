"""Host-side checks of libsqw8a8.so that need no GPU: the library loads, it
exports every function include/sq_w8a8.h declares, and argument validation
returns the documented status before anything is launched.

The validation tests pass fabricated device addresses with arguments that
must fail validation.  They run only in a process that sees no GPU: there a
validation regression that let a call through would fail its launch (no
device) instead of running a kernel on a wild address.  Where a GPU is
visible they are skipped (the same checks run in every CPU test run)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sq_w8a8.h")

import w8a8_int8_gemm_amd as sq  # noqa: E402


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(sq.LIB_PATH):
        from w8a8_int8_gemm_amd import build
        build.build()
    return sq.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(sq_[a-z0-9_]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("sq_calibrate", "sq_smooth_fold", "sq_quant_weight", "sq_w8a8_linear",
              "sq_quant_act", "sq_gemm_w8a8", "sq_linear_workspace_bytes", "sq_status_string",
              "sq_abi_version"):
        assert n in names, n


def test_library_exports_every_declared_symbol(L):
    for n in _declared_functions():
        assert hasattr(L, n), f"libsqw8a8.so does not export {n}"
    assert L.sq_abi_version() == 1


def test_status_strings(L):
    for code in range(8):
        s = sq.status_string(code)
        assert s.startswith("SQ_")
    assert "unknown" in sq.status_string(99)


def test_workspace_size(L):
    assert sq.sq_linear_workspace_bytes(0, 4096) == 0
    assert sq.sq_linear_workspace_bytes(1, 64) == 256 + 256
    assert sq.sq_linear_workspace_bytes(8192, 4096) == 8192 * 4096 + 8192 * 4


# fake, never-dereferenced device addresses; every call below fails validation
A16 = 0x7F0000000000
MIS = A16 + 8


def _gpu_visible() -> bool:
    # counting devices does not initialise the HIP runtime
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:  # noqa: BLE001 -- no torch: no GPU this process can reach
        return False


no_device = pytest.mark.skipif(
    _gpu_visible(), reason="passes fabricated device addresses: runs only where no GPU is "
    "visible, so a validation regression cannot launch a kernel on them")


@no_device
def test_calibrate_validation(L):
    c = L.sq_calibrate
    # K rules
    assert c(A16, sq.SQ_BF16, 10, 0, 0, 0, None, 1e-6, None, 0, 0, 0, 0.5, 0, A16, None, None, None) == sq.SQ_ERR_SHAPE
    assert c(A16, sq.SQ_BF16, 10, 96, 96, 0, None, 1e-6, None, 0, 0, 0, 0.5, 0, A16, None, None, None) == sq.SQ_ERR_UNSUPPORTED
    assert c(A16, sq.SQ_BF16, 10, 65536 + 64, 65600, 0, None, 1e-6, None, 0, 0, 0, 0.5, 0, A16, None, None, None) == sq.SQ_ERR_UNSUPPORTED
    # a required
    assert c(A16, sq.SQ_BF16, 10, 64, 64, 0, None, 1e-6, None, 0, 0, 0, 0.5, 0, None, None, None, None) == sq.SQ_ERR_NULL
    # dtype, leading dimension, alignment
    assert c(A16, sq.SQ_I8, 10, 64, 64, 0, None, 1e-6, None, 0, 0, 0, 0.5, 0, A16, None, None, None) == sq.SQ_ERR_DTYPE
    assert c(A16, sq.SQ_BF16, 10, 64, 32, 0, None, 1e-6, None, 0, 0, 0, 0.5, 0, A16, None, None, None) == sq.SQ_ERR_SHAPE
    assert c(A16, sq.SQ_BF16, -1, 64, 64, 0, None, 1e-6, None, 0, 0, 0, 0.5, 0, A16, None, None, None) == sq.SQ_ERR_SHAPE
    assert c(MIS, sq.SQ_BF16, 10, 64, 64, 0, None, 1e-6, None, 0, 0, 0, 0.5, 0, A16, None, None, None) == sq.SQ_ERR_UNSUPPORTED
    assert c(A16, sq.SQ_BF16, 10, 64, 68, 0, None, 1e-6, None, 0, 0, 0, 0.5, 0, A16, None, None, None) == sq.SQ_ERR_UNSUPPORTED
    # norm mode limits and flags
    # x_cal is required unless the activation pass is skipped; skipping it with
    # no weight leaves nothing to do
    assert c(None, sq.SQ_BF16, 10, 64, 64, 0, None, 1e-6, None, 0, 0, 0, 0.5, 0, A16, None, None, None) == sq.SQ_ERR_NULL
    assert c(None, sq.SQ_BF16, 10, 64, 64, 0, None, 1e-6, None, 0, 0, 0, 0.5, 2, A16, None, None, None) == sq.SQ_OK
    assert c(A16, sq.SQ_BF16, 10, 64, 64, 1, None, -1.0, None, 0, 0, 0, 0.5, 0, A16, None, None, None) == sq.SQ_ERR_SHAPE
    assert c(A16, sq.SQ_BF16, 10, 64, 64, 7, None, 1e-6, None, 0, 0, 0, 0.5, 0, A16, None, None, None) == sq.SQ_ERR_UNSUPPORTED
    assert c(A16, sq.SQ_BF16, 10, 64, 64, 0, None, 1e-6, None, 0, 0, 0, 0.5, 4, A16, None, None, None) == sq.SQ_ERR_UNSUPPORTED
    # weight side (activation pass skipped): alpha range, wmax/s required
    for bad in (-0.1, 1.5, float("nan"), float("inf")):
        assert c(None, 0, 0, 64, 64, 0, None, 1e-6, A16, sq.SQ_BF16, 64, 64, bad, 2, A16, A16, A16, None) == sq.SQ_ERR_ALPHA
    assert c(None, 0, 0, 64, 64, 0, None, 1e-6, A16, sq.SQ_BF16, 64, 64, 0.5, 2, A16, None, A16, None) == sq.SQ_ERR_NULL
    assert c(None, 0, 0, 64, 64, 0, None, 1e-6, A16, sq.SQ_BF16, 60, 56, 0.5, 2, A16, A16, A16, None) == sq.SQ_ERR_SHAPE


@no_device
def test_fold_and_quant_weight_validation(L):
    assert L.sq_smooth_fold(None, 64, None, A16, None, 0, 0, 0, None, None) == sq.SQ_ERR_NULL
    assert L.sq_smooth_fold(A16, 100, None, A16, None, 0, 0, 0, None, None) == sq.SQ_ERR_UNSUPPORTED
    assert L.sq_smooth_fold(A16, 64, None, A16, A16, sq.SQ_BF16, 64, 64, MIS, None) == sq.SQ_ERR_UNSUPPORTED
    q = L.sq_quant_weight
    assert q(None, sq.SQ_BF16, 64, 64, 64, None, A16, A16, None) == sq.SQ_ERR_NULL
    assert q(A16, sq.SQ_BF16, 64, 64, 64, None, None, A16, None) == sq.SQ_ERR_NULL
    assert q(A16, sq.SQ_BF16, 64, 12, 12, None, A16, A16, None) == sq.SQ_ERR_UNSUPPORTED   # ld 24 B
    assert q(A16, sq.SQ_F32, 64, 64, 32, None, A16, A16, None) == sq.SQ_ERR_SHAPE
    assert q(A16, sq.SQ_BF16, 64, 64, 64, None, MIS, A16, None) == sq.SQ_ERR_UNSUPPORTED
    assert q(A16, sq.SQ_I32, 64, 64, 64, None, A16, A16, None) == sq.SQ_ERR_DTYPE


@no_device
def test_act_gemm_linear_validation(L):
    a = L.sq_quant_act
    assert a(A16, sq.SQ_BF16, 4, 64, 64, 0, None, 1e-6, None, A16, None, None) == sq.SQ_ERR_NULL
    assert a(A16, sq.SQ_BF16, 4, 64, 64, 0, None, 1e-6, MIS, A16, None, None) == sq.SQ_ERR_UNSUPPORTED
    g = L.sq_gemm_w8a8
    assert g(None, A16, 4, 64, A16, A16, 8, None, A16, sq.SQ_BF16, 8, None, None) == sq.SQ_ERR_NULL
    assert g(A16, A16, 4, 64, A16, A16, 8, None, None, sq.SQ_BF16, 8, None, None) == sq.SQ_ERR_NULL
    assert g(A16, A16, 4, 64, A16, A16, 8, None, A16, sq.SQ_I8, 8, None, None) == sq.SQ_ERR_DTYPE
    assert g(A16, A16, 4, 64, A16, A16, 8, None, A16, sq.SQ_BF16, 4, None, None) == sq.SQ_ERR_SHAPE
    assert g(A16, A16, 4, 64, A16, A16, 8, None, A16, sq.SQ_BF16, 12, None, None) == sq.SQ_ERR_UNSUPPORTED
    assert g(A16, A16, 4, 80, A16, A16, 8, None, A16, sq.SQ_BF16, 8, None, None) == sq.SQ_ERR_UNSUPPORTED
    assert g(A16, A16, 4, 64, A16, A16, 8, None, None, sq.SQ_BF16, 8, MIS, None) == sq.SQ_ERR_UNSUPPORTED
    lin = L.sq_w8a8_linear
    # workspace missing, too small, misaligned
    assert lin(A16, sq.SQ_BF16, 4, 64, 64, 0, None, 1e-6, A16, A16, 8, None, A16, sq.SQ_BF16, 8,
               None, 0, None, None) == sq.SQ_ERR_WORKSPACE
    assert lin(A16, sq.SQ_BF16, 4, 64, 64, 0, None, 1e-6, A16, A16, 8, None, A16, sq.SQ_BF16, 8,
               A16, 16, None, None) == sq.SQ_ERR_WORKSPACE
    assert lin(A16, sq.SQ_BF16, 4, 64, 64, 0, None, 1e-6, A16, A16, 8, None, A16, sq.SQ_BF16, 8,
               A16 + 16, 1 << 20, None, None) == sq.SQ_ERR_WORKSPACE
    assert lin(A16, sq.SQ_BF16, 4, 64, 64, 0, None, 1e-6, None, A16, 8, None, A16, sq.SQ_BF16, 8,
               A16, 1 << 20, None, None) == sq.SQ_ERR_NULL
    # empty inputs are accepted and launch nothing
    assert a(A16, sq.SQ_BF16, 0, 64, 64, 0, None, 1e-6, A16, A16, None, None) == sq.SQ_OK
    assert g(A16, A16, 0, 64, A16, A16, 8, None, A16, sq.SQ_BF16, 8, None, None) == sq.SQ_OK
    assert lin(A16, sq.SQ_BF16, 0, 64, 64, 0, None, 1e-6, A16, A16, 8, None, A16, sq.SQ_BF16, 8,
               None, 0, None, None) == sq.SQ_OK


@no_device
def test_static_step_validation(L):
    st = L.sq_act_static_scale
    assert st(None, None, 64, A16, None) == sq.SQ_ERR_NULL
    assert st(A16, None, 64, None, None) == sq.SQ_ERR_NULL
    assert st(A16, None, 0, A16, None) == sq.SQ_ERR_SHAPE
    assert st(A16, None, 96, A16, None) == sq.SQ_ERR_UNSUPPORTED
    qs = L.sq_quant_act_static
    assert qs(A16, sq.SQ_BF16, 4, 64, 64, 0, None, 1e-6, None, A16, A16, None, None) == sq.SQ_ERR_NULL
    assert qs(A16, sq.SQ_BF16, 4, 64, 64, 0, None, 1e-6, A16, None, A16, None, None) == sq.SQ_ERR_NULL
    assert qs(A16, sq.SQ_BF16, 4, 64, 64, 0, None, 1e-6, A16, MIS, A16, None, None) == sq.SQ_ERR_UNSUPPORTED
    assert qs(A16, sq.SQ_BF16, 0, 64, 64, 0, None, 1e-6, A16, A16, A16, None, None) == sq.SQ_OK
    ls = L.sq_w8a8_linear_static
    assert ls(A16, sq.SQ_BF16, 4, 64, 64, 0, None, 1e-6, None, A16, A16, 8, None, A16,
              sq.SQ_BF16, 8, A16, 1 << 20, None, None) == sq.SQ_ERR_NULL
    assert ls(A16, sq.SQ_BF16, 4, 64, 64, 0, None, 1e-6, A16, A16, A16, 8, None, A16,
              sq.SQ_BF16, 8, None, 0, None, None) == sq.SQ_ERR_WORKSPACE


@no_device
def test_fp8_validation(L):
    qw = L.sq_quant_weight_fp8
    assert qw(None, sq.SQ_BF16, 64, 64, 64, None, A16, A16, None) == sq.SQ_ERR_NULL
    assert qw(A16, sq.SQ_BF16, 64, 12, 12, None, A16, A16, None) == sq.SQ_ERR_UNSUPPORTED   # ld 24 B
    qa = L.sq_quant_act_fp8
    assert qa(A16, sq.SQ_BF16, 4, 64, 64, 0, None, 1e-6, None, A16, None, None) == sq.SQ_ERR_NULL
    assert qa(A16, sq.SQ_BF16, 4, 64, 64, 0, None, 1e-6, MIS, A16, None, None) == sq.SQ_ERR_UNSUPPORTED
    assert qa(A16, sq.SQ_BF16, 0, 64, 64, 0, None, 1e-6, A16, A16, None, None) == sq.SQ_OK
    g = L.sq_gemm_fp8
    assert g(None, A16, 4, 64, A16, A16, 8, None, A16, sq.SQ_BF16, 8, None, None) == sq.SQ_ERR_NULL
    assert g(A16, A16, 4, 80, A16, A16, 8, None, A16, sq.SQ_BF16, 8, None, None) == sq.SQ_ERR_UNSUPPORTED
    assert g(A16, A16, 0, 64, A16, A16, 8, None, A16, sq.SQ_BF16, 8, None, None) == sq.SQ_OK
    lin = L.sq_w8a8_linear_fp8
    assert lin(A16, sq.SQ_BF16, 4, 64, 64, 0, None, 1e-6, A16, A16, 8, None, A16, sq.SQ_BF16, 8,
               None, 0, None, None) == sq.SQ_ERR_WORKSPACE


@no_device
def test_static_fp8_validation(L):
    st = L.sq_act_static_scale_fp8
    assert st(None, None, 64, A16, None) == sq.SQ_ERR_NULL
    assert st(A16, None, 64, None, None) == sq.SQ_ERR_NULL
    assert st(A16, None, 0, A16, None) == sq.SQ_ERR_SHAPE
    assert st(A16, None, 96, A16, None) == sq.SQ_ERR_UNSUPPORTED
    qs = L.sq_quant_act_static_fp8
    assert qs(A16, sq.SQ_BF16, 4, 64, 64, 0, None, 1e-6, None, A16, A16, None, None) == sq.SQ_ERR_NULL
    assert qs(A16, sq.SQ_BF16, 4, 64, 64, 0, None, 1e-6, A16, None, A16, None, None) == sq.SQ_ERR_NULL
    assert qs(A16, sq.SQ_BF16, 4, 64, 64, 0, None, 1e-6, A16, MIS, A16, None, None) == sq.SQ_ERR_UNSUPPORTED
    assert qs(A16, sq.SQ_BF16, 0, 64, 64, 0, None, 1e-6, A16, A16, A16, None, None) == sq.SQ_OK
    ls = L.sq_w8a8_linear_static_fp8
    assert ls(A16, sq.SQ_BF16, 4, 64, 64, 0, None, 1e-6, None, A16, A16, 8, None, A16,
              sq.SQ_BF16, 8, A16, 1 << 20, None, None) == sq.SQ_ERR_NULL
    assert ls(A16, sq.SQ_BF16, 4, 64, 64, 0, None, 1e-6, A16, A16, A16, 8, None, A16,
              sq.SQ_BF16, 8, None, 0, None, None) == sq.SQ_ERR_WORKSPACE


@no_device
def test_layernorm_and_fold_prev_validation(L):
    c = L.sq_calibrate_ln
    assert c(A16, sq.SQ_BF16, 8, 64, 64, None, None, 1e-6, None, sq.SQ_BF16, 0, 0, 0.5, 0,
             None, None, None, None) == sq.SQ_ERR_NULL
    assert c(A16, sq.SQ_BF16, 8, 64, 64, None, None, 1e-6, None, sq.SQ_BF16, 0, 0, 0.5, 8,
             A16, None, None, None) == sq.SQ_ERR_UNSUPPORTED      # unknown flag
    assert c(A16, sq.SQ_BF16, 8, 64, 64, None, None, -1.0, None, sq.SQ_BF16, 0, 0, 0.5, 0,
             A16, None, None, None) == sq.SQ_ERR_SHAPE
    assert c(None, sq.SQ_BF16, 0, 64, 64, None, None, 1e-6, A16, sq.SQ_BF16, 8, 8, 1.5, 2,
             A16, A16, A16, None) == sq.SQ_ERR_ALPHA
    assert c(None, sq.SQ_BF16, 0, 64, 64, None, None, 1e-6, A16, sq.SQ_BF16, 8, 8, 0.5, 0,
             A16, A16, A16, None) == sq.SQ_ERR_NULL               # x_cal without the skip flag
    f = L.sq_smooth_fold_ln
    assert f(A16, 64, None, None, A16, None, None) == sq.SQ_ERR_NULL
    assert f(A16, 96, None, None, A16, A16, None) == sq.SQ_ERR_UNSUPPORTED
    q = L.sq_quant_act_ln
    assert q(A16, sq.SQ_BF16, 4, 64, 64, None, A16, 1e-6, A16, A16, None, None, None) == sq.SQ_ERR_NULL
    assert q(A16, sq.SQ_BF16, 4, 64, 64, A16, None, 1e-6, A16, A16, None, None, None) == sq.SQ_ERR_NULL
    assert q(A16, sq.SQ_BF16, 4, 64, 64, A16, MIS, 1e-6, A16, A16, None, None, None) == sq.SQ_ERR_UNSUPPORTED
    assert q(A16, sq.SQ_BF16, 0, 64, 64, A16, A16, 1e-6, A16, A16, None, None, None) == sq.SQ_OK
    lin = L.sq_w8a8_linear_ln
    assert lin(A16, sq.SQ_BF16, 4, 64, 64, None, A16, 1e-6, A16, A16, 8, None, A16, sq.SQ_BF16, 8,
               A16, 1 << 20, None, None, None) == sq.SQ_ERR_NULL
    assert lin(A16, sq.SQ_BF16, 4, 64, 64, A16, A16, 1e-6, A16, A16, 8, None, A16, sq.SQ_BF16, 8,
               None, 0, None, None, None) == sq.SQ_ERR_WORKSPACE
    fp = L.sq_fold_prev_linear
    assert fp(None, 64, A16, sq.SQ_BF16, 8, 64, A16, 64, None, None, None) == sq.SQ_ERR_NULL
    assert fp(A16, 64, A16, sq.SQ_BF16, 8, 32, A16, 64, None, None, None) == sq.SQ_ERR_SHAPE
    assert fp(A16, 64, A16, sq.SQ_BF16, 8, 64, A16, 62, None, None, None) == sq.SQ_ERR_SHAPE
    assert fp(A16, 64, A16, sq.SQ_BF16, 8, 64, A16, 66, None, None, None) == sq.SQ_ERR_UNSUPPORTED
    assert fp(A16, 64, A16, sq.SQ_BF16, 8, 64, A16, 64, A16, None, None) == sq.SQ_ERR_NULL
    assert fp(A16, 64, A16, sq.SQ_I8, 8, 64, A16, 64, None, None, None) == sq.SQ_ERR_DTYPE


@no_device
def test_gptq_validation(L):
    g = L.sq_quant_weight_gptq
    ws = L.sq_gptq_workspace_bytes(8, 64, 64)
    assert ws > 64 * 64 * 8 * 2
    assert L.sq_gptq_workspace_bytes(0, 64, 64) == 0
    args = [A16, sq.SQ_BF16, 8, 64, 0, None, 1e-6, A16, sq.SQ_BF16, 64, 64, 64, None, 0.01, A16,
            A16, None, A16, ws, None]

    def call(**kw):
        a = list(args)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return g(*a)

    assert call(a14=None) == sq.SQ_ERR_NULL                   # wq
    assert call(a15=None) == sq.SQ_ERR_NULL                   # w_scale
    assert call(a7=None) == sq.SQ_ERR_NULL                    # w
    assert call(a2=0) == sq.SQ_ERR_SHAPE                      # no calibration tokens
    assert call(a13=-1.0) == sq.SQ_ERR_SHAPE                  # damp
    assert call(a10=12, a11=12) == sq.SQ_ERR_UNSUPPORTED      # ldw of 24 bytes
    assert call(a9=16384 + 64, a3=16448, a11=64) == sq.SQ_ERR_UNSUPPORTED   # k too large
    assert call(a17=None) == sq.SQ_ERR_WORKSPACE
    assert call(a18=ws - 1) == sq.SQ_ERR_WORKSPACE
    assert call(a17=MIS) == sq.SQ_ERR_WORKSPACE


@no_device
def test_noalloc_validation(L):
    f = L.sq_w8a8_linear_noalloc
    assert f(None, sq.SQ_BF16, 4, 64, 64, 0, None, 1e-6, A16, A16, 8, None, A16, sq.SQ_BF16, 8,
             None, None) == sq.SQ_ERR_NULL
    assert f(A16, sq.SQ_BF16, 4, 96, 96, 0, None, 1e-6, A16, A16, 8, None, A16, sq.SQ_BF16, 8,
             None, None) == sq.SQ_ERR_UNSUPPORTED
    # past the scratch array: refused before the device is touched
    t = (64 << 20) // 4096
    assert f(A16, sq.SQ_BF16, t, 4096, 4096, 0, None, 1e-6, A16, A16, 8, None, A16, sq.SQ_BF16, 8,
             None, None) == sq.SQ_ERR_WORKSPACE


@no_device
def test_row_limits(L):
    big = (1 << 24) + 1
    assert L.sq_quant_act(A16, sq.SQ_BF16, big, 64, 64, 0, None, 1e-6, A16, A16, None,
                          None) == sq.SQ_ERR_UNSUPPORTED
    assert L.sq_gemm_w8a8(A16, A16, big, 64, A16, A16, 8, None, A16, sq.SQ_BF16, 8, None,
                          None) == sq.SQ_ERR_UNSUPPORTED
    assert L.sq_gemm_w8a8(A16, A16, 8, 64, A16, A16, big, None, A16, sq.SQ_BF16, big + 7, None,
                          None) == sq.SQ_ERR_UNSUPPORTED


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(sq, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(sq, "_lib", None)
    with pytest.raises(ImportError):
        sq.lib()
