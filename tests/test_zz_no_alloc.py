"""sq_w8a8_linear_noalloc -- the forward without a workspace argument, for
callers that cannot allocate -- against sq_w8a8_linear with a workspace: the
same codes, steps and outputs bit for bit, on two calls in a row (the second
smaller, so the shared scratch array holds the first call's larger contents),
in plain and RMSNorm mode; and the size limit refused before any launch."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import synth  # noqa: E402
import w8a8_int8_gemm_amd as sq  # noqa: E402
from _gpu_util import DEV, f32, gpu_calibrate, gpu_prepare_weight, say, to_dev, to_np  # noqa: E402

SCRATCH_BYTES = 64 << 20     # SQ_NOALLOC_SCRATCH_BYTES


def _case(name, sizes):
    wl = synth.WORKLOADS[name].with_sizes(**sizes)
    inp = synth.make_inputs(wl)
    g = None if inp.gamma is None else to_dev(inp.gamma)
    w = to_dev(inp.w)
    _, _, s = gpu_calibrate(to_dev(inp.x_cal), w, wl.alpha, norm=wl.norm, gamma=g)
    gp, wq, wsc = gpu_prepare_weight(w, s, g)
    return wl, to_dev(inp.x), gp, wq, wsc, to_dev(inp.bias)


def _run(fn, wl, x, gp, wq, wsc, b, **kw):
    T, K, N = wl.T, wl.K, wl.N
    y = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
    rr = f32(T) if wl.norm else None
    fn(x, gp, wq, wsc, y, norm=wl.norm, bias=b, dbg_row_rscale=rr, **kw)
    return y, rr


def test_noalloc_equals_workspace_linear():
    # the second call is smaller: the scratch array still holds the first
    # call's codes beyond what the second writes
    cases = [("rmsnorm_qkv", dict(T=1100, Tc=256, K=2048, N=1032)),
             ("qproj_prefill", dict(T=129, Tc=200, K=512, N=264))]
    for name, sizes in cases:
        say(f"noalloc linear {name} {sizes}")
        wl, x, gp, wq, wsc, b = _case(name, sizes)
        T, K = wl.T, wl.K
        work = torch.empty(sq.sq_linear_workspace_bytes(T, K), dtype=torch.uint8, device=DEV)
        y_ref, r_ref = _run(lambda *a, **k: sq.sq_w8a8_linear(*a[:5], work, **k),
                            wl, x, gp, wq, wsc, b)
        y_na, r_na = _run(sq.sq_w8a8_linear_noalloc, wl, x, gp, wq, wsc, b)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_np(y_na), to_np(y_ref))
        if wl.norm:
            np.testing.assert_array_equal(to_np(r_na), to_np(r_ref))
        # the codes and steps the no-allocation call left in its scratch equal
        # the workspace call's (read back through the debug outputs of a third
        # call that supplies its own buffers for them)
        xq, xs = torch.empty((T, K), dtype=torch.int8, device=DEV), f32(T)
        y_dbg = torch.empty_like(y_ref)
        sq.sq_w8a8_linear_noalloc(x, gp, wq, wsc, y_dbg, norm=wl.norm, bias=b, dbg_xq=xq,
                                  dbg_x_scale=xs)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(to_np(xq), to_np(work[:T * K].view(torch.int8)).reshape(T, K))
        np.testing.assert_array_equal(to_np(y_dbg), to_np(y_ref))


def test_noalloc_refuses_inputs_past_its_scratch():
    say("noalloc size limit")
    K = 4096
    T = SCRATCH_BYTES // K          # codes alone fill the array; the steps do not fit
    x = torch.zeros((T, K), dtype=torch.bfloat16, device=DEV)
    wq = torch.zeros((8, K), dtype=torch.int8, device=DEV)
    y = torch.full((T, 8), 3.0, dtype=torch.bfloat16, device=DEV)
    assert sq.sq_linear_workspace_bytes(T, K) > SCRATCH_BYTES
    with pytest.raises(sq.SQError) as e:
        sq.sq_w8a8_linear_noalloc(x, None, wq, f32(8, 1.0), y)
    assert e.value.status == sq.SQ_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
    # the most tokens that fit
    T2 = T
    while sq.sq_linear_workspace_bytes(T2, K) > SCRATCH_BYTES:
        T2 -= 1
    assert T2 == T - 16
    y2 = torch.empty((T2, 8), dtype=torch.bfloat16, device=DEV)
    sq.sq_w8a8_linear_noalloc(x[:T2], None, wq, f32(8, 1.0), y2)
    torch.cuda.synchronize()
    assert bool((y2 == 0).all())    # zero input, zero weight codes, no bias
