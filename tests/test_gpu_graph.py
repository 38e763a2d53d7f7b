"""The forward captured in a HIP graph (torch.cuda.graph drives stream
capture; the library launches on the capturing stream and allocates nothing
inside the calls).  Every replay must equal the eager result bit for bit;
replays are interleaved with eager work and synchronizations, and the
captured inputs are rewritten between replays so each replay recomputes.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import synth  # noqa: E402
import w8a8_int8_gemm_amd as sq  # noqa: E402
from _gpu_util import DEV, f32, gpu_calibrate, gpu_prepare_weight, say, to_dev  # noqa: E402


@pytest.mark.parametrize("name,sizes", [("decode", dict(T=16, Tc=64, K=4096, N=4096)),
                                        ("rmsnorm_qkv", dict(T=300, Tc=256, K=1024, N=640)),
                                        # several GEMM tiles per workgroup (363 of 128 x 384)
                                        ("qproj_prefill", dict(T=4200, Tc=256, K=512, N=4104))])
def test_linear_graph_replays_match_eager(name, sizes):
    wl = synth.WORKLOADS[name].with_sizes(**sizes)
    say(f"graph replay {name} {sizes}")
    inp = synth.make_inputs(wl)
    T, K, N = wl.T, wl.K, wl.N
    g = None if inp.gamma is None else to_dev(inp.gamma)
    w = to_dev(inp.w)
    _, _, s = gpu_calibrate(to_dev(inp.x_cal), w, wl.alpha, norm=wl.norm, gamma=g)
    gp, wq, wsc = gpu_prepare_weight(w, s, g)
    bias = to_dev(inp.bias)
    x_static = to_dev(inp.x).clone()
    y_static = torch.empty((T, N), dtype=torch.bfloat16, device=DEV)
    work = torch.empty(sq.sq_linear_workspace_bytes(T, K), dtype=torch.uint8, device=DEV)

    def forward(x, y):
        sq.sq_w8a8_linear(x, gp, wq, wsc, y, work, norm=wl.norm, bias=bias)

    # inputs for the replays: the workload's tokens, scaled and permuted
    rng = np.random.default_rng(9)
    xs = [x_static.clone()]
    for i in range(3):
        xs.append(x_static[torch.from_numpy(rng.permutation(T)).to(DEV)] * (0.5 + i))
    eager = []
    for x in xs:
        y = torch.empty_like(y_static)
        forward(x, y)
        eager.append(y)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm the library up off the default stream
        forward(x_static, y_static)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        forward(x_static, y_static)
    torch.cuda.synchronize()
    for rep in range(2):
        for i, x in enumerate(xs):
            x_static.copy_(x)
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(y_static, eager[i]), (rep, i)
            # eager work between replays
            other = torch.empty_like(y_static)
            forward(xs[(i + 1) % len(xs)], other)
            torch.cuda.synchronize()
            assert torch.equal(other, eager[(i + 1) % len(xs)])


def test_calibrate_and_prepare_graph_replays():
    """The offline phase too (its zero fills are kernels, not memsets):
    calibrate, fold and quantize the weight inside one graph."""
    wl = synth.WORKLOADS["qproj_prefill"].with_sizes(T=8, Tc=512, K=1024, N=768)
    say("graph replay calibrate + prepare")
    inp = synth.make_inputs(wl)
    K, N = wl.K, wl.N
    xc_static, w_static = to_dev(inp.x_cal).clone(), to_dev(inp.w).clone()
    a, wm, s, gp, wsc = f32(K), f32(K), f32(K), f32(K), f32(N)
    wq = torch.empty((N, K), dtype=torch.int8, device=DEV)

    def prepare():
        sq.sq_calibrate(xc_static, w_static, wl.alpha, a, wm, s)
        sq.sq_smooth_fold(s, None, gp)
        sq.sq_quant_weight(w_static, s, wq, wsc)

    def snapshot():
        return [t.clone() for t in (a, wm, s, gp, wsc, wq)]

    variants = [(xc_static.clone(), w_static.clone())]
    for f in (2.0, 0.25):
        variants.append((variants[0][0] * f, (variants[0][1] * (1.0 / f))))
    eager = []
    for xc, ww in variants:
        xc_static.copy_(xc)
        w_static.copy_(ww)
        prepare()
        torch.cuda.synchronize()
        eager.append(snapshot())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        prepare()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        prepare()
    torch.cuda.synchronize()
    for rep in range(2):
        for i, (xc, ww) in enumerate(variants):
            xc_static.copy_(xc)
            w_static.copy_(ww)
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for got, want in zip(snapshot(), eager[i]):
                assert torch.equal(got, want), (rep, i)
