#!/usr/bin/env python3
"""Benchmark of the SmoothQuant W8A8 linear on one MI355X.

One step is one pass of the whole path over one batch of the 4096-wide
query-projection prefill workload (T = 8192 tokens, K = N = 4096, 8192
calibration tokens, alpha 0.5, bf16 in and out), inputs resident in HBM:

  sq_calibrate    activation absmax over X_cal, weight absmax, s
  sq_smooth_fold  gamma' = 1/s
  sq_quant_weight per-output-channel INT8 weight (fold fused)
  sq_quant_act    per-token INT8 activations          } together: sq_w8a8_linear
  sq_gemm_w8a8    INT8 MFMA GEMM + dequant/bias epilogue }

`value` is 2*T*K*N integer ops per step / step time (TOPS).  Every kernel is
also timed on its own with HIP events on the stream it runs on; the roofline
object is for the GEMM (MFMA bound, against the INT8 dense peak).  The steps
take their inputs in turn from --sets copies in HBM, so the 256 MB Infinity
Cache does not hold a step's inputs from the step before.  The CPU oracle is
timed on the host on the same inputs (a bounded sample of tokens).

Untimed extras on the same line: the layer's output error against the fp64
product per migration strength alpha (and without smoothing), with per-token
and with static per-tensor activation steps; the static-step activation
quantizer's time next to the per-token one; and the decode-shaped GEMM
(16 x 8192 x 8192, HBM bound) in GB/s.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-extras]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W8A8 smoothed linear TOPS + % of MI355X INT8 MFMA peak (T=8192,K=N=4096)"
PEAK_INT8_TOPS = 5000.0     # MI355X dense INT8 MFMA, 5.0 POP/s
PEAK_SCLK_GHZ = 2.4         # the shader clock that peak is quoted at
N_XCD, N_SIMD = 8, 1024     # MI355X: 8 XCDs, 256 compute units x 4 SIMDs
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, 8 TB/s
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense FP8 MFMA, 5.0 PFLOP/s
WORKLOAD = "qproj_prefill"
COUNTERS = os.path.join(ROOT, "profiles", "gemm_w8a8_qproj_prefill_counters.json")


def _parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--rocpd-summary", metavar="DB", default=None,
                    help="print a text summary of a rocprofv3 result database (kernel "
                         "durations, or counters per kernel) instead of benchmarking")
    ap.add_argument("--counters-json", metavar="PATH", default=None,
                    help="with --rocpd-summary of FETCH_SIZE and WRITE_SIZE databases "
                         "(comma-separated), write the GEMM's HBM bytes per launch, scaled "
                         "by the copy probe, to PATH")
    ap.add_argument("--sets", type=int, default=3,
                    help="copies of the input set (X_cal, X, W) in HBM, used in turn by the "
                         "steps, so that no step finds its inputs in the 256 MB Infinity Cache")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the untimed extras: the error per alpha and the decode GEMM")
    ap.add_argument("--gemm-loop", type=float, default=0.0, metavar="SECONDS",
                    help="instead of benchmarking, run only the headline GEMM back to back for "
                         "this long (for sampling power and clocks from outside) and print the "
                         "time per launch")
    ap.add_argument("--only", choices=("gptq", "decoder_layer", "configs", "rmsnorm_qkv",
                                       "gate_up", "decode"),
                    default=None,
                    help="instead of benchmarking, run only this extra and print its JSON "
                         "(for profiling one part on its own)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the timed steps, run one plain elementwise copy kernel over "
                         "this many MiB (reads and writes that many bytes): the reference "
                         "that scales the HBM byte counters of a profiling run")
    return ap.parse_args()


class HipTimer:
    """Timing events from the HIP runtime this process already runs (the copy
    torch loaded, found in /proc/self/maps, so that no second runtime is
    loaded), created with hipEventDisableSystemFence: recording one then ends
    with no system-scope release, which on this GPU writes back and
    invalidates the L2 and holds the stream for microseconds.  The events
    only time work: the host reads them after a device synchronize."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        path = next((ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln),
                    None)
        if path is None:
            raise RuntimeError("no HIP runtime loaded in this process")
        self._c = ctypes
        self.L = ctypes.CDLL(path)
        self.L.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                               ctypes.c_void_p]
        self.L.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self) -> int:
        e = self._c.c_void_p()
        rc = self.L.hipEventCreateWithFlags(self._c.byref(e), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")
        return e.value

    def record(self, e: int, stream) -> None:
        rc = self.L.hipEventRecord(e, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def ms(self, a: int, b: int) -> float:
        f = self._c.c_float()
        rc = self.L.hipEventElapsedTime(self._c.byref(f), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return f.value

    def destroy(self, events) -> None:
        for e in events:
            self.L.hipEventDestroy(e)


def _kernel_hash() -> str:
    """Hash of the GEMM's device code: k_gemm.hip up to its host-launcher
    section, and the device helpers of sq_common.h, with comments and
    whitespace removed (a comment edit does not invalidate the counters)."""
    import re
    h = hashlib.sha256()
    for f in ("k_gemm.hip", "sq_common.h"):
        with open(os.path.join(ROOT, "w8a8_int8_gemm_amd", "csrc", f), encoding="utf-8") as fh:
            text = fh.read()
        if f == "k_gemm.hip":
            text = text.split("// host launcher", 1)[0]
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def _counters():
    """The committed rocprofv3 counter record of the GEMM, if it was taken on
    the current kernel source; else {}."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return {}
    return c if c.get("kernel_source_sha256_16") == _kernel_hash() else {}


def _traffic(gemm_launch_bytes_alg: float):
    """HBM bytes per GEMM launch from the committed counter record, or None."""
    return _counters().get("hbm_bytes_per_launch")


def _clock_fields(achieved_tops: float) -> dict:
    """The shader clock the counter pass observed over a GEMM launch
    (GRBM_GUI_ACTIVE cycles per XCD / launch time), the INT8 peak at that
    clock, this run's fraction of it, and the share of cycles MFMA-busy."""
    c = _counters()
    if "sclk_ghz" not in c:
        return {"sclk_ghz": None}
    peak = PEAK_INT8_TOPS * c["sclk_ghz"] / PEAK_SCLK_GHZ
    return {"sclk_ghz": c["sclk_ghz"], "peak_at_sclk": peak, "frac_at_sclk": achieved_tops / peak,
            "mfma_busy": c.get("mfma_busy")}


def _rocpd_rows(db):
    import sqlite3
    con = sqlite3.connect(db)
    names = {r[0] for r in con.execute("select name from sqlite_master where type='view'")}
    out = {"trace": [], "pmc": []}
    if "kernels" in names:
        durs = {}
        for n, d in con.execute("select name, duration from kernels"):
            durs.setdefault(n, []).append(d)
        rows = []
        for n, ds in durs.items():
            ds.sort()
            m = len(ds) // 2
            med = ds[m] if len(ds) % 2 else 0.5 * (ds[m - 1] + ds[m])
            rows.append((n, len(ds), sum(ds) / len(ds), ds[0], ds[-1], med, sum(ds)))
        out["trace"] = [r[:6] for r in sorted(rows, key=lambda r: -r[6])]
    if "counters_collection" in names:
        out["pmc"] = list(con.execute(
            "select kernel_name, counter_name, avg(value), count(*), avg(duration) "
            "from counters_collection group by kernel_name, counter_name order by kernel_name"))
    return out


def _short(name: str) -> str:
    return name.split("(")[0].replace("void ", "")[:70]


def rocpd_summary(dbs: str, counters_json=None) -> None:
    """Text summary of rocprofv3 result databases (durations in microseconds)."""
    fetch = write = copy_fetch = copy_write = None
    grbm = mfma = gemm_us = None
    for db in dbs.split(","):
        rows = _rocpd_rows(db)
        print(f"# {db}")
        if rows["trace"] and not rows["pmc"]:
            print(f"{'kernel':70s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} "
                  f"{'median_us':>10s}")
            for n, c, a, lo, hi, med in rows["trace"]:
                print(f"{_short(n):70s} {c:6d} {a / 1e3:10.2f} {lo / 1e3:10.2f} {hi / 1e3:10.2f} "
                      f"{med / 1e3:10.2f}")
        for kn, cn, v, c, d in rows["pmc"]:
            print(f"{_short(kn):70s} {cn:28s} {v:18.1f}  n={c:<4d} avg_us={d / 1e3:.2f}")
            if "k_gemm_w8a8" in kn and cn == "FETCH_SIZE":
                fetch = v * 1024.0
            if "k_gemm_w8a8" in kn and cn == "WRITE_SIZE":
                write = v * 1024.0
            if "neg_kernel" in kn and cn == "FETCH_SIZE":
                copy_fetch = v * 1024.0
            if "neg_kernel" in kn and cn == "WRITE_SIZE":
                copy_write = v * 1024.0
            if "k_gemm_w8a8<256, 256" in kn and cn == "GRBM_GUI_ACTIVE":
                grbm, gemm_us = v, d / 1e3
            if "k_gemm_w8a8<256, 256" in kn and cn == "SQ_VALU_MFMA_BUSY_CYCLES":
                mfma = v
    if counters_json and fetch is not None and write is not None and copy_fetch and copy_write:
        probe = float(os.environ.get("COPY_PROBE_BYTES", 256 << 20))
        ff, wf = probe / copy_fetch, probe / copy_write
        rec = {"kernel_source_sha256_16": _kernel_hash(), "fetch_factor": ff, "write_factor": wf,
               "fetch_bytes_per_launch": fetch * ff, "write_bytes_per_launch": write * wf,
               "hbm_bytes_per_launch": fetch * ff + write * wf}
        if grbm and mfma and gemm_us:
            cyc = grbm / N_XCD                          # GPU cycles per XCD over a launch
            rec["sclk_ghz"] = cyc / (gemm_us * 1e3)
            rec["mfma_busy"] = mfma / N_SIMD / cyc
        with open(counters_json, "w") as f:
            json.dump(rec, f, indent=1)
        print(f"# scale factors: fetch {ff:.3f} write {wf:.3f}; GEMM HBM bytes per launch "
              f"{rec['hbm_bytes_per_launch'] / 2**20:.1f} MiB -> {counters_json}")
        if "sclk_ghz" in rec:
            print(f"# GEMM: {rec['sclk_ghz']:.2f} GHz average shader clock, "
                  f"{rec['mfma_busy']:.1%} of cycles MFMA-busy")


def alpha_sweep(sq, torch, inp, wl, x_cal, x, w, bias, dev, sample=256):
    """Relative Frobenius error of the W8A8 layer output against X W + b in
    fp64, per migration strength alpha and without smoothing (s = 1), over a
    sample of tokens.  Untimed; the GPU computes every layer output, numpy
    computes the fp64 reference of the sampled rows."""
    import numpy as np

    T, K, N = wl.T, wl.K, wl.N
    rows = np.linspace(0, T - 1, sample).astype(np.int64)

    def f64(bits):
        return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    ref = f64(inp.x[rows]) @ f64(inp.w) + inp.bias.astype(np.float64)[None, :]
    ref_norm = float(np.linalg.norm(ref))
    e = lambda n: torch.empty(n, dtype=torch.float32, device=dev)  # noqa: E731
    a, wm, s, gp, wsc, xs = e(K), e(K), e(K), e(K), e(N), e(T)
    wq = torch.empty((N, K), dtype=torch.int8, device=dev)
    xq = torch.empty((T, K), dtype=torch.int8, device=dev)
    y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    wq8 = torch.empty((N, K), dtype=torch.uint8, device=dev)
    xq8 = torch.empty((T, K), dtype=torch.uint8, device=dev)
    d = e(1)
    sq.sq_calibrate(x_cal, None, 0.5, a)           # activation absmax once
    res, res_static, res_fp8, res_fp8s = {}, {}, {}, {}
    for alpha in (None, 0.1, 0.25, 0.5, 0.75, 1.0):
        key = "unsmoothed" if alpha is None else f"{alpha:g}"
        gamma_f, s_arg = None, None                # unsmoothed: s = 1, gamma_f = 1
        if alpha is not None:
            sq.sq_calibrate(None, w, alpha, a, wm, s)   # s from the stored absmax
            sq.sq_smooth_fold(s, None, gp)
            gamma_f, s_arg = gp, s
        sq.sq_quant_weight(w, s_arg, wq, wsc)
        for mode, out in (("per_token", res), ("static", res_static), ("fp8", res_fp8),
                          ("fp8_static", res_fp8s)):
            if mode == "static":                   # one step from the calibration maximum
                sq.sq_act_static_scale(a, gamma_f, d)
                sq.sq_quant_act_static(x, gamma_f, d, xq, xs)
                sq.sq_gemm_w8a8(xq, xs, wq, wsc, y, bias=bias)
            elif mode == "fp8":                    # E4M3 weights and per-token activations
                sq.sq_quant_weight_fp8(w, s_arg, wq8, wsc)
                sq.sq_quant_act_fp8(x, gamma_f, xq8, xs)
                sq.sq_gemm_fp8(xq8, xs, wq8, wsc, y, bias=bias)
            elif mode == "fp8_static":             # E4M3, one static activation step
                sq.sq_act_static_scale_fp8(a, gamma_f, d)
                sq.sq_quant_act_static_fp8(x, gamma_f, d, xq8, xs)
                sq.sq_gemm_fp8(xq8, xs, wq8, wsc, y, bias=bias)
            else:
                sq.sq_quant_act(x, gamma_f, xq, xs)
                sq.sq_gemm_w8a8(xq, xs, wq, wsc, y, bias=bias)
            torch.cuda.synchronize()
            yb = y[torch.from_numpy(rows).to(dev)].view(torch.int16).cpu().numpy().view(np.uint16)
            out[key] = float(np.linalg.norm(f64(yb) - ref)) / ref_norm
    res["static_per_tensor"] = res_static
    res["fp8_e4m3_per_token"] = res_fp8
    res["fp8_e4m3_static_per_tensor"] = res_fp8s
    res["tokens"] = int(sample)
    res["reference"] = ("X W + b in fp64 over evenly spaced tokens; relative Frobenius norm; "
                        "top level: INT8 per-token activation steps")
    return res


def hbm_ceilings(torch, dev, T=8192, K=4096, copies=3, iters=20):
    """Practical HBM ceilings on this machine, measured in the same run with the
    vendor's own kernels of the same traffic shape as the path's memory-bound
    kernels, on `copies` rotating inputs (past the Infinity Cache):
      column_absmax: torch.amax over dim 0 of |X| for X [T, K] bf16 (reads 2 B
                     per element, writes K floats) -- the calibration pass;
      read2_write1:  X [T, K] bf16 -> int8 (reads 2 B, writes 1 B per element)
                     -- the activation and weight quantizers' traffic;
      copy:          a [T, K] fp32 copy (reads 4 B, writes 4 B per element)."""
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    xs = [torch.randn((T, K), dtype=torch.bfloat16, device=dev, generator=g) for _ in range(copies)]
    o8 = torch.empty((T, K), dtype=torch.int8, device=dev)
    f32 = [x.float() for x in xs[:2]]
    of = torch.empty_like(f32[0])
    am = torch.empty(K, dtype=torch.bfloat16, device=dev)

    def timed(fn, n):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    out = {}
    us = timed(lambda i: torch.amax(xs[i % copies], dim=0, out=am), iters)
    out["column_max"] = {"us": us, "GB/s": 2.0 * T * K / (us * 1e-6) / 1e9,
                         "note": "torch.amax over dim 0: the calibration pass's traffic"}
    us = timed(lambda i: o8.copy_(xs[i % copies]), iters)
    out["read2_write1"] = {"us": us, "GB/s": 3.0 * T * K / (us * 1e-6) / 1e9,
                           "note": "bf16 -> int8 conversion: the quantizers' traffic"}
    us = timed(lambda i: of.copy_(f32[i % 2]), iters)
    out["copy"] = {"us": us, "GB/s": 8.0 * T * K / (us * 1e-6) / 1e9, "note": "fp32 copy"}
    for v in out.values():
        v["frac_of_peak"] = v["GB/s"] / PEAK_HBM_GBS
    out["workload"] = f"[{T}, {K}] inputs, {copies} rotating copies, vendor kernels"
    del xs, f32
    return out


def vendor_int8_gemm(torch, xq, wq, iters=20):
    """Reference point only: the vendor library's INT8 GEMM (torch._int_mm,
    hipBLASLt on this stack) on the same codes, int32 output without the
    epilogue, event-timed."""
    wt = wq.t()
    try:
        torch._int_mm(xq, wt)
    except Exception as e:  # noqa: BLE001 -- a missing backend is reported, not fatal
        return {"error": str(e)[:200]}
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        torch._int_mm(xq, wt)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / iters
    T, K = xq.shape
    N = wq.shape[0]
    return {"op": "torch._int_mm (hipBLASLt), int32 out, same shape", "us": us,
            "tops": 2.0 * T * K * N / (us * 1e-6) / 1e12}


def fp8_timing(sq, torch, sets, wl, s, gp, bias, dev, iters=20):
    """Event times of the FP8 E4M3 weight and activation quantizers and the
    FP8 GEMM on the headline shape (rotating input sets), the GEMM against
    the dense FP8 matrix peak."""
    T, K, N = wl.T, wl.K, wl.N
    wq8 = torch.empty((N, K), dtype=torch.uint8, device=dev)
    xq8 = [torch.empty((T, K), dtype=torch.uint8, device=dev) for _ in sets]
    wsc = torch.empty(N, dtype=torch.float32, device=dev)
    xs = [torch.empty(T, dtype=torch.float32, device=dev) for _ in sets]
    y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    calls = {
        "quant_weight_fp8": lambda i: sq.sq_quant_weight_fp8(sets[i][2], s, wq8, wsc,
                                                             stream=stream),
        "quant_act_fp8": lambda i: sq.sq_quant_act_fp8(sets[i][1], gp, xq8[i], xs[i],
                                                       stream=stream),
        "gemm_fp8": lambda i: sq.sq_gemm_fp8(xq8[i], xs[i], wq8, wsc, y, bias=bias,
                                             stream=stream),
    }
    out = {}
    for name, fn in calls.items():
        for i in range(len(sets)):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(iters):
            fn(i % len(sets))
        e1.record(stream)
        torch.cuda.synchronize()
        out[name + "_us"] = e0.elapsed_time(e1) * 1e3 / iters
    ops = 2.0 * T * K * N
    ach = ops / (out["gemm_fp8_us"] * 1e-6) / 1e12
    out["gemm_fp8"] = {"achieved": ach, "unit": "TFLOP/s", "peak": PEAK_FP8_TFLOPS,
                       "frac": ach / PEAK_FP8_TFLOPS}
    return out


def static_act_timing(sq, torch, sets, gp, a, xq, xs, dev, iters=20):
    """Event time of the static-step activation quantizer (no per-token
    maximum) next to the per-token one, on the rotating input sets."""
    d = torch.empty(1, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    sq.sq_act_static_scale(a, gp, d, stream=stream)
    out = {}
    for name, fn in (("per_token", lambda x: sq.sq_quant_act(x, gp, xq, xs, stream=stream)),
                     ("static", lambda x: sq.sq_quant_act_static(x, gp, d, xq, xs,
                                                                 stream=stream))):
        for i in range(len(sets)):
            fn(sets[i][1])
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(iters):
            fn(sets[i % len(sets)][1])
        e1.record(stream)
        torch.cuda.synchronize()
        out[name + "_us"] = e0.elapsed_time(e1) * 1e3 / iters
    return out


def gemm_loop(sq, torch, inp, wl, d, dev, seconds):
    """The headline GEMM alone, back to back for `seconds`, on the workload's own
    quantized operands (calibrate, fold, quantize once, untimed)."""
    T, K, N = wl.T, wl.K, wl.N
    x_cal, x, w, bias = d(inp.x_cal), d(inp.x), d(inp.w), d(inp.bias)
    e = lambda n: torch.empty(n, dtype=torch.float32, device=dev)  # noqa: E731
    a, wm, s, gp, wsc, xs = e(K), e(K), e(K), e(K), e(N), e(T)
    wq = torch.empty((N, K), dtype=torch.int8, device=dev)
    xq = torch.empty((T, K), dtype=torch.int8, device=dev)
    y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    sq.sq_calibrate(x_cal, w, wl.alpha, a, wm, s)
    sq.sq_smooth_fold(s, None, gp)
    sq.sq_quant_weight(w, s, wq, wsc)
    sq.sq_quant_act(x, gp, xq, xs)
    torch.cuda.synchronize()
    n = 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_end = time.time() + seconds
    e0.record()
    while time.time() < t_end:
        for _ in range(50):
            sq.sq_gemm_w8a8(xq, xs, wq, wsc, y, bias=bias)
        torch.cuda.synchronize()
        n += 50
    e1.record()
    torch.cuda.synchronize()
    print(json.dumps({"gemm_loop_launches": n, "us_per_launch": e0.elapsed_time(e1) * 1e3 / n}),
          flush=True)


def decode_gemm(sq, torch, dev, T=16, K=8192, N=8192, copies=5, iters=50):
    """Decode-shaped INT8 GEMM (16 tokens, K = N = 8192): HBM-bound on the
    64 MiB weight.  Five weight copies (320 MiB) are used in turn so that the
    weight never sits in the Infinity Cache.  Returns the event time per call
    and the algorithmic bytes moved per second."""
    g = torch.Generator(device=dev)
    g.manual_seed(105)
    wqs = [torch.randint(-127, 128, (N, K), dtype=torch.int8, device=dev, generator=g)
           for _ in range(copies)]
    xq = torch.randint(-127, 128, (T, K), dtype=torch.int8, device=dev, generator=g)
    xs = torch.rand(T, device=dev, generator=g) * 1e-2
    ws = torch.rand(N, device=dev, generator=g) * 1e-3
    y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    for i in range(copies):
        sq.sq_gemm_w8a8(xq, xs, wqs[i], ws, y, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(iters):
        sq.sq_gemm_w8a8(xq, xs, wqs[i % copies], ws, y, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / iters
    byts = K * N + T * K + 4.0 * (T + N) + 2.0 * T * N
    gbs = byts / (us * 1e-6) / 1e9
    return {"workload": f"decode T={T} K={K} N={N}", "us": us, "achieved": gbs, "unit": "GB/s",
            "frac_of_peak": gbs / PEAK_HBM_GBS,
            "algorithmic": "K*N weight bytes + T*K + scales + 2*T*N output bytes per call"}


def block_timing(sq, torch, dev, T=2048, H=4096, KV=1024, I=14336, iters=10):
    """The online forward of one decoder layer's four W8A8 linears, wired as
    the pages map them: RMSNorm -> q|k|v and RMSNorm -> gate|up through the
    fused norm + smooth + quantize kernel, o_proj and down_proj plain per-token
    (Llama-8B-like shapes, T tokens of prefill).  Weights are random INT8
    codes with random steps (timing only).  Also the LayerNorm form of the
    q|k|v input's quantizer and its calibration pass, in GB/s."""
    g = torch.Generator(device=dev)
    g.manual_seed(107)
    stream = torch.cuda.current_stream()

    def act(t, k):
        x = torch.randn((t, k), device=dev, generator=g)
        x[:, :16] *= 30.0
        return x.to(torch.bfloat16)

    def weight(k, n):
        wq = torch.randint(-127, 128, (n, k), dtype=torch.int8, device=dev, generator=g)
        return wq, torch.rand(n, device=dev, generator=g) * 1e-3

    layers = {"qkv": (H, H + 2 * KV, True), "o_proj": (H, H, False),
              "gate_up": (H, 2 * I, True), "down": (I, H, False)}
    out, tot_ops, tot_us = {}, 0.0, 0.0
    for name, (K, N, norm) in layers.items():
        x = act(T, K)
        wq, wsc = weight(K, N)
        gam = torch.rand(K, device=dev, generator=g) + 0.5 if norm else None
        y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
        work = torch.empty(sq.sq_linear_workspace_bytes(T, K), dtype=torch.uint8, device=dev)

        def call():
            sq.sq_w8a8_linear(x, gam, wq, wsc, y, work, norm=norm, stream=stream)

        call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / iters
        ops = 2.0 * T * K * N
        out[name] = {"K": K, "N": N, "norm": norm, "us": us, "tops": ops / (us * 1e-6) / 1e12}
        tot_ops += ops
        tot_us += us
    out["layer_linears_tops"] = tot_ops / (tot_us * 1e-6) / 1e12
    out["layer_linears_us"] = tot_us

    # LayerNorm form: quantizer on the q|k|v input, calibration over 16384 tokens
    x = act(T, H)
    xc = act(16384, H)
    gam = torch.rand(H, device=dev, generator=g) + 0.5
    bet = torch.randn(H, device=dev, generator=g) * 0.1
    xq = torch.empty((T, H), dtype=torch.int8, device=dev)
    xs = torch.empty(T, dtype=torch.float32, device=dev)
    a = torch.empty(H, dtype=torch.float32, device=dev)
    for name, fn, byts in (
            ("quant_act_ln", lambda: sq.sq_quant_act_ln(x, gam, bet, xq, xs, stream=stream),
             3.0 * T * H + 4.0 * T),
            ("calibrate_ln", lambda: sq.sq_calibrate_ln(xc, None, 0.5, a, gamma=gam, beta=bet,
                                                        stream=stream), 2.0 * 16384 * H)):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(iters):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / iters
        out[name] = {"us": us, "gbs": byts / (us * 1e-6) / 1e9}
    out["shapes"] = (f"T={T}, hidden {H}, q|k|v {H}+{KV}+{KV}, gate|up 2x{I}, down {I}->{H}; "
                     "LayerNorm calibration over 16384 tokens")
    return out


def decode_calibration(sq, torch, dev, Tc=262144, K=8192, iters=5):
    """The decode workload's calibration pass: per-channel absmax of a
    262144 x 8192 bf16 calibration set (4 GiB, 24 outlier channels x60),
    far larger than the Infinity Cache.  Drawn on the GPU (N(0,1) bf16)."""
    g = torch.Generator(device=dev)
    g.manual_seed(105)
    xc = torch.randn((Tc, K), dtype=torch.bfloat16, device=dev, generator=g)
    for c in torch.randperm(K, generator=torch.Generator().manual_seed(105))[:24].tolist():
        xc[:, c].mul_(60.0)
    a = torch.empty(K, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    sq.sq_calibrate(xc, None, 0.5, a, stream=stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(iters):
        sq.sq_calibrate(xc, None, 0.5, a, stream=stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / iters
    del xc
    byts = 2.0 * Tc * K
    return {"workload": f"calibration absmax Tc={Tc} K={K} bf16", "us": us,
            "achieved": byts / (us * 1e-6) / 1e9, "unit": "GB/s",
            "frac_of_peak": byts / (us * 1e-6) / 1e9 / PEAK_HBM_GBS,
            "algorithmic": "2 bytes per calibration element"}


def decode_linear_graph(sq, torch, dev, T=16, K=8192, N=8192, iters=50):
    """The decode linear (quantizer + GEMM, one sq_w8a8_linear call) launched
    eagerly and replayed from a captured HIP graph: the launch cost the graph
    removes at 16 tokens."""
    g = torch.Generator(device=dev)
    g.manual_seed(106)
    x = torch.randn((T, K), dtype=torch.bfloat16, device=dev, generator=g)
    wq = torch.randint(-127, 128, (N, K), dtype=torch.int8, device=dev, generator=g)
    wsc = torch.rand(N, device=dev, generator=g) * 1e-3
    y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    work = torch.empty(sq.sq_linear_workspace_bytes(T, K), dtype=torch.uint8, device=dev)

    def fwd():
        sq.sq_w8a8_linear(x, None, wq, wsc, y, work)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / iters

    eager_us = timed(fwd)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fwd()
    graph_us = timed(graph.replay)
    return {"workload": f"decode linear T={T} K={K} N={N} (weight in cache)", "eager_us": eager_us,
            "graph_replay_us": graph_us}


def config_step(sq, torch, dev, name, steps=10, warmup=3, nsets=3):
    """The same whole step (calibrate, fold, quantize the weight, quantize the
    activation, the GEMM) on another workload's own synthetic inputs: the
    RMSNorm -> q|k|v and the MLP gate|up configurations.  As in the headline,
    the steps take X_cal, X and W in turn from `nsets` copies in HBM, so the
    Infinity Cache does not hold a step's inputs from the step before.  The
    timed steps carry no events; a breakdown pass times every call with
    fence-free HIP events, and each kernel gets its own roofline entry."""
    import numpy as np

    import synth

    wl = synth.WORKLOADS[name]
    T, K, N, Tc = wl.T, wl.K, wl.N, wl.Tc
    inp = synth.make_inputs(wl)

    def d(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    sets = [(d(inp.x_cal), d(inp.x), d(inp.w)) for _ in range(nsets)]
    bias = d(inp.bias)
    gamma = None if inp.gamma is None else d(inp.gamma)
    del inp
    f = lambda n: torch.empty(n, dtype=torch.float32, device=dev)  # noqa: E731
    a, wm, s, gp, wsc, xs = f(K), f(K), f(K), f(K), f(N), f(T)
    rr = f(T) if wl.norm else None
    wq = torch.empty((N, K), dtype=torch.int8, device=dev)
    xq = torch.empty((T, K), dtype=torch.int8, device=dev)
    y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    names = ["calibrate", "smooth_fold", "quant_weight", "quant_act", "gemm"]

    def calls(i):
        x_cal, x, w = sets[i % nsets]
        return [
            lambda: sq.sq_calibrate(x_cal, w, wl.alpha, a, wm, s, norm=wl.norm, gamma=gamma,
                                    stream=stream),
            lambda: sq.sq_smooth_fold(s, gamma, gp, stream=stream),
            lambda: sq.sq_quant_weight(w, s, wq, wsc, stream=stream),
            lambda: sq.sq_quant_act(x, gp, xq, xs, norm=wl.norm, row_rscale=rr, stream=stream),
            lambda: sq.sq_gemm_w8a8(xq, xs, wq, wsc, y, bias=bias, stream=stream),
        ]

    for i in range(warmup):
        for c in calls(i):
            c()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        for c in calls(warmup + i):
            c()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    hip = HipTimer()
    evs = [[hip.event() for _ in range(len(names) + 1)] for _ in range(steps)]
    for i in range(steps):
        hip.record(evs[i][0], stream)
        for j, c in enumerate(calls(warmup + steps + i)):
            c()
            hip.record(evs[i][j + 1], stream)
    torch.cuda.synchronize()
    per = {n: sum(hip.ms(evs[i][j], evs[i][j + 1]) for i in range(steps)) / steps * 1e3
           for j, n in enumerate(names)}
    hip.destroy([e for row in evs for e in row])
    ops = 2.0 * T * K * N
    lin = per["quant_act"] + per["gemm"]

    def hbm(byts, us):
        ach = byts / (us * 1e-6) / 1e9
        return {"bound": "hbm", "us": us, "achieved": ach, "unit": "GB/s",
                "frac": ach / PEAK_HBM_GBS, "algorithmic_bytes": byts}

    g_ach = ops / (per["gemm"] * 1e-6) / 1e12
    roof = {
        "gemm": {"bound": "mfma", "us": per["gemm"], "achieved": g_ach, "unit": "TOP/s",
                 "peak": PEAK_INT8_TOPS, "frac": g_ach / PEAK_INT8_TOPS,
                 "algorithmic": f"2*T*K*N = {ops:.4g} int8 ops"},
        "calibrate": hbm(2.0 * Tc * K + 2.0 * K * N + 12.0 * K, per["calibrate"]),
        "quant_weight": hbm(3.0 * K * N + 4.0 * (N + K), per["quant_weight"]),
        "quant_act": hbm(3.0 * T * K + 4.0 * (T + K), per["quant_act"]),
    }
    return {"workload": f"{name}: T={T} K={K} N={N} calib_tokens={Tc} norm={wl.norm}",
            "input_sets": nsets, "ms_per_step": ms, "step_tops": ops / (ms * 1e-3) / 1e12,
            "linear_us": lin, "linear_tops": ops / (lin * 1e-6) / 1e12, "calls_us": per,
            "roofline": roof}


def gptq_timing(sq, torch, inp, wl, d, dev, iters=2):
    """GPTQ rounding of the headline weight (K = N = 4096) with the Hessian of
    the 8192 calibration tokens: one sq_quant_weight_gptq call, event-timed,
    and its weight error through the calibration x^ next to round-to-nearest
    (computed on the GPU in fp64 from the codes)."""
    T, K, N = wl.Tc, wl.K, wl.N
    x_cal, w = d(inp.x_cal), d(inp.w)
    f = lambda n: torch.empty(n, dtype=torch.float32, device=dev)  # noqa: E731
    a, wm, s, gp, wsc, wsr = f(K), f(K), f(K), f(K), f(N), f(N)
    sq.sq_calibrate(x_cal, w, wl.alpha, a, wm, s)
    sq.sq_smooth_fold(s, None, gp)
    wq = torch.empty((N, K), dtype=torch.int8, device=dev)
    wr = torch.empty((N, K), dtype=torch.int8, device=dev)
    sq.sq_quant_weight(w, s, wr, wsr)
    work = torch.empty(sq.sq_gptq_workspace_bytes(T, K, N), dtype=torch.uint8, device=dev)
    sq.sq_quant_weight_gptq(x_cal, gp, w, s, wq, wsc, work)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        sq.sq_quant_weight_gptq(x_cal, gp, w, s, wq, wsc, work)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    del work
    # proxy error through the calibration x^ (fp64 on the GPU, reporting only)
    xh = (x_cal.double() * gp.double()).float().double()
    what = (w.float() * s[:, None]).double()

    def werr(codes, step):
        return float(torch.linalg.norm(xh @ (what - codes.double().t() * step.double()[None, :])))

    ratio = werr(wq, wsc) / werr(wr, wsr)
    return {"workload": f"GPTQ K={K} N={N} calibration tokens {T}", "ms": ms,
            "calibration_weight_error_vs_round_to_nearest": ratio}


def cpu_baseline(inp, wl, target_s: float):
    import numpy as np  # noqa: F401

    import oracle
    threads = oracle.max_threads()

    def run(rows):
        t = time.perf_counter()
        _, _, s = oracle.calibrate(inp.x_cal[:rows], inp.w, wl.alpha)
        gp, qw, ws = oracle.prepare_weight(inp.w, s)
        oracle.linear(inp.x[:rows], gp, qw, ws, inp.bias)
        return time.perf_counter() - t

    probe = min(wl.T, 256)
    tp = run(probe)
    t_fixed = run(8)
    per_row = max((tp - t_fixed) / max(probe - 8, 1), 1e-9)
    rows = int(min(wl.T, max(probe, (target_s - t_fixed) / per_row)))
    rows = max(64, rows // 64 * 64) if rows < wl.T else wl.T
    # the whole workload fits the time budget several times over: repeat it
    # until about target_s of CPU time has run (at most 8 passes)
    times = [run(rows)]
    while rows == wl.T and sum(times) < target_s and len(times) < 8:
        times.append(run(rows))
    secs = sum(times)
    ops = 2.0 * rows * wl.K * wl.N * len(times)
    return {
        "value": ops / secs / 1e12, "unit": "TOPS", "cores": threads, "kind": "oracle",
        "seconds": secs, "passes": len(times),
        "sample": (f"the whole step (calibration over {rows} tokens, fold and quantization of the "
                   f"full {wl.K}x{wl.N} weight, forward of {rows} of the {wl.T} tokens), "
                   f"{len(times)} pass(es); value = 2*{rows}*K*N ops per pass / wall time, "
                   f"plain-C oracle with OpenMP"),
    }


def main():
    args = _parse()
    if args.rocpd_summary:
        rocpd_summary(args.rocpd_summary, args.counters_json)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "bench.py measures one GPU only: the layer's multi-GPU "
                          "sharding is a design note, not built; run with --gpus 1"}))
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import w8a8_int8_gemm_amd as sq

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU (cuda:0)")
    sq.lib()   # fails loudly when the HIP library is missing
    dev = torch.device("cuda:0")
    wl = synth.WORKLOADS[WORKLOAD]
    T, K, N, Tc = wl.T, wl.K, wl.N, wl.Tc
    print(f"generating {WORKLOAD}: T={T} K={K} N={N} Tc={Tc}", file=sys.stderr, flush=True)
    inp = synth.make_inputs(wl)

    def d(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    if args.gemm_loop > 0:
        gemm_loop(sq, torch, inp, wl, d, dev, args.gemm_loop)
        return
    if args.only == "gptq":
        print(json.dumps(gptq_timing(sq, torch, inp, wl, d, dev)), flush=True)
        return
    if args.only == "decoder_layer":
        print(json.dumps(block_timing(sq, torch, dev)), flush=True)
        return
    if args.only in ("configs", "rmsnorm_qkv", "gate_up"):
        names = ("rmsnorm_qkv", "gate_up") if args.only == "configs" else (args.only,)
        print(json.dumps({n: config_step(sq, torch, dev, n) for n in names}), flush=True)
        return
    if args.only == "decode":
        print(json.dumps({"decode_gemm": decode_gemm(sq, torch, dev),
                          "decode_calibration": decode_calibration(sq, torch, dev)}), flush=True)
        return
    nsets = max(1, args.sets)
    sets = [(d(inp.x_cal), d(inp.x), d(inp.w)) for _ in range(nsets)]
    bias = d(inp.bias)
    f = lambda n: torch.empty(n, dtype=torch.float32, device=dev)  # noqa: E731
    a, wm, s, gp, wsc, xs = f(K), f(K), f(K), f(K), f(N), f(T)
    wq = torch.empty((N, K), dtype=torch.int8, device=dev)
    xq = torch.empty((T, K), dtype=torch.int8, device=dev)
    y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()
    names = ["calibrate", "smooth_fold", "quant_weight", "quant_act", "gemm"]

    def step(ev=None, i=0, every_call=False):
        # The timed steps record two events per step, on either side of the
        # GEMM (its duration feeds the roofline); every_call records one
        # between all five calls (the breakdown pass).  The events skip the
        # system-scope fence (HipTimer), so each costs the stream about half
        # a microsecond instead of several.
        x_cal, x, w = sets[i % nsets]
        if every_call:
            hip.record(ev[0], stream)
        sq.sq_calibrate(x_cal, w, wl.alpha, a, wm, s, stream=stream)
        if every_call:
            hip.record(ev[1], stream)
        sq.sq_smooth_fold(s, None, gp, stream=stream)
        if every_call:
            hip.record(ev[2], stream)
        sq.sq_quant_weight(w, s, wq, wsc, stream=stream)
        if every_call:
            hip.record(ev[3], stream)
        sq.sq_quant_act(x, gp, xq, xs, stream=stream)
        if ev is not None:
            hip.record(ev[4], stream)
        sq.sq_gemm_w8a8(xq, xs, wq, wsc, y, bias=bias, stream=stream)
        if ev is not None:
            hip.record(ev[5], stream)

    for i in range(args.warmup):
        step(i=i)
    torch.cuda.synchronize()
    hip = HipTimer()
    evs = [[hip.event() for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i], i=args.warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps
    gemm_ms = sum(hip.ms(e[4], e[5]) for e in evs) / args.steps
    print(f"timed {args.steps} steps: {ms_step:.4f} ms/step", file=sys.stderr, flush=True)
    # per-call breakdown: the same steps again, every call bracketed (untimed)
    bevs = [[hip.event() for _ in range(6)] for _ in range(args.steps)]
    tb0 = time.perf_counter()
    for i in range(args.steps):
        step(bevs[i], i=args.warmup + args.steps + i, every_call=True)
    torch.cuda.synchronize()
    breakdown_ms_step = (time.perf_counter() - tb0) * 1e3 / args.steps
    kern_ms = {n: sum(hip.ms(e[j], e[j + 1]) for e in bevs) / args.steps
               for j, n in enumerate(names)}
    hip.destroy([e for row in evs + bevs for e in row])
    breakdown_gemm_ms = kern_ms["gemm"]
    kern_ms["gemm"] = gemm_ms
    if args.copy_probe_mib > 0:
        n = args.copy_probe_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    ops = 2.0 * T * K * N
    value = ops / (ms_step * 1e-3) / 1e12
    # algorithmic bytes (or ops) per launch of each call
    alg = {
        "calibrate": ("GB/s", 2.0 * Tc * K + 2.0 * K * N + 12.0 * K),
        "smooth_fold": ("GB/s", 8.0 * K),
        "quant_weight": ("GB/s", 2.0 * K * N + 1.0 * K * N + 4.0 * N + 4.0 * K),
        "quant_act": ("GB/s", 2.0 * T * K + 1.0 * T * K + 4.0 * T + 4.0 * K),
        "gemm": ("TOPS", ops),
    }
    kernels = {}
    for n in names:
        unit, amount = alg[n]
        secs = kern_ms[n] * 1e-3
        ach = amount / secs / (1e9 if unit == "GB/s" else 1e12)
        peak = PEAK_HBM_GBS if unit == "GB/s" else PEAK_INT8_TOPS
        kernels[n] = {"us": kern_ms[n] * 1e3, "achieved": ach, "unit": unit, "frac_of_peak": ach / peak}

    gemm_s = kern_ms["gemm"] * 1e-3
    g_ach = ops / gemm_s / 1e12
    roofline = {"bound": "mfma", "achieved": g_ach, "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                "frac": g_ach / PEAK_INT8_TOPS, "traffic": _traffic(T * K + N * K + 2.0 * T * N),
                **_clock_fields(g_ach),
                "kernel": "k_gemm_w8a8 (sq_gemm_w8a8)",
                "algorithmic": f"2*T*K*N = {ops:.4g} int8 ops per launch"}
    linear_s = (kern_ms["quant_act"] + kern_ms["gemm"]) * 1e-3

    out = {
        "metric": METRIC, "value": value, "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "i8", "data": "synthetic",
        "config": {"workload": WORKLOAD, "T": T, "K": K, "N": N, "calib_tokens": Tc,
                   "alpha": wl.alpha, "x_dtype": "bf16", "w_dtype": "bf16", "y_dtype": "bf16",
                   "bias": True,
                   "step": "sq_calibrate + sq_smooth_fold + sq_quant_weight + sq_quant_act + "
                           "sq_gemm_w8a8"},
        "pct_of_int8_peak": 100.0 * value / PEAK_INT8_TOPS,
        "linear_tops": ops / linear_s / 1e12,
        "roofline": roofline,
        "kernels": kernels,
        "kernels_note": ("gemm: HIP events recorded on either side of the GEMM in the timed "
                         "steps; the other calls: a breakdown pass after the timed steps with an "
                         "event recorded between every two calls (all events created with "
                         "hipEventDisableSystemFence; that pass: "
                         f"{breakdown_ms_step * 1e3:.1f} us per step, GEMM bracket "
                         f"{breakdown_gemm_ms * 1e3:.1f} us)"),
        "device": torch.cuda.get_device_properties(0).name,
    }
    if not args.no_extras:
        x_cal, x, w = sets[0]
        out["alpha_sweep"] = alpha_sweep(sq, torch, inp, wl, x_cal, x, w, bias, dev)
        out["quant_act_static_vs_per_token"] = static_act_timing(sq, torch, sets, gp, a, xq, xs,
                                                                 dev)
        out["decode_gemm"] = decode_gemm(sq, torch, dev)
        out["fp8"] = fp8_timing(sq, torch, sets, wl, s, gp, bias, dev)
        out["vendor_int8_gemm"] = vendor_int8_gemm(torch, xq, wq)
        out["hbm_ceilings"] = hbm_ceilings(torch, dev)
        out["decoder_layer"] = block_timing(sq, torch, dev)
        out["decode_calibration"] = decode_calibration(sq, torch, dev)
        out["configs"] = {n: config_step(sq, torch, dev, n) for n in ("rmsnorm_qkv", "gate_up")}
        out["gptq"] = gptq_timing(sq, torch, inp, wl, d, dev)
        out["decode_linear_graph"] = decode_linear_graph(sq, torch, dev)
    if not args.no_cpu_baseline:
        print("timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(inp, wl, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
