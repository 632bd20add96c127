#!/usr/bin/env python3
"""conv2d forward throughput on one MI355X, against the kernel's roofline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--layer CID:LI | --separable | --all]

A step is one forward pass of the workload layer through the timed C entry
``conv2d_fwd_nhwc_packed`` (channels-last activations already resident in
HBM, weights packed once beforehand): host plan -> kernel with the fused
bias+ReLU epilogue.  The default workload is the 3x3 bf16 layer
N=32, 128x112x112 -> 256, stride 1, pad 1, bias+ReLU (implicit GEMM with
M=256, K=1152, N*Ho*Wo=401408).  ``--layer`` / ``--all`` time the other
workload layers (one JSON line each); ``--separable`` times the
depthwise-separable pair of config 3 as one fused pass
(``conv2d_fwd_separable_nhwc``: 3x3 depthwise + bias + ReLU, then the 1x1
144 -> 24, the intermediate kept on chip).

Timing: W untimed warm-up steps, then exactly K steps between two
torch.cuda.synchronize() calls (wall clock -> ms_per_step and value).  The
defaults (W = 300, K = 500; under 0.2 s of GPU time on the 3x3 layer) put the
timed steps past the GPU's power-management transient: on the 3x3 layer
launch durations rise from ~215 us to 250-290 us around launches 7-30 and
settle at ~211 us within about 100 launches (``--launch-times`` prints every
launch's duration).  Input
and output buffers rotate over R sets whose total size is >= 512 MB, so the
256 MB Infinity Cache cannot hold the working set across steps.  Each launch
is also bracketed by HIP events on the stream it runs on; their mean is the
kernel duration used for the roofline figures.

Roofline: achieved = algorithmic FLOPs (2*N*Ho*Wo*Cout*(Cin/G)*Kh*Kw) or
algorithmic bytes (x, w, bias and y each moved once) per launch / mean launch
duration; peak = MI355X dense bf16 MFMA 2516.6 TFLOP/s (256 CU x 2.4 GHz x
4096 FLOP/clk), fp32 vector 157.3 TFLOP/s, or HBM3E 8000 GB/s.  traffic is the
HBM byte count measured with rocprofv3 counters for this kernel source, read
from profiles/traffic.json, or null when the kernel source changed since.

The roofline block also gives the launch durations' mean and p10/p50/p90.
Beside the timed entry, ``nchw_entry`` times ``conv2d_fwd`` on the pages'
own layouts (weight repack and both layout passes per call; never the
headline value); ``--no-nchw`` skips it.

cpu_baseline: the fp64 oracle (test infrastructure) on a bounded sample of the
same workload -- whole images, all channels -- run on the host cores until
about --cpu-seconds have passed, scaled to the metric's unit.  The first line
also carries ``single_thread``: the oracle on one host thread over the whole
fp32 first layer and the whole depthwise-separable pair.

``--hbm-ceiling`` only times a plain device copy that moves each HBM-bound
layer's total bytes (context for their HBM fractions).

``--power SECONDS`` adds ``sustained``: after the timed steps the layer runs
back to back for SECONDS while amd-smi reads the socket power and the
graphics clock every two seconds (the clock the chip holds under the kernel,
against the 2.4 GHz the spec peaks assume).  It never enters value or the
roofline figures, and the default line does not take it (so a kernel trace
of the default command covers exactly the launches the line is computed
from).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import conv_inputs as ci  # noqa: E402

PEAK_BF16_TFLOPS = 2516.6
PEAK_FP32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
ROTATE_BYTES = 512 << 20
METRIC = "conv2d fwd TFLOP/s (GB/s for depthwise) and % of MI355X roofline, 1 GPU"
KERNEL_SOURCES = {"direct": ["direct.hip"], "depthwise": ["depthwise.hip", "dwrow.hpp"],
                  "gemm1x1": ["pointwise.hip", "igemm.hip"], "igemm_gather": ["igemm.hip"],
                  "igemm_halo": ["igemm_halo.hip", "igemm_halo_s2.hip", "halo.hpp"],
                  "separable": ["separable.hip", "dwrow.hpp"],
                  "transposed_igemm_gather": ["igemm.hip"], "transposed_direct": ["transposed.hip"],
                  "transposed_gemm1x1": ["pointwise.hip"], "transposed_igemm_halo": ["transposed.hip"],
                  "winograd": ["winograd.hip"]}


FORCED_PATH = None  # set by --path: the kernel path forced for the timed layers
LAUNCH_TIMES = False  # set by --launch-times: report every launch's duration


def out_hw(ly):
    if ly.transposed:
        ho = (ly.H - 1) * ly.stride - 2 * ly.pad + ly.dilation * (ly.Kh - 1) + ly.out_pad + 1
        wo = (ly.W - 1) * ly.stride - 2 * ly.pad + ly.dilation * (ly.Kw - 1) + ly.out_pad + 1
        return ho, wo
    ho = (ly.H + 2 * ly.pad - ly.dilation * (ly.Kh - 1) - 1) // ly.stride + 1
    wo = (ly.W + 2 * ly.pad - ly.dilation * (ly.Kw - 1) - 1) // ly.stride + 1
    return ho, wo


def _landing_pairs(n_in, k, stride, pad, dil, n_out):
    """(input, tap) pairs along one axis whose product lands inside the output
    of a transposed convolution."""
    return sum(1 for i in range(n_in) for t in range(k) if 0 <= i * stride - pad + t * dil < n_out)


def algorithmic(ly):
    """Nominal FLOPs and bytes (each tensor moved once) of one launch.  A
    transposed layer counts the products that land inside its output."""
    ho, wo = out_hw(ly)
    esz = 4 if ly.dtype == ci.F32 else 2
    if ly.transposed:
        flops = 2 * ly.N * ly.Cout * (ly.Cin // ly.groups) \
            * _landing_pairs(ly.H, ly.Kh, ly.stride, ly.pad, ly.dilation, ho) \
            * _landing_pairs(ly.W, ly.Kw, ly.stride, ly.pad, ly.dilation, wo)
    else:
        flops = 2 * ly.N * ho * wo * ly.Cout * (ly.Cin // ly.groups) * ly.Kh * ly.Kw
    nbytes = esz * (ly.N * ly.Cin * ly.H * ly.W + ly.Cout * (ly.Cin // ly.groups) * ly.Kh * ly.Kw
                    + ly.N * ly.Cout * ho * wo)
    if ly.epilogue & ci.EPI_BIAS:
        nbytes += 4 * ly.Cout
    return flops, nbytes


def bound_of(ly):
    """Binding roof: FLOP/byte against the ridge of the layer's dtype."""
    flops, nbytes = algorithmic(ly)
    peak = PEAK_FP32_TFLOPS if ly.dtype == ci.F32 else PEAK_BF16_TFLOPS
    ridge = peak * 1e12 / (PEAK_HBM_GBS * 1e9)
    return ("mfma" if ly.dtype != ci.F32 else "alu") if flops / nbytes >= ridge else "hbm"


def source_digest(path_name):
    csrc = os.path.join(ROOT, "cnn_convolution_conv2d_amd", "csrc")
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[path_name] + ["common.hpp", "mfma.hpp"]:
        h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(key, path_name):
    """HBM bytes per launch from rocprofv3 counters, if taken on this source."""
    f = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(f):
        return None
    entry = json.load(open(f)).get(key)
    if not entry or entry.get("source_digest") != source_digest(path_name):
        return None
    return entry.get("hbm_bytes_per_launch")


def _builder():
    """The library's build module, loaded by path: importing it through the
    package would first load the (possibly stale or missing) library."""
    import importlib.util
    path = os.path.join(ROOT, "cnn_convolution_conv2d_amd", "build.py")
    spec = importlib.util.spec_from_file_location("conv2d_build", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def host_cpu():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def launch_stats(launch_ms):
    """Mean and p10/p50/p90 of the per-launch HIP-event durations, in us
    (with --launch-times also every launch's duration, in launch order)."""
    us = np.asarray(launch_ms) * 1e3
    p10, p50, p90 = np.percentile(us, [10, 50, 90])
    out = {"kernel_mean_us": round(float(us.mean()), 3), "kernel_median_us": round(float(p50), 3),
           "kernel_p10_us": round(float(p10), 3), "kernel_p90_us": round(float(p90), 3)}
    if LAUNCH_TIMES:
        out["launch_us"] = [round(float(v), 1) for v in us]
    return out


_SINGLE_THREAD_CHILD = r"""
import json, sys, time
sys.path.insert(0, sys.argv[1])
import conv_inputs as ci
import oracle
out = {}
for cid, li in ((1, 0), (3, 0), (3, 1)):
    ly = ci.layer(cid, li)
    x, w, b = ci.layer_tensors(cid, li)
    relu = bool(ly.epilogue & ci.EPI_RELU)
    oracle.conv2d(x[:1], w, b, ly.stride, ly.pad, ly.dilation, ly.groups, relu=relu, with_scale=False)
    t0 = time.perf_counter()
    oracle.conv2d(x, w, b, ly.stride, ly.pad, ly.dilation, ly.groups, relu=relu, with_scale=False)
    out[f"cfg{cid}:{ly.name}"] = time.perf_counter() - t0
out["threads"] = oracle.num_threads()
print(json.dumps(out))
"""


def oracle_single_thread():
    """The oracle on one host thread over the whole fp32 first layer and the
    whole depthwise-separable pair (each layer separately), in a child
    process started with OMP_NUM_THREADS=1; seconds and GFLOP/s per layer."""
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-c", _SINGLE_THREAD_CHILD, ROOT], env=env, capture_output=True,
                       text=True, timeout=300)
    if r.returncode != 0:
        return {"error": (r.stderr or "")[-300:]}
    t = json.loads(r.stdout.strip().splitlines()[-1])
    res = {"threads": t.pop("threads")}
    for key, sec in t.items():
        cid, name = key[3:].split(":", 1)
        ly = ci.layer(int(cid), name)
        flops, nbytes = algorithmic(ly)
        res[key] = {"seconds": round(sec, 4), "gflop_per_s": round(flops / sec / 1e9, 4),
                    "gb_per_s": round(nbytes / sec / 1e9, 4), "sample": f"all {ly.N} images"}
    return res


def cpu_baseline(cid, li, x, w, b, target_s, unit):
    """The fp64 oracle on whole images of the workload until target_s elapses."""
    import oracle
    ly = ci.layer(cid, li)
    flops, nbytes = algorithmic(ly)
    relu = bool(ly.epilogue & ci.EPI_RELU)
    k = 0
    t0 = time.perf_counter()
    while k < ly.N and (k == 0 or time.perf_counter() - t0 < target_s):
        if ly.transposed:
            oracle.conv_transpose2d(x[k:k + 1], w, b, ly.stride, ly.pad, ly.out_pad, ly.dilation, ly.groups,
                                    relu=relu)
        else:
            oracle.conv2d(x[k:k + 1], w, b, ly.stride, ly.pad, ly.dilation, ly.groups, relu=relu,
                          with_scale=False)
        k += 1
    dt = time.perf_counter() - t0
    frac = k / ly.N
    value = (flops * frac / dt / 1e12) if unit == "TFLOP/s" else (nbytes * frac / dt / 1e9)
    return {"value": round(value, 6), "unit": unit, "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"first {k} of {ly.N} images, all {ly.Cout} output channels, fp64 "
                      f"{'scatter' if ly.transposed else 'direct'} loop ({dt:.1f} s)",
            "host_cpu": host_cpu()}


def time_nchw_entry(c2, ly, x, w, b, ho, wo, tdt, dt_lib, dev, stream, steps, flops, nbytes, unit):
    """conv2d_fwd end to end on the pages' layouts (NCHW x and y, OIHW w):
    for bf16 this is the weight repack, the NCHW -> NHWC pass, the kernel and
    the NHWC -> NCHW pass per call, the conversion cost that can cancel a
    kernel's gain (lincklin.cn lesson 9, section 30).  One buffer set; the
    library's scratch is grown by the warm-up call.  Reported beside the
    timed entry, never as the headline value."""
    import torch
    xn = torch.from_numpy(x).to(dev).to(tdt)
    wn = torch.from_numpy(w).to(dev).to(tdt)
    bn = torch.from_numpy(b).to(dev) if b is not None else None
    yn = torch.empty((ly.N, ly.Cout, ho, wo), dtype=tdt, device=dev)

    def call():
        c2.conv2d_fwd(xn, wn, bn, yn, ly.N, ly.Cin, ly.H, ly.W, ly.Cout, ly.Kh, ly.Kw, ly.stride, ly.pad,
                      ly.dilation, ly.groups, dt_lib, ly.epilogue, stream)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    value = flops / (ms * 1e-3) / 1e12 if unit == "TFLOP/s" else nbytes / (ms * 1e-3) / 1e9
    del xn, wn, yn
    return {"entry": "conv2d_fwd (NCHW in and out, weights repacked per call)", "steps": steps,
            "ms_per_call": round(ms, 5), "value": round(value, 3), "unit": unit, "buffer_sets": 1}


HEADLINE_LAYER = "2:0"


def smi_sample(gpu):
    """One amd-smi reading of the GPU's socket power (W) and graphics clock
    (MHz, the mean over its graphics partitions, one per XCD)."""
    try:
        r = subprocess.run(["amd-smi", "metric", "-p", "-c", "-g", str(gpu)], capture_output=True, text=True,
                           timeout=20)
    except (OSError, subprocess.TimeoutExpired) as e:
        return {"error": str(e)[:200]}

    def num(t):
        v = t.split(":", 1)[1].split()
        try:
            return float(v[0])
        except (IndexError, ValueError):
            return None

    power, clocks, in_gfx = None, [], False
    for ln in r.stdout.splitlines():
        t = ln.strip()
        if t.startswith("SOCKET_POWER:") and power is None:
            power = num(t)
        elif t.endswith(":") and not t.startswith("CLK"):
            in_gfx = t.startswith("GFX_")
        elif in_gfx and t.startswith("CLK:"):
            c = num(t)
            if c is not None:
                clocks.append(c)
    if power is None and not clocks:
        return {"error": (r.stderr or r.stdout or "no output")[-200:]}
    return {"socket_power_w": power,
            "gfx_clock_mhz": round(sum(clocks) / len(clocks), 1) if clocks else None,
            "gfx_clocks_mhz": clocks}


def sustained_power(step, stream, seconds, gpu):
    """Launch STEP back to back for SECONDS, reading amd-smi every two seconds
    from the second second on: the power and clock the chip holds under the
    kernel (the spec peaks assume 2.4 GHz)."""
    import threading
    import torch
    samples, stop = [], threading.Event()

    def sampler():
        if stop.wait(2.0):
            return
        while not stop.is_set():
            samples.append(smi_sample(gpu))
            stop.wait(2.0)

    th = threading.Thread(target=sampler, daemon=True)
    t0 = time.perf_counter()
    th.start()
    n, spans = 0, []
    while time.perf_counter() - t0 < seconds:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(100):
            step(n + i)
        e1.record(stream)
        e1.synchronize()
        spans.append(e0.elapsed_time(e1) / 100)
        n += 100
    stop.set()
    th.join()
    good = [x for x in samples if "error" not in x]
    out = {"seconds": seconds, "launches": n, "mean_us": round(float(np.mean(spans)) * 1e3, 2),
           "samples": samples}
    for k in ("socket_power_w", "gfx_clock_mhz"):
        v = [x[k] for x in good if x.get(k) is not None]
        if v:
            out[k + "_mean"] = round(float(np.mean(v)), 1)
    return out


def bench_layer(cid, li, steps, warmup, cpu_seconds, with_cpu, winograd=False, with_nchw=True, power_seconds=0.0):
    import torch
    import cnn_convolution_conv2d_amd as c2

    ly = ci.layer(cid, li)
    ho, wo = out_hw(ly)
    dt_lib = c2.F32 if ly.dtype == ci.F32 else c2.BF16
    tdt = torch.float32 if ly.dtype == ci.F32 else torch.bfloat16
    esz = 4 if ly.dtype == ci.F32 else 2
    if winograd:
        path, pname = None, "winograd"
    elif ly.transposed:
        path = c2.conv2d_transpose_select_path(ly.N, ly.Cin, ly.H, ly.W, ly.Cout, ly.Kh, ly.Kw, ly.stride,
                                               ly.pad, ly.out_pad, ly.dilation, ly.groups, dt_lib)
        pname = "transposed_" + c2.PATH_NAMES[path]
    else:
        path = c2.conv2d_select_path(ly.N, ly.Cin, ly.H, ly.W, ly.Cout, ly.Kh, ly.Kw, ly.stride, ly.pad,
                                     ly.dilation, ly.groups, dt_lib)
        pname = c2.PATH_NAMES[path]
    flops, nbytes = algorithmic(ly)
    bound = bound_of(ly)

    x, w, b = ci.layer_tensors(cid, li)
    dev = torch.device("cuda", torch.cuda.current_device())
    stream = torch.cuda.current_stream()
    # inputs resident in HBM, channels-last, before the timed region
    x_nchw = torch.from_numpy(x).to(dev).to(tdt)
    w_dev = torch.from_numpy(w).to(dev).to(tdt)
    wbytes = c2.conv2d_winograd_weight_bytes(ly.Cout, ly.Cin, dt_lib) if winograd else \
        c2.conv2d_packed_weight_bytes(ly.Cout, ly.Cin, ly.Kh, ly.Kw, ly.groups, dt_lib)
    wp = torch.empty(wbytes // esz, dtype=tdt, device=dev)
    if winograd:
        c2.conv2d_winograd_transform_weights(w_dev, wp, ly.Cout, ly.Cin, dt_lib)
    elif ly.transposed:
        c2.conv2d_transpose_pack_weights(w_dev, wp, ly.Cin, ly.Cout, ly.Kh, ly.Kw, ly.groups, dt_lib)
    else:
        c2.conv2d_pack_weights(w_dev, wp, ly.Cout, ly.Cin, ly.Kh, ly.Kw, ly.groups, dt_lib)
    bias = torch.from_numpy(b).to(dev) if b is not None else None
    set_bytes = esz * (x.size + ly.N * ly.Cout * ho * wo)
    R = max(1, min(16, math.ceil(ROTATE_BYTES / set_bytes)))
    x0 = torch.empty((ly.N, ly.H, ly.W, ly.Cin), dtype=tdt, device=dev)
    c2.conv2d_nchw_to_nhwc(x_nchw, x0, ly.N, ly.Cin, ly.H, ly.W, dt_lib)
    xs = [x0] + [x0.clone() for _ in range(R - 1)]
    ys = [torch.empty((ly.N, ho, wo, ly.Cout), dtype=tdt, device=dev) for _ in range(R)]
    del x_nchw, w_dev

    def step(i):
        j = i % R
        if winograd:
            c2.conv2d_fwd_winograd_nhwc(xs[j], wp, bias, ys[j], ly.N, ly.Cin, ly.H, ly.W, ly.Cout, ly.pad, dt_lib,
                                        ly.epilogue, stream)
        elif ly.transposed:
            c2.conv2d_transpose_fwd_nhwc_packed(xs[j], wp, bias, ys[j], ly.N, ly.Cin, ly.H, ly.W, ly.Cout,
                                                ly.Kh, ly.Kw, ly.stride, ly.pad, ly.out_pad, ly.dilation,
                                                ly.groups, dt_lib, ly.epilogue, stream)
        else:
            c2.conv2d_fwd_nhwc_packed(xs[j], wp, bias, ys[j], ly.N, ly.Cin, ly.H, ly.W, ly.Cout, ly.Kh,
                                      ly.Kw, ly.stride, ly.pad, ly.dilation, ly.groups, dt_lib,
                                      ly.epilogue, stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = np.array([a.elapsed_time(e) for a, e in ev])
    mean_ms = float(launch_ms.mean())
    ms_per_step = wall * 1e3 / steps
    power = sustained_power(step, stream, power_seconds, torch.cuda.current_device()) if power_seconds > 0 else None

    unit = "TFLOP/s" if bound in ("mfma", "alu") else "GB/s"
    if unit == "TFLOP/s":
        value = flops / (ms_per_step * 1e-3) / 1e12
        achieved = flops / (mean_ms * 1e-3) / 1e12
        peak = PEAK_FP32_TFLOPS if ly.dtype == ci.F32 else PEAK_BF16_TFLOPS
    else:
        value = nbytes / (ms_per_step * 1e-3) / 1e9
        achieved = nbytes / (mean_ms * 1e-3) / 1e9
        peak = PEAK_HBM_GBS
    # a forced path's counters are kept under their own key
    key = f"cfg{cid}:{ly.name}" + (":winograd" if winograd else "") + (f":{pname}" if FORCED_PATH else "")
    traffic = measured_traffic(key, pname)
    nchw = None
    if with_nchw and not winograd and not ly.transposed:
        nchw = time_nchw_entry(c2, ly, x, w, b, ho, wo, tdt, dt_lib, dev, stream, max(5, min(steps, 20)),
                               flops, nbytes, unit)
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if ly.dtype == ci.F32 else "bf16",
        "data": "synthetic (seeded, workload shapes and distributions; no dataset)",
        "config": {
            "workload": f"cfg{cid} {ly.name}: {'transposed ' if ly.transposed else ''}N={ly.N} Cin={ly.Cin} "
                        f"{ly.H}x{ly.W} -> Cout={ly.Cout} {ho}x{wo} "
                        f"{ly.Kh}x{ly.Kw} s{ly.stride} p{ly.pad} d{ly.dilation} g{ly.groups}"
                        f"{' bias' if ly.epilogue & ci.EPI_BIAS else ''}"
                        f"{' relu' if ly.epilogue & ci.EPI_RELU else ''}",
            "layout": "NHWC activations, " + ("Winograd-transformed weights" if winograd else "packed weights"),
            "path": pname,
            "gflop_per_step": round(flops / 1e9, 4), "algorithmic_mb_per_step": round(nbytes / 1e6, 3),
            "rotating_buffer_sets": R, "device": torch.cuda.get_device_name(dev),
        },
        "roofline": {
            "bound": bound, "achieved": round(achieved, 3), "peak": peak,
            "unit": "TFLOP/s" if unit == "TFLOP/s" else "GB/s",
            "frac": round(achieved / peak, 4), "traffic": traffic,
            **launch_stats(launch_ms),
        },
    }
    if nchw is not None:
        line["nchw_entry"] = nchw
    if power is not None:
        line["sustained"] = power
    if winograd:
        # FLOP/s above count the convolution's own multiply-adds; the matrix
        # cores execute 16/36 of them (F(2x2,3x3)) on the transformed data
        line["config"]["mfma_gflop_per_step"] = round(flops * 16 / 36 / 1e9, 4)
        line["config"]["flop_count"] = "direct convolution's 2*N*Ho*Wo*Cout*Cin*9"
    if with_cpu:
        line["cpu_baseline"] = cpu_baseline(cid, li, x, w, b, cpu_seconds, unit)
    return line


def separable_algorithmic():
    """Nominal FLOPs (depthwise + 1x1) and bytes (x, both weights, both
    biases and y, each once; the intermediate never reaches memory) of the
    fused depthwise-separable pass."""
    dw, pw = ci.layer(3, 0), ci.layer(3, 1)
    fd, _ = algorithmic(dw)
    fp, _ = algorithmic(pw)
    ho, wo = out_hw(dw)
    nbytes = 2 * (dw.N * dw.Cin * dw.H * dw.W + dw.Cin * 9 + pw.Cout * pw.Cin + dw.N * pw.Cout * ho * wo)
    nbytes += 4 * (dw.Cin if dw.epilogue & ci.EPI_BIAS else 0)
    nbytes += 4 * (pw.Cout if pw.epilogue & ci.EPI_BIAS else 0)
    return fd + fp, nbytes


def separable_cpu_baseline(x, wdw, bdw, wpw, bpw, target_s):
    """The oracle's block (depthwise, bf16 intermediate, 1x1) on whole images
    of the workload until target_s elapses; GB/s of the fused pass."""
    import oracle
    dw, pw = ci.layer(3, 0), ci.layer(3, 1)
    _, nbytes = separable_algorithmic()
    k = 0
    t0 = time.perf_counter()
    while k < dw.N and (k == 0 or time.perf_counter() - t0 < target_s):
        oracle.separable(x[k:k + 1], wdw, wpw, bdw, bpw, dw.stride, dw.pad,
                         dw_relu=bool(dw.epilogue & ci.EPI_RELU), pw_relu=bool(pw.epilogue & ci.EPI_RELU))
        k += 1
    dt = time.perf_counter() - t0
    return {"value": round(nbytes * (k / dw.N) / dt / 1e9, 6), "unit": "GB/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"first {k} of {dw.N} images, all channels, fp64 depthwise + 1x1 ({dt:.1f} s)",
            "host_cpu": host_cpu()}


def bench_separable(steps, warmup, cpu_seconds, with_cpu):
    """Config 3's pair as one fused pass, timed like a layer."""
    import torch
    import cnn_convolution_conv2d_amd as c2

    dw, pw = ci.layer(3, 0), ci.layer(3, 1)
    ho, wo = out_hw(dw)
    N, C, Cout = dw.N, dw.Cin, pw.Cout
    flops, nbytes = separable_algorithmic()
    x, wdw, bdw = ci.layer_tensors(3, 0)
    _, wpw, bpw = ci.layer_tensors(3, 1, N=1, H=1, W=1)
    dev = torch.device("cuda", torch.cuda.current_device())
    stream = torch.cuda.current_stream()
    wd = torch.from_numpy(wdw).to(dev).to(torch.bfloat16)
    wdp = torch.empty(c2.conv2d_packed_weight_bytes(C, C, 3, 3, C, c2.BF16) // 2, dtype=torch.bfloat16,
                      device=dev)
    c2.conv2d_pack_weights(wd, wdp, C, C, 3, 3, C, c2.BF16)
    wpd = torch.from_numpy(wpw.reshape(Cout, C)).to(dev).to(torch.bfloat16).contiguous()
    bdd = torch.from_numpy(bdw).to(dev) if bdw is not None else None
    bpd = torch.from_numpy(bpw).to(dev) if bpw is not None else None
    set_bytes = 2 * (x.size + N * Cout * ho * wo)
    R = max(1, min(16, math.ceil(ROTATE_BYTES / set_bytes)))
    x_nchw = torch.from_numpy(x).to(dev).to(torch.bfloat16)
    x0 = torch.empty((N, dw.H, dw.W, C), dtype=torch.bfloat16, device=dev)
    c2.conv2d_nchw_to_nhwc(x_nchw, x0, N, C, dw.H, dw.W, c2.BF16)
    xs = [x0] + [x0.clone() for _ in range(R - 1)]
    ys = [torch.empty((N, ho, wo, Cout), dtype=torch.bfloat16, device=dev) for _ in range(R)]
    del x_nchw, wd

    def step(i):
        j = i % R
        c2.conv2d_fwd_separable_nhwc(xs[j], wdp, bdd, wpd, bpd, ys[j], N, C, dw.H, dw.W, Cout,
                                     dw.stride, dw.pad, c2.BF16, dw.epilogue, pw.epilogue, stream)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = np.array([a.elapsed_time(e) for a, e in ev])
    mean_ms = float(launch_ms.mean())
    ms_per_step = wall * 1e3 / steps
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (mean_ms * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded, workload shapes and distributions; no dataset)",
        "config": {
            "workload": f"cfg3 fused depthwise-separable: N={N} C={C} {dw.H}x{dw.W}, 3x3 depthwise "
                        f"s{dw.stride} p{dw.pad} bias relu -> 1x1 {C}->{Cout}",
            "layout": "NHWC activations, packed weights", "path": "separable",
            "gflop_per_step": round(flops / 1e9, 4), "algorithmic_mb_per_step": round(nbytes / 1e6, 3),
            "rotating_buffer_sets": R, "device": torch.cuda.get_device_name(dev),
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 3), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic("cfg3:separable", "separable"),
            **launch_stats(launch_ms),
        },
    }
    if with_cpu:
        line["cpu_baseline"] = separable_cpu_baseline(x, wdw, bdw, wpw, bpw, cpu_seconds)
    return line


def hbm_ceiling(steps):
    """What a plain device copy (torch's copy kernel) reaches when it moves
    the same total bytes as each HBM-bound layer (x read + y written, bf16):
    a copy of (R + W) / 2 bytes into another buffer.  Buffer sets rotate as in
    the layer timing.  Context for the HBM roofline fractions: a streaming
    kernel with no arithmetic at the layer's size, not a bound on it."""
    import torch
    dev = torch.device("cuda", torch.cuda.current_device())
    lines = []
    for cid, li in ((3, 0), (3, 1), (5, 0), (5, 2), (6, 1)):
        ly = ci.layer(cid, li)
        ho, wo = out_hw(ly)
        rb, wb = 2 * ly.N * ly.H * ly.W * ly.Cin, 2 * ly.N * ho * wo * ly.Cout
        half = (rb + wb) // 4  # bf16 elements of each side of the copy
        R = max(2, min(16, math.ceil(ROTATE_BYTES / (rb + wb))))
        xs = [torch.randn(half, device=dev).to(torch.bfloat16) for _ in range(R)]
        ys = [torch.empty(half, dtype=torch.bfloat16, device=dev) for _ in range(R)]
        for i in range(5):
            ys[i % R].copy_(xs[i % R])
        torch.cuda.synchronize()
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(steps):
            ys[i % R].copy_(xs[i % R])
        e.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(e) * 1e3 / steps
        moved = 4 * half
        lines.append({"workload": f"cfg{cid} {ly.name}", "layer_read_mb": round(rb / 1e6, 2),
                      "layer_write_mb": round(wb / 1e6, 2), "copy_mb_each_way": round(2 * half / 1e6, 2),
                      "us": round(us, 2), "gb_per_s": round(moved / us / 1e3, 1),
                      "frac_of_8tb": round(moved / us / 1e3 / PEAK_HBM_GBS, 4), "buffer_sets": R})
        del xs, ys
    return lines


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--layer", default=HEADLINE_LAYER, help="workload layer as CID:LAYER_INDEX")
    ap.add_argument("--all", action="store_true", help="time every workload layer and the fused pair")
    ap.add_argument("--separable", action="store_true",
                    help="time the fused depthwise-separable pair of config 3")
    ap.add_argument("--winograd", action="store_true",
                    help="time the 3x3 layer through the Winograd F(2x2,3x3) entry")
    ap.add_argument("--path", default="auto",
                    choices=["auto", "direct", "depthwise", "gemm1x1", "igemm", "igemm_gather", "igemm_halo"],
                    help="force the library's kernel path (conv2d_set_path_override) for the timed layers")
    ap.add_argument("--launch-times", action="store_true",
                    help="add every timed launch's duration (us, in launch order) to the JSON line")
    ap.add_argument("--power", type=float, default=0.0, metavar="SECONDS",
                    help="after the timed steps, launch the layer back to back for SECONDS and read the "
                         "socket power and graphics clock with amd-smi every two seconds")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-nchw", action="store_true",
                    help="skip timing the NCHW entry conv2d_fwd beside the timed entry")
    ap.add_argument("--hbm-ceiling", action="store_true",
                    help="only time a plain device copy moving each HBM-bound layer's total bytes")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 5 plain device copies of 256 MiB (known HBM traffic), for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE")
    a = ap.parse_args(argv)
    global FORCED_PATH, LAUNCH_TIMES
    LAUNCH_TIMES = a.launch_times
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py: the library and this benchmark use one GPU (asked for --gpus {a.gpus}, "
              f"WORLD_SIZE {world}); a multi-GPU split of the batch is not implemented.",
              file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    if a.copy_calibration:
        n = 256 << 20
        src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                          "dispatches": 5}))
        return 0
    if a.hbm_ceiling:
        for ln in hbm_ceiling(a.steps):
            print(json.dumps(ln), flush=True)
        return 0
    _builder().ensure_built()  # rebuilds a missing or stale library
    if a.winograd and not a.all:
        cid, li = (int(v) for v in a.layer.split(":"))
        print(json.dumps(bench_layer(cid, li, a.steps, a.warmup, a.cpu_seconds, with_cpu=not a.no_cpu_baseline,
                                     winograd=True, power_seconds=a.power)), flush=True)
        return 0
    if a.separable and not a.all:
        print(json.dumps(bench_separable(a.steps, a.warmup, a.cpu_seconds,
                                         with_cpu=not a.no_cpu_baseline)), flush=True)
        return 0
    layers = [(c, i) for c in sorted(ci.WORKLOADS) for i in range(len(ci.WORKLOADS[c].layers))] \
        if a.all else [tuple(int(v) for v in a.layer.split(":"))]
    if a.path != "auto":
        import cnn_convolution_conv2d_amd as c2
        FORCED_PATH = a.path
        c2.conv2d_set_path_override(getattr(c2, "PATH_" + a.path.upper()))
    for cid, li in layers:
        line = bench_layer(cid, li, a.steps, a.warmup, a.cpu_seconds,
                           with_cpu=not a.no_cpu_baseline, with_nchw=not a.no_nchw, power_seconds=a.power)
        if not a.no_cpu_baseline and (cid, li) == layers[0]:
            line["cpu_baseline"]["single_thread"] = oracle_single_thread()
        print(json.dumps(line), flush=True)
        if a.all and cid == 2:
            print(json.dumps(bench_layer(cid, li, a.steps, a.warmup, a.cpu_seconds,
                                         with_cpu=not a.no_cpu_baseline, winograd=True)), flush=True)
        if a.all and cid == 3 and li == len(ci.WORKLOADS[3].layers) - 1:
            print(json.dumps(bench_separable(a.steps, a.warmup, a.cpu_seconds,
                                             with_cpu=not a.no_cpu_baseline)), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
