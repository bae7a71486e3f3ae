#!/usr/bin/env python3
"""Benchmark of libfno's spectral convolution on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3] [--variant fused|unfused]
                    [--pass forward|backward|layer|filter|linconv]

One step = one full spectral-convolution call (forward pruned FFT, per-mode
channel mix, inverse pruned FFT) over one batch of synthetic inputs already
resident in device memory.  Default workload: the 128x128 grid shaped like the
TurboFNO blog's PDE step (B=32, Cin=Cout=64, modes 32x32).  Buffer sets
(x, out) rotate so repeated calls cannot be served from the 256 MiB
last-level cache when one set is larger than it.

The timed region runs K steps twice: first plainly between two HIP events
(ms_per_step, value), then again with every kernel launched with its own
start / stop HIP events, which take that kernel's start and end timestamps
(per-kernel times, roofline).  The second pass is separate because
launch-carried events lengthen the gaps between kernels.

Prints ONE JSON line.  `value` is compulsory bytes (x + W + out) per second
in GB/s; the line also carries calls/s, the fraction of the 8 TB/s HBM peak,
a `roofline` entry for the longest-running kernel (its share of x + W + out
per launch over its average launch time: the first transform reads x, the
mix reads W, the last transform writes out; the truncated spectra it also
moves appear as `spectra_ratio`), a `whole_call` entry (x + W + out over the
call time), a `mix` entry for the matrix-core channel mix (8 flops per
complex multiply-add against the fp32 MFMA peak, and the 6 the 3M form
executes) when the workload uses it, a `cpu_baseline` entry (the fp64 CPU
oracle timed on this host on a bounded sample), `parity` (the benched
output against that oracle output), and `workloads`: the other four
workloads timed in the same run (ms per call, GB/s, calls/s, per-kernel
times) with their parity against the oracle on a sample of batch items.

--pass backward times both gradients of a real loss (compulsory bytes: x, W,
dL/dout read, dL/dx, dL/dW written); --pass layer times the operator with
the fused layer tail gelu(conv + bias + branch) (adds the branch read);
--pass filter times the diagonal global filter (x and the mask read, out
written); --pass linconv times the zero-padded linear convolution with a
5x5 (1D: 7-tap) kernel and 'same' output (x and the kernel read, out
written; the kernel's weight spectrum is prepared before the timed region).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
MFMA_FP32_PEAK_TFLOPS = 157.3     # dense fp32 matrix-core peak of one MI355X
ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from fft_spectral_convolution_amd.inputs import CONFIGS, make_inputs  # noqa: E402


# Algorithmic bytes each kernel must move per launch (read once + write once),
# by kernel name (per-unit figures: x, W, out and the truncated spectra).
def kernel_bytes(name: str, cfg, backward: bool = False) -> int:
    """Bytes of kernel `name` (a repeat launch carries ":n").  In the backward
    pass the first transform runs on dL/dout (Cout channels) and the inverse
    writes dL/dx (Cin channels): both see the channel counts swapped; the
    second forward transform (":2") runs on x."""
    if backward and not name.endswith(":2"):
        import dataclasses
        cfg = dataclasses.replace(cfg, Cin=cfg.Cout, Cout=cfg.Cin)
    c8 = 8
    m_modes = cfg.my if cfg.kind == "1d" else 2 * cfg.mx * cfg.my
    if cfg.kind == "1d":
        n_in = cfg.B * cfg.Cin * cfg.W * 4
        n_out = cfg.B * cfg.Cout * cfg.W * 4
        xh = cfg.B * cfg.Cin * cfg.my * c8
        yh = cfg.B * cfg.Cout * cfg.my * c8
        wb = cfg.my * cfg.Cin * cfg.Cout * c8
        r_in = r_out = 0
    else:
        m = 2 * cfg.mx * cfg.my
        n_in = cfg.B * cfg.Cin * cfg.H * cfg.W * 4
        n_out = cfg.B * cfg.Cout * cfg.H * cfg.W * 4
        xh = cfg.B * cfg.Cin * m * c8
        yh = cfg.B * cfg.Cout * m * c8
        wb = m * cfg.Cin * cfg.Cout * c8
        r_in = cfg.B * cfg.Cin * cfg.H * cfg.my * c8
        r_out = cfg.B * cfg.Cout * cfg.H * cfg.my * c8
    table = {
        "rows_fwd": n_in + (r_in if cfg.kind == "2d" else xh),
        "cols_fwd": r_in + xh,
        "mix_valu": xh + wb + yh,
        "mix_mfma": xh + wb + yh,
        "mix_mfma_adj": xh + wb + yh,
        "cols_inv": yh + r_out,
        "rows_inv": (r_out if cfg.kind == "2d" else yh) + n_out,
        "fwd2d": n_in + xh,
        "inv2d": yh + n_out,
        # the whole call in one kernel: the spectra never leave the chip
        "conv_fused": n_in + wb + n_out,
        # backward pass: the weight gradient reads both truncated spectra and
        # writes a weight-sized gradient; the adjoint transposes the weight
        # fused layer tail: the inverse also reads the branch (output-sized)
        "inv2d_gelu": yh + 2 * n_out,
        "rows_inv_gelu": (r_out if cfg.kind == "2d" else yh) + 2 * n_out,
        # diagonal filter: both truncated spectra and the (mode, channel) mask
        "mix_diag": xh + yh + (m_modes * cfg.Cin * c8),
        "fwd2d_diag": n_in + xh + (m_modes * cfg.Cin * c8),
        "mask_transpose": 2 * m_modes * cfg.Cin * c8,
        "wgrad": xh + yh + wb,
        "wadjoint": 2 * wb,
        # sum of the batch splits' partial weight gradients (when the batch
        # is split): counted as its one compulsory write
        "wgrad_reduce": wb,
    }
    return table[name.split(":")[0]]


def compulsory_share(name: str, cfg, backward: bool = False) -> int:
    """The kernel's share of the compulsory bytes x + W + out: the first
    transform reads x, the mix reads W, the last transform writes out (the
    truncated spectra between kernels are not compulsory).  Kernels that
    only move spectra (the column passes of the staged schedule) have none."""
    if backward and not name.endswith(":2"):
        import dataclasses
        cfg = dataclasses.replace(cfg, Cin=cfg.Cout, Cout=cfg.Cin)
    n_in = 4 * int(np.prod(cfg.x_shape))
    n_out = 4 * int(np.prod(cfg.out_shape))
    wb = 8 * int(np.prod(cfg.w_shape))
    base = name.split(":")[0]
    share = {
        "fwd2d": n_in, "rows_fwd": n_in, "fwd2d_diag": n_in,
        "mix_mfma": wb, "mix_valu": wb, "mix_mfma_adj": wb, "mix_fused": wb,
        "inv2d": n_out, "rows_inv": n_out, "inv2d_gelu": 2 * n_out, "rows_inv_gelu": 2 * n_out,
        "wgrad": wb, "wgrad_reduce": 0,
        "conv_fused": n_in + wb + n_out,
    }
    return share.get(base, 0)


def load_traffic(kernel: str, workload: str):
    """Measured HBM bytes per launch from committed rocprofv3 counter runs, if
    they were taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            rec = json.load(f)
        entry = rec.get(workload, {}).get(kernel)
        if not entry:
            return None
        import hashlib
        h = hashlib.sha256()
        for src in sorted(entry["sources"]):
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != entry["sources_sha256"]:
            return None
        return int(entry["bytes_per_launch"])
    except Exception:
        return None


def cpu_baseline(cfg, x, w, budget_s: float = 12.0, g=None, compulsory=None, layer=None, mask=None, kernel=None):
    """Time the fp64 oracle (as it stands) on this host on a bounded sample
    (the backward pass when the output gradient g is given, the operator with
    the layer tail when layer = (bias, branch) is).  Returns the baseline
    entry, the oracle's output on the first nb batch items and nb."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    except Exception:
        threads = 1
    # one batch item first, to size the sample
    def call(nb):
        if kernel is not None:
            if cfg.kind == "1d":
                kk = kernel.shape[-1]
                return oracle.linear_conv1d_ref(x[:nb], kernel, (kk - 1) // 2, cfg.W)
            kh, kw = kernel.shape[-2:]
            return oracle.linear_conv2d_ref(x[:nb], kernel, (kh - 1) // 2, (kw - 1) // 2, cfg.H, cfg.W)
        if mask is not None:
            if cfg.kind == "1d":
                return oracle.spectral_filter1d_ref(x[:nb], mask, cfg.my)
            return oracle.spectral_filter2d_ref(x[:nb], mask, cfg.mx, cfg.my)
        if layer is not None:
            bias, branch = layer
            if cfg.kind == "1d":
                return oracle.spectral_conv1d_gelu_ref(x[:nb], w, cfg.my, bias=bias, branch=branch[:nb])
            return oracle.spectral_conv2d_gelu_ref(x[:nb], w, cfg.mx, cfg.my, bias=bias, branch=branch[:nb])
        if g is not None:
            if cfg.kind == "1d":
                return oracle.spectral_conv1d_backward_ref(x[:nb], w, g[:nb], cfg.my)
            return oracle.spectral_conv2d_backward_ref(x[:nb], w, g[:nb], cfg.mx, cfg.my)
        if cfg.kind == "1d":
            return oracle.spectral_conv1d_ref(x[:nb], w, cfg.my)
        return oracle.spectral_conv2d_ref(x[:nb], w, cfg.mx, cfg.my)

    t0 = time.perf_counter()
    call(1)
    t1 = time.perf_counter() - t0
    nb = int(max(1, min(cfg.B, budget_s / max(t1, 1e-3))))
    reps = 0
    t0 = time.perf_counter()
    while True:
        ref = call(nb)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s * 0.5 or reps >= 3:
            break
    per_item = el / (reps * nb)
    call_time = per_item * cfg.B
    return {
        "value": round((compulsory or cfg.compulsory_bytes) / call_time / 1e9, 6),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{reps} oracle call(s) on {nb} of {cfg.B} batch items of the same workload "
                   f"({el:.1f} s total); scaled to the full batch: {call_time:.3f} s per layer call"),
        "calls_per_s": round(1.0 / call_time, 6),
        "os_cpu_count": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
    }, ref, nb


def device_memory_report(dev: int) -> dict:
    """HBM figures as the HIP runtime reports them for device `dev`: memory
    bus width (bits) and peak memory clock (kHz), from hipDeviceGetAttribute
    (hipDeviceAttributeMemoryBusWidth = 59 and hipDeviceAttributeMemoryClockRate
    = 60 in ROCm 7's hip_runtime_api.h), and the peak they imply.  HBM3E
    moves four transfers per reported memory clock (MI355X: 2.0 GHz, 8 Gbps
    per pin), so the peak is 4 x clock x width / 8 (8192 bits: 8.19 TB/s,
    the published ~8 TB/s).  The runtime library is the one already loaded
    in this process (same soname)."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so.7")
        v = ctypes.c_int(0)
        vals = {}
        for name, attr in (("bus_width_bits", 59), ("memory_clock_khz", 60)):
            vals[name] = v.value if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, dev) == 0 else None
    except OSError as e:
        return {"error": str(e)}
    # the enum values are those of ROCm 7; a runtime that numbers them
    # differently would answer another attribute: keep only plausible values
    if not (vals["bus_width_bits"] and 256 <= vals["bus_width_bits"] <= 65536):
        vals["bus_width_bits"] = None
    if not (vals["memory_clock_khz"] and 100_000 <= vals["memory_clock_khz"] <= 20_000_000):
        vals["memory_clock_khz"] = None
    if vals["bus_width_bits"] and vals["memory_clock_khz"]:
        vals["derived_peak_gbs"] = round(4.0 * vals["memory_clock_khz"] * 1e3 * vals["bus_width_bits"] / 8 / 1e9, 1)
    vals["nominal_peak_gbs"] = HBM_PEAK_GBS
    return vals


def build_step(fno, torch, dev, cfg, which, variant, x_np, w_np, nsets):
    """Device buffers and the step function of one workload and pass.  Returns
    (step, outs, compulsory, extras) with extras holding the host arrays the
    oracle needs for that pass."""
    xs = [torch.from_numpy(x_np).to(dev)]
    for _ in range(nsets - 1):
        xs.append(xs[0].clone())
    outs = [torch.empty(cfg.out_shape, dtype=torch.float32, device=dev) for _ in range(nsets)]
    w = torch.from_numpy(w_np).to(dev)
    compulsory = cfg.compulsory_bytes
    extras = {"g": None, "layer": None, "mask": None, "kernel": None, "lens": None, "touched_extra": 0}
    if which == "backward":
        # step: both gradients of a real loss, given a synthetic dL/dout of the
        # output's shape; compulsory bytes: x, w, dL/dout read, dL/dx, dL/dw written
        g_np = np.random.default_rng(1).uniform(-1.0, 1.0, size=cfg.out_shape).astype(np.float32)
        gs = [torch.from_numpy(g_np).to(dev)]
        for _ in range(nsets - 1):
            gs.append(gs[0].clone())
        compulsory = 2 * int(x_np.nbytes) + 2 * int(w_np.nbytes) + int(g_np.nbytes)
        gxs = [torch.empty_like(xs[0]) for _ in range(nsets)]
        gw = torch.empty_like(w)
        extras["g"] = g_np
        extras["touched_extra"] = nsets * x_np.nbytes + w_np.nbytes
        if cfg.kind == "1d":
            step = lambda i: fno.fno_spectral_conv1d_backward(xs[i % nsets], w, gs[i % nsets], cfg.my,
                                                              grad_x=gxs[i % nsets], grad_w=gw)
        else:
            step = lambda i: fno.fno_spectral_conv2d_backward(xs[i % nsets], w, gs[i % nsets], cfg.mx, cfg.my,
                                                              grad_x=gxs[i % nsets], grad_w=gw)
        outs = gxs
    elif which == "layer":
        # step: out = gelu(conv + bias[o] + branch), branch an output-sized
        # tensor; compulsory bytes: x, w, bias, branch read, out written
        rng = np.random.default_rng(2)
        br_np = rng.standard_normal(cfg.out_shape).astype(np.float32)
        bias_np = rng.standard_normal(cfg.Cout).astype(np.float32)
        extras["layer"] = (bias_np, br_np)
        bias = torch.from_numpy(bias_np).to(dev)
        brs = [torch.from_numpy(br_np).to(dev)]
        for _ in range(nsets - 1):
            brs.append(brs[0].clone())
        compulsory = cfg.compulsory_bytes + int(br_np.nbytes) + 4 * cfg.Cout
        extras["touched_extra"] = nsets * 4 * int(np.prod(cfg.out_shape))
        if cfg.kind == "1d":
            step = lambda i: fno.fno_spectral_conv1d_gelu(xs[i % nsets], w, cfg.my, bias=bias, branch=brs[i % nsets],
                                                          out=outs[i % nsets])
        else:
            step = lambda i: fno.fno_spectral_conv2d_gelu(xs[i % nsets], w, cfg.mx, cfg.my, bias=bias,
                                                          branch=brs[i % nsets], out=outs[i % nsets])
    elif which == "filter":
        # step: out = C2R(truncate(R2C(x)) * mask); compulsory bytes: x and
        # the mask read, out written
        rng = np.random.default_rng(3)
        mshape = (cfg.my, cfg.Cin) if cfg.kind == "1d" else (2, cfg.mx, cfg.my, cfg.Cin)
        mask_np = (rng.standard_normal(mshape) + 1j * rng.standard_normal(mshape)).astype(np.complex64)
        mask = torch.from_numpy(mask_np).to(dev)
        extras["mask"] = mask_np
        compulsory = 2 * int(x_np.nbytes) + int(mask_np.nbytes)
        if cfg.kind == "1d":
            step = lambda i: fno.fno_spectral_filter1d(xs[i % nsets], mask, cfg.my, out=outs[i % nsets])
        else:
            step = lambda i: fno.fno_spectral_filter2d(xs[i % nsets], mask, cfg.mx, cfg.my, out=outs[i % nsets])
    elif which == "linconv":
        # step: out = crop(C2R(R2C(pad x) * wspec)), 'same' output; the weight
        # spectrum of the kernel is prepared once (kernels are fixed across
        # calls); compulsory bytes: x and the kernel read, out written
        rng = np.random.default_rng(4)
        kshape = (cfg.Cout, cfg.Cin, 7) if cfg.kind == "1d" else (cfg.Cout, cfg.Cin, 5, 5)
        k_np = (rng.standard_normal(kshape) / np.sqrt(np.prod(kshape[1:]))).astype(np.float32)
        kd = torch.from_numpy(k_np).to(dev)
        compulsory = cfg.compulsory_bytes - int(w_np.nbytes) + int(k_np.nbytes)
        extras["kernel"] = k_np
        lens = ([fno.fno_linear_conv_length(cfg.W, 7)] if cfg.kind == "1d"
                else [fno.fno_linear_conv_length(cfg.H, 5), fno.fno_linear_conv_length(cfg.W, 5)])
        if 0 in lens:
            sys.exit(f"--pass linconv: the padded lengths of workload {cfg.name} exceed the transforms' range")
        extras["lens"] = lens
        if cfg.kind == "1d":
            wspec = fno.fno_linear_conv1d_prepare(kd, cfg.W)
            step = lambda i: fno.fno_linear_conv1d(xs[i % nsets], kd, wspec=wspec, out=outs[i % nsets])
        else:
            wspec = fno.fno_linear_conv2d_prepare(kd, cfg.H, cfg.W)
            step = lambda i: fno.fno_linear_conv2d(xs[i % nsets], kd, wspec=wspec, out=outs[i % nsets])
    elif cfg.kind == "1d":
        fn = fno.fno_spectral_conv1d if variant == "fused" else fno.fno_spectral_conv1d_unfused
        step = lambda i: fn(xs[i % nsets], w, cfg.my, out=outs[i % nsets])
    else:
        fn = fno.fno_spectral_conv2d if variant == "fused" else fno.fno_spectral_conv2d_unfused
        step = lambda i: fn(xs[i % nsets], w, cfg.mx, cfg.my, out=outs[i % nsets])
    return step, outs, compulsory, extras


def buffer_sets(cfg) -> int:
    """Enough (x, out) sets that the rotation exceeds the 256 MiB last-level cache."""
    set_bytes = 4 * (np.prod(cfg.x_shape) + np.prod(cfg.out_shape))
    return int(max(1, min(4, -(-3 * 256 * 2**20 // set_bytes))))


def time_steps(fno, torch, stream, step, steps, warmup):
    """Warm up, then time `steps` plain steps between two HIP events on the
    call's stream (ms per step), then the same steps again with every kernel
    launched with its own start / stop events (per-kernel times)."""
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    kernels = fno.fno_last_kernels()
    # a kernel that runs more than once per step gets its launch number
    seen = {}
    for j, k in enumerate(kernels):
        seen[k] = seen.get(k, 0) + 1
        if seen[k] > 1:
            kernels[j] = f"{k}:{seen[k]}"
    nk = len(kernels)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * nk)] for _ in range(steps)]
    for row in evs:                      # torch creates the HIP event on first record
        for e in row:
            e.record(stream)
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        step(i)
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # launch-carried events change the gaps between kernels, so this pass
    # does not set ms_per_step
    for i in range(steps):
        fno.fno_set_timing_events(evs[i])
        step(i)
    torch.cuda.synchronize()
    fno.fno_set_timing_events(None)
    ms = start.elapsed_time(stop) / steps
    per_kernel_ms = [float(np.mean([evs[i][2 * k].elapsed_time(evs[i][2 * k + 1]) for i in range(steps)]))
                     for k in range(nk)]
    spans_us = [evs[i][0].elapsed_time(evs[i][2 * nk - 1]) * 1e3 for i in range(steps)]
    return ms, kernels, per_kernel_ms, spans_us, wall


def oracle_out(cfg, x, w, nb):
    import oracle
    if cfg.kind == "1d":
        return oracle.spectral_conv1d_ref(x[:nb], w, cfg.my)
    return oracle.spectral_conv2d_ref(x[:nb], w, cfg.mx, cfg.my)


def parity(got, ref) -> dict:
    """Relative L2 and max-abs error (relative to max|ref|) of the GPU output
    against the oracle on the same batch items."""
    g = got.astype(np.float64)
    rel = float(np.linalg.norm((g - ref).ravel()) / max(np.linalg.norm(ref.ravel()), 1e-300))
    mx = float(np.max(np.abs(g - ref)) / max(np.max(np.abs(ref)), 1e-300))
    return {"rel_l2": float(f"{rel:.3e}"), "max_abs_rel": float(f"{mx:.3e}"),
            "pass": bool(rel <= 1e-5 and mx <= 1e-4)}


def workload_summary(fno, torch, dev, stream, name, steps, warmup, oracle_budget_s=2.0) -> dict:
    """ms per call, GB/s, HBM %, calls/s and per-kernel times of the plain
    operator on workload `name`, plus its parity against the oracle on as many
    batch items as ~oracle_budget_s of oracle time allows."""
    cfg = CONFIGS[name]
    x_np, w_np = make_inputs(cfg, 0)
    nsets = buffer_sets(cfg)
    step, outs, compulsory, _ = build_step(fno, torch, dev, cfg, "forward", "fused", x_np, w_np, nsets)
    ms, kernels, pk, _, _ = time_steps(fno, torch, stream, step, steps, warmup)
    gbs = compulsory / (ms * 1e-3) / 1e9
    set_bytes = 4 * (np.prod(cfg.x_shape) + np.prod(cfg.out_shape))
    resident = bool(nsets * set_bytes + w_np.nbytes <= 256 * 2**20)
    got = outs[(steps - 1) % nsets][:1].cpu().numpy()
    t0 = time.perf_counter()
    ref = oracle_out(cfg, x_np, w_np, 1)
    t1 = time.perf_counter() - t0
    nb = int(max(1, min(cfg.B, oracle_budget_s / max(t1, 1e-3))))
    if nb > 1:
        got = outs[(steps - 1) % nsets][:nb].cpu().numpy()
        ref = oracle_out(cfg, x_np, w_np, nb)
    res = {
        "workload": f"{cfg.name}: {cfg.describe()}",
        "ms_per_step": round(ms, 6),
        "calls_per_s": round(1e3 / ms, 3),
        "gbs": round(gbs, 3),
        "hbm_pct": round(100.0 * gbs / HBM_PEAK_GBS, 3),
        "cache_resident": resident,
        "kernels_us": {k: round(t * 1e3, 3) for k, t in zip(kernels, pk)},
        "parity": dict(parity(got, ref), batch_items=nb),
    }
    if resident:
        res["note"] = "every buffer fits the 256 MiB last-level cache: GB/s is not an HBM rate; calls/s is the figure"
    del outs
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c3", choices=sorted(CONFIGS))
    ap.add_argument("--variant", default="fused", choices=["fused", "unfused"])
    ap.add_argument("--pass", dest="which", default="forward",
                    choices=["forward", "backward", "layer", "filter", "linconv"],
                    help="time the operator (default), its backward pass (both gradients), the operator "
                         "with the fused layer tail gelu(conv + bias + branch), or the diagonal global "
                         "filter (one complex weight per kept mode and channel), or the zero-padded linear "
                         "convolution with a 5x5 (1D: 7-tap) kernel, 'same' output, weight spectrum prepared "
                         "once outside the timed region")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the other four workloads (timed and parity-checked in the same run by default)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--stream-ceilings", action="store_true",
                    help="time torch's own write (fill_), read (sum) and copy (copy_) kernels over rotated "
                         "256 MiB buffers: the box's practical streaming rates, a calibration only")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device copies of MIB MiB (scale for HBM byte counters) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the batch would shard across GPUs with W replicated; not built).", file=sys.stderr)
        sys.exit(2)

    import torch
    import fft_spectral_convolution_amd as fno

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.stream_ceilings:
        # four 256 MiB buffers rotated, so that the 256 MiB last-level cache
        # never holds the buffer an operation touches
        n = 256 * 2**20 // 4
        bufs = [torch.ones(n, dtype=torch.float32, device=dev) for _ in range(4)]
        res = {}
        for name, moved, op in (("write", 1, lambda i: bufs[i % 4].fill_(1.0)),
                                ("read", 1, lambda i: bufs[i % 4].sum()),
                                ("copy", 2, lambda i: bufs[(i + 1) % 4].copy_(bufs[i % 4]))):
            ts = []
            for i in range(24):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                op(i)
                e1.record()
                e1.synchronize()
                if i >= 4:
                    ts.append(e0.elapsed_time(e1) * 1e-3)
            med = float(np.median(ts))
            res[name] = {"gbs": round(moved * n * 4 / med / 1e9, 1), "us": round(med * 1e6, 1)}
        # Reuse through the last-level (memory-side) cache: time a copy out of
        # S (32, 64, 128 MiB) into D after a 1 GiB flush, right after S was
        # written (fill_) and right after S was read (sum).  If the cache kept
        # S, the copy's read half would be faster than after the flush.
        del bufs
        flush = torch.empty(2**28, dtype=torch.float32, device=dev)        # 1 GiB
        reuse = {}
        for mib in (32, 64, 128):
            m = mib * 2**20 // 4
            S = torch.ones(m, dtype=torch.float32, device=dev)
            D = torch.empty_like(S)

            def t_copy(pre):
                ts = []
                for i in range(9):
                    flush.fill_(0.0)
                    flush.sum()
                    pre()
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record()
                    D.copy_(S)
                    e1.record()
                    e1.synchronize()
                    if i >= 2:
                        ts.append(e0.elapsed_time(e1) * 1e3)
                return round(float(np.median(ts)), 2)
            reuse[f"{mib}MiB"] = {"copy_after_flush_us": t_copy(lambda: None),
                                  "copy_after_write_us": t_copy(lambda: S.fill_(2.0)),
                                  "copy_after_read_us": t_copy(lambda: S.sum())}
            del S, D
        print(json.dumps({"stream_ceilings": res, "bytes_per_buffer": n * 4,
                          "note": "torch fill_ / sum / copy_ on rotated 256 MiB buffers, median of 20",
                          "cache_reuse": reuse,
                          "cache_reuse_note": "copy of S into D (us, median of 7) after a 1 GiB flush, "
                                              "after S was written, after S was read"}))
        return
    if args.calibrate_copy:
        n = args.calibrate_copy * 2**20 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": n * 4, "calibrate_copy_bytes_written": n * 4, "copies": 5}))
        return
    cfg = CONFIGS[args.workload]
    x_np, w_np = make_inputs(cfg, 0)
    nsets = buffer_sets(cfg)
    set_bytes = 4 * (np.prod(cfg.x_shape) + np.prod(cfg.out_shape))
    step, outs, compulsory, extras = build_step(fno, torch, dev, cfg, args.which, args.variant, x_np, w_np, nsets)
    stream = torch.cuda.current_stream(dev)
    ms_per_step, kernels, per_kernel_ms, spans_us, wall = time_steps(fno, torch, stream, step, args.steps,
                                                                     args.warmup)
    nk = len(kernels)
    dom = int(np.argmax(per_kernel_ms))
    dom_name = kernels[dom]
    # the linear convolution runs on the padded grid at full modes: its kernels'
    # bytes are those of that grid (rows counted at the padded length)
    kcfg = cfg
    if args.which == "linconv":
        import dataclasses
        lens = extras["lens"]
        if cfg.kind == "1d":
            kcfg = dataclasses.replace(cfg, W=lens[0], my=lens[0] // 2 + 1)
        else:
            kcfg = dataclasses.replace(cfg, H=lens[0], W=lens[1], mx=lens[0] // 2, my=lens[1] // 2 + 1)
    bwd = args.which == "backward"
    # Roofline of the longest kernel on its share of the compulsory bytes
    # (x + W + out: the first transform's x, the mix's W, the last
    # transform's out); the truncated spectra it also moves are reported as
    # the ratio of all its bytes to that share.
    dom_share = compulsory_share(dom_name, cfg, bwd) if args.which in ("forward", "backward", "layer") else 0
    dom_all = kernel_bytes(dom_name, kcfg, bwd)
    dom_alg = dom_share if dom_share > 0 else dom_all
    achieved = dom_alg / (per_kernel_ms[dom] * 1e-3) / 1e9
    traffic = load_traffic(dom_name, cfg.name if args.which == "forward" else f"{cfg.name}/{args.which}")
    gbs = compulsory / (ms_per_step * 1e-3) / 1e9
    # bytes of all buffers the timed steps touch
    touched = nsets * set_bytes + w_np.nbytes + extras["touched_extra"]
    per_kernel = {}
    for k, t in zip(kernels, per_kernel_ms):
        share = compulsory_share(k, cfg, bwd) if args.which in ("forward", "backward", "layer") else 0
        allb = kernel_bytes(k, kcfg, bwd)
        per_kernel[k] = {
            "us": round(t * 1e3, 3),
            "compulsory_bytes": share,
            "frac_compulsory": round(share / (t * 1e-3) / 1e9 / HBM_PEAK_GBS, 5) if share else None,
            "all_bytes": allb,
            "gbs_all_bytes": round(allb / (t * 1e-3) / 1e9, 3),
        }
    line = {
        "metric": "spectral-conv GB/s (HBM % of peak) and layer calls/s vs fp64 CPU oracle",
        "value": round(gbs, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {cfg.describe()}",
            "variant": args.variant,
            "pass": args.which,
            "x_dist": cfg.dist,
            "compulsory_bytes": compulsory,
            "buffer_sets": nsets,
            # every buffer a step touches fits the 256 MiB last-level cache:
            # the GB/s figure is then not an HBM rate
            "cache_resident": bool(touched <= 256 * 2**20),
        },
        "calls_per_s": round(1e3 / ms_per_step, 3),
        "hbm_pct": round(100.0 * gbs / HBM_PEAK_GBS, 3),
        "hbm_device": device_memory_report(torch.cuda.current_device()),
        "wall_s_timed": round(wall, 4),
        "kernels": {k: round(t * 1e3, 3) for k, t in zip(kernels, per_kernel_ms)},
        "kernels_unit": "us per launch (start/stop events carried by each launch)",
        "kernel_bytes": per_kernel,
        "step_span_us": {"median": round(float(np.median(spans_us)), 3), "min": round(float(np.min(spans_us)), 3),
                         "note": "first kernel start to last kernel stop of each step, event-carrying pass"},
        "roofline": {
            "kernel": dom_name,
            "bound": "hbm",
            "achieved": round(achieved, 3),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 5),
            "traffic": traffic,
            "algorithmic_bytes": dom_alg,
            "algorithmic_bytes_note": ("the kernel's share of x + W + out" if dom_share > 0 else
                                       "all bytes the kernel must move (it has no share of x + W + out)"),
            "bytes_incl_spectra": dom_all,
            "spectra_ratio": round(dom_all / dom_alg, 4),
            "avg_launch_us": round(per_kernel_ms[dom] * 1e3, 3),
        },
        "whole_call": {
            "achieved": round(gbs, 3),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 5),
            "bytes_incl_spectra": int(sum(kernel_bytes(k, kcfg, bwd) for k in kernels)),
            "spectra_ratio": round(sum(kernel_bytes(k, kcfg, bwd) for k in kernels) / compulsory, 4),
        },
    }
    if "mix_mfma" in kernels and args.which != "backward":
        # the matrix-core stage against the fp32 MFMA peak: the method's count
        # of 8 flops per complex multiply-add (frac), and what the 3M form
        # executes (three real products, 6 flops per complex multiply-add)
        k = kernels.index("mix_mfma")
        macs = kcfg.B * kcfg.Cin * kcfg.Cout * (kcfg.my if kcfg.kind == "1d" else 2 * kcfg.mx * kcfg.my)
        t = per_kernel_ms[k] * 1e-3
        line["mix"] = {
            "kernel": "mix_mfma",
            "bound": "mfma",
            "achieved": round(8.0 * macs / t / 1e12, 3),
            "peak": MFMA_FP32_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(8.0 * macs / t / 1e12 / MFMA_FP32_PEAK_TFLOPS, 5),
            "flops_note": "achieved/frac count 8 flops per complex multiply-add; *_executed_3m count the 6 the 3M form runs",
            "flops_complex_8": 8 * macs,
            "flops_executed_3m": 6 * macs,
            "achieved_executed_3m": round(6.0 * macs / t / 1e12, 3),
            "frac_executed_3m": round(6.0 * macs / t / 1e12 / MFMA_FP32_PEAK_TFLOPS, 5),
            "w_gbs": round(compulsory_share("mix_mfma", kcfg) / t / 1e9, 3),
            "all_bytes_gbs": round(kernel_bytes("mix_mfma", kcfg) / t / 1e9, 3),
            "avg_launch_us": round(per_kernel_ms[k] * 1e3, 3),
        }
    if not args.no_cpu_baseline:
        cb, ref, nb = cpu_baseline(cfg, x_np, w_np, args.cpu_budget, g=extras["g"], compulsory=compulsory,
                                   layer=extras["layer"], mask=extras["mask"], kernel=extras["kernel"])
        line["cpu_baseline"] = cb
        if args.which in ("forward", "layer", "filter", "linconv"):
            # parity of the benched output (the last timed step's) on the
            # batch items the oracle leg computed
            got = outs[(args.steps - 1) % nsets][:nb].cpu().numpy()
            line["parity"] = dict(parity(got, ref), batch_items=nb,
                                  note="last timed step's output against the cpu_baseline leg's oracle output")
    if not args.no_workloads and args.which == "forward" and args.variant == "fused":
        del outs, step
        torch.cuda.empty_cache()
        line["workloads"] = {n: workload_summary(fno, torch, dev, stream, n, args.steps, args.warmup)
                             for n in sorted(CONFIGS) if n != cfg.name}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
