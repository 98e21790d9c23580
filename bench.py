#!/usr/bin/env python3
"""Throughput of the Sign-Muon optimizer step on one MI355X.

A step is one call of signmuon_step: every worker's momentum update,
Frobenius normalisation, Newton-Schulz iterations, sign and 1-bit packing,
then the majority vote and the weight update, for every matrix of the
workload. Inputs are seeded synthetic gradients already resident in HBM.

Default workload: GPT-2 small (nanoGPT, 124M) weight matrices -- 12 layers of
768x2304, 768x768, 768x3072, 3072x768 (84.9M parameters) -- with 8 workers,
bf16 momentum and Newton-Schulz operands, fp32 weights, 1 iteration.

Prints one JSON line: params/s (each parameter counted once per step), the
per-kernel timing measured with HIP events between the library's launches
inside the timed region, the dominant kernel's roofline, and the CPU oracle
timed on a bounded sample of the same workload on this host.
"""
import argparse
import ctypes
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "Sign-Muon params/s per step at 1 GPU; NS MFMA util %; vote+update HBM GB/s"
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # dense MFMA
PEAK_FP32_TFLOPS = 157.3


def log(msg):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gpt2s_mw8_k1")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the int8-payload and comparison-step timings (profiler runs, so "
                         "that per-kernel statistics cover the benchmarked step only)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run one plain copy kernel of this size first (counter calibration)")
    return ap.parse_args()


class Hip:
    """Event calls of the HIP runtime (events must live on the library's stream)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def event(self):
        e = ctypes.c_void_p()
        if self.lib.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e.value

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        if self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, e):
        self.lib.hipEventDestroy(e)

    def record(self, e, stream):
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        if self.lib.hipEventRecord(e, stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def sync(self, e):
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventSynchronize(e)


def work_per_kind(wl):
    """Algorithmic work of each kernel kind in one step: flops for the
    Newton-Schulz GEMMs, HBM bytes for the streaming kernels."""
    s_g = 4 if wl.grad_dtype == "f32" else 2
    s_m = 4 if wl.mom_dtype == "f32" else 2
    mw, k = wl.workers, wl.ns_iters
    n = wl.params
    gram = sum(mw * min(R, C) ** 2 * max(R, C) for R, C in wl.shapes) * k
    prod = sum(mw * 2 * min(R, C) ** 2 * max(R, C) for R, C in wl.shapes) * k
    unfused = sum(R * C for R, C in wl.shapes if C % 64 != 0) if k > 0 else n
    return {
        "momentum": ("hbm", mw * n * (s_g + 2 * s_m)),
        "ns_gram": ("mfma", gram),
        "ns_product": ("mfma", prod),
        "sign_pack": ("hbm", mw * unfused * (4 + 1 / 8)),
        "vote_update": ("hbm", n * (mw / 8 + 8)),
    }


def kernel_table(wl, per_kind_ms):
    """Per kernel kind: ms per step and, for the kinds with an algorithmic
    work count, the achieved rate and its fraction of the peak."""
    work = work_per_kind(wl)
    mfma_peak = PEAK_BF16_TFLOPS if wl.ns_dtype == "bf16" else PEAK_FP32_TFLOPS
    kernels = {}
    for name, ms in per_kind_ms.items():
        entry = {"ms": round(ms, 5)}
        if name in work and work[name][1] > 0:
            bound, amount = work[name]
            if bound == "hbm":
                ach = amount / (ms * 1e-3) / 1e9
                entry.update(bound="hbm", achieved=round(ach, 1), unit="GB/s",
                             frac=round(ach / PEAK_HBM_GBS, 4), algorithmic_bytes=int(amount))
            else:
                ach = amount / (ms * 1e-3) / 1e12
                entry.update(bound="mfma", achieved=round(ach, 1), unit="TFLOP/s",
                             frac=round(ach / mfma_peak, 4), algorithmic_flops=int(amount))
        kernels[name] = entry
    return kernels


def build_state(sm, wl, dev, threads=16):
    """Device buffers of a workload (step 0 gradients from the seeded
    generator, zero momentum, initial W), as the benchmark passes them: packed
    signs and W, no U and no vote output."""
    import torch

    import synthetic
    mom_t = torch.bfloat16 if wl.mom_dtype == "bf16" else torch.float32
    mats = []

    def draw(jm):
        j, m = jm
        return jm, synthetic.gradient(wl, j, m, 0)

    grads = [torch.empty((wl.workers, R, C), dtype=torch.float32, device=dev) for R, C in wl.shapes]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        for (j, m), g in ex.map(draw, [(j, m) for j in range(len(wl.shapes)) for m in range(wl.workers)]):
            grads[j][m].copy_(torch.from_numpy(g))
    for j, (R, C) in enumerate(wl.shapes):
        mats.append(sm.Matrix(
            grad=grads[j],
            momentum=torch.zeros((wl.workers, R, C), dtype=mom_t, device=dev),
            packed=torch.zeros((wl.workers, sm.signmuon_packed_words(R * C)), dtype=torch.int64,
                               device=dev),
            weight=torch.from_numpy(synthetic.initial_weight(wl, j)).to(dev)))
    return mats


def params_of(sm, wl):
    code = {"f32": sm.F32, "bf16": sm.BF16}
    return sm.Params(workers=wl.workers, beta=wl.beta, eta=wl.eta, ns_iters=wl.ns_iters,
                     post_polar_iters=wl.post_polar_iters, grad_dtype=code[wl.grad_dtype],
                     mom_dtype=code[wl.mom_dtype], ns_dtype=code[wl.ns_dtype],
                     norm=sm.NORM_SPECTRAL if wl.norm == "spectral" else sm.NORM_FROBENIUS,
                     power_iters=wl.power_iters)


# The other configurations of the measurement plan, each timed in the same run
# (they are parity cases; the benchmarked line is the GPT-2 small one), and
# the benchmarked workload with spectral scaling (its `power` kind is the
# power iteration): (workload, warmup steps, timed steps).
OTHER_CONFIGS = (("square256_mw4_k1", 5, 20), ("resnet50_4shapes_mw4_k1", 5, 20),
                 ("resnet50_4shapes_mw4_k5", 3, 10), ("gpt2s_mw16_k5_t3", 2, 5),
                 ("block4096_mw16_k5", 1, 3), ("gpt2s_mw8_k1_spectral", 3, 10))


def time_other_configs(sm, hip, dev, configs=OTHER_CONFIGS):
    """Each configuration as whole traced steps on its own buffers: ms per step
    (wall clock over the timed steps), params/s and the per-kernel table."""
    import torch

    import synthetic
    out = {}
    for name, warmup, steps in configs:
        wl = synthetic.WORKLOADS[name]
        t0 = time.perf_counter()
        mats = build_state(sm, wl, dev)
        params = params_of(sm, wl)
        ws = sm.workspace_tensor(mats, params, dev)
        step = sm.Prepared(mats, params, ws)
        for _ in range(warmup):
            step.step()
        traces = [sm.Trace([hip.event() for _ in range(128)]) for _ in range(steps)]
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for tr in traces:
            step.step_traced(tr)
        torch.cuda.synchronize()
        ms = 1e3 * (time.perf_counter() - t1) / steps
        per_kind, _ = traced_kernel_ms(sm, hip, traces)
        for tr in traces:
            for e in list(tr._events):
                hip.destroy(e)
        kernels = kernel_table(wl, per_kind)
        gram, prod = per_kind.get("ns_gram", 0.0), per_kind.get("ns_product", 0.0)
        peak = PEAK_BF16_TFLOPS if wl.ns_dtype == "bf16" else PEAK_FP32_TFLOPS
        ns_util = (100.0 * wl.ns_flops() / ((gram + prod) * 1e-3) / (peak * 1e12)
                   if gram + prod > 0 else None)
        out[name] = {"description": wl.description, "params": wl.params, "workers": wl.workers,
                     "ns_iters": wl.ns_iters, "ns_dtype": wl.ns_dtype, "steps": steps,
                     "ms_per_step": round(ms, 4), "params_per_s": round(wl.params / (ms * 1e-3), 1),
                     "steps_per_s": round(1e3 / ms, 2),
                     "ns_mfma_util_pct": None if ns_util is None else round(ns_util, 2),
                     "kernels_ms_per_step": kernels}
        log(f"[bench] {name}: {ms:.3f} ms per step ({time.perf_counter() - t0:.1f} s with set-up)")
        del mats, ws, step
        torch.cuda.empty_cache()
    return out


def time_standalone_pack(sm, wl, hip, dev, reps=10):
    """signmuon_sign_pack on a [workers][n] U of the workload's size (n = all
    its parameters), bf16 and fp32, timed between HIP events; algorithmic
    bytes: U read once, the packed bits written once."""
    import torch
    stream = torch.cuda.current_stream().cuda_stream
    n, mw = wl.params, wl.workers
    out = {}
    for name, dt, code, size in (("bf16", torch.bfloat16, sm.BF16, 2), ("fp32", torch.float32, sm.F32, 4)):
        u = torch.randn((mw, n), dtype=dt, device=dev)
        packed = torch.empty((mw, sm.signmuon_packed_words(n)), dtype=torch.int64, device=dev)
        ev = [hip.event() for _ in range(2)]
        sm.signmuon_sign_pack(u, n, mw, packed)
        hip.record(ev[0], stream)
        for _ in range(reps):
            sm.signmuon_sign_pack(u, n, mw, packed)
        hip.record(ev[1], stream)
        hip.sync(ev[1])
        ms = hip.elapsed_ms(ev[0], ev[1]) / reps
        for e in ev:
            hip.destroy(e)
        nbytes = mw * n * (size + 1 / 8)
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"ms": round(ms, 5), "bound": "hbm", "achieved": round(gbs, 1), "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": int(nbytes),
                     "workers": mw, "n": n}
        del u, packed
    torch.cuda.empty_cache()
    return out


def time_int8_payload(sm, mats, wl, code, hip, dev, reps=10):
    """The whole step with the int8 payload on the workload's matrices: the
    last Newton-Schulz product writes each worker's signs as int8, and one
    batched launch takes the vote as the sign of their integer sum and
    updates W. Timed as whole traced steps (HIP events on the library's
    stream); the vote kernel's rate is its algorithmic bytes over its time."""
    import torch
    norm = sm.NORM_SPECTRAL if wl.norm == "spectral" else sm.NORM_FROBENIUS
    i8 = [sm.Matrix(grad=m.grad, momentum=m.momentum, weight=m.weight,
                    signs_i8=torch.empty((wl.workers,) + m.shape, dtype=torch.int8, device=dev))
          for m in mats]
    p8 = sm.Params(workers=wl.workers, beta=wl.beta, eta=wl.eta, ns_iters=wl.ns_iters,
                   grad_dtype=code[wl.grad_dtype], mom_dtype=code[wl.mom_dtype],
                   ns_dtype=code[wl.ns_dtype], norm=norm, power_iters=wl.power_iters,
                   payload=sm.PAYLOAD_INT8)
    ws8 = sm.workspace_tensor(i8, p8, dev)
    step8 = sm.Prepared(i8, p8, ws8)
    step8.step()
    traces = [sm.Trace([hip.event() for _ in range(64)]) for _ in range(reps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for tr in traces:
        step8.step_traced(tr)
    torch.cuda.synchronize()
    ms_step = 1e3 * (time.perf_counter() - t0) / reps
    kinds_ms, launches = traced_kernel_ms(sm, hip, traces)
    for tr in traces:
        for e in list(tr._events):
            hip.destroy(e)
    out = {"ms_per_step": round(ms_step, 5), "params_per_s": round(wl.params / (ms_step * 1e-3), 1),
           "kernels_ms": {k: round(v, 5) for k, v in kinds_ms.items()}}
    vms = kinds_ms.get("vote_update_int8")
    if vms:
        nbytes = wl.params * (wl.workers + 8)
        gbs = nbytes / (vms * 1e-3) / 1e9
        out["vote_update_int8"] = {"ms": round(vms, 5), "bound": "hbm", "achieved": round(gbs, 1),
                                   "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                                   "algorithmic_bytes": int(nbytes),
                                   "launches": launches.get("vote_update_int8", 0)}
    return out


def traced_kernel_ms(sm, hip, traces):
    """Per kernel kind, the summed time per step from the events recorded
    around each launch of signmuon_step_traced, and the launch counts."""
    per_kind_ms, launch_count = {}, {}
    for kd in traces[0].kinds():
        launch_count[sm.KERNEL_KINDS[kd]] = launch_count.get(sm.KERNEL_KINDS[kd], 0) + 1
    for tr in traces:
        kinds = tr.kinds()
        if tr.launches + 1 > len(tr._events):
            raise RuntimeError("trace capacity too small")
        evs = list(tr._events)
        for i, kd in enumerate(kinds):
            name = sm.KERNEL_KINDS[kd]
            per_kind_ms[name] = per_kind_ms.get(name, 0.0) + hip.elapsed_ms(evs[i], evs[i + 1])
    return {k: v / len(traces) for k, v in per_kind_ms.items()}, launch_count


def time_comparison_steps(sm, mats, wl, code, hip, dev, reps=10):
    """The comparison steps on the workload's matrices, each timed as whole
    calls between HIP events on the library's stream:
      muon:   the full-precision Muon step of one worker (worker 0's
              gradients, its own momentum, the workload's Newton-Schulz
              settings, W <- fmaf(-eta, U, W) on a copy of W);
      signum: majority-vote signum with momentum, i.e. the whole step with
              k = 0, over all the workload's workers."""
    import torch
    stream = torch.cuda.current_stream().cuda_stream
    mom_t = torch.bfloat16 if wl.mom_dtype == "bf16" else torch.float32
    norm = sm.NORM_SPECTRAL if wl.norm == "spectral" else sm.NORM_FROBENIUS
    s_g = 4 if wl.grad_dtype == "f32" else 2
    s_m = 4 if wl.mom_dtype == "f32" else 2
    mfma_peak = PEAK_BF16_TFLOPS if wl.ns_dtype == "bf16" else PEAK_FP32_TFLOPS

    def timed(call):
        ev = [hip.event() for _ in range(2)]
        call()
        total = 0.0
        for _ in range(reps):
            hip.record(ev[0], stream)
            call()
            hip.record(ev[1], stream)
            hip.sync(ev[1])
            total += hip.elapsed_ms(ev[0], ev[1])
        for e in ev:
            hip.destroy(e)
        return total / reps

    out = {}
    if wl.ns_iters >= 1:
        one = [sm.Matrix(grad=m.grad[0:1], momentum=torch.zeros((1,) + m.shape, dtype=mom_t, device=dev),
                         weight=m.weight.clone()) for m in mats]
        p1 = sm.Params(workers=1, beta=wl.beta, eta=wl.eta, ns_iters=wl.ns_iters,
                       grad_dtype=code[wl.grad_dtype], mom_dtype=code[wl.mom_dtype],
                       ns_dtype=code[wl.ns_dtype], norm=norm, power_iters=wl.power_iters)
        ws1 = sm.workspace_tensor(one, p1, dev)
        muon = sm.Prepared(one, p1, ws1)
        ms = timed(muon.muon_step)
        flops = sum(3 * min(R, C) ** 2 * max(R, C) for R, C in wl.shapes) * wl.ns_iters
        out["muon"] = {"workers": 1, "ms_per_step": round(ms, 5),
                       "params_per_s": round(wl.params / (ms * 1e-3), 1),
                       "ns_flops": int(flops),
                       "step_mfma_frac": round(flops / (ms * 1e-3) / (mfma_peak * 1e12), 4)}
        del one, ws1, muon
    p0 = sm.Params(workers=wl.workers, beta=wl.beta, eta=wl.eta, ns_iters=0,
                   grad_dtype=code[wl.grad_dtype], mom_dtype=code[wl.mom_dtype],
                   ns_dtype=code[wl.ns_dtype])
    ws0 = sm.workspace_tensor(mats, p0, dev)
    signum = sm.Prepared(mats, p0, ws0)
    ms = timed(signum.step)
    traces = [sm.Trace([hip.event() for _ in range(16)]) for _ in range(reps)]
    for tr in traces:
        signum.step_traced(tr)
    torch.cuda.synchronize()
    kinds_ms, _ = traced_kernel_ms(sm, hip, traces)
    for tr in traces:
        for e in list(tr._events):
            hip.destroy(e)
    mw, n = wl.workers, wl.params
    # momentum (G read, M read and written) with the signs packed in the same pass, then the
    # vote (the packed bits read, W read and written)
    nbytes = mw * n * (s_g + 2 * s_m + 1 / 8) + n * (mw / 8 + 8)
    gbs = nbytes / (ms * 1e-3) / 1e9
    out["signum"] = {"workers": mw, "ms_per_step": round(ms, 5),
                     "params_per_s": round(n / (ms * 1e-3), 1),
                     "algorithmic_bytes": int(nbytes), "achieved": round(gbs, 1), "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "kernels_ms": {k: round(v, 5) for k, v in kinds_ms.items()}}
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl, js=(0, 1, 2, 3), others=True):
    """The oracle, single-threaded, on a bounded sample of the workload: the
    matrices js (for GPT-2 small, the four matrices of one transformer layer)
    with all workers, one full step each (momentum, normalisation,
    Newton-Schulz, sign/pack, vote, update)."""
    import numpy as np

    import oracle
    import synthetic
    ns = oracle.BF16 if wl.ns_dtype == "bf16" else oracle.F32
    js = [j for j in js if j < len(wl.shapes)]
    total_s, params = 0.0, 0
    # one core: the oracle is single-threaded; pin the process to the core it
    # runs on for the timed calls, and restore the affinity afterwards
    saved = os.sched_getaffinity(0)
    core = min(saved)
    os.sched_setaffinity(0, {core})
    for j in js:
        R, C = wl.shapes[j]
        g = synthetic.gradients(wl, j, 0)
        m = np.zeros((wl.workers, R, C), np.uint16 if wl.mom_dtype == "bf16" else np.float32)
        w = synthetic.initial_weight(wl, j)
        t0 = time.perf_counter()
        oracle.step_matrix(g, m, w, wl.beta, wl.eta, wl.ns_iters, ns, post_k=wl.post_polar_iters,
                       norm=oracle.NORM_SPECTRAL if wl.norm == "spectral" else oracle.NORM_FROB,
                       power_iters=wl.power_iters)
        total_s += time.perf_counter() - t0
        params += R * C
    other = cpu_baseline_other(wl, js, total_s) if others else None
    os.sched_setaffinity(0, saved)
    shapes = ", ".join(f"{wl.shapes[j][0]}x{wl.shapes[j][1]}" for j in js)
    out = {"value": params / total_s, "unit": "params/s", "cores": 1, "kind": "oracle",
           "cpu_model": cpu_model(), "host_threads": len(saved), "pinned_core": core,
           "sample": f"{wl.name} matrices {js[0]}-{js[-1]} ({shapes}; {params} params), all "
                     f"{wl.workers} workers, one full step each: {total_s:.1f} s single-threaded "
                     f"on this host's CPU"}
    if other is not None:
        out["other_configs"] = other
    return out


def oracle_multiply_adds(wl):
    """Multiply-adds of the oracle's Newton-Schulz for one whole step (it
    forms the whole Gram matrix: 2 r^2 c per worker, matrix and iteration)."""
    return sum(2 * min(R, C) ** 2 * max(R, C) for R, C in wl.shapes) * wl.workers * wl.ns_iters


def cpu_baseline_other(wl_main, js_main, main_s):
    """The oracle (one core, the caller pins it) on the other configurations:
    whole steps where they take seconds (the 256x256 and ResNet-50 k = 1
    workloads), and, for the three that would take minutes to hours,
    extrapolations from measured samples, labelled as such."""
    import numpy as np

    import oracle
    import synthetic

    def full_step(name):
        wl = synthetic.WORKLOADS[name]
        ns = oracle.BF16 if wl.ns_dtype == "bf16" else oracle.F32
        t = 0.0
        for j, (R, C) in enumerate(wl.shapes):
            g = synthetic.gradients(wl, j, 0)
            m = np.zeros((wl.workers, R, C), np.uint16 if wl.mom_dtype == "bf16" else np.float32)
            w = synthetic.initial_weight(wl, j)
            t0 = time.perf_counter()
            oracle.step_matrix(g, m, w, wl.beta, wl.eta, wl.ns_iters, ns)
            t += time.perf_counter() - t0
        return {"params_per_s": wl.params / t, "seconds_per_step": round(t, 3), "kind": "measured",
                "sample": f"one whole step ({len(wl.shapes)} matrices, {wl.workers} workers)"}

    out = {n: full_step(n) for n in ("square256_mw4_k1", "resnet50_4shapes_mw4_k1")}
    # GPT-2 shapes with 16 workers and 5 iterations: the main sample's layer of
    # the same shapes (all 8 workers, k = 1) scaled by layers, workers and k
    for name in ("gpt2s_mw16_k5_t3",):
        wl = synthetic.WORKLOADS[name]
        layers = len(wl.shapes) / len(js_main)
        t = main_s * layers * (wl.workers / wl_main.workers) * (wl.ns_iters / wl_main.ns_iters)
        out[name] = {"params_per_s": wl.params / t, "seconds_per_step": round(t, 1),
                     "kind": "extrapolated",
                     "sample": f"the measured {wl_main.name} layer ({main_s:.1f} s for the same four "
                               f"shapes, {wl_main.workers} workers, k = {wl_main.ns_iters}) scaled "
                               f"linearly by {layers:.0f} layers, {wl.workers} workers and "
                               f"k = {wl.ns_iters}"}
    # the transformer block: one worker's Newton-Schulz on a 512 x 4096 slab of
    # its gradient (k = 1), scaled by the oracle's multiply-adds
    wl = synthetic.WORKLOADS["block4096_mw16_k5"]
    g = synthetic.gradient(wl, 0, 0, 0)[:512]
    m = np.zeros(g.shape, np.uint16)
    t0 = time.perf_counter()
    oracle.momentum(g, m, wl.beta)
    x0 = oracle.normalise(m)[1]
    oracle.newton_schulz(x0, 1, oracle.BF16)
    dt = time.perf_counter() - t0
    rate = 2 * 512 * 512 * 4096 / dt
    t = oracle_multiply_adds(wl) / rate
    out[wl.name] = {"params_per_s": wl.params / t, "seconds_per_step": round(t, 1),
                    "kind": "extrapolated",
                    "sample": f"one worker's momentum and Newton-Schulz (k = 1) on a 512x4096 slab "
                              f"of a 4096x4096 gradient: {dt:.1f} s, {rate / 1e9:.2f} G multiply-adds/s; "
                              f"the whole step's {oracle_multiply_adds(wl):.3g} Newton-Schulz "
                              f"multiply-adds at that rate"}
    for v in out.values():
        v["params_per_s"] = round(v["params_per_s"], 1)
    return out


def library_source_hash():
    """sha256 over the library's kernel and host sources (csrc/, sorted)."""
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "sign_muon_step_amd", "csrc")
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            with open(os.path.join(d, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def counter_traffic(wl, kind):
    """HBM bytes per step of kernel kind `kind` (all its launches in a step)
    from the committed rocprofv3 counter summary of this workload (FETCH_SIZE
    and WRITE_SIZE, each scaled by the factor a plain copy kernel gives the
    same counter). None when there is no summary or the library sources
    changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{wl.name}.md")
    if not os.path.exists(path):
        return None
    fields, rows = {}, {}
    with open(path) as f:
        for line in f:
            parts = line.split()
            if len(parts) == 2 and parts[0] in ("source_sha256", "fetch_factor", "write_factor"):
                fields[parts[0]] = parts[1]
            elif len(parts) == 4 and parts[0] == "kind":
                rows[parts[1]] = (float(parts[2]), float(parts[3]))
    if fields.get("source_sha256") != library_source_hash():
        return None
    if kind not in rows:
        return None
    fetch_kib, write_kib = rows[kind]
    return int(1024 * (fetch_kib * float(fields["fetch_factor"]) +
                       write_kib * float(fields["write_factor"])))


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sign_muon_step_amd as sm
    import synthetic

    wl = synthetic.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    code = {"f32": sm.F32, "bf16": sm.BF16}
    mom_t = torch.bfloat16 if wl.mom_dtype == "bf16" else torch.float32

    log(f"[bench] generating {wl.name}: {len(wl.shapes)} matrices, {wl.params} params, "
        f"{wl.workers} workers")
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=16) as ex:
        grads = list(ex.map(lambda j: synthetic.gradients(wl, j, 0), range(len(wl.shapes))))
    mats = []
    for j, (R, C) in enumerate(wl.shapes):
        mats.append(sm.Matrix(
            grad=torch.from_numpy(grads[j]).to(dev),
            momentum=torch.zeros((wl.workers, R, C), dtype=mom_t, device=dev),
            packed=torch.zeros((wl.workers, sm.signmuon_packed_words(R * C)), dtype=torch.int64,
                               device=dev),
            weight=torch.from_numpy(synthetic.initial_weight(wl, j)).to(dev)))
        grads[j] = None
    params = sm.Params(workers=wl.workers, beta=wl.beta, eta=wl.eta, ns_iters=wl.ns_iters,
                       post_polar_iters=wl.post_polar_iters, grad_dtype=code[wl.grad_dtype],
                       mom_dtype=code[wl.mom_dtype], ns_dtype=code[wl.ns_dtype],
                       norm=sm.NORM_SPECTRAL if wl.norm == "spectral" else sm.NORM_FROBENIUS,
                       power_iters=wl.power_iters)
    ws = sm.workspace_tensor(mats, params, dev)
    torch.cuda.synchronize()
    log(f"[bench] inputs resident in HBM after {time.perf_counter() - t0:.1f} s; workspace "
        f"{0 if ws is None else ws.numel() / 2**20:.0f} MiB")

    if args.calibrate_copy_mib:
        src = torch.ones(args.calibrate_copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy kernel: {args.calibrate_copy_mib} MiB read, "
            f"{args.calibrate_copy_mib} MiB written")
        del src, dst

    hip = Hip()
    cap = 64
    traces = [sm.Trace([hip.event() for _ in range(cap)]) for _ in range(args.steps)]

    # buffers checked and marshalled once, as an optimizer keeps them across steps
    step = sm.Prepared(mats, params, ws)
    for _ in range(args.warmup):
        step.step()
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps done; timing {args.steps} steps")

    t0 = time.perf_counter()
    for i in range(args.steps):
        step.step_traced(traces[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / args.steps

    # per-kernel time per step, from the events around each launch
    per_kind_ms, launch_count = traced_kernel_ms(sm, hip, traces)
    launches = traces[0].launches
    # each step's own duration: its first event to its last
    step_ms = sorted(hip.elapsed_ms(tr._events[0], tr._events[tr.launches]) for tr in traces)
    ms_median = step_ms[len(step_ms) // 2]
    for tr in traces:
        for e in list(tr._events):
            hip.destroy(e)

    work = work_per_kind(wl)
    mfma_peak = PEAK_BF16_TFLOPS if wl.ns_dtype == "bf16" else PEAK_FP32_TFLOPS
    kernels = kernel_table(wl, per_kind_ms)
    dominant = max((k for k in kernels if "bound" in kernels[k]), key=lambda k: kernels[k]["ms"])
    d = kernels[dominant]
    roofline = {"bound": d["bound"], "achieved": d["achieved"],
                "peak": PEAK_HBM_GBS if d["bound"] == "hbm" else mfma_peak, "unit": d["unit"],
                "frac": d["frac"], "traffic": counter_traffic(wl, dominant), "kernel": dominant,
                "launches_per_step": launch_count.get(dominant, 0), "per": "step"}
    ns_ms = per_kind_ms.get("ns_gram", 0.0) + per_kind_ms.get("ns_product", 0.0)
    ns_flops = work["ns_gram"][1] + work["ns_product"][1]
    ns_util = 100.0 * ns_flops / (ns_ms * 1e-3) / (mfma_peak * 1e12) if ns_ms > 0 else None
    vote_gbs = kernels.get("vote_update", {}).get("achieved")

    int8 = comparison = others = pack = None
    if not args.no_extras:
        log("[bench] timing the step with the int8 payload")
        int8 = time_int8_payload(sm, mats, wl, code, hip, dev)
        log("[bench] timing the comparison steps (Muon, one worker; majority-vote signum)")
        comparison = time_comparison_steps(sm, mats, wl, code, hip, dev)
        log("[bench] timing the other configurations")
        del step, ws, mats
        torch.cuda.empty_cache()
        others = time_other_configs(sm, hip, dev)
        log("[bench] timing the standalone sign + pack")
        pack = time_standalone_pack(sm, wl, hip, dev)

    base = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        base = cpu_baseline(wl, others=not args.no_extras)

    params_per_s = wl.params / (ms_per_step * 1e-3)
    out = {
        "metric": METRIC, "value": round(params_per_s, 1), "unit": "params/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.ns_dtype, "data": "synthetic",
        "config": {"workload": wl.name, "description": wl.description,
                   "matrices": len(wl.shapes), "params": wl.params, "workers": wl.workers,
                   "ns_iters": wl.ns_iters, "post_polar_iters": wl.post_polar_iters,
                   "grad_dtype": wl.grad_dtype, "momentum_dtype": wl.mom_dtype,
                   "ns_dtype": wl.ns_dtype, "weight_dtype": "f32", "norm": wl.norm,
                   "power_iters": wl.power_iters},
        "ms_per_step_median": round(ms_median, 4),
        "steps_per_s": round(1e3 / ms_per_step, 2),
        "worker_params_per_s": round(params_per_s * wl.workers, 1),
        "ns_mfma_util_pct": None if ns_util is None else round(ns_util, 2),
        "vote_update_hbm_gbs": vote_gbs,
        "kernels_ms_per_step": kernels,
        "launches_per_step": launches,
        "int8_payload": int8,
        "comparison_steps": comparison,
        "other_configs": others,
        "standalone_sign_pack": pack,
        "roofline": roofline,
        "cpu_baseline": base,
    }
    log("[bench] " + ", ".join(f"{k} {v['ms']:.3f} ms" + (f" ({v['frac'] * 100:.1f}% of "
                                                          f"{v['bound']})" if "frac" in v else "")
                               for k, v in kernels.items()))
    if int8:
        log(f"[bench] int8 payload: step {int8['ms_per_step']:.3f} ms" +
            (f", vote_update_int8 {int8['vote_update_int8']['ms']:.3f} ms "
             f"({int8['vote_update_int8']['frac'] * 100:.1f}% of hbm)" if "vote_update_int8" in int8 else ""))
    if comparison:
        log("[bench] comparison steps: " + ", ".join(f"{k} {v['ms_per_step']:.3f} ms per step"
                                                     for k, v in comparison.items()))
    print(json.dumps(out), flush=True)
    del np


if __name__ == "__main__":
    main()
