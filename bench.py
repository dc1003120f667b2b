"""Benchmark of the fused W8A8 MoE expert block on one MI355X.

One step = one call of moe_w8a8_forward (routing, quantisation, GEMM1 with
SwiGLU, requantisation, GEMM2, combine, shared expert) over one batch of the
DeepSeek-V4-Flash-shaped decode workload: T = 8 token rows, hidden 4096,
expert intermediate 2048, 256 routed experts resident, top-8, one shared
expert of intermediate 2048, int8 weights with fp32 per-channel scales.

Inputs are resident in HBM before timing. The routed and shared weights are
held in `--layers` copies at distinct addresses and step i uses copy
i % layers, as consecutive MoE layers of a model would, so every step streams
its experts' weights from HBM rather than from the 256 MB last-level cache.

Prints one JSON line: the metric (µs per MoE layer), the achieved HBM GB/s of
the layer, the roofline of the dominant kernel (GEMM1) from HIP events bound
to that kernel's launch (hipExtLaunchKernel) in every timed step, and the CPU
oracle's time on this host as a baseline. Memory-bound GEMMs are also set
against measured ceilings: a read probe with their weight-stream pattern
(moe_w8a8_read_probe) and, for batches past decode, whose GEMMs write tens
of MB of output rows while their weights stream, a probe of each GEMM's own
read and write bytes (moe_w8a8_read_write_probe).

`--weight-format mxfp4` times the FP4-weight / FP8-activation variant of the
same workload instead (E2M1 weights with E8M0 block scales, 0.53 bytes per
weight element), `--quant-group G` the variant with one activation scale per
row and group of G elements; the default line is the INT8 block with one
scale per row.
"""
from __future__ import annotations

import argparse
import ctypes
import dataclasses
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import moe_expert_ffn_route_amd as moe  # noqa: E402
from moe_expert_ffn_route_amd import binding, synth  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_I8_PEAK_TOPS = 5000.0  # MI355X dense int8 matrix rate, published (no sparsity)
MFMA_F8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 matrix rate, published (an FP8 x FP4 product runs at it)
MFMA_I8_OPS_PER_CLK_CU = 8192  # the per-CU rate at which 256 CUs at 2.4 GHz reach the published figure
HIP_ATTR_CLOCK_RATE = 5  # hipDeviceAttributeClockRate (peak clock, kHz) in hip_runtime_api.h
START_GATE_CYCLES = 2_000_000  # about 1 ms of a one-thread sleep kernel (see start_gate)


def start_gate(stream, enabled=True):
    """Enqueue a bounded one-thread sleep kernel (torch.cuda._sleep, about
    1 ms) on `stream` ahead of a timed region's start event. The GPU is idle
    after the synchronisation that opens the region, so without it the start
    event would fire at once and the region would also time the host's
    latency to enqueue the first step; with it the host has enqueued the
    first steps by the time the start event fires, and the region times the
    device running the K steps back to back. Returns whether it gated (False
    when disabled or when this torch build has no sleep kernel)."""
    sleep = getattr(torch.cuda, "_sleep", None)
    if not enabled or sleep is None:
        return False
    with torch.cuda.stream(stream):
        sleep(START_GATE_CYCLES)
    return True


def log(*a):
    print(*a, file=sys.stderr, flush=True)


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence in hip_runtime_api.h
_hip_rt = None


def hip_runtime() -> ctypes.CDLL:
    """The HIP runtime torch has loaded (the same library instance, so its
    events and streams are shared with torch and libmoe_w8a8)."""
    global _hip_rt
    if _hip_rt is None:
        torch.cuda.init()
        with open("/proc/self/maps") as f:
            paths = [ln.split()[-1] for ln in f if "libamdhip64" in ln]
        if not paths:
            raise RuntimeError("the HIP runtime is not loaded")
        _hip_rt = ctypes.CDLL(paths[0])
        P = ctypes.c_void_p
        _hip_rt.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(P), ctypes.c_uint]
        _hip_rt.hipEventRecord.argtypes = [P, P]
        _hip_rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), P, P]
        _hip_rt.hipEventDestroy.argtypes = [P]
        _hip_rt.hipStreamWaitEvent.argtypes = [P, P, ctypes.c_uint]
    return _hip_rt


class TimingEvent:
    """A HIP event used only for timing, created with hipEventDisableSystemFence
    so that recording it (or binding it to a kernel launch) adds no
    system-scope cache writeback and invalidation to the stream. The host reads
    results only after a device synchronisation, so nothing relies on the
    fence. Offers what this file uses of torch.cuda.Event: record(stream),
    elapsed_time(end) in ms and the raw handle `cuda_event`."""

    def __init__(self, fence_free: bool = True):
        rt = hip_runtime()
        h = ctypes.c_void_p()
        flags = HIP_EVENT_DISABLE_SYSTEM_FENCE if fence_free else 0
        if rt.hipEventCreateWithFlags(ctypes.byref(h), flags) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
        self.cuda_event = h.value

    def record(self, stream):
        if hip_runtime().hipEventRecord(self.cuda_event, stream.cuda_stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end: "TimingEvent") -> float:
        ms = ctypes.c_float()
        if hip_runtime().hipEventElapsedTime(ctypes.byref(ms), self.cuda_event, end.cuda_event) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def __del__(self):
        if _hip_rt is not None and self.cuda_event:
            _hip_rt.hipEventDestroy(self.cuda_event)


def weight_bytes_per_element(spec) -> float:
    """1 for INT8 weights; 1/2 + 1/32 for FP4 elements with one E8M0 scale per 32."""
    return 0.5 + 1.0 / 32 if spec.weight_format == "mxfp4" else 1.0


def algorithmic_bytes(case, counts):
    """Bytes the layer must move at least once: every touched expert's weights
    and scales, the shared expert's, the activations in and out."""
    s = case.spec
    H, I, Is, T, K = s.H, s.I, s.I_s, s.T, s.K
    wb = weight_bytes_per_element(s)
    touched = int((counts > 0).sum())
    per_expert = int(3 * H * I * wb) + 4 * (2 * I + H)
    shared = (int(3 * H * Is * wb) + 4 * (2 * Is + H)) if Is else 0
    act = 2 * T * H + 8 * T * K + 2 * T * H * (2 if Is else 1)
    if case.smooth is not None:
        act += 4 * s.E_loc * H
    gemm1 = touched * (int(2 * I * H * wb) + 8 * I) + ((int(2 * Is * H * wb) + 8 * Is) if Is else 0)
    routed_rows = int(counts.sum())
    t_act = T if case.mask is None else int(np.count_nonzero(case.mask))
    rows = routed_rows + (t_act if Is else 0)
    G = getattr(s, "quant_group", 0)
    ngx, ngh = (H // G, max(I, Is) // G) if G else (1, 1)  # activation scales per row
    gemm1 += rows * (H + 4 * ngx + 4 * max(I, Is))  # q_x and its scales read, h written
    gemm2 = touched * (int(H * I * wb) + 4 * H) + ((int(H * Is * wb) + 4 * H) if Is else 0)
    gemm2 += routed_rows * (I + 4 * ngh + 2 * H) + ((t_act * (Is + 4 * ngh + 2 * H)) if Is else 0)  # q_h, hs in; z out
    return touched * per_expert + shared + act, gemm1, gemm2, touched, rows


def gemm_write_bytes(case, counts):
    """Bytes each GEMM writes (part of its algorithmic bytes): GEMM1 the fp32 h
    rows (4 * max(I, I_s) per grouped row), GEMM2 the bf16 z rows and shared
    output rows (2 * H per routed row and per active token)."""
    s = case.spec
    routed = int(counts.sum())
    t_act = s.T if case.mask is None else int(np.count_nonzero(case.mask))
    rows = routed + (t_act if s.I_s else 0)
    return rows * 4 * max(s.I, s.I_s), rows * 2 * s.H


def layer_ops(case, counts):
    """Integer multiply-adds (x2) of the two GEMMs: 2 * rows * 3 * H * I for
    the routed rows and the same with I_s for the shared rows."""
    s = case.spec
    routed = int(counts.sum())
    t_act = s.T if case.mask is None else int(np.count_nonzero(case.mask))
    return 2 * 3 * s.H * (routed * s.I + (t_act * s.I_s if s.I_s else 0))


def gemm_ops(case, counts):
    """Integer operations (2 per multiply-add) of GEMM1 and of GEMM2 over the
    real rows: rows x 2I x H and rows x H x I, with I_s for the shared rows."""
    s = case.spec
    routed = int(counts.sum())
    t_act = s.T if case.mask is None else int(np.count_nonzero(case.mask))
    sh = t_act * s.I_s if s.I_s else 0
    return 2 * 2 * s.H * (routed * s.I + sh), 2 * s.H * (routed * s.I + sh)


def mfma_peak_on_device():
    """int8 MFMA peak re-derived from the device: CUs x peak clock x the
    per-CU rate; None when the clock cannot be read."""
    props = torch.cuda.get_device_properties(0)
    for name in ("libamdhip64.so", "/opt/rocm/lib/libamdhip64.so"):
        try:
            hip = ctypes.CDLL(name)
            break
        except OSError:
            hip = None
    if hip is None:
        return None
    khz = ctypes.c_int(0)
    if hip.hipDeviceGetAttribute(ctypes.byref(khz), HIP_ATTR_CLOCK_RATE, torch.cuda.current_device()) != 0:
        return None
    if not 500_000 <= khz.value <= 5_000_000:
        return None
    cus = props.multi_processor_count
    return {"cus": cus, "clock_mhz": khz.value / 1e3,
            "tops": round(cus * khz.value * 1e3 * MFMA_I8_OPS_PER_CLK_CU / 1e12, 1)}


READ_PROBE_BYTES = 8 << 30  # 32x the 256 MB memory-side cache, so the probe's own ramp and tail are < 1 %


def hbm_read_probe(stream, fence_free, reps=5):
    """The HBM read rate this device reaches: moe_w8a8_read_probe (the GEMMs'
    weight-stream access pattern, nothing else) over an 8 GiB range, one
    untimed pass, then `reps` timed passes (HIP events on the launch stream).
    Returns the median GB/s and the passes' figures."""
    buf = torch.empty(READ_PROBE_BYTES, dtype=torch.uint8, device="cuda")  # contents are never used
    evs = [TimingEvent(fence_free) for _ in range(reps + 1)]
    with torch.cuda.stream(stream):
        moe.moe_w8a8_read_probe(buf, stream=stream)
        for i in range(reps):
            evs[i].record(stream)
            moe.moe_w8a8_read_probe(buf, stream=stream)
        evs[reps].record(stream)
    torch.cuda.synchronize()
    gbs = [READ_PROBE_BYTES / (evs[i].elapsed_time(evs[i + 1]) * 1e-3) / 1e9 for i in range(reps)]
    del buf
    return {"gbps": round(float(np.median(gbs)), 1), "passes_gbps": [round(g, 1) for g in gbs],
            "bytes": READ_PROBE_BYTES, "entry_point": "moe_w8a8_read_probe",
            "pattern": "1 KB contiguous per wave load, non-temporal, 8 loads in flight per wave, whole chip"}


def hbm_read_write_probe(stream, fence_free, read_bytes, write_bytes, reps=5):
    """The time a GEMM's byte mix takes on this device: moe_w8a8_read_write_probe
    reads `read_bytes` (rounded down to whole 256 KB work items, the time scaled
    back up) with the larger-batch GEMMs' weight-stream pattern and writes
    `write_bytes` in equal shares at the items' ends, as those GEMMs write their
    output rows. One untimed pass, then `reps` timed passes; returns the median
    time in µs and the passes' figures."""
    item = 256 * 1024
    src_bytes = (read_bytes // item) * item
    dst_bytes = min((write_bytes // 16) * 16, src_bytes)
    src = torch.empty(src_bytes, dtype=torch.uint8, device="cuda")  # contents are never used
    dst = torch.empty(max(16, dst_bytes), dtype=torch.uint8, device="cuda")
    evs = [TimingEvent(fence_free) for _ in range(reps + 1)]
    with torch.cuda.stream(stream):
        moe.moe_w8a8_read_write_probe(src, src_bytes, dst, dst_bytes, stream=stream)
        for i in range(reps):
            evs[i].record(stream)
            moe.moe_w8a8_read_write_probe(src, src_bytes, dst, dst_bytes, stream=stream)
        evs[reps].record(stream)
    torch.cuda.synchronize()
    us = [evs[i].elapsed_time(evs[i + 1]) * 1e3 * read_bytes / src_bytes for i in range(reps)]
    del src, dst
    return {"us": round(float(np.median(us)), 2), "passes_us": [round(u, 2) for u in us],
            "read_bytes": read_bytes, "write_bytes": write_bytes, "entry_point": "moe_w8a8_read_write_probe"}


def gemm_traffic(workload, kernel_prefix):
    """HBM bytes per launch of the kernel whose name starts with
    `kernel_prefix`, from the committed rocprofv3 counter summary of this
    workload (read requests counted by size, 32 / 64 / 128 bytes; write
    bytes from WRITE_SIZE), or None when there is none or when a source file
    it lists has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"gemm_hbm_traffic__{workload}.md")
    if not os.path.exists(path):
        return None
    rec = None
    with open(path) as f:
        for line in f:
            if line.startswith("TRAFFIC_JSON: "):
                rec = json.loads(line[len("TRAFFIC_JSON: "):])
    if rec is None:
        return None
    h = hashlib.sha256()
    for name in rec.get("sources", []):
        with open(os.path.join(ROOT, "moe_expert_ffn_route_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    if not rec.get("sources") or h.hexdigest() != rec.get("source_sha256"):
        return None
    for k, v in rec["kernels"].items():
        if k.startswith(kernel_prefix):
            return int(v["read_bytes"] + v["write_bytes"])
    return None


def gemm1_kernel_prefix(case, mx):
    """Name prefix of the GEMM1 kernel the library picks for this batch (the
    work-item rules of the C ABI: 16-row items up to 16 tokens; FP4 weights
    and group-wise scales 32-row items when the local experts can average 16
    rows, on the two-tile kernels; otherwise 256-row tall items when they can
    average 256 rows, else 32-row wide items)."""
    s = case.spec
    grp = getattr(s, "quant_group", 0)
    rows_per_expert = s.T * s.K // s.ep_size
    if s.T <= 16:
        return "void gemm_mx_kernel<1," if mx else "void gemm_kernel<1,"
    if mx or grp:
        two_tiles = rows_per_expert >= 16 * s.E_loc
        if mx:
            return "void gemm_mx_wide_kernel<1," if two_tiles else "void gemm_mx_kernel<1,"
        return "void gemm_wide_kernel<1," if two_tiles else "void gemm_kernel<1,"
    if s.T >= 256 and rows_per_expert >= 256 * s.E_loc:
        return "void gemm_tall_kernel<1,"
    return "void gemm_wide_kernel<1,"


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(case, budget_s=12.0, max_reps=40, tokens=None, threads=1):
    """The CPU oracle as it stands, on the same batch (or on `tokens` of it):
    single-threaded, or with the tokens split over `threads` host threads
    (each running the unchanged single-threaded C forward on its subset).
    Returns (mean µs per run, runs, output of the last run)."""
    import oracle  # test infrastructure: only this leg of the benchmark uses it
    oracle.lib()
    times = []
    out = None
    t_end = time.perf_counter() + budget_s
    while len(times) < max_reps and (not times or time.perf_counter() < t_end):
        t0 = time.perf_counter()
        out = oracle.forward(case, tokens=tokens, threads=threads)
        times.append(time.perf_counter() - t0)
    return float(np.mean(times)) * 1e6, len(times), out


class Leg:
    """Resident inputs of one workload: weight copies (shared with another leg
    where the model is the same), activations, and a Runner."""

    def __init__(self, case, layers, dims):
        self.case, self.layers, self.dims = case, layers, dims
        self.runner = moe.Runner(dims)


def measure(leg, steps, warmup, stream, fence_free, kernel_events=True, graphs=None, after_step=None, gate=True):
    """Time `steps` forwards of one leg (step i on weight copy i % copies).
    Returns µs per step, GEMM1 / GEMM2 kernel durations from events bound to
    their launches, per-stage times (marker events, separate pass) and the
    per-step distribution (one marker per step boundary, separate pass).
    after_step(i), if given, is called after step i is enqueued (in every
    pass). gate: open the timed region and the per-step pass with start_gate."""
    runner, layers = leg.runner, leg.layers
    hook = after_step or (lambda i: None)
    n_ev = len(binding.STAGES) + 1
    events = [[TimingEvent(fence_free) for _ in range(n_ev)] for _ in range(steps)]
    kevents = [[TimingEvent(fence_free) for _ in range(4)] for _ in range(steps)]
    for evs in events + kevents:
        for e in evs:
            e.record(stream)  # materialise the HIP event handles
    torch.cuda.synchronize()
    # timed region: the library binds two events to the GEMM1 launch itself
    # (its start and end); the per-stage pass below records a marker event
    # between every two stages and binds GEMM2's pair (GEMM1 only in the timed
    # region: each bound event costs a few µs of the step)
    k_arrays = [(ctypes.c_void_p * 4)(evs[0].cuda_event, evs[1].cuda_event, None, None) for evs in kevents]
    k2_arrays = [(ctypes.c_void_p * 4)(None, None, evs[2].cuda_event, evs[3].cuda_event) for evs in kevents]
    all_arrays = [(ctypes.c_void_p * n_ev)(*[e.cuda_event for e in evs]) for evs in events]
    k_dbg = [binding.Debug(kernel_events=ctypes.cast(p, ctypes.c_void_p).value) for p in k_arrays]
    all_dbg = [binding.Debug(stage_events=ctypes.cast(p, ctypes.c_void_p).value,
                             kernel_events=ctypes.cast(q, ctypes.c_void_p).value)
               for p, q in zip(all_arrays, k2_arrays)]

    with torch.cuda.stream(stream):
        for i in range(warmup):
            runner(layers[i % len(layers)], stream=stream)
            hook(i)
    torch.cuda.synchronize()
    if graphs:
        for i in range(warmup):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()

    t_start = TimingEvent(fence_free)
    t_stop = TimingEvent(fence_free)
    torch.cuda.synchronize()
    gated = start_gate(stream, gate)
    with torch.cuda.stream(stream):
        t_start.record(stream)
        for i in range(steps):
            if graphs:
                graphs[i % len(graphs)].replay()
            else:
                runner(layers[i % len(layers)], dbg=k_dbg[i] if kernel_events else None, stream=stream)
            hook(i)
        t_stop.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_stop) / steps
    g1_us = None
    if kernel_events and not graphs:
        g1_us = float(np.mean([kevents[i][0].elapsed_time(kevents[i][1]) for i in range(steps)])) * 1e3

    with torch.cuda.stream(stream):
        for i in range(steps):
            runner(layers[i % len(layers)], dbg=all_dbg[i], stream=stream)
            hook(i)
    torch.cuda.synchronize()
    stage_us = {name: float(np.mean([events[i][j].elapsed_time(events[i][j + 1]) for i in range(steps)]) * 1e3)
                for j, name in enumerate(binding.STAGES)}
    g2_us = float(np.mean([kevents[i][2].elapsed_time(kevents[i][3]) for i in range(steps)])) * 1e3
    timing = "kernel-bound HIP events in the timed steps"
    if g1_us is None:
        g1_us = stage_us["gemm1"]
        timing = "marker HIP events between stages (per-stage pass)"
    timing += ", hipEventDisableSystemFence" if fence_free else ", default event flags"
    timing += ", region opened behind a 1 ms sleep kernel" if gated else ", region opened on an idle GPU"

    bounds = [TimingEvent(fence_free) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    start_gate(stream, gate)
    with torch.cuda.stream(stream):
        bounds[0].record(stream)
        for i in range(steps):
            if graphs:
                graphs[i % len(graphs)].replay()
            else:
                runner(layers[i % len(layers)], stream=stream)
            hook(i)
            bounds[i + 1].record(stream)
    torch.cuda.synchronize()
    step_samples = [bounds[i].elapsed_time(bounds[i + 1]) * 1e3 for i in range(steps)]
    p10, p50, p90 = (float(v) for v in np.percentile(step_samples, [10, 50, 90]))
    out = runner.output.float()
    if not torch.isfinite(out).all():
        raise RuntimeError("non-finite output")
    return dict(us=ms_per_step * 1e3, ms_per_step=ms_per_step, g1_us=g1_us, g2_us=g2_us, stage_us=stage_us,
                p=(p10, p50, p90), timing=timing, counts=runner.expert_token_nums.cpu().numpy())


def large_batch_record(base_case, layers, wkeys, weight_layout, steps, warmup, stream, fence_free, gate=True):
    """The T = 512 half of the metric: the large-batch workload (same model as
    the decode workload, so the resident weight copies are reused; only the
    512 tokens' activations are generated), timed like the decode step.
    Returns the record's fields: µs per layer, int8 TOP/s over the layer and
    its fraction of the MFMA peak, the layer's algorithmic GB/s, and each
    GEMM's kernel-bound duration with its algorithmic HBM bandwidth."""
    spec4 = synth.WORKLOADS[4]
    s1 = base_case.spec
    assert (spec4.weight_seed, spec4.H, spec4.I, spec4.E_g, spec4.I_s) == (s1.weight_seed, s1.H, s1.I, s1.E_g, s1.I_s)
    case4 = synth.make_case(spec4, weights=(base_case.w1, base_case.w1s, base_case.w2, base_case.w2s))
    act = moe.upload(case4, weights={k: layers[0][k] for k in wkeys})
    legs = [dict(act, **{k: lay[k] for k in wkeys}) for lay in layers]
    dims4 = moe.dims_of_case(case4)
    dims4.weight_layout = weight_layout
    leg = Leg(case4, legs, dims4)
    m = measure(leg, steps, warmup, stream, fence_free, gate=gate)
    counts = m["counts"]
    layer_bytes, g1_bytes, g2_bytes, touched, rows = algorithmic_bytes(case4, counts)
    g1_write, g2_write = gemm_write_bytes(case4, counts)
    g1_ops, g2_ops = gemm_ops(case4, counts)
    us = m["us"]
    tops = layer_ops(case4, counts) / (us * 1e-6) / 1e12
    return {
        "workload": spec4.name, "tokens": spec4.T, "touched_experts": touched, "grouped_rows": rows,
        "us_per_layer": round(us, 2),
        "step_us_p10_p50_p90": [round(v, 2) for v in m["p"]],
        "tops": round(tops, 1), "mfma_i8_frac": round(tops / MFMA_I8_PEAK_TOPS, 4),
        "hbm_gbps": round(layer_bytes / (us * 1e-6) / 1e9, 1),
        "hbm_frac": round(layer_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "gemm1": {"avg_us": round(m["g1_us"], 2), "algorithmic_bytes": g1_bytes, "write_bytes": g1_write,
                  "achieved_gbps": round(g1_bytes / (m["g1_us"] * 1e-6) / 1e9, 1),
                  "hbm_frac": round(g1_bytes / (m["g1_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                  "tops": round(g1_ops / (m["g1_us"] * 1e-6) / 1e12, 1),
                  "traffic": gemm_traffic(spec4.name, gemm1_kernel_prefix(case4, False))},
        "gemm2": {"avg_us": round(m["g2_us"], 2), "algorithmic_bytes": g2_bytes, "write_bytes": g2_write,
                  "achieved_gbps": round(g2_bytes / (m["g2_us"] * 1e-6) / 1e9, 1),
                  "hbm_frac": round(g2_bytes / (m["g2_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                  "tops": round(g2_ops / (m["g2_us"] * 1e-6) / 1e12, 1)},
        "stage_us": {k: round(v, 2) for k, v in m["stage_us"].items()},
        "timing": m["timing"],
        "bound": "hbm (about 36 int8 operations per weight byte, far below the MFMA ridge of about 625)",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1, help="must be 1: the block runs on one GPU")
    ap.add_argument("--steps", type=int, default=50, help="timed steps (one forward each)")
    ap.add_argument("--warmup", type=int, default=10, help="untimed steps before the timed region")
    ap.add_argument("--config", type=int, default=1,
                    help="workload index (0-4; 1 is the headline decode step; 5 is the supplementary "
                         "compute-bound probe)")
    ap.add_argument("--layers", type=int, default=4, help="weight copies cycled through to keep the cache cold")
    ap.add_argument("--row-major", action="store_true",
                    help="stream the weights in their row-major layout instead of the packed one")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip timing the CPU oracle (cpu_baseline and cpu_baseline_all_cores)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB 5 times (calibrates HBM byte counters)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one step per weight copy into HIP graphs and time their replays")
    ap.add_argument("--fuse-route-scale", action="store_true",
                    help="fold the routing weight into the GEMM2 row scale (combine only sums)")
    ap.add_argument("--requant-in-epilogue", type=int, choices=[0, 1], default=0,
                    help="1: requantise h in GEMM1's epilogue (last-arriving workgroup per chunk) instead of a "
                         "launch of its own (decode batches)")
    ap.add_argument("--weight-format", choices=["int8", "mxfp4"], default="int8",
                    help="mxfp4: FP4 weights with E8M0 block scales and FP8 activations (always packed)")
    ap.add_argument("--quant-group", type=int, default=0, choices=[0, 64, 128, 256],
                    help="group-wise activation scales (quant_mode 2) with groups of this many elements")
    ap.add_argument("--fenced-events", action="store_true",
                    help="time with default HIP events (each record adds a system-scope cache writeback) "
                         "instead of events created with hipEventDisableSystemFence")
    ap.add_argument("--warm-next-shared", action="store_true",
                    help="after each layer, warm the next layer's shared-expert GEMM1 weights on a second stream "
                         "(moe_w8a8_warm), overlapping that layer's routing launch")
    ap.add_argument("--no-large-batch", action="store_true",
                    help="skip the T = 512 leg (large_batch_t512) of the default decode line")
    ap.add_argument("--no-start-gate", action="store_true",
                    help="start the timed region on an idle GPU (the region then also times the host's latency "
                         "to enqueue the first step) instead of behind a 1 ms sleep kernel")
    ap.add_argument("--no-kernel-events", action="store_true",
                    help="time the steps without the GEMM kernel events (GEMM times then come from the "
                         "per-stage pass)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(expert parallelism across GPUs is not part of this library)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        n = args.copy_probe << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n, "copy_probe_bytes_written": n, "launches": 5}), flush=True)
        return
    moe.library()  # fail loudly if the HIP library is missing

    spec = synth.WORKLOADS[args.config]
    mx = args.weight_format == "mxfp4"
    if mx:
        if args.row_major:
            print("--weight-format mxfp4 needs packed weights", file=sys.stderr)
            sys.exit(2)
        spec = dataclasses.replace(spec, name=spec.name + "_mxfp4", weight_format="mxfp4")
    if args.quant_group:
        if mx:
            print("--quant-group applies to INT8 weights", file=sys.stderr)
            sys.exit(2)
        spec = dataclasses.replace(spec, name=f"{spec.name}_g{args.quant_group}", quant_group=args.quant_group)
    log(f"[bench] workload {spec.name}: generating inputs")
    t0 = time.perf_counter()
    case = synth.make_case(spec) if (mx or args.quant_group) else synth.workload_case(args.config)
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f}s; uploading")
    dev = moe.upload(case)  # FP4 weights are packed by upload (moe_w8a8_pack_weights_mx)
    if not args.row_major and not mx:
        dev = moe.pack_weights(dev)  # one-time re-layout at load time (moe_w8a8_pack_weights)
        torch.cuda.synchronize()
    wkeys = [k for k in ("gmm1_weight", "gmm1_weight_scale", "gmm2_weight", "gmm2_weight_scale",
                         "share_gmm1_weight", "share_gmm1_weight_scale", "share_gmm2_weight",
                         "share_gmm2_weight_scale") if dev.get(k) is not None]
    layers = [dev] + [dict(dev, **{k: dev[k].clone() for k in wkeys}) for _ in range(max(0, args.layers - 1))]
    dims = moe.dims_of_case(case)
    dims.weight_layout = moe.MOE_WEIGHT_ROW_MAJOR if args.row_major else moe.MOE_WEIGHT_PACKED
    dims.weight_format = moe.MOE_WEIGHT_MXFP4 if mx else moe.MOE_WEIGHT_INT8
    dims.fuse_route_scale = int(args.fuse_route_scale)
    dims.requant_in_epilogue = args.requant_in_epilogue
    leg = Leg(case, layers, dims)
    runner = leg.runner
    stream = torch.cuda.Stream()
    fence_free = not args.fenced_events

    graphs = []
    if args.graph:
        # one graph per weight copy; the GEMM1 events of the timed region are
        # not recorded inside graphs (stage times come from the per-stage pass)
        with torch.cuda.stream(stream):
            runner(layers[0], stream=stream)
        torch.cuda.synchronize()
        for li in range(len(layers)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                runner(layers[li], stream=stream)
            graphs.append(g)
        torch.cuda.synchronize()

    after_step = None
    if args.warm_next_shared:
        if not spec.I_s or graphs:
            print("--warm-next-shared needs a shared expert and stream launches", file=sys.stderr)
            sys.exit(2)
        # after layer i is enqueued, a second stream waits for it and warms
        # layer i + 1's shared-expert GEMM1 weights and scales, which then
        # overlap layer i + 1's routing launch (HBM otherwise idle)
        # (fence-free events: the warm only reads weights, so the wait orders
        # launches and needs no cache writeback; a default event's record
        # would add one per step)
        side = torch.cuda.Stream()
        marks = [TimingEvent(fence_free) for _ in range(len(layers))]

        def after_step(i):
            nxt = layers[(i + 1) % len(layers)]
            ev = marks[i % len(layers)]
            ev.record(stream)
            if hip_runtime().hipStreamWaitEvent(side.cuda_stream, ev.cuda_event, 0) != 0:
                raise RuntimeError("hipStreamWaitEvent failed")
            moe.moe_w8a8_warm(nxt["share_gmm1_weight"], stream=side)
            moe.moe_w8a8_warm(nxt["share_gmm1_weight_scale"], stream=side)
    log(f"[bench] warmup {args.warmup} steps, timing {args.steps} steps (three passes)")
    m = measure(leg, args.steps, args.warmup, stream, fence_free, kernel_events=not args.no_kernel_events,
                graphs=graphs, after_step=after_step, gate=not args.no_start_gate)
    counts = m["counts"]
    g1_us, g2_us, stage_us, timing = m["g1_us"], m["g2_us"], m["stage_us"], m["timing"]
    p10, p50, p90 = m["p"]
    ms_per_step = m["ms_per_step"]

    layer_bytes, gemm1_bytes, gemm2_bytes, touched, rows = algorithmic_bytes(case, counts)
    us = ms_per_step * 1e3
    g1_gbs = gemm1_bytes / (g1_us * 1e-6) / 1e9
    traffic = None if args.row_major else gemm_traffic(spec.name, gemm1_kernel_prefix(case, mx))
    tops = layer_ops(case, counts) / (us * 1e-6) / 1e12
    g1_ops, g2_ops = gemm_ops(case, counts)
    # the roofline that binds GEMM1: HBM below the ridge (peak ops / peak
    # bytes per second), the int8 MFMA rate above it
    mfma_peak = MFMA_F8_PEAK_TFLOPS if mx else MFMA_I8_PEAK_TOPS
    mfma_unit = "TFLOP/s (fp8 x fp4)" if mx else "TOP/s (int8)"
    if g1_ops / gemm1_bytes > mfma_peak * 1e12 / (HBM_PEAK_GBS * 1e9):
        g1_tops = g1_ops / (g1_us * 1e-6) / 1e12
        roofline = {"kernel": "gemm1_swiglu", "bound": "mfma", "achieved": round(g1_tops, 1),
                    "peak": mfma_peak, "unit": mfma_unit, "frac": round(g1_tops / mfma_peak, 4),
                    "traffic": traffic, "algorithmic_ops": g1_ops, "algorithmic_bytes": gemm1_bytes,
                    "hbm_gbps": round(g1_gbs, 1), "avg_us": round(g1_us, 2), "timing": timing}
    else:
        roofline = {"kernel": "gemm1_swiglu", "bound": "hbm", "achieved": round(g1_gbs, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(g1_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "algorithmic_bytes": gemm1_bytes, "avg_us": round(g1_us, 2), "timing": timing}
    log("[bench] HBM read probe")
    read_probe = hbm_read_probe(stream, fence_free)
    if roofline["bound"] == "hbm":
        roofline["measured_peak"] = read_probe["gbps"]
        roofline["frac_of_measured_peak"] = round(g1_gbs / read_probe["gbps"], 4)
    gemm2_rec = {"achieved": round(gemm2_bytes / (g2_us * 1e-6) / 1e9, 1), "unit": "GB/s",
                 "algorithmic_bytes": gemm2_bytes, "avg_us": round(g2_us, 2),
                 "tops": round(g2_ops / (g2_us * 1e-6) / 1e12, 1)}
    if spec.T > 16 and roofline["bound"] == "hbm":
        # batches past decode write tens of MB of output rows while their
        # weights stream: each GEMM is also set against a probe of its own
        # read and write bytes
        log("[bench] read-write probes (each GEMM's byte mix)")
        for rec_g, total, w, g_us in ((roofline, gemm1_bytes, gemm_write_bytes(case, counts)[0], g1_us),
                                      (gemm2_rec, gemm2_bytes, gemm_write_bytes(case, counts)[1], g2_us)):
            rw = hbm_read_write_probe(stream, fence_free, total - w, w)
            rec_g["write_bytes"] = w
            rec_g["read_write_probe"] = rw
            rec_g["frac_of_read_write_probe"] = round(rw["us"] / g_us, 4)
    headline = args.config == 1 and not mx and not args.quant_group
    rec = {
        "metric": ("µs per MoE layer (T=8 decode); achieved HBM GB/s in hbm_gbps; INT8 TOP/s at T=512 in "
                   "large_batch_t512.tops") if headline else "µs per MoE layer; achieved HBM GB/s in hbm_gbps",
        "value": round(us, 2),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3 x fp4e2m1 (fp32 accumulate)" if mx else "int8",
        "data": "synthetic",
        "config": {"workload": spec.name, "tokens": spec.T, "hidden": spec.H, "inter": spec.I,
                   "experts": spec.E_g, "topk": spec.K, "share_inter": spec.I_s,
                   "touched_experts": touched, "grouped_rows": rows, "weight_copies": len(layers),
                   "weight_layout": "row_major" if args.row_major else "packed",
                   "weight_format": args.weight_format,
                   "activation_scales": f"per row and {args.quant_group} elements" if args.quant_group else "per row",
                   "route_scale": "fused_gemm2" if args.fuse_route_scale else "combine",
                   "requant": "gemm1_epilogue" if args.requant_in_epilogue and spec.T <= 16 else "own_launch",
                   "launch": "hip_graph" if graphs else "stream",
                   "warm_next_shared": bool(args.warm_next_shared)},
        "hbm_gbps": round(layer_bytes / (us * 1e-6) / 1e9, 1),
        "tokens_per_s": round(spec.T / (us * 1e-6), 1),
        "step_us_p10_p50_p90": [round(p10, 2), round(p50, 2), round(p90, 2)],  # one event per step boundary
        "tops": round(tops, 2),
        "mfma_i8_frac": None if mx else round(tops / MFMA_I8_PEAK_TOPS, 5),
        "mfma_i8_peak_derived": mfma_peak_on_device(),
        "hbm_read_probe": read_probe,
        "stage_us": {k: round(v, 2) for k, v in stage_us.items()},  # separate pass, every stage bracketed
        "roofline": roofline,
        "gemm2": gemm2_rec,
    }
    if headline and not args.no_large_batch and not graphs:
        log("[bench] large-batch leg (T = 512, same resident weights)")
        rec["large_batch_t512"] = large_batch_record(case, layers, wkeys, dims.weight_layout, args.steps,
                                                     args.warmup, stream, fence_free,
                                                     gate=not args.no_start_gate)
        for g in ("gemm1", "gemm2"):
            lb = rec["large_batch_t512"][g]
            lb["frac_of_measured_peak"] = round(lb["achieved_gbps"] / read_probe["gbps"], 4)
            # the same byte mix (reads, and the writes among the algorithmic
            # bytes) as a probe: the ceiling for a kernel that must write its
            # output rows while its weights stream
            w = lb["write_bytes"]
            rw = hbm_read_write_probe(stream, fence_free, lb["algorithmic_bytes"] - w, w)
            lb["read_write_probe"] = rw
            lb["frac_of_read_write_probe"] = round(rw["us"] / lb["avg_us"], 4)
    if args.no_cpu_baseline:
        rec["cpu_baseline"] = None
    else:
        log("[bench] CPU oracle baseline")
        if mx:
            # the FP4 oracle is slower per product: two tokens, scaled to the batch
            n_tok = min(2, spec.T)
            cpu_us, reps, _ = cpu_baseline(case, tokens=list(range(n_tok)))
            cpu_us *= spec.T / max(1, n_tok)
            sample = (f"tokens 0-{n_tok - 1} of this workload (routing of the whole batch), {reps} runs, "
                      f"time scaled by {spec.T}/{n_tok} to the batch, single-threaded C oracle")
        else:
            cpu_us, reps, ref1 = cpu_baseline(case)
            sample = f"the full batch of this workload, {reps} runs, single-threaded C oracle"
        rec["cpu_baseline"] = {"value": round(cpu_us, 1), "unit": "us", "cores": 1, "kind": "oracle",
                               "sample": sample, "host_cpu": host_cpu_model(),
                               "host_threads_available": os.cpu_count()}
        if not mx:
            # the same oracle on every host thread: tokens split over threads
            # (one token per thread at most, so a batch of T tokens uses at
            # most T threads); bit-identical to the single-threaded run
            n_thr = max(1, min(os.cpu_count() or 1, spec.T))
            cpu_all, reps_all, ref_all = cpu_baseline(case, budget_s=6.0, threads=n_thr)
            for k in ("output", "share_output", "expert_token_nums"):
                a, b = ref1[k], ref_all[k]
                if (a is None) != (b is None) or (a is not None and not np.array_equal(a, b)):
                    raise RuntimeError(f"threaded oracle differs from the single-threaded run in {k}")
            rec["cpu_baseline_all_cores"] = {
                "value": round(cpu_all, 1), "unit": "us", "cores": n_thr, "kind": "oracle",
                "sample": (f"the full batch of this workload, {reps_all} runs, tokens split over {n_thr} host "
                           "threads, each running the single-threaded C oracle; output bit-identical to the "
                           "single-threaded run"),
                "host_cpu": host_cpu_model(), "host_threads_available": os.cpu_count()}
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
