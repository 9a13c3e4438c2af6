#!/usr/bin/env python3
"""Benchmark of the MI355X selective scan: one JSON line on stdout.

A step is one fused selective-scan forward (ssm_scan_fwd) over the
Mamba-130M-shaped layer: batch 8, L 2048, D 1536 (d_model 768 x expand 2),
N 16, bf16 inputs and output, fp32 state, SiLU(z) gate, D skip, dt bias with
softplus, zero-order-hold discretization.  Inputs are resident in HBM before
the timed region; three independent input sets (203 MB each) rotate from step
to step so that the 256 MB Infinity Cache cannot serve a step from the previous
one.  Before the warm-up steps the scan runs back to back, untimed, for about
100 ms, long enough for the GPU clock to settle under load (it ramps up over
the first ~30 ms), so the timed steps see the steady state.  `value` is
algorithmic bytes per step / measured step time.

Also reported, outside `value`: the same scan under the exponential-Euler rule,
the extended scan (initial state, lengths, document resets), the backward pass,
the block's convolution (sequence and decoding step), the Mamba-2 / SSD layer
on the matrix cores, the scan on the Mamba-1.4B and long-sequence layers,
the decode step (ssm_step) on its
workload (batch 256, D 5120, N 16, 1000 consecutive tokens), the kernel
roofline for the dominant kernel, and the fp64 CPU oracle timed on the host.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu]

For profilers (rocprofv3) a reduced mode runs a few launches of one kernel on
one input set and prints no JSON:
    python bench.py --only scan [--dt-mode zoh|euler] [--launches 3] [--kernel wave]
    python bench.py --only decode [--launches 3]
    python bench.py --only conv [--launches 3]
    python bench.py --only ssd [--launches 3]
    python bench.py --only bwd [--dt-mode zoh|euler] [--launches 3]   # the backward, Mamba-130M layer
    python bench.py --only train [--launches 3]  # the forward keeping checkpoints, then the backward from them
    python bench.py --only tpar [--launches 3]   # the time-parallel scan with four waves per row, forced, Mamba-130M layer at batch 1
    python bench.py --only seq [--launches 3]    # the sequential scan (2 states per lane), forced, Mamba-130M layer
    python bench.py --only copy     # a plain 256 MiB device copy, for counter calibration
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
# ALU roofline of the scan.  Per state update the method does 2 multiplies and
# 2 FMAs (6 flops: Delta A, (Delta u) B, the state FMA, the readout FMA) and one
# exponential.  MI355X has 256 CUs of 4 SIMDs x 16 fp32 lanes at 2.4 GHz:
# 39.3e12 fp32 lane-instructions per second, i.e. 78.6 TFLOP/s counting an FMA
# as 2 flops.  The published 157.3 TFLOP/s needs packed fp32 (two FMAs per
# lane-instruction), which this build turns off, so the roofline's peak is 78.6.
VALU_LANE_OPS = 256 * 4 * 16 * 2.4e9
FP32_TFLOPS = 2 * VALU_LANE_OPS / 1e12
FP32_PUBLISHED_TFLOPS = 157.3
FLOPS_PER_UPDATE = 6
# The fewest VALU instructions a state update needs besides its exponential:
# Euler: Delta*A', (Delta u)*B, the state FMA, the readout FMA; ZOH adds the
# (abar - 1) factor (an FMA) and the 1/A weight (a multiply) of the input term.
VALU_PER_UPDATE = {"zoh": 6, "euler": 4}
METRIC = "selective-scan fwd achieved HBM GB/s (% of peak) and B·L·D elems/s; decode tok/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def scan_bytes(b, L, D, N, io_bytes, gate):
    """Algorithmic bytes of one scan: every input read once, y and the final
    state written once (u, raw delta, [z], y: b L D; B, C: b L N; A: D N fp32;
    D, bias: D fp32 each; last_state: b D N fp32)."""
    streamed = 3 if gate else 2
    return (streamed + 1) * b * L * D * io_bytes + 2 * b * L * N * io_bytes + 4 * D * N + 8 * D \
        + 4 * b * D * N


def step_bytes(b, D, N, io_bytes, gate):
    """Algorithmic bytes of one decode step: state read + written (fp32), u, raw
    delta, [z] read and y written (b D), B, C (b N), A (D N), D and bias (D)."""
    streamed = 3 if gate else 2
    return 8 * b * D * N + (streamed + 1) * b * D * io_bytes + 2 * b * N * io_bytes + 4 * D * N + 8 * D


def alu_rates(dev, blocks=2048, iters=4096, reps=7):
    """Measured issue rates of the chip (the library's probe kernels): fp32 FMA
    and v_exp_f32 lane-operations per second, and the issue slots one
    exponential takes inside a stream of FMAs (8 exponentials and 32 FMAs per
    iteration, against the FMA-only rate).  blocks x 256 lanes fill every
    SIMD with 8 waves; each probe is timed with HIP events on torch's current
    stream (where the library launches), median of `reps` launches."""
    import torch
    import selective_state_space_66_amd as ssm
    sink = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    lanes = blocks * 256
    ms = {}
    for op in ("fma", "exp", "mix"):
        ssm.alu_probe(op, sink, blocks, iters)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            a.record()
            ssm.alu_probe(op, sink, blocks, iters)
            b.record()
        torch.cuda.synchronize()
        ms[op] = float(np.median([a.elapsed_time(b) for a, b in ev]))
    n = lanes * iters
    fma = 8 * n / (ms["fma"] * 1e-3)
    exp = 8 * n / (ms["exp"] * 1e-3)
    exp_slots = (ms["mix"] * 1e-3 * fma / n - 32) / 8
    return {"fma_lane_ops_per_s": float(f"{fma:.4g}"), "exp_lane_ops_per_s": float(f"{exp:.4g}"),
            "exp_slots_in_fma_stream": round(exp_slots, 3),
            "fma_frac_of_nominal": round(fma / VALU_LANE_OPS, 4),
            "probe_ms": {k: round(v, 4) for k, v in ms.items()},
            "probe": f"{blocks} blocks x 256 lanes x {iters} iterations of 8 FMAs, 8 exponentials, "
                     "or 8 x (exponential + 4 FMAs); 8 independent chains per lane"}


def alu_figures(updates, ms, mode, rates):
    """The scan's compute position: the method's flops per second against the
    fp32 FMA peak (and the published packed-fp32 peak), and the kernel time
    against the measured ALU floor -- the fewest VALU instructions per update
    plus one exponential at its measured cost, issued at the measured FMA rate."""
    tflops = FLOPS_PER_UPDATE * updates / (ms * 1e-3) / 1e12
    out = {"TFLOPs": round(tflops, 3), "frac_fp32": round(tflops / FP32_TFLOPS, 4),
           "frac_published_fp32": round(tflops / FP32_PUBLISHED_TFLOPS, 4)}
    if rates:
        slots = VALU_PER_UPDATE[mode] + rates["exp_slots_in_fma_stream"]
        floor_ms = updates * slots / rates["fma_lane_ops_per_s"] * 1e3
        out["floor"] = {"slots_per_update": round(slots, 3), "floor_ms": round(floor_ms, 5),
                        "frac": round(floor_ms / ms, 4)}
    return out


# The sources each measured kernel is built from: its own file, plus the shared
# device and launch headers and the C-ABI file that picks its launch shape.
KERNEL_SOURCES = {
    "scan_fwd_mamba130m_zoh": ["scan_fwd.hip", "scan_tpar.hip", "scan_wave8.hip", "ssm_wave8.h"],
    "step_decode_zoh": ["step.hip"],
    "conv1d_fwd_conv130m": ["conv1d.hip"],
    "ssd_fwd_ssd130m": ["ssd.hip"],
    "conv1d_bwd_conv130m": ["conv1d.hip"],
    "scan_bwd_mamba130m_zoh": ["scan_bwd.hip", "scan_bwd_wave.hip", "ssm_bwd.h"],
}
COMMON_SOURCES = ["ssm_device.h", "ssm_launch.h", "ssm_api.hip"]


def kernel_source_hash(kernel_key):
    """Hash of the sources the kernel `kernel_key` is built from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "selective_state_space_66_amd", "csrc")
    for f in sorted(KERNEL_SOURCES[kernel_key] + COMMON_SOURCES):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the kernel's current sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(kernel_key)
    if not ent or ent.get("source_hash") != kernel_source_hash(kernel_key):
        return None
    return ent.get("bytes_per_launch")


def to_dev(x, io, dev):
    import torch
    if x is None:
        return None
    if io == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dev)


def launched_scan_kernel(name, io):
    """The one kernel a forward call without lengths or document starts runs,
    from the library's name for its layout and the call's io type: the 16-lane
    layout takes eight tokens per lane for bf16 io, four otherwise; from 8192
    rows the eight-token kernel takes the bf16 calls it fits."""
    split = "scan_wave8_kernel (time-parallel, 16 lanes per row, 8 tokens per lane) for bf16 io"
    if name.startswith(split):
        return name[:name.index(" for bf16 io")] if io == "bf16" else name.split(", else ", 1)[1]
    if name.startswith("scan_wave8_kernel / scan_wave_kernel"):
        tpl = 8 if io == "bf16" else 4
        return (f"{'scan_wave8_kernel' if tpl == 8 else 'scan_wave_kernel'} "
                f"(time-parallel, 16 lanes per row, {tpl} tokens per lane)")
    return name


def upload_scan(inp, dev):
    io = inp["io"]
    return dict(u=to_dev(inp["u"], io, dev), delta=to_dev(inp["delta"], io, dev),
                A=to_dev(inp["A"], "f32", dev), B=to_dev(inp["B"], io, dev),
                C=to_dev(inp["C"], io, dev), D=to_dev(inp["D"], "f32", dev),
                z=to_dev(inp["z"], io, dev), delta_bias=to_dev(inp["delta_bias"], "f32", dev))


def time_scan(sets, steps, warmup, dt_mode, extras=None, stats=False, kernel=None):
    """Run warmup steps, then `steps` timed by the wall clock (bracketed by
    device synchronisations), then `steps` more with HIP events around each
    launch, rotating over the input sets.  Returns (wall ms per step, mean
    per-launch kernel ms from the events), and with `stats` also the median
    and the minimum of the per-launch times.  `extras` (h0, seq_lens, reset)
    selects the extended scan."""
    import torch
    import selective_state_space_66_amd as ssm
    outs = [(torch.empty_like(s["u"]), torch.empty(s["u"].shape[0], s["u"].shape[2], s["A"].shape[1],
                                                    dtype=torch.float32, device=s["u"].device))
            for s in sets]
    ex = extras or {}

    def launch(i):
        s = sets[i % len(sets)]
        y, last = outs[i % len(sets)]
        ssm.scan_fwd(s["u"], s["delta"], s["A"], s["B"], s["C"], D=s["D"], z=s["z"],
                     delta_bias=s["delta_bias"], softplus=True, dt_mode=dt_mode, y=y,
                     last_state=last, kernel=kernel, **ex)

    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    # wall time of `steps` back-to-back steps, nothing else on the stream
    t0 = time.perf_counter()
    for i in range(steps):
        launch(warmup + i)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    # then the same steps again with HIP events around each launch (kernel time)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        launch(warmup + steps + i)
        ev[i][1].record()
    torch.cuda.synchronize()
    times = [a.elapsed_time(b) for a, b in ev]
    kern = float(np.mean(times))
    if stats:
        return wall, kern, float(np.median(times)), float(np.min(times))
    return wall, kern


def settle_clock(sets, ms=100.0):
    """Launch the ZOH scan back to back, untimed, for about `ms` milliseconds.
    Under sustained load the GPU's clock ramps up over the first tens of
    milliseconds: on this layer the scan went from about 210 to 182.5 us per
    launch over its first ~140 launches (30 ms) and then held there.  Running
    this before the warm-up steps makes the timed steps measure the steady
    state, whatever the warm-up count.  Returns the number of launches."""
    import torch
    import selective_state_space_66_amd as ssm
    outs = [(torch.empty_like(s["u"]), torch.empty(s["u"].shape[0], s["u"].shape[2], s["A"].shape[1],
                                                    dtype=torch.float32, device=s["u"].device))
            for s in sets]
    n = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(20):
            s = sets[n % len(sets)]
            y, last = outs[n % len(sets)]
            ssm.scan_fwd(s["u"], s["delta"], s["A"], s["B"], s["C"], D=s["D"], z=s["z"],
                         delta_bias=s["delta_bias"], softplus=True, dt_mode="zoh", y=y,
                         last_state=last)
            n += 1
        torch.cuda.synchronize()
    return n


def time_narrow(dev, steps, warmup, rates=None):
    """The scan where (batch x channel) rows are few, so the sequential kernel
    leaves most of the GPU idle: the pages' speed-benchmark shape (batch 1,
    L 2048, D 1024, N 16), the Mamba-130M layer at batch 1 (1 x 2048 x 1536)
    and a long narrow sequence (1 x 65536 x 128), bf16, gate, ZOH.  Timed
    with the library's own choice (a time-parallel scan) and with the
    sequential kernel forced, for comparison."""
    import workloads as W
    import selective_state_space_66_amd as ssm
    out = {}
    shapes = (("paper_speed_benchmark", (1, 2048, 1024)), ("mamba130m_batch1", (1, 2048, 1536)),
              ("long_narrow", (1, 65536, 128)))
    for name, (b, L, D) in shapes:
        cfg = W.ScanConfig(name, b, L, D, 16, "bf16", True, 7)
        sets = [upload_scan(W.scan_inputs(cfg), dev)]
        res = {}
        for label, kern in (("auto", None), ("sequential", "seq1")):
            res[label] = time_scan(sets, steps, warmup, "zoh", kernel=kern)[1]
        upd = b * L * D * 16
        out[name] = {"workload": f"ssm_scan_fwd: batch {b}, L {L}, D {D}, N 16, bf16, gate, ZOH",
                     "kernel": launched_scan_kernel(ssm.scan_kernel_name(b, L, D, 16), "bf16"),
                     "kernel_ms": round(res["auto"], 5),
                     "sequential_kernel_ms": round(res["sequential"], 5),
                     "speedup": round(res["sequential"] / res["auto"], 2),
                     "alu": alu_figures(upd, res["auto"], "zoh", rates)}
        del sets
    return out


def time_layers(dev, steps, warmup, rates=None):
    """The scan forward on the two larger layers of the workload set, ZOH and
    exponential-Euler: the Mamba-1.4B-shaped layer (8 x 2048 x 4096, N 16,
    bf16, gate) and the long-sequence selective-copying-like case (4 x 65536 x
    2048, N 16, bf16, no gate), on the seeded inputs the parity tests check.
    Each input set is far larger than the 256 MB Infinity Cache, so one set is
    reused from launch to launch."""
    import torch
    import workloads as W
    import selective_state_space_66_amd as ssm
    out = {}
    for name, nsteps in (("mamba1p4b", steps), ("longseq", max(10, steps // 4))):
        cfg = W.SCAN_CONFIGS[name]
        t0 = time.perf_counter()
        sets = [upload_scan(W.scan_inputs(cfg), dev)]
        torch.cuda.synchronize()
        log(f"[bench] {name}: inputs generated and uploaded in {time.perf_counter() - t0:.1f} s")
        _, kern, kmed, kmin = time_scan(sets, nsteps, max(2, warmup // 5), "zoh", stats=True)
        kern_e = time_scan(sets, nsteps, max(2, warmup // 5), "euler")[1]
        nbytes = scan_bytes(cfg.batch, cfg.L, cfg.dim, cfg.N, 2, cfg.gate)
        upd = cfg.batch * cfg.L * cfg.dim * cfg.N
        gbs = nbytes / (kern * 1e-3) / 1e9
        out[name] = {"workload": f"ssm_scan_fwd: batch {cfg.batch}, L {cfg.L}, D {cfg.dim}, N {cfg.N}, "
                                 f"bf16, {'gate' if cfg.gate else 'no gate'}, ZOH",
                     "kernel": launched_scan_kernel(ssm.scan_kernel_name(cfg.batch, cfg.L, cfg.dim, cfg.N),
                                                    cfg.io),
                     "launches": nsteps, "kernel_ms": round(kern, 5),
                     "kernel_ms_median": round(kmed, 5), "kernel_ms_min": round(kmin, 5),
                     "GB/s": round(gbs, 2),
                     "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
                     "elems_per_s": float(f"{cfg.batch * cfg.L * cfg.dim / (kern * 1e-3):.4g}"),
                     "updates_per_s": float(f"{upd / (kern * 1e-3):.4g}"),
                     "alu": alu_figures(upd, kern, "zoh", rates),
                     "algorithmic_bytes": nbytes,
                     "euler": {"kernel_ms": round(kern_e, 5),
                               "GB/s": round(nbytes / (kern_e * 1e-3) / 1e9, 2),
                               "pct_hbm_peak": round(100.0 * nbytes / (kern_e * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                               "updates_per_s": float(f"{upd / (kern_e * 1e-3):.4g}"),
                               "alu": alu_figures(upd, kern_e, "euler", rates)}}
        del sets
        torch.cuda.empty_cache()
    return out


def time_tiny(dev, steps=200):
    """The tiny fp32 workload (batch 1, L 256, D 64, N 16, no gate): launch-bound
    on the GPU; timed per launch with events, both rules."""
    import torch
    import workloads as W
    import selective_state_space_66_amd as ssm
    cfg = W.SCAN_CONFIGS["tiny"]
    inp = W.scan_inputs(cfg)
    s = upload_scan(inp, dev)
    out = {"workload": "ssm_scan_fwd: batch 1, L 256, D 64, N 16, fp32 io, no gate, D skip, "
                       "softplus(delta + bias)",
           "kernel": launched_scan_kernel(ssm.scan_kernel_name(cfg.batch, cfg.L, cfg.dim, cfg.N), cfg.io)}
    for mode in ("zoh", "euler"):
        out[mode] = {"kernel_us": round(time_scan([s], steps, 20, mode)[1] * 1e3, 2)}
    return out


def settle_launches(launch, ms=30.0):
    """Untimed launches of `launch(i)` for about `ms` milliseconds: workloads
    whose inputs are generated on the host just before find the clock lowered
    by the idle time, and it ramps up again under load (see settle_clock).
    Returns the number of launches."""
    import torch
    n = 0
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(20):
            launch(n)
            n += 1
        torch.cuda.synchronize()
    return n


def time_decode(cfg, nsteps, dev, npool=8, nstates=1):
    """ssm_step over nsteps consecutive tokens on the full state; the token inputs
    cycle through `npool` distinct seeded token batches resident in HBM.  With
    nstates > 1 the steps rotate over that many independent state caches (4 x
    84 MB exceed the 256 MB Infinity Cache, so every step streams its state
    from and to HBM)."""
    import torch
    import selective_state_space_66_amd as ssm
    import workloads as W
    A, D, bias = W.channel_params(cfg.seed, cfg.dim, cfg.N)
    Ad, Dd, bd = to_dev(A, "f32", dev), to_dev(D, "f32", dev), to_dev(bias, "f32", dev)
    states = [to_dev(W.step_state0(cfg), "f32", dev) for _ in range(nstates)]
    pool = []
    for s in range(npool):
        inp = W.step_inputs(cfg, s)
        pool.append({k: to_dev(inp[k], cfg.io, dev) for k in ("u", "delta", "B", "C", "z")})
    ys = [torch.empty_like(p["u"]) for p in pool]

    def one(i):
        p = pool[i % npool]
        ssm.step(states[i % nstates], p["u"], p["delta"], Ad, p["B"], p["C"], D=Dd, z=p["z"],
                 delta_bias=bd, y=ys[i % npool])

    for i in range(20):
        one(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(nsteps):
        one(i)
    e1.record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    return wall_s, e0.elapsed_time(e1) / nsteps


def time_bwd(sets, steps, warmup, dev):
    """ssm_scan_bwd on the Mamba-130M layer (ZOH, gate, D, bias), rotating the
    input sets, one dy per set; one workspace reused."""
    import torch
    import selective_state_space_66_amd as ssm
    s0 = sets[0]
    batch, L, dim = s0["u"].shape
    N = s0["A"].shape[1]
    ws = torch.empty(ssm.scan_bwd_workspace_size(batch, L, dim, N), dtype=torch.uint8, device=dev)
    gen = torch.Generator(device="cpu").manual_seed(12)
    dys = [torch.randn((batch, L, dim), generator=gen).to(torch.bfloat16).to(dev) for _ in sets]

    def launch(i):
        s = sets[i % len(sets)]
        ssm.scan_bwd(s["u"], s["delta"], s["A"], s["B"], s["C"], dys[i % len(sets)], D=s["D"],
                     z=s["z"], delta_bias=s["delta_bias"], workspace=ws)

    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        launch(warmup + i)
        ev[i][1].record()
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in ev])), ws.numel()


def time_train(sets, steps, warmup, dev):
    """The training path on the same layer: ssm_scan_fwd_ckpt (the forward that
    keeps the state every 16 tokens) and ssm_scan_bwd_ex from those checkpoints,
    rotating the input sets; returns (forward ms, backward ms) per launch."""
    import torch
    import selective_state_space_66_amd as ssm
    s0 = sets[0]
    batch, L, dim = s0["u"].shape
    N = s0["A"].shape[1]
    ws = torch.empty(ssm.scan_bwd_workspace_size(batch, L, dim, N), dtype=torch.uint8, device=dev)
    gen = torch.Generator(device="cpu").manual_seed(13)
    dys = [torch.randn((batch, L, dim), generator=gen).to(torch.bfloat16).to(dev) for _ in sets]
    outs = [ssm.scan_fwd_train(s["u"], s["delta"], s["A"], s["B"], s["C"], D=s["D"], z=s["z"],
                               delta_bias=s["delta_bias"]) for s in sets]

    def fwd(i):
        s, (y, last, ck) = sets[i % len(sets)], outs[i % len(sets)]
        ssm.scan_fwd_train(s["u"], s["delta"], s["A"], s["B"], s["C"], D=s["D"], z=s["z"],
                           delta_bias=s["delta_bias"], y=y, last_state=last, ckpt=ck)

    def bwd(i):
        s, (_, _, ck) = sets[i % len(sets)], outs[i % len(sets)]
        ssm.scan_bwd(s["u"], s["delta"], s["A"], s["B"], s["C"], dys[i % len(sets)], D=s["D"],
                     z=s["z"], delta_bias=s["delta_bias"], workspace=ws, ckpt=ck)

    res = []
    for launch in (fwd, bwd):
        for i in range(warmup):
            launch(i)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for i in range(steps):
            ev[i][0].record()
            launch(warmup + i)
            ev[i][1].record()
        torch.cuda.synchronize()
        res.append(float(np.mean([a.elapsed_time(b) for a, b in ev])))
    del outs, ws
    return res[0], res[1]


def ssd_bytes(b, L, H, P, N, gate):
    """Algorithmic bytes of the SSD layer (bf16 io): x, [z] read and y written
    once, B and C read once, dt (fp32) read once, A, D, dt_bias, and the final
    state written (fp32)."""
    return (3 if gate else 2) * b * L * H * P * 2 + 2 * b * L * N * 2 + 4 * b * L * H + 12 * H \
        + 4 * b * H * P * N


def ssd_mfma_flops(b, L, H, N):
    """MFMA work of the chunked SSD kernel (64-token chunks, 64 channels per
    head): the causal tiles of C B^T, C H^T, the masked scores times x, and the
    state update, as 16x16x32 products of 16384 flops."""
    chunks = b * H * ((L + 63) // 64)
    per_chunk = 10 * (N // 32) + 16 * (N // 32) + 24 + (4 * N // 16) * 2
    return chunks * per_chunk * 16384


def time_ssd(dev, steps, warmup, nsets=3):
    """The Mamba-2 / SSD layer (ssm_ssd_fwd) on the Mamba-2-130M shape, rotating
    input sets (3 x ~160 MB > the 256 MB Infinity Cache)."""
    import torch
    import selective_state_space_66_amd as ssm
    import workloads as W
    cfg = W.SSD_CONFIGS["ssd130m"]
    sets = []
    for k in range(nsets):
        c = W.SSDConfig(cfg.name, cfg.batch, cfg.L, cfg.nheads, cfg.P, cfg.N, cfg.io, cfg.gate,
                        cfg.seed + 100 * k)
        inp = W.ssd_inputs(c)
        sets.append({kk: to_dev(inp[kk], "f32" if kk in ("dt", "A", "D", "dt_bias") else "bf16", dev)
                     for kk in ("x", "z", "dt", "A", "D", "dt_bias", "B", "C")})
    out = {}
    for mode in ("euler", "zoh"):
        ys = [(torch.empty_like(s["x"]), torch.empty((cfg.batch, cfg.nheads, cfg.P, cfg.N),
                                                     dtype=torch.float32, device=dev)) for s in sets]

        def launch(i):
            s = sets[i % nsets]
            y, last = ys[i % nsets]
            ssm.ssd_fwd(s["x"], s["dt"], s["A"], s["B"], s["C"], D=s["D"], z=s["z"],
                        dt_bias=s["dt_bias"], dt_mode=mode, y=y, last_state=last)

        settle_launches(launch)
        for i in range(warmup):
            launch(i)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(steps)]
        for i in range(steps):
            ev[i][0].record()
            launch(warmup + i)
            ev[i][1].record()
        torch.cuda.synchronize()
        out[mode] = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    nb = ssd_bytes(cfg.batch, cfg.L, cfg.nheads, cfg.P, cfg.N, cfg.gate)
    fl = ssd_mfma_flops(cfg.batch, cfg.L, cfg.nheads, cfg.N)
    ms = out["euler"]
    return {"workload": f"ssm_ssd_fwd: batch {cfg.batch}, L {cfg.L}, {cfg.nheads} heads x {cfg.P}, "
                        f"N {cfg.N}, bf16, gate, D (Mamba-2-130M shape)",
            "kernel_ms": round(ms, 5), "zoh_kernel_ms": round(out["zoh"], 5),
            "roofline": {"bound": "hbm", "achieved": round(nb / (ms * 1e-3) / 1e9, 2),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes": nb, "traffic": measured_traffic("ssd_fwd_ssd130m")},
            "mfma": {"achieved_TFLOPs": round(fl / (ms * 1e-3) / 1e12, 2), "peak_TFLOPs": 2500.0,
                     "flops": fl}}


def conv_bwd_bytes(b, L, D, k, io_bytes):
    """Algorithmic bytes of the convolution's backward pass: x and dout read,
    dx written once; weights and bias read, their gradients written."""
    return 3 * b * L * D * io_bytes + 4 * D * (k + 1) * 2


def conv_bytes(b, L, D, k, io_bytes):
    """Algorithmic bytes of the sequence convolution: x read and out written once,
    the decoding window written, weights and bias read."""
    return 2 * b * L * D * io_bytes + b * (k - 1) * D * io_bytes + 4 * D * k + 4 * D


def time_conv(dev, steps, warmup, nsets=4):
    """The block's convolution on the Mamba-130M layer's input (bf16, k = 4),
    rotating `nsets` input sets (4 x 100 MB of x and out > the 256 MB Infinity
    Cache); and its decoding step on the decode workload's width (the window
    stays cache-resident across steps, as in a real decoding loop)."""
    import torch
    import selective_state_space_66_amd as ssm
    import workloads as W
    cfg = W.CONV_CONFIGS["conv130m"]
    sets = []
    for k in range(nsets):
        c = W.ConvConfig(cfg.name, cfg.batch, cfg.L, cfg.dim, cfg.k, cfg.io, cfg.seed + 100 * k)
        inp = W.conv_inputs(c)
        sets.append((to_dev(inp["x"], cfg.io, dev), to_dev(inp["w"], "f32", dev),
                     to_dev(inp["bias"], "f32", dev)))
    outs = [(torch.empty_like(x), torch.empty((cfg.batch, cfg.k - 1, cfg.dim), dtype=x.dtype,
                                              device=dev)) for x, _, _ in sets]

    def launch(i):
        x, w, b = sets[i % nsets]
        o, win = outs[i % nsets]
        ssm.conv1d_fwd(x, w, bias=b, out=o, window_out=win)

    settle_launches(launch)
    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        launch(warmup + i)
        ev[i][1].record()
    torch.cuda.synchronize()
    fwd_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))

    # the backward pass on the same layer: dout per set, one workspace
    gen = torch.Generator(device="cpu").manual_seed(14)
    douts = [torch.randn(x.shape, generator=gen).to(x.dtype).to(dev) for x, _, _ in sets]
    ws = torch.empty(ssm.conv1d_bwd_workspace_size(cfg.batch, cfg.L, cfg.dim, cfg.k),
                     dtype=torch.uint8, device=dev)

    def launch_bwd(i):
        x, w, b = sets[i % nsets]
        ssm.conv1d_bwd(x, w, douts[i % nsets], bias=b, workspace=ws)

    settle_launches(launch_bwd)
    for i in range(warmup):
        launch_bwd(i)
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record()
        launch_bwd(warmup + i)
        ev[i][1].record()
    torch.cuda.synchronize()
    bwd_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    bwd_b = conv_bwd_bytes(cfg.batch, cfg.L, cfg.dim, cfg.k, 2)

    dcfg = W.CONV_CONFIGS["conv_decode"]
    w, b = W.conv_params(dcfg.seed, dcfg.dim, dcfg.k)
    wd, bd = to_dev(w, "f32", dev), to_dev(b, "f32", dev)
    win = to_dev(W.conv_window0(dcfg), dcfg.io, dev)
    toks = [to_dev(W.conv_step_inputs(dcfg, s), dcfg.io, dev) for s in range(8)]
    o = torch.empty_like(toks[0])
    for i in range(20):
        ssm.conv1d_step(win, toks[i % 8], wd, bias=bd, out=o)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(dcfg.steps):
        ssm.conv1d_step(win, toks[i % 8], wd, bias=bd, out=o)
    e1.record()
    torch.cuda.synchronize()
    step_us = e0.elapsed_time(e1) / dcfg.steps * 1e3
    fwd_b = conv_bytes(cfg.batch, cfg.L, cfg.dim, cfg.k, 2)
    step_b = 8 * dcfg.batch * dcfg.dim * 2 + 4 * dcfg.dim * (dcfg.k + 1)
    return {"workload": f"ssm_conv1d_fwd: batch {cfg.batch}, L {cfg.L}, D {cfg.dim}, k {cfg.k}, "
                        "bf16, SiLU",
            "kernel_ms": round(fwd_ms, 5),
            "GB/s": round(fwd_b / (fwd_ms * 1e-3) / 1e9, 2),
            "hbm_frac": round(fwd_b / (fwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": fwd_b,
            "traffic": measured_traffic("conv1d_fwd_conv130m"),
            "step": {"workload": f"ssm_conv1d_step: batch {dcfg.batch}, D {dcfg.dim}, k {dcfg.k}, "
                                 "bf16, SiLU", "us_per_step": round(step_us, 3),
                     "GB/s": round(step_b / (step_us * 1e-6) / 1e9, 2)},
            "backward": {"workload": "ssm_conv1d_bwd on the same layer: dx, dweight, dbias "
                                     "(its finalize kernel included)",
                         "kernel_ms": round(bwd_ms, 5),
                         "GB/s": round(bwd_b / (bwd_ms * 1e-3) / 1e9, 2),
                         "hbm_frac": round(bwd_b / (bwd_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes": bwd_b,
                         "traffic": measured_traffic("conv1d_bwd_conv130m")}}


def copy_bandwidth(dev, nbytes=256 << 20, reps=20):
    """A plain device copy of nbytes (torch's copy kernel): read + write bytes per
    second, the practical HBM ceiling the kernels are compared with."""
    import torch
    x = torch.ones(nbytes // 2, dtype=torch.bfloat16, device=dev)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record()
        y.copy_(x)
        b.record()
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
    return 2 * nbytes / (ms * 1e-3) / 1e9


def host_facts():
    """The host the oracle runs on: CPU model, CPUs online, CPUs this process
    may use, and the threads the oracle takes (that share)."""
    import oracle
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {"cpu_model": model, "nproc": os.cpu_count(), "affinity_cpus": affinity,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "oracle_threads": oracle.host_threads()}


def _oracle_scan_seconds(inp, io, threads, mode="zoh"):
    import oracle
    import workloads as W
    f = lambda k: W.as_f64(inp[k], io)
    args = [f("u"), f("delta"), inp["A"], f("B"), f("C")]
    t0 = time.perf_counter()
    oracle.scan_fwd(*args, D=inp["D"], z=f("z") if inp["z"] is not None else None,
                    delta_bias=inp["delta_bias"], softplus=True, dt_mode=mode, nthreads=threads)
    return time.perf_counter() - t0


def cpu_baselines(inp1, threads):
    """The fp64 oracle, as it stands, timed on the host for every workload:
    whole where that takes seconds (the tiny case, the Mamba-130M layer), on a
    stated channel subset or a run of steps otherwise (extrapolated by the
    subset's share of the updates, which the oracle's cost is linear in).
    On `threads` host threads, and on one core for the first three."""
    import oracle
    import workloads as W
    out = {}

    def rec(name, seconds, updates, frac, sample, one_core=None):
        full = seconds / frac
        r = {"sample": sample, "seconds": round(seconds, 3), "updates": updates,
             "updates_per_s": float(f"{updates / seconds:.4g}"),
             "full_seconds" + ("" if frac == 1 else "_extrapolated"): round(full, 2)}
        if one_core is not None:  # (seconds, updates) of the one-core run
            r["one_core_seconds"] = round(one_core[0], 3)
            r["one_core_updates_per_s"] = float(f"{one_core[1] / one_core[0]:.4g}")
            r["one_core_full_seconds" + ("" if frac == 1 else "_extrapolated")] = \
                round(one_core[0] * updates / frac / one_core[1], 2)
        out[name] = r

    cfg = W.SCAN_CONFIGS["tiny"]
    inp = W.scan_inputs(cfg)
    upd = cfg.batch * cfg.L * cfg.dim * cfg.N
    rec("tiny", _oracle_scan_seconds(inp, cfg.io, threads), upd, 1.0, "whole (1 x 256 x 64, N 16)",
        (_oracle_scan_seconds(inp, cfg.io, 1), upd))

    cfg = W.SCAN_CONFIGS["mamba130m"]
    upd = cfg.batch * cfg.L * cfg.dim * cfg.N
    rec("mamba130m", _oracle_scan_seconds(inp1, cfg.io, threads), upd, 1.0,
        "whole (8 x 2048 x 1536, N 16, gate)", (_oracle_scan_seconds(inp1, cfg.io, 1), upd))

    cfg = W.SCAN_CONFIGS["mamba1p4b"]
    ch = np.arange(1024)
    inp = W.scan_inputs(cfg, channels=ch)
    upd = cfg.batch * cfg.L * len(ch) * cfg.N
    one = W.scan_inputs(cfg, channels=np.arange(256))
    rec("mamba1p4b", _oracle_scan_seconds(inp, cfg.io, threads), upd, len(ch) / cfg.dim,
        "channels 0-1023 of 4096 (8 x 2048, N 16, gate); one core on channels 0-255",
        (_oracle_scan_seconds(one, cfg.io, 1), upd // 4))
    del inp, one

    cfg = W.SCAN_CONFIGS["longseq"]
    ch = np.arange(128)
    inp = W.scan_inputs(cfg, channels=ch)
    upd = cfg.batch * cfg.L * len(ch) * cfg.N
    rec("longseq", _oracle_scan_seconds(inp, cfg.io, threads), upd, len(ch) / cfg.dim,
        "channels 0-127 of 2048 (4 x 65536, N 16)")
    del inp

    cfg = W.STEP_CONFIGS["decode"]
    A, D, bias = W.channel_params(cfg.seed, cfg.dim, cfg.N)
    st = W.step_state0(cfg).astype(np.float64)
    nsteps = 10
    toks = W.step_inputs_range(cfg, 0, nsteps)
    f = lambda x: W.as_f64(x, cfg.io)
    toks = [{k: f(t[k]) for k in ("u", "delta", "B", "C", "z")} for t in toks]
    t0 = time.perf_counter()
    for t in toks:
        _, st = oracle.step(st, t["u"], t["delta"], A, t["B"], t["C"], D=D, z=t["z"],
                            delta_bias=bias, nthreads=threads, inplace=True)
    sec = time.perf_counter() - t0
    upd = nsteps * cfg.batch * cfg.dim * cfg.N
    rec("decode", sec, upd, nsteps / cfg.steps, f"{nsteps} of the 1000 steps on the whole "
        "256 x 5120 x 16 state")
    out["decode"]["tok_per_s"] = round(nsteps * cfg.batch / sec, 1)
    return out


def profile_only(what, launches, dt_mode, kernel=None):
    """A few launches of one kernel for an external profiler (no timing, no JSON);
    kernel forces one scan kernel for `scan`."""
    import torch
    import selective_state_space_66_amd as ssm
    import workloads as W
    dev = torch.device("cuda:0")
    if what == "copy":
        x = torch.ones(128 * 1024 * 1024, dtype=torch.bfloat16, device=dev)
        y = torch.empty_like(x)
        for _ in range(launches):
            y.copy_(x)
    elif what == "scan":
        cfg = W.SCAN_CONFIGS["mamba130m"]
        s = upload_scan(W.scan_inputs(cfg), dev)
        y = torch.empty_like(s["u"])
        last = torch.empty(cfg.batch, cfg.dim, cfg.N, device=dev)
        for _ in range(launches):
            ssm.scan_fwd(s["u"], s["delta"], s["A"], s["B"], s["C"], D=s["D"], z=s["z"],
                         delta_bias=s["delta_bias"], dt_mode=dt_mode, y=y, last_state=last,
                         kernel=kernel)
    elif what == "bwd":
        cfg = W.SCAN_CONFIGS["mamba130m"]
        s = upload_scan(W.scan_inputs(cfg), dev)
        ws = torch.empty(ssm.scan_bwd_workspace_size(cfg.batch, cfg.L, cfg.dim, cfg.N),
                         dtype=torch.uint8, device=dev)
        gen = torch.Generator(device="cpu").manual_seed(12)
        dy = torch.randn((cfg.batch, cfg.L, cfg.dim), generator=gen).to(torch.bfloat16).to(dev)
        for _ in range(launches):
            ssm.scan_bwd(s["u"], s["delta"], s["A"], s["B"], s["C"], dy, D=s["D"], z=s["z"],
                         delta_bias=s["delta_bias"], dt_mode=dt_mode, workspace=ws)
    elif what == "train":
        # the training path: the forward that keeps the state every 16 tokens,
        # then the backward from those checkpoints
        cfg = W.SCAN_CONFIGS["mamba130m"]
        s = upload_scan(W.scan_inputs(cfg), dev)
        ws = torch.empty(ssm.scan_bwd_workspace_size(cfg.batch, cfg.L, cfg.dim, cfg.N),
                         dtype=torch.uint8, device=dev)
        gen = torch.Generator(device="cpu").manual_seed(13)
        dy = torch.randn((cfg.batch, cfg.L, cfg.dim), generator=gen).to(torch.bfloat16).to(dev)
        y, last, ck = ssm.scan_fwd_train(s["u"], s["delta"], s["A"], s["B"], s["C"], D=s["D"], z=s["z"],
                                         delta_bias=s["delta_bias"], dt_mode=dt_mode)
        for _ in range(launches):
            ssm.scan_fwd_train(s["u"], s["delta"], s["A"], s["B"], s["C"], D=s["D"], z=s["z"],
                               delta_bias=s["delta_bias"], dt_mode=dt_mode, y=y, last_state=last, ckpt=ck)
            ssm.scan_bwd(s["u"], s["delta"], s["A"], s["B"], s["C"], dy, D=s["D"], z=s["z"],
                         delta_bias=s["delta_bias"], dt_mode=dt_mode, workspace=ws, ckpt=ck)
    elif what in ("tpar", "seq"):
        # the time-parallel kernel with four waves per row on the Mamba-130M
        # layer at batch 1, or the sequential kernel (2 states per lane) on the
        # Mamba-130M layer, forced
        kern = "tpar" if what == "tpar" else "seq2"
        cfg = (W.ScanConfig("mamba130m_batch1", 1, 2048, 1536, 16, "bf16", True, 7) if what == "tpar"
               else W.SCAN_CONFIGS["mamba130m"])
        s = upload_scan(W.scan_inputs(cfg), dev)
        y = torch.empty_like(s["u"])
        last = torch.empty(cfg.batch, cfg.dim, cfg.N, device=dev)
        for _ in range(launches):
            ssm.scan_fwd(s["u"], s["delta"], s["A"], s["B"], s["C"], D=s["D"], z=s["z"],
                         delta_bias=s["delta_bias"], dt_mode=dt_mode, y=y, last_state=last,
                         kernel=kern)
    elif what == "decode":
        time_decode(W.STEP_CONFIGS["decode"], launches, dev, npool=2)
    elif what == "ssd":
        cfg = W.SSD_CONFIGS["ssd130m"]
        inp = W.ssd_inputs(cfg)
        t = {k: to_dev(inp[k], "f32" if k in ("dt", "A", "D", "dt_bias") else "bf16", dev)
             for k in ("x", "z", "dt", "A", "D", "dt_bias", "B", "C")}
        for _ in range(launches):
            ssm.ssd_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], D=t["D"], z=t["z"],
                        dt_bias=t["dt_bias"])
    elif what == "conv":
        cfg = W.CONV_CONFIGS["conv130m"]
        inp = W.conv_inputs(cfg)
        x = to_dev(inp["x"], cfg.io, dev)
        w, b = to_dev(inp["w"], "f32", dev), to_dev(inp["bias"], "f32", dev)
        for _ in range(launches):
            ssm.conv1d_fwd(x, w, bias=b)
    elif what == "conv_bwd":
        cfg = W.CONV_CONFIGS["conv130m"]
        inp = W.conv_inputs(cfg)
        x = to_dev(inp["x"], cfg.io, dev)
        w, b = to_dev(inp["w"], "f32", dev), to_dev(inp["bias"], "f32", dev)
        gen = torch.Generator(device="cpu").manual_seed(14)
        dout = torch.randn(x.shape, generator=gen).to(x.dtype).to(dev)
        for _ in range(launches):
            ssm.conv1d_bwd(x, w, dout, bias=b)
    torch.cuda.synchronize()
    log(f"[bench] profile-only {what}: {launches} launches done")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--only", choices=["scan", "seq", "bwd", "train", "tpar", "decode", "conv", "conv_bwd",
                                       "ssd", "copy"],
                    default=None,
                    help="profiling mode: a few launches of one kernel, no JSON")
    ap.add_argument("--launches", type=int, default=3)
    ap.add_argument("--dt-mode", choices=["zoh", "euler"], default="zoh")
    ap.add_argument("--kernel", default=None,
                    help="profiling mode, scan: force one scan kernel (seq1, seq2, seq4, tpar, wave, wave4)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the scan shards by batch or channel with no communication between GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import selective_state_space_66_amd as ssm
    import workloads as W
    ssm.load_library()  # fail loudly if the HIP library is missing
    if args.only:
        profile_only(args.only, args.launches, args.dt_mode, args.kernel)
        return
    dev = torch.device("cuda:0")

    cfg = W.SCAN_CONFIGS["mamba130m"]
    log(f"[bench] generating inputs for {cfg}")
    inp0 = W.scan_inputs(cfg)
    sets = [upload_scan(inp0, dev)]
    for k in (1, 2):  # two more independent sets (other seeds) for cache rotation
        other = W.ScanConfig(cfg.name, cfg.batch, cfg.L, cfg.dim, cfg.N, cfg.io, cfg.gate,
                             cfg.seed + 100 * k)
        sets.append(upload_scan(W.scan_inputs(other), dev))
    nbytes = scan_bytes(cfg.batch, cfg.L, cfg.dim, cfg.N, 2, cfg.gate)
    elems = cfg.batch * cfg.L * cfg.dim

    scan_kernel = launched_scan_kernel(ssm.scan_kernel_name(cfg.batch, cfg.L, cfg.dim, cfg.N), cfg.io)
    settle = settle_clock(sets)
    log(f"[bench] {settle} untimed launches while the clock settles")
    rates = alu_rates(dev)
    log(f"[bench] ALU rates: FMA {rates['fma_lane_ops_per_s']:.4g}/s, exp {rates['exp_lane_ops_per_s']:.4g}/s, "
        f"{rates['exp_slots_in_fma_stream']} FMA slots per exponential in an FMA stream")
    settle_clock(sets, ms=30.0)
    log(f"[bench] timing ZOH scan ({scan_kernel})")
    wall_ms, kern_ms, kern_med, kern_min = time_scan(sets, args.steps, args.warmup, "zoh", stats=True)
    log(f"[bench] zoh: wall {wall_ms:.4f} ms/step, kernel {kern_ms:.4f} ms")
    # the same scan with the sequential kernel forced, for comparison
    seq_kern_ms = time_scan(sets, args.steps, args.warmup, "zoh", kernel="seq2")[1]
    log(f"[bench] zoh, sequential kernel forced: {seq_kern_ms:.4f} ms")
    log("[bench] timing exponential-Euler scan")
    e_wall, e_kern = time_scan(sets, args.steps, args.warmup, "euler")
    log(f"[bench] euler: wall {e_wall:.4f} ms/step, kernel {e_kern:.4f} ms")

    # the extended scan: chunked prefill from an initial state, ragged lengths
    # and packed documents (a reset every 512 tokens)
    rng = np.random.default_rng(11)
    lens = [cfg.L, cfg.L - 48, cfg.L // 2 + 1, cfg.L, 1000, cfg.L, 1537, cfg.L]
    reset = np.zeros((cfg.batch, cfg.L), dtype=np.uint8)
    reset[:, 512::512] = 1
    extras = {"h0": torch.from_numpy(rng.normal(size=(cfg.batch, cfg.dim, cfg.N)).astype(np.float32)).to(dev),
              "seq_lens": torch.tensor(lens, dtype=torch.int32, device=dev),
              "reset": torch.from_numpy(reset).to(dev)}
    log("[bench] timing the extended scan (h0, lengths, resets)")
    x_wall, x_kern = time_scan(sets, args.steps, args.warmup, "zoh", extras)
    x_bytes = nbytes + 4 * cfg.batch * cfg.dim * cfg.N + cfg.batch * cfg.L + 4 * cfg.batch
    x_updates = sum(lens) * cfg.dim * cfg.N
    log(f"[bench] extended: wall {x_wall:.4f} ms/step, kernel {x_kern:.4f} ms")

    log("[bench] timing the backward pass")
    b_ms, b_ws = time_bwd(sets, max(5, args.steps // 5), 2, dev)
    tf_ms, tb_ms = time_train(sets, max(5, args.steps // 5), 2, dev)
    log(f"[bench] backward: {b_ms:.4f} ms per call (workspace {b_ws / 1e6:.1f} MB)")

    log("[bench] timing the convolution")
    del sets
    torch.cuda.empty_cache()
    conv = time_conv(dev, args.steps, args.warmup)
    log("[bench] timing the Mamba-2 / SSD layer")
    torch.cuda.empty_cache()
    ssd = time_ssd(dev, args.steps, args.warmup)
    log(f"[bench] ssd: {ssd['kernel_ms']:.4f} ms")
    log(f"[bench] conv: {conv['kernel_ms']:.4f} ms, step {conv['step']['us_per_step']:.2f} us")
    log("[bench] timing the scan on the Mamba-1.4B and long-sequence layers")
    torch.cuda.empty_cache()
    layers = time_layers(dev, args.steps, args.warmup, rates)
    log("[bench] layers: " + ", ".join(f"{k} {v['kernel_ms']:.4f} ms ({v['GB/s']:.0f} GB/s), "
                                       f"Euler {v['euler']['kernel_ms']:.4f} ms"
                                       for k, v in layers.items()))
    log("[bench] timing the scan on few, narrow rows")
    torch.cuda.empty_cache()
    narrow = time_narrow(dev, args.steps, args.warmup, rates)
    log("[bench] timing the tiny workload")
    tiny = time_tiny(dev)
    log("[bench] narrow: " + ", ".join(f"{k} {v['kernel_ms']:.4f} ms (sequential {v['sequential_kernel_ms']:.4f})"
                                       for k, v in narrow.items()))

    dcfg = W.STEP_CONFIGS["decode"]
    d_bytes = step_bytes(dcfg.batch, dcfg.dim, dcfg.N, 2, dcfg.gate)
    # a model decodes layer after layer, so each layer's state comes from HBM:
    # the steps rotate over four state caches (336 MB, past the 256 MB
    # Infinity Cache); one state stepped over and over stays cache-resident
    log("[bench] timing decode steps over 4 state caches (HBM-resident)")
    d_wall_s, d_kern_ms = time_decode(dcfg, args.decode_steps, dev, nstates=4)
    log("[bench] timing decode steps on one state cache (cache-resident)")
    d1_wall_s, d1_kern_ms = time_decode(dcfg, max(100, args.decode_steps // 5), dev)
    log("[bench] timing a plain device copy")
    copy_gbs = copy_bandwidth(dev)
    for v in layers.values():
        v["pct_copy_bw"] = round(100.0 * v["GB/s"] / copy_gbs, 2)
        v["euler"]["pct_copy_bw"] = round(100.0 * v["euler"]["GB/s"] / copy_gbs, 2)

    cpu = None
    if not args.no_cpu:
        facts = host_facts()
        threads = facts["oracle_threads"]
        log(f"[bench] timing the fp64 oracle on {threads} host threads ({facts})")
        per = cpu_baselines(inp0, threads)
        c1 = per["mamba130m"]
        cpu = {"value": round(nbytes / c1["seconds"] / 1e9, 4), "unit": "GB/s", "cores": threads,
               "kind": "oracle",
               "sample": f"the whole workload ({cfg.batch}x{cfg.L}x{cfg.dim}, N {cfg.N}, ZOH, "
                         f"gate): {c1['seconds']:.2f} s wall on {threads} threads, "
                         f"{elems / c1['seconds']:.4g} elems/s",
               "host": facts, "one_core": {"value": round(nbytes / c1["one_core_seconds"] / 1e9, 4),
                                           "unit": "GB/s", "seconds": c1["one_core_seconds"]},
               "workloads": per}
        log(f"[bench] oracle: " + ", ".join(f"{k} {v['seconds']:.2f} s" for k, v in per.items()))

    gbs = nbytes / (wall_ms * 1e-3) / 1e9
    achieved = nbytes / (kern_ms * 1e-3) / 1e9
    updates = elems * cfg.N
    tflops = FLOPS_PER_UPDATE * updates / (kern_ms * 1e-3) / 1e12
    traffic = measured_traffic("scan_fwd_mamba130m_zoh")
    out = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_launches": settle,
        "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "mamba130m-layer selective scan fwd: batch 8, L 2048, D 1536, N 16, "
                               "bf16 io, fp32 state, silu(z) gate, D skip, softplus(delta+bias), ZOH",
                   "batch": cfg.batch, "seq_len": cfg.L, "dim": cfg.dim, "d_state": cfg.N,
                   "io_dtype": "bf16", "dt_mode": "zoh", "parallelism": "none (1 GPU)"},
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "copy_GBps": round(copy_gbs, 1),
        "pct_copy_bw": round(100.0 * gbs / copy_gbs, 2),
        "elems_per_s": float(f"{elems / (wall_ms * 1e-3):.4g}"),
        "updates_per_s": float(f"{elems * cfg.N / (wall_ms * 1e-3):.4g}"),
        "algorithmic_bytes_per_step": nbytes,
        "roofline": {"bound": "alu", "achieved": round(tflops, 3), "peak": round(FP32_TFLOPS, 2),
                     "unit": "TFLOP/s", "frac": round(tflops / FP32_TFLOPS, 4),
                     "traffic": traffic,
                     "peak_basis": "256 CU x 4 SIMD x 16 lanes x 2.4 GHz x 2 flops per fp32 FMA "
                                   "(packed fp32 off in this build)",
                     "published_fp32_peak": FP32_PUBLISHED_TFLOPS,
                     "frac_published_fp32": round(tflops / FP32_PUBLISHED_TFLOPS, 4),
                     "kernel": scan_kernel, "instance": "ZOH, bf16 io, gate",
                     "kernel_ms": round(kern_ms, 5), "kernel_ms_median": round(kern_med, 5),
                     "kernel_ms_min": round(kern_min, 5),
                     "per_launch": {"updates": updates, "flops": FLOPS_PER_UPDATE * updates,
                                    "algorithmic_bytes": nbytes},
                     "hbm": {"achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(achieved / HBM_PEAK_GBS, 4)},
                     "alu_floor": alu_figures(updates, kern_ms, "zoh", rates)["floor"],
                     "alu_rates": rates},
        "cpu_baseline": cpu,
        "sequential_kernel": {"kernel": "scan_fwd_kernel (sequential, 2 states per lane), forced",
                              "kernel_ms": round(seq_kern_ms, 5),
                              "alu": alu_figures(updates, seq_kern_ms, "zoh", rates)},
        "euler": {"ms_per_step": round(e_wall, 5), "GB/s": round(nbytes / (e_wall * 1e-3) / 1e9, 2),
                  "kernel_ms": round(e_kern, 5),
                  "alu": alu_figures(updates, e_kern, "euler", rates)},
        "scan_ex": {"workload": "ssm_scan_fwd_ex on the same layer, ZOH: h0 given, lengths "
                                f"{lens}, a document start every 512 tokens",
                    "kernel_ms": round(x_kern, 5),
                    "GB/s": round(x_bytes / (x_kern * 1e-3) / 1e9, 2),
                    "alu": alu_figures(x_updates, x_kern, "zoh", rates)},
        "bwd": {"workload": "ssm_scan_bwd on the same layer, ZOH, gate, D, bias: du, d delta, dz, "
                            "dA, dB, dC, dD, d bias (states recomputed from the inputs)",
                "kernels": "scan_bwd_wave_kernel (time-parallel, rows of 16 lanes; every tile here has "
                           "|A| >= 1/2), then the dB/dC and dA/dD/dbias finalize kernels",
                "ms": round(b_ms, 4), "x_forward": round(b_ms / kern_ms, 2),
                "traffic": measured_traffic("scan_bwd_mamba130m_zoh"),
                "updates_per_s": float(f"{elems * cfg.N / (b_ms * 1e-3):.4g}"),
                "workspace_MB": round(b_ws / 1e6, 1),
                "training": {"workload": "ssm_scan_fwd_ckpt (keeps the state every 16 tokens) then "
                                         "ssm_scan_bwd_ex from those checkpoints, same layer",
                             "forward_ms": round(tf_ms, 4), "backward_ms": round(tb_ms, 4),
                             "step_ms": round(tf_ms + tb_ms, 4),
                             "step_ms_without_checkpoints": round(kern_ms + b_ms, 4)}},
        "conv": conv,
        "ssd": ssd,
        "layers": layers,
        "tiny": tiny,
        "time_parallel": narrow,
        "decode": {"workload": "ssm_step: batch 256, D 5120, N 16, bf16 io, fp32 state, gate, ZOH; "
                               "consecutive steps rotate over 4 state caches (HBM-resident)",
                   "steps": args.decode_steps,
                   "tok_per_s": round(dcfg.batch * args.decode_steps / d_wall_s, 1),
                   "us_per_step": round(d_kern_ms * 1e3, 3),
                   "GB/s": round(d_bytes / (d_kern_ms * 1e-3) / 1e9, 2),
                   "pct_hbm_peak": round(100.0 * d_bytes / (d_kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                   "pct_copy_bw": round(100.0 * d_bytes / (d_kern_ms * 1e-3) / 1e9 / copy_gbs, 2),
                   "algorithmic_bytes": d_bytes, "traffic": measured_traffic("step_decode_zoh"),
                   "cache_resident": {"steps": max(100, args.decode_steps // 5), "state_caches": 1,
                                      "tok_per_s": round(dcfg.batch * max(100, args.decode_steps // 5)
                                                         / d1_wall_s, 1),
                                      "us_per_step": round(d1_kern_ms * 1e3, 3),
                                      "GB/s": round(d_bytes / (d1_kern_ms * 1e-3) / 1e9, 2)}},
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
