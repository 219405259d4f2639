"""Benchmark of the MI355X selective scan (one GPU).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Default workload: the Mamba-2.8B-shaped layer scan, B=4 D=5120 N=16 L=2048,
bf16 inputs/outputs, fp32 state and arithmetic, final state returned.  A
step is one call of mamba_scan_fwd over one batch (inputs resident in HBM;
three input sets rotate so the 256 MB last-level cache cannot hold a step's
inputs from an earlier step).  Prints one JSON line.

Other workloads: --workload long_b1 (B=1 D=4096 L=131072, chunked along L),
mamba130m_layer, tiny_fp32, decode48 (48 layers x 128 steps of
mamba_state_update at B=128 D=4096, the 48-layer step replayed as a graph),
conv_2.8b_layer (causal conv1d + SiLU at B=4 D=5120 L=2048 K=4) and
conv_decode48 (48 layers x 128 steps of the one-token conv update),
bwd_2.8b_layer (the scan's backward pass at the 2.8B-layer shape) and
ssd_2.7b_layer (the Mamba-2 layer forward: B=4, 80 heads x 64 channels,
N=128, L=2048, on the matrix cores).

--copy-calibration runs only a plain device copy of known size (used to
scale rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "scan HBM GB/s (% of MI355X peak) + B·D·L elems/s at Mamba-2.8B layer shape"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, AMD published
CUS, SIMDS_PER_CU, LANES_PER_SIMD, CLOCK_GHZ = 256, 4, 16, 2.4
# fp32 VALU lane-operations per second without packed math: 256 x 4 x 16 x 2.4e9
VALU_PEAK_TOPS = CUS * SIMDS_PER_CU * LANES_PER_SIMD * CLOCK_GHZ / 1e3
# Algorithmic fp32 operations of one ZOH state update (delta*A, exp, (e-1)/A,
# B*u, *coef, e*h + input, C*h accumulate): 6 VALU + 1 transcendental; the
# transcendental occupies the VALU issue slot it is issued in.
OPS_PER_UPDATE = 7
OPS_PER_UPDATE_DELTA_B = 5   # delta A', exp2, (delta u) B, the h fma, the readout fma
# Counter-derived HBM traffic of the scan kernel (rocprofv3 FETCH_SIZE and
# WRITE_SIZE, scaled by the same counters on a plain copy of known size); used
# only while the kernel sources still hash to the recorded value.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_mamba2.8b_layer_traffic.txt")
SCAN_SOURCES = ["selective_state_space_75_amd/csrc/scan_v4.hpp", "selective_state_space_75_amd/csrc/scan_v4_bf16.hip",
                "selective_state_space_75_amd/csrc/scan_v4_f32.hip", "selective_state_space_75_amd/csrc/kernels.hpp",
                "selective_state_space_75_amd/csrc/device_math.hpp", "selective_state_space_75_amd/csrc/abi.hip"]
ROW_SOURCES = ["selective_state_space_75_amd/csrc/scan_row.hip", "selective_state_space_75_amd/csrc/kernels.hpp",
               "selective_state_space_75_amd/csrc/device_math.hpp", "selective_state_space_75_amd/csrc/abi.hip"]
# Counter summaries per scan workload (taken with the kernel the planner picks
# for it; the sources hashed are those of that kernel).
SCAN_TRAFFIC = {
    "mamba2.8b_layer": TRAFFIC_FILE,
    "mamba130m_layer": os.path.join(ROOT, "profiles", "scan_mamba130m_layer_traffic.txt"),
    "long_b1": os.path.join(ROOT, "profiles", "scan_long_b1_traffic.txt"),
}


def kernel_sources(kernel):
    """Source files of a scan kernel (by its mamba_scan_kernel name)."""
    return ROW_SOURCES if kernel.startswith("row") else SCAN_SOURCES
# Shader clock measured on the 2.8B-layer scan (rocprofv3 GRBM counters over
# the kernel's duration); the ALU peak is also given at this clock.
CLOCK_FILE = os.path.join(ROOT, "profiles", "scan_mamba2.8b_layer_sq_counters.txt")
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "state_update_decode48_traffic.txt")
CONV_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "conv1d_2.8b_layer_traffic.txt")
CONV_SOURCES = ["selective_state_space_75_amd/csrc/conv1d.hip", "selective_state_space_75_amd/csrc/kernels.hpp",
                "selective_state_space_75_amd/csrc/device_math.hpp", "selective_state_space_75_amd/csrc/abi.hip"]
BWD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "scan_bwd_2.8b_layer_traffic.txt")
BWD_SOURCES = ["selective_state_space_75_amd/csrc/scan_bwd.hip", "selective_state_space_75_amd/csrc/kernels.hpp",
               "selective_state_space_75_amd/csrc/device_math.hpp", "selective_state_space_75_amd/csrc/abi.hip"]
DECODE_SOURCES = ["selective_state_space_75_amd/csrc/state_update.hip", "selective_state_space_75_amd/csrc/kernels.hpp",
                  "selective_state_space_75_amd/csrc/device_math.hpp", "selective_state_space_75_amd/csrc/abi.hip"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def to_dev(a, dev):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(a.astype(np.float32, copy=False)).to(dev)


def cpu_threads():
    env = os.environ.get("OMP_NUM_THREADS")
    n = int(env) if env and env.isdigit() and int(env) > 0 else (os.cpu_count() or 1)
    return max(1, min(16, n))


# ----------------------------------------------------------------------------- CPU oracle baseline
def cpu_baseline_scan(cfg, x, seconds: float, channels: int = 0, single_channels: int = 0):
    """Time the fp64 oracle (as it stands) on a bounded sample of the workload,
    repeated until about `seconds` of wall time; report the median run.

    channels > 0 samples the first `channels` channels of batch row 0 (whole
    sequence) instead of the whole workload; single_channels, likewise, the
    sample of the one-thread run.  Rates are per unit of work (bytes and
    elements scale with the sampled channels), so they compare with the
    whole-workload GPU rate."""
    import oracle
    from selective_state_space_75_amd import workloads as W
    nth = cpu_threads()
    f64 = lambda a: W.as_f32(a).astype(np.float64)  # noqa: E731
    total_ch = cfg.B * cfg.D

    def args_for(nch):
        if nch <= 0 or nch >= total_ch:
            return (f64(x["u"]), f64(x["delta_raw"]), f64(x["z"]), f64(x["Bt"]), f64(x["Ct"]),
                    x["A"].astype(np.float64), x["Dskip"].astype(np.float64),
                    x["delta_bias"].astype(np.float64)), 1.0, "whole workload"
        nch = min(nch, cfg.D)
        sl = lambda a: f64(a[0:1, 0:nch, :])  # noqa: E731
        return ((sl(x["u"]), sl(x["delta_raw"]), sl(x["z"]), f64(x["Bt"][0:1]), f64(x["Ct"][0:1]),
                 x["A"][0:nch].astype(np.float64), x["Dskip"][0:nch].astype(np.float64),
                 x["delta_bias"][0:nch].astype(np.float64)), nch / total_ch,
                "channels 0..%d of batch row 0 (%.4g of the workload), whole sequence" % (nch - 1, nch / total_ch))

    args, frac, what = args_for(channels)
    times = []
    t_all = time.perf_counter()
    while len(times) < 3 or (time.perf_counter() - t_all < seconds and len(times) < 200):
        t0 = time.perf_counter()
        oracle.scan(*args, nthreads=nth)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    nbytes = cfg.algorithmic_bytes() * frac
    out = {"value": round(nbytes / t / 1e9, 4), "unit": "GB/s", "cores": nth, "kind": "oracle",
           "sample": "%s (B=%d D=%d N=%d L=%d%s), fp64 C oracle, %d runs in %.1f s, median %.3f s per run; "
                     "GB/s = the sample's share of the workload's algorithmic bytes / run time"
                     % (what, cfg.B, cfg.D, cfg.N, cfg.L, ", final state" if cfg.final_state else "", len(times),
                        time.perf_counter() - t_all, t),
           "elems_per_s": round(cfg.elements * frac / t, 1),
           "updates_per_s": round(cfg.updates * frac / t, 1)}
    del args
    if nth > 1:
        # one run on a single thread, for the per-core rate
        args1, frac1, what1 = args_for(single_channels if single_channels else channels)
        t0 = time.perf_counter()
        oracle.scan(*args1, nthreads=1)
        t1 = time.perf_counter() - t0
        out["single_thread"] = {"value": round(cfg.algorithmic_bytes() * frac1 / t1 / 1e9, 4), "unit": "GB/s",
                                "run_s": round(t1, 3), "sample": what1,
                                "elems_per_s": round(cfg.elements * frac1 / t1, 1),
                                "updates_per_s": round(cfg.updates * frac1 / t1, 1)}
    return out


def cpu_baseline_decode(cfg, layers=(0, 47), steps: int = 128):
    """The fp64 oracle's decode step on layers {0, 47} x `steps` steps (step-major
    within the sample), extrapolated to all layers: the sample is 2 of the 48
    layers, so the whole workload takes 24 times as long."""
    import oracle
    from selective_state_space_75_amd import workloads as W
    nth = cpu_threads()
    f64 = lambda a: W.as_f32(a).astype(np.float64)  # noqa: E731
    prm, states = {}, {}
    for l in layers:
        A, Dskip, bias, st0 = W.decode_layer_params(cfg, l)
        prm[l] = (A.astype(np.float64), Dskip.astype(np.float64), bias.astype(np.float64))
        states[l] = st0.astype(np.float64)
    t_run = 0.0
    for s in range(steps):
        for l in layers:
            si = W.decode_step_inputs(cfg, l, s)
            ins = (f64(si["u"]), f64(si["delta_raw"]), f64(si["z"]), f64(si["Bt"]), f64(si["Ct"]))
            t0 = time.perf_counter()
            _, states[l] = oracle.state_update(states[l], *ins, *prm[l], nthreads=nth)
            t_run += time.perf_counter() - t0
    scale = cfg.layers / len(layers)
    per_ls = cfg.bytes_per_layer_step()
    total_s = t_run * scale
    return {"value": round(per_ls * len(layers) * steps / t_run / 1e9, 4), "unit": "GB/s", "cores": nth,
            "kind": "oracle",
            "sample": "layers %s x %d steps of the decode workload (B=%d D=%d N=%d), fp64 C oracle, %.1f s; "
                      "extrapolated x%g to all %d layers" % (list(layers), steps, cfg.B, cfg.D, cfg.N, t_run, scale,
                                                            cfg.layers),
            "extrapolated": True, "extrapolated_total_s": round(total_s, 2),
            "tokens_per_s": round(cfg.B * steps / total_s, 2),
            "layer_step_ms": round(t_run * 1e3 / (len(layers) * steps), 3)}


def settle(step, ms):
    """Untimed launches of the step for `ms` milliseconds of wall time, before
    the counted warm-up steps.  Timed right after the GPU sat idle (input
    generation, a CPU baseline) the first launches on MI355X run up to 1.6x
    slower for about 20-30 ms while the clocks come up (measured at the
    2.8B-layer scan: 0.40 ms per launch over the first 25 launches, 0.243 ms
    from the 50th on); a short timed region would measure that ramp instead of
    the steady state.  Returns what ran, for the JSON line."""
    import torch
    if ms <= 0:
        return {"ms": 0, "launches": 0}
    n = 0
    t_end = time.perf_counter() + ms / 1e3
    while time.perf_counter() < t_end:
        step(n)
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()   # keep the queue short, so wall time is GPU time
    torch.cuda.synchronize()
    return {"ms": ms, "launches": n}


def source_digest(files):
    """sha256 over the sources with comments and whitespace removed, so that
    only a change of the code itself invalidates a recorded measurement."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in files:
        src = open(os.path.join(ROOT, f), encoding="utf-8").read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        h.update(re.sub(r"\s+", "", src).encode())
    return h.hexdigest()


def measured_clock_ghz(path=CLOCK_FILE):
    """Shader clock (GHz) recorded in the committed counter summary, or None."""
    if not os.path.exists(path):
        return None
    for line in open(path, encoding="utf-8"):
        if line.startswith("measured_clock_ghz:"):
            return float(line.split(":", 1)[1])
    return None


def recorded_traffic(path=TRAFFIC_FILE, sources=SCAN_SOURCES):
    """(bytes per launch, note) from the committed counter summary, or (None,
    reason) when it is missing or the kernel sources changed since."""
    if not os.path.exists(path):
        return None, "no counter summary"
    kv = {}
    for line in open(path, encoding="utf-8"):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != source_digest(sources):
        return None, "kernel changed since the counters were taken"
    return int(kv["hbm_bytes_per_launch"]), kv.get("summary", "")


# ----------------------------------------------------------------------------- scan benchmark
def scan_config(workload, seq_len=0):
    """The scan workload's configuration; seq_len > 0 keeps its batch,
    channels, states, dtype and seed at another sequence length."""
    from selective_state_space_75_amd import workloads as W
    cfg = W.SCAN_CONFIGS[workload]
    if seq_len:
        cfg = W.ScanConfig("%s_L%d" % (cfg.name, seq_len), cfg.B, cfg.D, cfg.N, seq_len, cfg.dtype,
                           cfg.seed, cfg.dskip, cfg.final_state)
    return cfg


def scan_kernel_name(cfg, args):
    """The kernel the library runs for this workload (mamba_scan_kernel)."""
    import selective_state_space_75_amd as m
    return m.scan_kernel(cfg.B, cfg.D, cfg.N, cfg.L)


def bench_scan(args, dev):
    import torch
    import selective_state_space_75_amd as m
    from selective_state_space_75_amd import workloads as W
    cfg = scan_config(args.workload, args.seq_len)
    log("workload %s: B=%d D=%d N=%d L=%d %s" % (cfg.name, cfg.B, cfg.D, cfg.N, cfg.L, cfg.dtype))
    x = W.scan_inputs(cfg)
    sets = []
    for k in range(args.sets):
        if k == 0:
            xs = x
        else:
            xs = W.scan_inputs(W.ScanConfig(cfg.name, cfg.B, cfg.D, cfg.N, cfg.L, cfg.dtype, cfg.seed + 100 * k,
                                            cfg.dskip, cfg.final_state))
        t = {k2: to_dev(xs[k2], dev) for k2 in ("u", "delta_raw", "z", "Bt", "Ct", "A", "Dskip", "delta_bias")}
        sets.append(t)
    odt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    ys = [torch.empty((cfg.B, cfg.D, cfg.L), dtype=odt, device=dev) for _ in sets]
    hs = [torch.empty((cfg.B, cfg.D, cfg.N), dtype=torch.float32, device=dev) for _ in sets]
    wsb = m.workspace_size(cfg.B, cfg.D, cfg.N, cfg.L)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        t = sets[i % len(sets)]
        m.scan_fwd(t["u"], t["delta_raw"], t["z"], t["Bt"], t["Ct"], t["A"], t["Dskip"], t["delta_bias"],
                   return_final_state=cfg.final_state, y=ys[i % len(sets)], final_state=hs[i % len(sets)],
                   workspace=ws if wsb else None, stream=stream, delta_b=args.delta_b)

    settled = settle(step, args.settle_ms)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    # the launch stream is torch's current stream, so these events bracket the kernel itself
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch_ms = [a.elapsed_time(b) for a, b in ev]
    ms_step = wall * 1e3 / args.steps
    kern_ms = float(np.mean(per_launch_ms))
    nbytes = cfg.algorithmic_bytes()
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    opu = OPS_PER_UPDATE_DELTA_B if args.delta_b else OPS_PER_UPDATE
    ops = cfg.updates * opu
    achieved_tops = ops / (kern_ms * 1e-3) / 1e12
    kernel = scan_kernel_name(cfg, args)
    if cfg.name in SCAN_TRAFFIC and not args.delta_b and getattr(args, "scan_kernel", "planner") == "planner":
        traffic, traffic_note = recorded_traffic(SCAN_TRAFFIC[cfg.name], kernel_sources(kernel))
    else:
        traffic, traffic_note = None, "not measured for this variant"
    clock = measured_clock_ghz()
    p10, p50, p90 = (float(v) for v in np.percentile(per_launch_ms, [10, 50, 90]))
    line = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle": settled, "ms_per_step": round(ms_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "io_dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "D": cfg.D, "N": cfg.N, "L": cfg.L,
                   "final_state": cfg.final_state, "global_batch": cfg.B, "seq_len": cfg.L,
                   "discretization": "delta_b" if args.delta_b else "zoh", "parallelism": "none (1 GPU)",
                   "scan_kernel": kernel},
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "elems_per_s": round(cfg.elements / (ms_step * 1e-3), 1),
        "kernel_ms_mean": round(kern_ms, 5), "kernel_ms_min": round(float(np.min(per_launch_ms)), 5),
        "kernel_ms_p10_p50_p90": [round(p10, 5), round(p50, 5), round(p90, 5)],
        "input_sets": len(sets),
        # the first input set's arrays (as generated, bf16 as bit patterns), to pin the workload
        "inputs": {"numpy": np.__version__,
                   "sha256": {k2: W.sha256(x[k2]) for k2 in ("u", "delta_raw", "z", "Bt", "Ct", "A", "Dskip",
                                                            "delta_bias")}},
        "algorithmic_bytes": nbytes,
        "roofline": {"bound": "alu", "achieved": round(achieved_tops, 3), "peak": round(VALU_PEAK_TOPS, 2),
                     "unit": "TOP/s", "frac": round(achieved_tops / VALU_PEAK_TOPS, 4), "traffic": traffic,
                     "traffic_note": traffic_note,
                     "ops_per_update": opu, "updates_per_launch": cfg.updates,
                     "op": "fp32 VALU lane-operations (%d per state update + 1 exp2); peak = 256 CUs x 64 "
                           "lanes x 2.4 GHz, non-packed" % (opu - 1),
                     "clock_ghz_measured": clock,
                     "frac_at_measured_clock": (round(achieved_tops / (VALU_PEAK_TOPS * clock / CLOCK_GHZ), 4)
                                                if clock else None),
                     "hbm_achieved_gbs_kernel": round(nbytes / (kern_ms * 1e-3) / 1e9, 2)},
    }
    return line, cfg, x


# ----------------------------------------------------------------------------- decode benchmark
def bench_decode(args, dev):
    import torch
    import selective_state_space_75_amd as m
    from selective_state_space_75_amd import workloads as W
    cfg = W.DECODE_CONFIGS["decode48"]
    log("decode48: %d layers x %d steps, B=%d D=%d N=%d" % (cfg.layers, cfg.steps, cfg.B, cfg.D, cfg.N))
    layers = []
    pool = 4   # distinct per-layer token inputs cycled over steps (inputs are ~4% of the bytes)
    for l in range(cfg.layers):
        A, Dskip, bias, st0 = W.decode_layer_params(cfg, l)
        toks = []
        for s in range(pool):
            si = W.decode_step_inputs(cfg, l, s)
            toks.append({k: to_dev(v, dev) for k, v in si.items()})
        layers.append({"A": to_dev(A, dev), "Dskip": to_dev(Dskip, dev), "bias": to_dev(bias, dev),
                       "state": to_dev(st0, dev), "toks": toks,
                       "y": torch.empty((cfg.B, cfg.D), dtype=torch.bfloat16, device=dev)})
        if l % 12 == 11:
            log("  layer %d ready" % (l + 1))
    stream = torch.cuda.Stream(dev)
    graphs = []
    torch.cuda.synchronize()
    for s in range(pool):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for L_ in layers:
                tk = L_["toks"][s]
                m.state_update(L_["state"], tk["u"], tk["delta_raw"], tk["z"], tk["Bt"], tk["Ct"], L_["A"],
                               L_["Dskip"], L_["bias"], y=L_["y"], stream=stream)
        graphs.append(g)
    # capture does not execute; restore the states it did not touch anyway
    settled = settle(lambda i: graphs[i % pool].replay(), args.settle_ms)
    for i in range(args.warmup):
        graphs[i % pool].replay()
    torch.cuda.synchronize()
    steps = args.decode_steps
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(torch.cuda.current_stream(dev))
    for s in range(steps):
        graphs[s % pool].replay()
    ev1.record(torch.cuda.current_stream(dev))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = ev0.elapsed_time(ev1)
    per_ls = cfg.bytes_per_layer_step()
    total = per_ls * cfg.layers * steps
    gbs = total / (wall) / 1e9
    kern_us = gpu_ms * 1e3 / (cfg.layers * steps)
    traffic, traffic_note = recorded_traffic(DECODE_TRAFFIC_FILE, DECODE_SOURCES)
    line = {
        "metric": "decode state-update HBM GB/s, 48 layers x 128 steps (B=128, D=4096, N=16)",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
        "settle": settled, "ms_per_step": round(wall * 1e3 / steps, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "io_dtype": "bf16", "data": "synthetic",
        "config": {"workload": "decode48", "layers": cfg.layers, "steps": steps, "B": cfg.B, "D": cfg.D,
                   "N": cfg.N, "order": "step-major, 48-layer step replayed as a HIP graph"},
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(cfg.B * steps / wall, 1),
        "layer_step_us_mean": round(kern_us, 3),
        "roofline": {"bound": "hbm", "achieved": round(per_ls / (kern_us * 1e-6) / 1e9, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(per_ls / (kern_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "traffic_note": traffic_note, "bytes_per_layer_step": per_ls,
                     "launch_time": "graph replay time / launches (inter-kernel gaps included)"},
    }
    return line


def bench_conv(args, dev):
    """Causal conv1d + SiLU over the 2.8B-layer shape; HBM-bound."""
    import torch
    import selective_state_space_75_amd as m
    from selective_state_space_75_amd import workloads as W
    cfg = W.CONV_CONFIGS[args.workload]
    log("conv workload %s: B=%d D=%d L=%d K=%d %s" % (cfg.name, cfg.B, cfg.D, cfg.L, cfg.K, cfg.dtype))
    sets = []
    for k in range(args.sets):
        xs = W.conv_inputs(cfg.B, cfg.D, cfg.L, cfg.K, cfg.dtype, cfg.seed + 100 * k)
        sets.append({n: to_dev(v, dev) for n, v in xs.items()})
    odt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    ys = [torch.empty((cfg.B, cfg.D, cfg.L), dtype=odt, device=dev) for _ in sets]
    fss = [torch.empty((cfg.B, cfg.D, cfg.K), dtype=torch.float32, device=dev) for _ in sets]
    stream = torch.cuda.current_stream(dev)

    def step(i):
        t = sets[i % len(sets)]
        m.conv1d_fwd(t["x"], t["w"], t["bias"], return_final_state=True, y=ys[i % len(sets)],
                     final_state=fss[i % len(sets)], stream=stream)

    settled = settle(step, args.settle_ms)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [a.elapsed_time(b) for a, b in ev]
    kern_ms = float(np.mean(per))
    ms_step = wall * 1e3 / args.steps
    nbytes = cfg.algorithmic_bytes()
    ach = nbytes / (kern_ms * 1e-3) / 1e9
    traffic, note = recorded_traffic(CONV_TRAFFIC_FILE, CONV_SOURCES)
    return {
        "metric": "causal conv1d + SiLU HBM GB/s (% of MI355X peak) at Mamba-2.8B layer shape",
        "value": round(nbytes / (ms_step * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle": settled, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "io_dtype": cfg.dtype, "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "D": cfg.D, "L": cfg.L, "K": cfg.K, "input_sets": len(sets)},
        "elems_per_s": round(cfg.elements / (ms_step * 1e-3), 1),
        "kernel_ms_mean": round(kern_ms, 5),
        "kernel_ms_p10_p50_p90": [round(float(v), 5) for v in np.percentile(per, [10, 50, 90])],
        "roofline": {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic, "traffic_note": note,
                     "algorithmic_bytes": nbytes},
    }


def bench_conv_decode(args, dev):
    """48 layers x 128 steps of the one-token conv update (B=128 D=4096 K=4),
    step-major, the 48-layer step replayed as a graph."""
    import torch
    import selective_state_space_75_amd as m
    from selective_state_space_75_amd import workloads as W
    cfg = W.CONV_UPDATE_CONFIGS[args.workload]
    log("conv decode: %d layers x %d steps, B=%d D=%d K=%d" % (cfg.layers, cfg.steps, cfg.B, cfg.D, cfg.K))
    pool = 4
    layers = []
    for l in range(cfg.layers):
        w, bias, st0 = W.conv_update_layer(cfg, l)
        layers.append({"w": to_dev(w, dev), "bias": to_dev(bias, dev), "state": to_dev(st0, dev),
                       "x": [to_dev(W.conv_update_step(cfg, l, s), dev) for s in range(pool)],
                       "y": torch.empty((cfg.B, cfg.D), dtype=torch.bfloat16, device=dev)})
    stream = torch.cuda.Stream(dev)
    graphs = []
    torch.cuda.synchronize()
    for s in range(pool):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for L_ in layers:
                m.conv1d_update(L_["state"], L_["x"][s], L_["w"], L_["bias"], y=L_["y"], stream=stream)
        graphs.append(g)
    settled = settle(lambda i: graphs[i % pool].replay(), args.settle_ms)
    for i in range(args.warmup):
        graphs[i % pool].replay()
    torch.cuda.synchronize()
    steps = args.decode_steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(torch.cuda.current_stream(dev))
    for s in range(steps):
        graphs[s % pool].replay()
    e1.record(torch.cuda.current_stream(dev))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_ls = cfg.bytes_per_layer_step()
    kern_us = e0.elapsed_time(e1) * 1e3 / (cfg.layers * steps)
    ach = per_ls / (kern_us * 1e-6) / 1e9
    return {
        "metric": "conv1d one-token update HBM GB/s, 48 layers x 128 steps (B=128, D=4096, K=4)",
        "value": round(per_ls * cfg.layers * steps / wall / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "settle": settled, "ms_per_step": round(wall * 1e3 / steps, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "io_dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "layers": cfg.layers, "steps": steps, "B": cfg.B, "D": cfg.D, "K": cfg.K,
                   "order": "step-major, 48-layer step replayed as a HIP graph"},
        "layer_step_us_mean": round(kern_us, 3),
        "roofline": {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None, "bytes_per_layer_step": per_ls,
                     "launch_time": "graph replay time / launches (inter-kernel gaps included)"},
    }


# fp32 lane-operations of one state update in the backward pass, counted as the
# method needs them once: the forward step (6 + exp) and the reverse step (the
# state adjoint, the four input coefficients' partials, dB/dC/du/ddelta/dA
# accumulations and exp of the step again: 22).
OPS_PER_UPDATE_BWD = 29


def bench_bwd(args, dev):
    """Backward pass at the 2.8B-layer shape: bf16 inputs, dy and input gradients."""
    import torch
    import selective_state_space_75_amd as m
    from selective_state_space_75_amd import workloads as W
    cfg = W.SCAN_CONFIGS["mamba2.8b_layer"]
    log("bwd workload: B=%d D=%d N=%d L=%d" % (cfg.B, cfg.D, cfg.N, cfg.L))
    sets = []
    for k in range(2):
        xs = W.scan_inputs(W.ScanConfig(cfg.name, cfg.B, cfg.D, cfg.N, cfg.L, cfg.dtype, cfg.seed + 100 * k,
                                        cfg.dskip, cfg.final_state))
        t = {k2: to_dev(xs[k2], dev) for k2 in ("u", "delta_raw", "z", "Bt", "Ct", "A", "Dskip", "delta_bias")}
        dy = W._normal_f32([cfg.seed + 100 * k, 77], cfg.B * cfg.D * cfg.L).reshape(cfg.B, cfg.D, cfg.L)
        t["dy"] = torch.from_numpy(dy).to(dev).to(torch.bfloat16)
        sets.append(t)
    ws = torch.empty(m.scan_bwd_workspace_size(cfg.B, cfg.D, cfg.N, cfg.L), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        t = sets[i % len(sets)]
        m.scan_bwd(t["u"], t["delta_raw"], t["z"], t["Bt"], t["Ct"], t["A"], t["Dskip"], t["delta_bias"], t["dy"],
                   workspace=ws, stream=stream)

    settled = settle(step, args.settle_ms)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    steps = min(args.steps, 20)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [a.elapsed_time(b) for a, b in ev]
    call_ms = float(np.mean(per))
    e = cfg.elements
    bc = cfg.B * cfg.N * cfg.L
    nbytes = e * 2 * 4 + bc * 2 * 2 + e * 2 * 3 + bc * 4 * 2 + cfg.D * (cfg.N + 3) * 4 * 2
    ops = cfg.updates * OPS_PER_UPDATE_BWD
    ach = ops / (call_ms * 1e-3) / 1e12
    traffic, traffic_note = recorded_traffic(BWD_TRAFFIC_FILE, BWD_SOURCES)
    return {
        "metric": "scan backward: algorithmic GB/s and fp32 lane-op rate at Mamba-2.8B layer shape",
        "value": round(nbytes / (wall / steps) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "settle": settled, "ms_per_step": round(wall * 1e3 / steps, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "io_dtype": "bf16", "data": "synthetic",
        "config": {"workload": "bwd_2.8b_layer", "B": cfg.B, "D": cfg.D, "N": cfg.N, "L": cfg.L,
                   "grads": "du, ddelta, dz bf16; dB, dC, dA, dD, dbias fp32"},
        "call_ms_mean": round(call_ms, 5), "algorithmic_bytes": nbytes,
        "roofline": {"bound": "alu", "achieved": round(ach, 3), "peak": round(VALU_PEAK_TOPS, 2), "unit": "TOP/s",
                     "frac": round(ach / VALU_PEAK_TOPS, 4), "traffic": traffic, "traffic_note": traffic_note,
                     "ops_per_update": OPS_PER_UPDATE_BWD,
                     "launch_time": "whole call: segment summary, carry, segment recompute and two reduce kernels"},
    }


# MI355X dense bf16 matrix peak (AMD published, without sparsity).
MFMA_BF16_PEAK_TFLOPS = 2500.0
SSD_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ssd_2.7b_layer_traffic.txt")
SSD_SOURCES = ["selective_state_space_75_amd/csrc/ssd.hip", "selective_state_space_75_amd/csrc/kernels.hpp",
               "selective_state_space_75_amd/csrc/device_math.hpp", "selective_state_space_75_amd/csrc/abi.hip"]


def ssd_mfma_flops(cfg) -> int:
    """Matrix-core flops of the chunked algorithm (the split operands counted
    twice): per 64-channel block and 32-step chunk, C B^T on 3 of 4 16x16 tiles
    (K = N), G x (K = 32, two parts), C H (K = N, two parts) and B^T (w o x)
    (K = 32, two parts).  The segment-state launch, which repeats B^T (w o x)
    over all segments but the last when L is cut into segments, is not
    counted."""
    q, pb = 32, 64
    per_chunk = 2 * (3 * 16 * 16 * cfg.N + 2 * q * pb * q + 2 * q * pb * cfg.N + 2 * cfg.N * pb * q)
    chunks = (cfg.L + q - 1) // q
    return per_chunk * chunks * cfg.B * cfg.H * (cfg.P // pb)


def bench_ssd(args, dev):
    """Mamba-2 (SSD) layer forward: B=4, 80 heads x 64 channels, N=128, L=2048."""
    import torch
    import selective_state_space_75_amd as m
    from selective_state_space_75_amd import workloads as W
    cfg = W.SSD_CONFIGS[args.workload]
    log("ssd workload %s: B=%d H=%d P=%d N=%d L=%d" % (cfg.name, cfg.B, cfg.H, cfg.P, cfg.N, cfg.L))
    sets = []
    for k in range(args.sets):
        xs = W.ssd_inputs(cfg.B, cfg.H, cfg.P, cfg.N, cfg.L, cfg.seed + 100 * k, cfg.gate)
        sets.append({n: (None if v is None else to_dev(v, dev)) for n, v in xs.items() if n != "dt"})
    ys = [torch.empty((cfg.B, cfg.D, cfg.L), dtype=torch.bfloat16, device=dev) for _ in sets]
    stream = torch.cuda.current_stream(dev)

    def step(i):
        t = sets[i % len(sets)]
        m.ssd_fwd(t["x"], t["delta_raw"], t["z"], t["Bt"], t["Ct"], t["A"], t["Dskip"], t["delta_bias"], P=cfg.P,
                  y=ys[i % len(sets)], stream=stream)

    settled = settle(step, args.settle_ms)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [a.elapsed_time(b) for a, b in ev]
    kern_ms = float(np.mean(per))
    ms_step = wall * 1e3 / args.steps
    nbytes = cfg.algorithmic_bytes()
    ach = nbytes / (kern_ms * 1e-3) / 1e9
    flops = ssd_mfma_flops(cfg)
    traffic, note = recorded_traffic(SSD_TRAFFIC_FILE, SSD_SOURCES)
    return {
        "metric": "Mamba-2 SSD layer HBM GB/s (% of MI355X peak) at a 2.7B-shaped layer",
        "value": round(nbytes / (ms_step * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle": settled, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "P": cfg.P, "N": cfg.N, "L": cfg.L,
                   "gate": cfg.gate, "input_sets": len(sets)},
        "elems_per_s": round(cfg.elements / (ms_step * 1e-3), 1),
        "kernel_ms_mean": round(kern_ms, 5),
        "kernel_ms_p10_p50_p90": [round(float(v), 5) for v in np.percentile(per, [10, 50, 90])],
        "roofline": {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic, "traffic_note": note,
                     "algorithmic_bytes": nbytes},
        "mfma": {"flops_per_launch": flops, "achieved_tflops": round(flops / (kern_ms * 1e-3) / 1e12, 1),
                 "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
                 "frac": round(flops / (kern_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
    }


def copy_calibration(args, dev):
    import torch
    n = args.copy_mb * (1 << 20) // 4
    a = torch.randn(n, device=dev)
    b = torch.empty_like(a)
    for _ in range(args.steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4,
                      "launches": args.steps}), flush=True)


def sub_args(args, **kw):
    """A copy of the command-line options for one of the nested workloads."""
    a = argparse.Namespace(**vars(args))
    a.seq_len = 0
    a.delta_b = False
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def headline(args, dev):
    """The default run: the 2.8B-layer scan line, with the other workloads of
    the path nested under "workloads" (each with its own roofline and CPU
    oracle baseline): the 48-layer decode step, the 130M layer and the
    batch-1 long sequence."""
    import torch
    from selective_state_space_75_amd import workloads as W
    line, cfg, x = bench_scan(sub_args(args, workload="mamba2.8b_layer"), dev)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle), mamba2.8b_layer ...")
        line["cpu_baseline"] = cpu_baseline_scan(cfg, x, args.cpu_seconds)
    del x
    if args.headline_only:
        return line
    nested = {}
    torch.cuda.empty_cache()
    dec = bench_decode(sub_args(args, warmup=min(args.warmup, 4)), dev)
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle), decode48 layers {0, 47} ...")
        dec["cpu_baseline"] = cpu_baseline_decode(W.DECODE_CONFIGS["decode48"])
    nested["decode48"] = dec
    torch.cuda.empty_cache()
    # (workload, timed steps, input sets, oracle sample channels, one-thread sample channels)
    for name, steps, sets, ch, ch1 in (("mamba130m_layer", min(args.steps, 50), 3, 0, 0),
                                       ("long_b1", min(args.steps, 10), 1, 512, 64)):
        ln, c, xx = bench_scan(sub_args(args, workload=name, steps=steps, sets=sets,
                                        warmup=min(args.warmup, 3)), dev)
        if not args.no_cpu_baseline:
            log("cpu baseline (oracle), %s ..." % name)
            ln["cpu_baseline"] = cpu_baseline_scan(c, xx, min(args.cpu_seconds, 6.0), channels=ch,
                                                   single_channels=ch1)
        del xx
        for k in ("metric", "n_gpus", "higher_is_better", "scaling", "data", "inputs"):
            ln.pop(k, None)
        nested[name] = ln
        torch.cuda.empty_cache()
    for k in ("metric", "n_gpus", "higher_is_better", "scaling", "data"):
        nested["decode48"].pop(k, None)
    line["workloads"] = nested
    return line


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed launches for this long before the warm-up steps (clock ramp; 0 = none)")
    ap.add_argument("--workload", default=None,
                    help="one workload only (default: the 2.8B-layer line with the decode, 130M-layer and "
                         "batch-1 long workloads nested)")
    ap.add_argument("--headline-only", action="store_true",
                    help="default run without the nested workloads")
    ap.add_argument("--sets", type=int, default=3, help="distinct input sets cycled over steps")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=128, help="decode48: timed steps (the workload has 128)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--copy-mb", type=int, default=1024)
    ap.add_argument("--seq-len", type=int, default=0,
                    help="scan workloads: another sequence length L (same B, D, N, dtype, seed)")
    ap.add_argument("--delta-b", action="store_true",
                    help="scan workloads: the simplified rule B-bar = delta B instead of zero-order hold")
    ap.add_argument("--scan-kernel", default="planner", choices=["planner", "wave_tile", "row", "row_lean", "general"],
                    help="diagnostic: force a scan kernel through the library's test knob")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        copy_calibration(args, dev)
        return
    from selective_state_space_75_amd import workloads as W
    if args.scan_kernel != "planner":
        import selective_state_space_75_amd as m
        m.set_test_knobs(scan_kernel=args.scan_kernel)
    if args.workload is None:
        line = headline(args, dev)
    elif args.workload == "decode48":
        line = bench_decode(args, dev)
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline_decode(W.DECODE_CONFIGS["decode48"])
    elif args.workload == "bwd_2.8b_layer":
        line = bench_bwd(args, dev)
    elif args.workload in W.CONV_CONFIGS:
        line = bench_conv(args, dev)
    elif args.workload in W.CONV_UPDATE_CONFIGS:
        line = bench_conv_decode(args, dev)
    elif args.workload in W.SSD_CONFIGS:
        line = bench_ssd(args, dev)
    else:
        line, cfg, x = bench_scan(args, dev)
        if not args.no_cpu_baseline and not args.delta_b:
            log("cpu baseline (oracle) ...")
            big = cfg.updates > 2e9
            line["cpu_baseline"] = cpu_baseline_scan(cfg, x, args.cpu_seconds, channels=512 if big else 0,
                                                     single_channels=64 if big else 0)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
