"""GPU parity of the one-state-per-lane (row) scan kernels against the oracle.

Both variants (row, and row_lean with fewer registers and less LDS per
workgroup) are selected with the scan_kernel test knob, so every case runs
them whatever the planner would choose: ragged channel counts (a workgroup's 16
channels and a wave's 4 only partly present), N < 16 (lanes holding no
state), one and two 32-step chunks, fp32 and bf16 inputs and outputs, the
simplified rule, the accurate flag, A = 0 and denormal A, small |A| in one
tile (the cancellation-free quotient for that workgroup only), absent z, D
and bias, the full 130M-layer and batch-1 long workloads (every output), and a
shape the planner itself gives to the lean kernel.
"""
import numpy as np
import pytest

from helpers import (BF16_MAX_ABS_FRAC, BF16_REL_L2, F32_OUT_REL_L2, BlockErr, assert_close, from_dev,
                     gpu_scan, log, oracle_scan, oracle_scan_blocks, rel_l2, upload_scan)
from selective_state_space_75_amd import workloads as W

pytestmark = pytest.mark.gpu

CASES = [
    # B, D, N, L, dtype, out, opts
    (1, 16, 16, 32, "f32", "f32", {}),
    (2, 70, 16, 64, "bf16", "bf16", {}),
    (3, 33, 5, 96, "bf16", "f32", {}),
    (2, 64, 7, 128, "f32", "f32", {"delta_b": True}),
    (2, 100, 16, 256, "bf16", "f32", {"accurate": True}),
    (2, 64, 16, 128, "f32", "f32", {"zero_A": True}),
    (2, 48, 16, 160, "bf16", "f32", {"small_A": True}),
    (1, 200, 16, 224, "f32", "f32", {"no_z": True, "no_dskip": True, "no_bias": True}),
    (4, 130, 16, 512, "bf16", "bf16", {"delta_b": True}),
    (1, 1, 1, 32, "f32", "f32", {}),
]


ROW_KERNELS = ["row", "row_lean"]

# The row kernel over L in chunks (forced chunk counts): chunk 0 in full and
# the middle chunks as summaries in one pass, the carry, then the other
# chunks from their carried states; ragged last chunks of 32 steps.
CHUNK_CASES = [
    # B, D, N, L, dtype, out, chunks, opts
    (1, 64, 16, 320, "bf16", "bf16", 3, {}),                      # chunks of 128, 128, 64
    (2, 70, 16, 640, "bf16", "f32", 4, {}),                       # 192 x 3 + 64, ragged channels
    (1, 33, 5, 96, "f32", "f32", 2, {}),                          # 64 + 32, N < 16
    (2, 48, 16, 256, "f32", "f32", 3, {"delta_b": True}),
    (1, 100, 16, 384, "bf16", "f32", 5, {"accurate": True}),      # 3 chunks of 128
    (2, 48, 16, 512, "bf16", "f32", 4, {"small_A": True}),
    (1, 40, 16, 448, "bf16", "bf16", 7, {"no_z": True, "no_dskip": True, "no_bias": True}),
]


@pytest.mark.parametrize("kernel", ROW_KERNELS)
@pytest.mark.parametrize("case", CASES, ids=lambda c: "B%dD%dN%dL%d_%s_%s_%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], "-".join(sorted(c[6])) or "plain"))
def test_row_kernel_cases(case, kernel, dev):
    import torch
    import selective_state_space_75_amd as m
    B, D, N, L, dt, odt, opts = case
    log("[%s] %s" % (kernel, case))
    x = W.custom_scan_inputs(B, D, N, L, dt, seed=6000 + B * 131 + D * 7 + L + N)
    if opts.get("zero_A"):
        A = x["A"].copy()
        A[::3, 1] = 0.0
        A[1::5, 4] = 1e-45
        x["A"] = A
    if opts.get("small_A"):
        A = x["A"].copy()
        A[:16, :] *= np.float32(1e-5)
        A[3, 2] = np.float32(-0.05)
        x["A"] = A
    t = upload_scan(x, dev)
    if opts.get("no_z"):
        t["z"] = None
    if opts.get("no_dskip"):
        t["Dskip"] = None
    if opts.get("no_bias"):
        t["delta_bias"] = None
    out_dtype = torch.float32 if odt == "f32" else torch.bfloat16
    with m.test_knobs(scan_kernel=kernel):
        assert m.scan_kernel(B, D, N, L) == kernel
        assert m.workspace_size(B, D, N, L) == 0
        y, hN = gpu_scan(t, return_final_state=True, out_dtype=out_dtype, delta_b=opts.get("delta_b", False),
                         accurate_expm1=opts.get("accurate", False))
    torch.cuda.synchronize()
    yr, hr = oracle_scan(x, use_z=not opts.get("no_z"), use_dskip=not opts.get("no_dskip"),
                         use_bias=not opts.get("no_bias"),
                         discretization="delta_b" if opts.get("delta_b") else "zoh")
    bf16 = dt == "bf16" or odt == "bf16"
    assert_close(from_dev(y), yr, bf16, "%s y" % kernel)
    e = rel_l2(from_dev(hN), hr)
    log("  final state rel_l2=%.3e" % e)
    assert e <= (2e-3 if dt == "bf16" else 1e-5)


@pytest.mark.parametrize("case", CHUNK_CASES, ids=lambda c: "B%dD%dN%dL%d_%s_%s_k%d_%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], "-".join(sorted(c[7])) or "plain"))
def test_row_kernel_chunked(case, dev):
    import torch
    import selective_state_space_75_amd as m
    B, D, N, L, dt, odt, chunks, opts = case
    log("[row chunked] %s" % (case,))
    x = W.custom_scan_inputs(B, D, N, L, dt, seed=6800 + B * 131 + D * 7 + L + N + chunks)
    if opts.get("small_A"):
        A = x["A"].copy()
        A[:16, :] *= np.float32(1e-5)
        x["A"] = A
    t = upload_scan(x, dev)
    if opts.get("no_z"):
        t["z"] = None
    if opts.get("no_dskip"):
        t["Dskip"] = None
    if opts.get("no_bias"):
        t["delta_bias"] = None
    out_dtype = torch.float32 if odt == "f32" else torch.bfloat16
    with m.test_knobs(scan_kernel="row", scan_chunks=chunks):
        assert m.scan_kernel(B, D, N, L) == "row"
        wsb = m.workspace_size(B, D, N, L)
        assert wsb > 0
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        y, hN = gpu_scan(t, return_final_state=True, out_dtype=out_dtype, delta_b=opts.get("delta_b", False),
                         accurate_expm1=opts.get("accurate", False), workspace=ws)
    torch.cuda.synchronize()
    yr, hr = oracle_scan(x, use_z=not opts.get("no_z"), use_dskip=not opts.get("no_dskip"),
                         use_bias=not opts.get("no_bias"),
                         discretization="delta_b" if opts.get("delta_b") else "zoh")
    bf16 = dt == "bf16" or odt == "bf16"
    assert_close(from_dev(y), yr, bf16, "row chunked y")
    e = rel_l2(from_dev(hN), hr)
    log("  final state rel_l2=%.3e" % e)
    assert e <= (2e-3 if dt == "bf16" else 1e-5)


@pytest.mark.parametrize("kernel", ROW_KERNELS)
def test_row_kernel_matches_wave_tile_kernel(kernel, dev):
    """On the fast quotient the row kernels keep the state scaled by A (g = A h,
    g_t = Abar_t (g_{t-1} + B_t u_t) - B_t u_t), which rounds differently from
    the wave-tile kernel's h_t = Abar_t h_{t-1} + ((Abar_t - 1)/A) B_t u_t: y
    and the final state agree with it to fp32 rounding."""
    import torch
    import selective_state_space_75_amd as m
    x = W.custom_scan_inputs(2, 256, 16, 1024, "bf16", seed=6500)
    t = upload_scan(x, dev)
    with m.test_knobs(scan_kernel=kernel):
        y1, h1 = gpu_scan(t, return_final_state=True, out_dtype=torch.float32)
    with m.test_knobs(scan_kernel="wave_tile"):
        y2, h2 = gpu_scan(t, return_final_state=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    eh = rel_l2(from_dev(h1), from_dev(h2))
    log("  %s vs wave-tile final state: rel_l2=%.3e" % (kernel, eh))
    assert eh <= 1e-6
    e = rel_l2(from_dev(y1), from_dev(y2))
    log("  %s vs wave-tile y: rel_l2=%.3e" % (kernel, e))
    assert e <= 1e-6


@pytest.mark.parametrize("name", ["mamba130m_layer", "long_b1"])
def test_row_kernel_full_workload(name, dev):
    """Every output of a full workload on both row kernels, bf16 and fp32
    output, against the oracle (run once, in 256-channel blocks); the batch-1
    long sequence also on the row kernel in one pass (its planned form is
    four chunks)."""
    import torch
    import selective_state_space_75_amd as m
    cfg = W.SCAN_CONFIGS[name]
    x = W.scan_inputs(cfg)
    t = upload_scan(x, dev)
    outs = {}
    variants = [(k, 0) for k in ROW_KERNELS] + ([("row", 1)] if name == "long_b1" else [])
    for kernel, chunks in variants:
        with m.test_knobs(scan_kernel=kernel, scan_chunks=chunks):
            wsb = m.workspace_size(cfg.B, cfg.D, cfg.N, cfg.L)
            ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None
            for odt in (torch.bfloat16, torch.float32):
                outs[("%s/%d" % (kernel, chunks), odt)] = gpu_scan(t, return_final_state=True, out_dtype=odt,
                                                                   workspace=ws)
    torch.cuda.synchronize()
    del t
    errs = {key: (BlockErr(), BlockErr()) for key in outs}
    for b, d0, d1, yr, hr in oracle_scan_blocks(x, block=256):
        for key, (ey, eh) in errs.items():
            y, hN = outs[key]
            ey.add(from_dev(y[b, d0:d1]), yr)
            eh.add(from_dev(hN[b, d0:d1]), hr)
    for kernel in sorted({k for k, _ in outs}):
        ey, eh = errs[(kernel, torch.bfloat16)]
        log("  %s %s y bf16: rel_l2=%.3e max_abs/max|y|=%.3e" % (name, kernel, ey.rel_l2, ey.max_abs_frac))
        assert ey.rel_l2 <= BF16_REL_L2 and ey.max_abs_frac <= BF16_MAX_ABS_FRAC
        ey, eh = errs[(kernel, torch.float32)]
        log("  %s %s y fp32: rel_l2=%.3e; final state rel_l2=%.3e" % (name, kernel, ey.rel_l2, eh.rel_l2))
        assert ey.rel_l2 <= F32_OUT_REL_L2 and eh.rel_l2 <= F32_OUT_REL_L2


def test_lean_row_kernel_on_planner_shape(dev):
    """A shape the planner gives to the lean row kernel (ten 16-channel tiles
    per CU: B=8, D=5120, L=1024), through the planner, every output and the
    final state against the oracle, bf16 and fp32 output."""
    import torch
    import selective_state_space_75_amd as m
    B, D, N, L = 8, 5120, 16, 1024
    assert m.scan_kernel(B, D, N, L) == "row_lean"
    assert m.workspace_size(B, D, N, L) == 0
    x = W.custom_scan_inputs(B, D, N, L, "bf16", seed=6700)
    t = upload_scan(x, dev)
    outs = {odt: gpu_scan(t, return_final_state=True, out_dtype=odt) for odt in (torch.bfloat16, torch.float32)}
    torch.cuda.synchronize()
    del t
    errs = {odt: (BlockErr(), BlockErr()) for odt in outs}
    for b, d0, d1, yr, hr in oracle_scan_blocks(x, block=1024):
        for odt, (ey, eh) in errs.items():
            y, hN = outs[odt]
            ey.add(from_dev(y[b, d0:d1]), yr)
            eh.add(from_dev(hN[b, d0:d1]), hr)
    ey, _ = errs[torch.bfloat16]
    log("  lean planner shape y bf16: rel_l2=%.3e max_abs/max|y|=%.3e" % (ey.rel_l2, ey.max_abs_frac))
    assert ey.rel_l2 <= BF16_REL_L2 and ey.max_abs_frac <= BF16_MAX_ABS_FRAC
    ey, eh = errs[torch.float32]
    log("  lean planner shape y fp32: rel_l2=%.3e; final state rel_l2=%.3e" % (ey.rel_l2, eh.rel_l2))
    assert ey.rel_l2 <= F32_OUT_REL_L2 and eh.rel_l2 <= F32_OUT_REL_L2
