"""The scan recorded into a HIP graph and replayed with new inputs.

The balanced split hands states between workgroups through flagged slots in
the workspace.  A replay cannot take a new launch tag from the host, so a scan
recorded while its stream captures clears the flags with a kernel of its own
on every replay.  Each replay here runs on new inputs copied into the captured
buffers, with eager scans and synchronisations between the replays, and must
equal the eager result bit for bit (and the oracle to the usual bar).  The
balanced cases force the wave-tile kernel; the last case runs the planner's
kernel at a shape where that is the lean row kernel (no workspace).
"""
import numpy as np
import pytest

from helpers import assert_close, from_dev, gpu_scan, log, oracle_scan, upload_scan
from selective_state_space_75_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", [(2, 10240, 16, 128, 0, "wave_tile"), (1, 4096, 16, 320, 5, "wave_tile"),
                                   (4, 5120, 16, 2048, 0, "wave_tile"), (8, 5120, 16, 1024, 0, "planner"),
                                   (1, 256, 16, 1024, 4, "row")],
                         ids=["balanced", "chunked_balanced", "mamba2.8b_layer", "lean_row", "row_chunked"])
def test_scan_graph_replays_match_eager(shape, dev):
    import torch
    import selective_state_space_75_amd as m
    B, D, N, L, chunks, kernel = shape
    with m.test_knobs(scan_chunks=chunks, scan_kernel=kernel):
        wsb = m.workspace_size(B, D, N, L)
        if kernel != "planner":
            assert wsb > 0, "shape should need a workspace (hand-over slots or chunk carries)"
        sets = [W.custom_scan_inputs(B, D, N, L, "bf16", seed=9900 + k) for k in range(3)]
        bufs = upload_scan(sets[0], dev)
        y = torch.empty((B, D, L), dtype=torch.bfloat16, device=dev)
        h = torch.empty((B, D, N), dtype=torch.float32, device=dev)
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None
        side = torch.cuda.Stream(dev)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            gpu_scan(bufs, return_final_state=True, y=y, final_state=h, workspace=ws)
        torch.cuda.synchronize()
        for rep in range(6):
            x = sets[rep % 3]
            src = upload_scan(x, dev)
            for k in bufs:
                bufs[k].copy_(src[k])
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            y_g, h_g = y.clone(), h.clone()
            # eager work between the replays, on the same workspace
            y_e, h_e = gpu_scan(src, return_final_state=True, workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(y_g, y_e) and torch.equal(h_g, h_e), "replay %d differs from the eager scan" % rep
            if rep < 3:
                yr, _ = oracle_scan(x)
                assert_close(from_dev(y_g), yr, True, "replay %d y" % rep)
        log("  %s: 6 replays equal the eager scans" % (shape,))
