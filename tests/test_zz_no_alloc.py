"""mamba_scan_fwd_noalloc against mamba_scan_fwd.

The entry point without a workspace takes its scratch memory from the
library's own per-GPU buffer.  Two calls in a row, the second on a smaller
input, must each equal mamba_scan_fwd on the same inputs bit for bit (the same
kernels run on the same values; only where the scratch lives differs), and
the oracle to the bf16 bar.  On the wave-tile kernel the first call takes the
chunked path (summary, carry, a balanced full pass), the second the balanced
split alone; on the planner's kernel both calls take the row kernel's two
passes over chunks with the carry between them.  All of them use the
scratch.  A shape whose plan needs more scratch than the buffer holds
is refused before any launch (a host-side check, tested with the CPU tests).
"""
import pytest

from helpers import assert_close, from_dev, log, oracle_scan, upload_scan
from selective_state_space_75_amd import workloads as W

pytestmark = pytest.mark.gpu

NOALLOC_BYTES = 8 << 20


def test_noalloc_matches_workspace_entry_point(dev):
    import selective_state_space_75_amd as m
    # the wave-tile kernel forced (the planner scans the first shape with the
    # row kernel over chunks, tested below)
    for i, (B, D, N, L) in enumerate([(1, 4096, 16, 16384), (2, 10240, 16, 128)]):
        with m.test_knobs(scan_kernel="wave_tile"):
            _call(m, i, B, D, N, L, dev)


def test_noalloc_matches_workspace_entry_point_row_chunks(dev):
    import selective_state_space_75_amd as m
    for i, (B, D, N, L) in enumerate([(1, 4096, 16, 16384), (1, 2048, 16, 8192)]):
        assert m.scan_kernel(B, D, N, L) == "row"
        _call(m, 10 + i, B, D, N, L, dev)


def _call(m, i, B, D, N, L, dev):
    import torch
    wsb = m.workspace_size(B, D, N, L)
    log("[noalloc] call %d: B=%d D=%d N=%d L=%d (scratch %d bytes)" % (i, B, D, N, L, wsb))
    assert 0 < wsb <= NOALLOC_BYTES, "the shape should use the scratch buffer"
    x = W.custom_scan_inputs(B, D, N, L, "bf16", seed=9700 + i)
    t = upload_scan(x, dev)
    y_ref, h_ref = m.scan_fwd(t["u"], t["delta_raw"], t["z"], t["Bt"], t["Ct"], t["A"], t["Dskip"],
                              t["delta_bias"], return_final_state=True)
    y = torch.empty((B, D, L), dtype=torch.bfloat16, device=dev)
    h = torch.empty((B, D, N), dtype=torch.float32, device=dev)
    m.scan_fwd_noalloc(t["u"], t["delta_raw"], t["z"], t["Bt"], t["Ct"], t["A"], t["Dskip"],
                       t["delta_bias"], y=y, final_state=h)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref) and torch.equal(h, h_ref), "call %d differs from mamba_scan_fwd" % i
    yr, _ = oracle_scan(x)
    assert_close(from_dev(y), yr, True, "noalloc call %d y" % i)
