"""MI355X (gfx950) Mamba-1 selective scan (S6) forward and selective state update,
with the causal conv1d + SiLU that produces the scan input, the scan's backward
pass, and the Mamba-2 (SSD) layer forward.

The computation runs in hand-written HIP kernels inside ``libmamba_scan.so``
(C ABI: ``include/mamba_scan.h``).  This package is the thin Python side:
``scan_fwd`` / ``scan_bwd`` / ``state_update`` / ``conv1d_fwd`` /
``conv1d_update`` / ``ssd_fwd`` marshal torch tensors to that library, and
``workloads`` draws the seeded synthetic inputs.
"""
from ._lib import (FLAG_ACCURATE_EXPM1, FLAG_DELTA_B, MambaError, conv1d_fwd, conv1d_update,  # noqa: F401
                   lib, scan_bwd, scan_bwd_workspace_size, scan_fwd, scan_fwd_noalloc, scan_kernel, set_test_knobs, ssd_fwd, ssd_workspace_size,
                   state_update, status_string, test_knobs, workspace_size)

__all__ = ["scan_fwd", "scan_bwd", "scan_bwd_workspace_size", "state_update", "conv1d_fwd", "conv1d_update",
           "ssd_fwd", "ssd_workspace_size", "workspace_size", "status_string", "lib", "MambaError", "FLAG_DELTA_B",
           "FLAG_ACCURATE_EXPM1", "set_test_knobs", "test_knobs", "scan_fwd_noalloc", "scan_kernel"]
