"""Complex-valued chunkwise state-space scan on AMD MI355X (gfx950).

The computation lives in ``libcssd.so`` (hand-written HIP kernels behind the C
ABI in ``include/cssd.h``); this package is a thin ctypes binding with the same
entry-point names.  Build the library with ``python -m
complex_valued_state_amd.build``.
"""
from ._binding import (CSSD_BF16, CSSD_F32, KERNEL_NAMES, LIB_PATH, CSSDError, cssd_backward,
                       cssd_backward_saved, cssd_born_attention,
                       cssd_backward_workspace_size, cssd_forward, cssd_forward_noalloc,
                       cssd_forward_workspace_size, CSSD_NOALLOC_SCRATCH_BYTES,
                       cssd_phase_scan, cssd_phase_scan_workspace_size, cssd_step,
                       cssd_step_infinite, cssd_step_n, cssd_version, load_library, profile,
                       status_string)

__all__ = ["cssd_forward", "cssd_forward_noalloc", "CSSD_NOALLOC_SCRATCH_BYTES", "cssd_backward", "cssd_backward_saved", "cssd_backward_workspace_size", "cssd_step",
           "cssd_step_n", "cssd_step_infinite", "cssd_phase_scan",
           "cssd_phase_scan_workspace_size", "cssd_born_attention",
           "cssd_forward_workspace_size", "cssd_version",
           "load_library", "profile", "status_string", "CSSDError", "CSSD_F32", "CSSD_BF16",
           "KERNEL_NAMES", "LIB_PATH"]
