"""MI355X-native (gfx950) DeltaProduct forward: hand-written HIP kernels
behind a C ABI (include/dp.h, libdp.so), with a thin ctypes binding."""
from .binding import (  # noqa: F401
    DPError, EXPORTS, Pipeline, STAGE_ALL, STAGE_SCAN, STAGE_UT, alloc_workspace, bwd, bwd_workspace_size, decode, fwd,
    fwd_varlen, fwd_varlen_noalloc, launch_info, load,
    osdn_bwd, osdn_bwd_workspace_size, osdn_fwd, osdn_fwd_workspace_size, osdn_precond, osdn_precond_bwd,
    osdn_precond_varlen, osdn_precond_varlen_workspace_size,
    osdn_precond_bwd_workspace_size, status_str, varlen_workspace_size, workspace_size,
)
