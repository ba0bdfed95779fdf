"""MI355X-native Mamba-2 SSD chunked scan: gfx950 HIP kernels behind a C ABI (libssd.so).

    from state_space_sequence_mamba_amd import conv1d_silu, ssd_fwd, ssd_step, conv1d_silu_step
"""
from .ssd import (  # noqa: F401
    SsdError, conv1d_silu, conv1d_silu_step, load_library, make_dims, ssd_bwd, ssd_bwd_workspace_size, ssd_fwd,
    ssd_fwd_workspace_size, ssd_status_string, ssd_step, launch_opts, fwd_state_path,
)
