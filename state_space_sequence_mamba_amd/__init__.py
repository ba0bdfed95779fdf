"""MI355X-native Mamba-2 SSD chunked scan: gfx950 HIP kernels behind a C ABI (libssd.so).

    from state_space_sequence_mamba_amd import ssd_fwd, ssd_step
"""
from .ssd import (  # noqa: F401
    SsdError, load_library, make_dims, ssd_fwd, ssd_fwd_workspace_size, ssd_status_string, ssd_step, tune_set,
)
