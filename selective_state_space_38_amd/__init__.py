"""MI355X (gfx950) selective-scan (Mamba S6) library: a C-ABI shared library
with hand-written HIP kernels, and a thin PyTorch binding."""

from .api import (  # noqa: F401
    selective_scan_fwd,
    selective_scan_fwd_aggregate,
    selective_scan_carry_combine,
    selective_scan_bwd,
    ckpt_buffer,
    record_buffer,
    selective_state_update,
    causal_conv1d_fwd,
    causal_conv1d_update,
    mamba_block_fwd,
    check_device_errors,
    fwd_plan,
)
