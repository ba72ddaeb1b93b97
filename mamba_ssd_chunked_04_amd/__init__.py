"""Mamba-2 SSD chunked forward on MI355X (gfx950).

The compute path is the HIP library libssd_mi355x.so (C ABI in
include/ssd_mi355x.h); this package only binds it.  PyTorch supplies device
memory and streams.
"""
from .binding import (EXPORTED_SYMBOLS, NOALLOC_MAX_SCRATCH, SSD_ERR_WORKSPACE,  # noqa: F401
                      SsdCall, SsdDesc, SsdError, load_library, make_desc, plan, prepare,
                      prepare_bwd, rmsnorm_gated, causal_conv1d, causal_conv1d_tokmajor, ssd_bwd,
                      ssd_fwd, status_str, workspace_size)

__all__ = ["ssd_fwd", "ssd_bwd", "prepare_bwd", "rmsnorm_gated", "causal_conv1d",
           "causal_conv1d_tokmajor", "prepare", "plan", "workspace_size", "load_library", "make_desc",
           "SsdCall", "SsdDesc", "SsdError", "status_str", "EXPORTED_SYMBOLS",
           "NOALLOC_MAX_SCRATCH", "SSD_ERR_WORKSPACE"]
