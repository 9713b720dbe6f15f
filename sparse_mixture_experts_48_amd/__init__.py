"""Top-K routed mixture-of-experts FFN layer (forward pass) for the AMD MI355X.

The compute lives in libmoe_mi355x.so (hand-written HIP for gfx950, C-ABI in
include/moe.h); this package holds its ctypes binding, the build script and the
seeded synthetic workloads.
"""
from . import workloads  # noqa: F401
from .binding import (MoeDesc, MoeError, MoELayer, Trace, backward, backward_workspace, capacity_slots,  # noqa: F401
                      combine, desc_of, expert_ffn, forward, forward_noalloc, header_symbols, lib, permute, route,
                      workspace, workspace_size)
