"""MI355X-native Kimi Delta Attention (KDA): chunked forward, decode step and backward.

The compute lives in libkda.so (hand-written HIP for gfx950, C ABI in
include/kda.h).  This package is a thin ctypes binding: it turns torch tensors
into C descriptors and passes the current HIP stream; every step of the forward
pass runs in the library's kernels.  There is no fallback: if libkda.so is
missing or the tensors are not on the GPU, the call raises.
"""
from .binding import (KdaError, kda_bwd, kda_bwd_workspace_size, kda_decode, kda_dv_slices, kda_fwd, kda_fwd_cp,  # noqa: F401
                      kda_fwd_fused,
                      kda_fwd_cp_packed_workspace_size, kda_fwd_cp_plan, kda_fwd_cp_workspace_size, kda_fwd_intra, kda_fwd_noalloc,
                      kda_fwd_noalloc_max_bytes, kda_fwd_qg, kda_fwd_scan, kda_fwd_trace, kda_fwd_workspace_size, kda_fwd_ws,
                      library_path, load_library)

__all__ = ["KdaError", "kda_bwd", "kda_bwd_workspace_size", "kda_decode", "kda_dv_slices", "kda_fwd", "kda_fwd_cp", "kda_fwd_cp_plan", "kda_fwd_fused",
           "kda_fwd_cp_packed_workspace_size", "kda_fwd_cp_workspace_size", "kda_fwd_intra", "kda_fwd_noalloc", "kda_fwd_noalloc_max_bytes", "kda_fwd_qg", "kda_fwd_scan",
           "kda_fwd_ws", "kda_fwd_trace", "kda_fwd_workspace_size",
           "library_path", "load_library"]
