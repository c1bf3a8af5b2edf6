"""Load-balanced split-KV decode attention with a fused RoPE/QK-Norm prologue, for MI355X.

The compute path is liblbsr.so (HIP kernels for gfx950 behind the C ABI in
include/lbsr.h); this package is its thin Python binding plus seeded input
generators (``workloads``).  Importing the package does not load the
library; the first call does, and raises ``LibraryNotBuilt`` if it is missing.
"""

from ._binding import LbsrError, LibraryNotBuilt, EXPORTS, LIB_PATH
from .decode import (DecodeConfig, Schedule, device_workers, workspace_layout,
                     alloc_workspace, rope_norm_kv_write, plan, attention, decode_step,
                     decode_step_timed, read_plan, read_error, xcd_rates,
                     xcd_weights_from_rates, prefill_attention, prefill_step,
                     prefill_attention_varlen, prefill_step_varlen,
                     prefill_workspace_size, alloc_prefill_workspace, stream_read,
                     decode_step_noalloc, pack_cache, unpack_cache)

__all__ = [
    "LbsrError", "LibraryNotBuilt", "EXPORTS", "LIB_PATH", "DecodeConfig", "Schedule",
    "device_workers", "workspace_layout", "alloc_workspace", "rope_norm_kv_write", "plan",
    "attention", "decode_step", "decode_step_timed", "read_plan", "read_error", "xcd_rates",
    "xcd_weights_from_rates", "prefill_attention", "prefill_step", "prefill_attention_varlen",
    "prefill_step_varlen", "prefill_workspace_size", "alloc_prefill_workspace", "stream_read",
    "decode_step_noalloc", "pack_cache", "unpack_cache",
]
