"""Paged KV-cache decode attention for AMD MI355X (gfx950).

The compute lives in libpa.so (hand-written HIP kernels behind the C ABI in include/pa.h);
this package is its thin Python binding. Importing it never falls back to any other code
path: if the library is missing, calls raise.
"""
from ._binding import (DECODE_KERNELS, PAError, lib_path, load, pa_copy_blocks, pa_decode,
                       pa_decode_append, pa_decode_noalloc, pa_decode_shared_prefix,
                       pa_decode_shared_prefix_workspace_size, pa_decode_workspace_size, pa_prefill,
                       pa_set_decode_kernel, pa_status_string, pa_swap_blocks, pa_write_kv)

SCRATCH_BYTES = 16 << 20  # PA_DECODE_SCRATCH_BYTES in include/pa.h

__all__ = ["DECODE_KERNELS", "PAError", "SCRATCH_BYTES", "lib_path", "load", "pa_copy_blocks",
           "pa_decode", "pa_decode_append", "pa_decode_noalloc", "pa_decode_shared_prefix",
           "pa_decode_shared_prefix_workspace_size", "pa_decode_workspace_size", "pa_prefill",
           "pa_set_decode_kernel", "pa_status_string", "pa_swap_blocks", "pa_write_kv"]
