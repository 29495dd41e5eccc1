"""CPU oracle for paged decode attention — TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this package.
It shares no code with the GPU library: the C part (pa_oracle.c, built by `build()` with the
host compiler into liboracle.so) is the plain definition in double precision, and
`blockwise.py` restates the pages' block-wise forms in numpy for the oracle's self-checks.

Sources:
  [PA-summary]  azimuth.plus, "Efficient Memory Management for Large Language Model Serving
                with PagedAttention" (summary of Kwon et al., SOSP 2023).
  [PA-tutorial] un.csdn.net, "PagedAttention实战：如何用Python手搓一个高效KV缓存管理器".

Every function here is pinned by tests/test_oracle_pins.py (closed forms, library routines,
invariants, brute force on tiny inputs, and a mutation test showing that planted mistakes fail
a pin). No function is "parity unpinned".
"""
from .core import (build, copy_blocks, decode, lib_path, num_threads, prefill, round_to,
                   set_num_threads,
                   run_prefill_step, run_step, swap_blocks, widen, write_kv)

__all__ = ["build", "copy_blocks", "decode", "lib_path", "num_threads", "prefill", "round_to",
           "set_num_threads",
           "run_prefill_step", "run_step", "swap_blocks", "widen", "write_kv"]
