"""Seeded synthetic inputs shared by the GPU library's tests/benchmark and the CPU oracle.

Input plumbing only: random content, storage formats, block placement and the host toy block
manager that decides slots and copy-on-write pairs. No attention arithmetic lives here.
"""
from .alloc import (BlockAllocator, InOrder, PoolExhausted, Sequence, append_tokens, block_tables_array,
                    fork, release, wasted_slots)
from .configs import (CONFIGS, DecodeStep, KVWrite, PrefillStep, config1, config2, config3,
                      config4, config5, logical_kv, make_config, make_prefill_step, make_step,
                      prefill_gqa, prefill_mha13b)
from .numfmt import (DTYPE_CODE, DTYPES, ELEM_BYTES, STORAGE, bf16_bits_to_f32, f32_to_bf16_bits,
                     full, inf_value, nan_value, to_float64, to_storage)

__all__ = [
    "BlockAllocator", "InOrder", "PoolExhausted", "Sequence", "append_tokens", "block_tables_array", "fork",
    "release", "wasted_slots", "CONFIGS", "DecodeStep", "KVWrite", "PrefillStep", "config1",
    "config2", "config3", "config4", "config5", "logical_kv", "make_config", "make_prefill_step",
    "make_step", "prefill_gqa", "prefill_mha13b", "DTYPE_CODE",
    "DTYPES", "ELEM_BYTES", "STORAGE", "bf16_bits_to_f32", "f32_to_bf16_bits", "full",
    "inf_value", "nan_value", "to_float64", "to_storage",
]
