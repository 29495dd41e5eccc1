"""Seeded synthetic inputs shared by the GPU library's tests/benchmark and the CPU oracle.

Input plumbing only: random content, storage formats, block placement and the host toy block
manager that decides slots and copy-on-write pairs. No attention arithmetic lives here.
"""
from .alloc import (BlockAllocator, InOrder, PoolExhausted, Sequence, append_tokens, block_tables_array,
                    fork, prefix_groups, release, wasted_slots)
from .configs import (DecodeStep, KVWrite, PrefillStep, gqa32_bf16, gqa_bf16, gqa_lengths,
                      logical_kv,
                      long_bf16, long_lengths, make_prefill_step, make_step, mha13b_f16,
                      mha13b_lengths, prefill_gqa, prefill_mha13b, prefill_mha13b_f32,
                      shared_prefix_f16, tiny_f32)
from .numfmt import (DTYPE_CODE, DTYPES, ELEM_BYTES, STORAGE, bf16_bits_to_f32, f32_to_bf16_bits,
                     full, inf_value, nan_value, to_float64, to_storage)

__all__ = [
    "BlockAllocator", "InOrder", "PoolExhausted", "Sequence", "append_tokens", "block_tables_array", "fork",
    "prefix_groups", "release", "wasted_slots", "DecodeStep", "KVWrite", "PrefillStep", "tiny_f32",
    "mha13b_f16", "mha13b_lengths", "gqa32_bf16", "gqa_bf16", "gqa_lengths", "long_bf16", "long_lengths", "shared_prefix_f16", "logical_kv", "make_prefill_step",
    "make_step", "prefill_gqa", "prefill_mha13b", "prefill_mha13b_f32", "DTYPE_CODE",
    "DTYPES", "ELEM_BYTES", "STORAGE", "bf16_bits_to_f32", "f32_to_bf16_bits", "full",
    "inf_value", "nan_value", "to_float64", "to_storage",
]
