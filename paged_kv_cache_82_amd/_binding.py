"""ctypes binding of libpa.so (C ABI in include/pa.h): argument marshalling only.

Functions take torch tensors that live on the GPU (PyTorch provides device memory and the
stream) and pass their data pointers, sizes and the current HIP stream to the library; every
step of the computation runs in the library's kernels. A missing library raises: there is no
other implementation to fall back to.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(PKG, "libpa.so")
_lock = threading.Lock()
_lib = None

PA_OK = 0
_DTYPE_NAMES = {"float32": 0, "float16": 1, "bfloat16": 2}


class PAError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({pa_status_string(status)})")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libpa.so (once). Raises FileNotFoundError if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        p = path or _LIB_PATH
        # PyTorch ships its own HIP runtime whose soname equals the system one but which torch
        # requests by another file name. Importing torch first makes libpa bind to that single
        # runtime; loading libpa first would put two HIP runtimes in the process, and torch's
        # streams and allocations would be foreign to the one libpa launches on.
        import torch  # noqa: F401

        if not os.path.exists(p):
            raise FileNotFoundError(
                f"{p} is missing: build it first (python -m paged_kv_cache_82_amd.build)")
        lib = ctypes.CDLL(p)
        P, I, I64, F, SZ = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                            ctypes.c_size_t)
        lib.pa_write_kv.argtypes = [P, P, P, P, P, I, I, I, I, I64, I, P]
        lib.pa_write_kv.restype = I
        lib.pa_decode_workspace_size.argtypes = [I, I, I, I, I, I, I, I]
        lib.pa_decode_workspace_size.restype = SZ
        lib.pa_decode.argtypes = [P, P, P, P, P, P, F, I, I, I, I, I, I, I64, I, I, P, SZ, I, P]
        lib.pa_decode.restype = I
        lib.pa_decode_noalloc.argtypes = [P, P, P, P, P, P, F, I, I, I, I, I, I, I64, I, I, I, P]
        lib.pa_decode_noalloc.restype = I
        lib.pa_decode_append.argtypes = [P, P, P, P, P, P, P, P, P, F, I, I, I, I, I, I, I64, I,
                                         I, P, SZ, I, P]
        lib.pa_decode_append.restype = I
        lib.pa_decode_shared_prefix.argtypes = [P, P, P, P, P, P, P, P, F, I, I, I, I, I, I, I,
                                                I64, I, I, I, I, P, SZ, I, P]
        lib.pa_decode_shared_prefix.restype = I
        lib.pa_decode_shared_prefix_workspace_size.argtypes = [I] * 10 + [I]
        lib.pa_decode_shared_prefix_workspace_size.restype = SZ
        lib.pa_set_decode_kernel.argtypes = [I]
        lib.pa_set_decode_kernel.restype = I
        lib.pa_prefill.argtypes = [P, P, P, P, P, P, P, F, I, I, I, I, I, I, I, I64, I, I, I, P]
        lib.pa_prefill.restype = I
        lib.pa_copy_blocks.argtypes = [P, P, P, I, I, I, I, I64, I, P]
        lib.pa_copy_blocks.restype = I
        lib.pa_swap_blocks.argtypes = [P, P, I64, P, P, I64, P, I, I, I, I, I, P]
        lib.pa_swap_blocks.restype = I
        lib.pa_status_string.argtypes = [I]
        lib.pa_status_string.restype = ctypes.c_char_p
        _lib = lib
        return lib


def pa_status_string(status: int) -> str:
    try:
        return load().pa_status_string(int(status)).decode()
    except FileNotFoundError:
        return "library not loaded"


def _dtype_code(t) -> int:
    name = str(t.dtype).replace("torch.", "")
    if name not in _DTYPE_NAMES:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DTYPE_NAMES[name]


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _check(fn: str, status: int) -> None:
    if status != PA_OK:
        raise PAError(fn, status)


def pa_write_kv(k_cache, v_cache, k_new, v_new, slot_mapping, stream=None) -> None:
    """k_cache/v_cache [N, Hkv, B, d]; k_new/v_new [n, Hkv, d]; slot_mapping int32 [n]."""
    N, Hkv, B, d = k_cache.shape
    n = slot_mapping.shape[0]
    _check("pa_write_kv", load().pa_write_kv(
        _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), n, Hkv, d,
        B, N, _dtype_code(k_cache), _stream(stream)))


def pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                             max_context_len, partition_tokens, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _DTYPE_NAMES[str(dtype).replace("torch.", "")]
    return int(load().pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                               block_size, max_context_len, partition_tokens,
                                               code))


def pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
              workspace=None, partition_tokens=0, stream=None) -> None:
    """out, q [S, Hq, d]; pools [N, Hkv, B, d]; block_tables int32 [S, M]; context_lens int32
    [S]; workspace: a device uint8 tensor of >= pa_decode_workspace_size bytes (any
    contents; None when that size is 0)."""
    S, Hq, d = q.shape
    N, Hkv, B, _ = k_cache.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pa_decode", load().pa_decode(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        _ptr(context_lens), float(scale), S, Hq, Hkv, d, B, block_tables.shape[1], N,
        int(max_context_len), int(partition_tokens), _ptr(workspace), ws_bytes,
        _dtype_code(q), _stream(stream)))


def pa_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                      max_context_len, partition_tokens=0, stream=None) -> None:
    """pa_decode with the split-K partials in the library's static per-GPU scratch array (no
    workspace argument, no allocation); raises PAError(PA_ERR_WORKSPACE) when the partition
    plan needs more than PA_DECODE_SCRATCH_BYTES."""
    S, Hq, d = q.shape
    N, Hkv, B, _ = k_cache.shape
    _check("pa_decode_noalloc", load().pa_decode_noalloc(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        _ptr(context_lens), float(scale), S, Hq, Hkv, d, B, block_tables.shape[1], N,
        int(max_context_len), int(partition_tokens), _dtype_code(q), _stream(stream)))


def pa_decode_append(out, q, k_cache, v_cache, k_new, v_new, slot_mapping, block_tables,
                     context_lens, scale, max_context_len, workspace=None, partition_tokens=0,
                     stream=None) -> None:
    """The decode step's KV write and attention in one launch: k_new, v_new [S, Hkv, d] are
    every sequence's newest token (position context_lens[s] - 1), attended to directly and
    stored at slot_mapping[s] (int32 [S]; negative: not stored). Workspace as pa_decode."""
    S, Hq, d = q.shape
    N, Hkv, B, _ = k_cache.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pa_decode_append", load().pa_decode_append(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new),
        _ptr(slot_mapping), _ptr(block_tables), _ptr(context_lens), float(scale), S, Hq, Hkv, d,
        B, block_tables.shape[1], N, int(max_context_len), int(partition_tokens),
        _ptr(workspace), ws_bytes, _dtype_code(q), _stream(stream)))


def pa_decode_shared_prefix_workspace_size(num_seqs, num_groups, num_q_heads, num_kv_heads,
                                           head_dim, block_size, max_context_len,
                                           max_prefix_len, max_group_size, partition_tokens,
                                           dtype) -> int:
    code = dtype if isinstance(dtype, int) else _DTYPE_NAMES[str(dtype).replace("torch.", "")]
    return int(load().pa_decode_shared_prefix_workspace_size(
        num_seqs, num_groups, num_q_heads, num_kv_heads, head_dim, block_size, max_context_len,
        max_prefix_len, max_group_size, partition_tokens, code))


def pa_decode_shared_prefix(out, q, k_cache, v_cache, block_tables, context_lens, prefix_lens,
                            group_start, scale, max_context_len, max_prefix_len, max_group_size,
                            workspace=None, partition_tokens=0, stream=None) -> None:
    """pa_decode for groups of sequences sharing a prefix. prefix_lens int32 [S] (tokens each
    sequence shares with its group), group_start int32 [G + 1] (group i = sequences
    group_start[i] .. group_start[i+1]-1), both on the device; max_* are host-known bounds."""
    S, Hq, d = q.shape
    N, Hkv, B, _ = k_cache.shape
    G = group_start.shape[0] - 1
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("pa_decode_shared_prefix", load().pa_decode_shared_prefix(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        _ptr(context_lens), _ptr(prefix_lens), _ptr(group_start), float(scale), S, G, Hq, Hkv,
        d, B, block_tables.shape[1], N, int(max_context_len), int(max_prefix_len),
        int(max_group_size), int(partition_tokens), _ptr(workspace), ws_bytes, _dtype_code(q),
        _stream(stream)))


DECODE_KERNELS = {"auto": 0, "valu": 1, "mfma": 2}


def pa_set_decode_kernel(kernel: str) -> None:
    """Process-wide decode kernel choice: "auto" (default), "valu" or "mfma"."""
    _check("pa_set_decode_kernel", load().pa_set_decode_kernel(DECODE_KERNELS[kernel]))


def pa_prefill(out, q, k_cache, v_cache, block_tables, context_lens, query_start, scale,
               max_query_len, max_context_len, stream=None) -> None:
    """Causal multi-query attention. out, q [Nq, Hq, d]; pools [N, Hkv, B, d]; block_tables
    int32 [S, M]; context_lens int32 [S]; query_start int32 [S + 1] (rows of q per sequence);
    max_query_len / max_context_len: host-known bounds on the per-sequence counts."""
    Nq, Hq, d = q.shape
    N, Hkv, B, _ = k_cache.shape
    S = context_lens.shape[0]
    if query_start.shape[0] != S + 1:
        raise ValueError("query_start must have num_seqs + 1 entries")
    _check("pa_prefill", load().pa_prefill(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        _ptr(context_lens), _ptr(query_start), float(scale), S, Nq, Hq, Hkv, d, B,
        block_tables.shape[1], N, int(max_query_len), int(max_context_len), _dtype_code(q),
        _stream(stream)))


def pa_copy_blocks(k_cache, v_cache, block_pairs, stream=None) -> None:
    """block_pairs int32 [n, 2] of (src, dst) physical block ids."""
    N, Hkv, B, d = k_cache.shape
    _check("pa_copy_blocks", load().pa_copy_blocks(
        _ptr(k_cache), _ptr(v_cache), _ptr(block_pairs), block_pairs.shape[0], Hkv, d, B, N,
        _dtype_code(k_cache), _stream(stream)))


def pa_swap_blocks(dst_k, dst_v, src_k, src_v, block_pairs, stream=None) -> None:
    """Whole-block moves between two pools [N, Hkv, B, d] (device or pinned host tensors);
    block_pairs int32 [n, 2] of (src, dst), on the device."""
    Nd, Hkv, B, d = dst_k.shape
    Ns = src_k.shape[0]
    if tuple(src_k.shape[1:]) != (Hkv, B, d) or src_k.dtype != dst_k.dtype:
        raise ValueError("pools differ in block shape or dtype")
    _check("pa_swap_blocks", load().pa_swap_blocks(
        _ptr(dst_k), _ptr(dst_v), Nd, _ptr(src_k), _ptr(src_v), Ns, _ptr(block_pairs),
        block_pairs.shape[0], Hkv, d, B, _dtype_code(dst_k), _stream(stream)))
