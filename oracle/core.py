"""ctypes wrapper of the C oracle (pa_oracle.c). TEST INFRASTRUCTURE ONLY.

Element types follow the workloads' storage convention: "f32" float32, "f16" float16, "bf16"
uint16 bit patterns. All arrays must be C-contiguous in their storage type.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pa_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

_CODE = {"f32": 0, "f16": 1, "bf16": 2}
_STORAGE = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}
_ERR = {-1: "invalid sizes", -2: "block id outside the pool or table",
        -3: "duplicate or overlapping indices", -4: "allocation failure"}

_lock = threading.Lock()
_libs: dict = {}


def lib_path() -> str:
    return LIB


def build(src: str = SRC, out: str = LIB, cc: str = "gcc") -> str:
    """Compile the oracle with the host C compiler (IEEE arithmetic, no fast-math)."""
    tmp = out + ".tmp"
    cmd = [cc, "-O2", "-fopenmp", "-Wall", "-shared", "-fPIC", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    with _lock:
        _libs.pop(out, None)
    return out


def _load(path: str | None = None) -> ctypes.CDLL:
    path = path or LIB
    with _lock:
        if path in _libs:
            return _libs[path]
        if not os.path.exists(path):
            if path != LIB:
                raise FileNotFoundError(path)
            build()
        lib = ctypes.CDLL(path)
        P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.oracle_decode.argtypes = [P, P, P, P, P, P, D, I, I, I, I, I, I, I64, I, P, I]
        lib.oracle_prefill.argtypes = [P, P, P, P, P, P, P, D, I, I, I, I, I, I, I, I64, I]
        lib.oracle_write_kv.argtypes = [P, P, P, P, P, I, I, I, I, I64, I]
        lib.oracle_copy_blocks.argtypes = [P, P, P, I, I, I, I, I64, I]
        lib.oracle_swap_blocks.argtypes = [P, P, I64, P, P, I64, P, I, I, I, I, I]
        lib.oracle_round.argtypes = [P, P, I64, I]
        lib.oracle_widen.argtypes = [P, P, I64, I]
        for f in (lib.oracle_decode, lib.oracle_prefill, lib.oracle_write_kv, lib.oracle_copy_blocks,
                  lib.oracle_swap_blocks,
                  lib.oracle_round, lib.oracle_widen, lib.oracle_num_threads):
            f.restype = I
        _libs[path] = lib
        return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what}: {_ERR.get(rc, rc)}")


def _need(a: np.ndarray, dtype: str, name: str) -> np.ndarray:
    if a.dtype != _STORAGE[dtype] or not a.flags.c_contiguous:
        raise TypeError(f"{name} must be C-contiguous {_STORAGE[dtype].__name__} for {dtype}")
    return a


def num_threads(lib: str | None = None) -> int:
    return int(_load(lib).oracle_num_threads())


def set_num_threads(n: int, lib: str | None = None) -> None:
    """Threads the oracle's later calls use; timing only, results do not depend on it."""
    f = _load(lib).oracle_set_num_threads
    f.argtypes = [ctypes.c_int]
    f.restype = None
    f(int(n))


def widen(a: np.ndarray, dtype: str, lib: str | None = None) -> np.ndarray:
    a = _need(np.ascontiguousarray(a), dtype, "a")
    out = np.empty(a.shape, np.float64)
    _check(_load(lib).oracle_widen(_ptr(out), _ptr(a), a.size, _CODE[dtype]), "widen")
    return out


def round_to(x: np.ndarray, dtype: str, lib: str | None = None) -> np.ndarray:
    """Round float64 values to `dtype`, nearest-even; returns the storage representation."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    r = np.empty_like(x)
    _check(_load(lib).oracle_round(_ptr(r), _ptr(x), x.size, _CODE[dtype]), "round")
    if dtype == "f32":
        return r.astype(np.float32)
    if dtype == "f16":
        return r.astype(np.float16)  # exact: r is representable
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)  # exact likewise


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, dtype: str,
           seq_list=None, lib: str | None = None) -> np.ndarray:
    """Attention outputs in float64, shape [len(seq_list) or S, Hq, d]."""
    for name, a in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _need(a, dtype, name)
    S, Hq, d = q.shape
    N, Hkv, B, d2 = k_cache.shape
    if d2 != d or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    bt = np.ascontiguousarray(block_tables, np.int32)
    cl = np.ascontiguousarray(context_lens, np.int32)
    sl = None if seq_list is None else np.ascontiguousarray(seq_list, np.int32)
    n = S if sl is None else len(sl)
    out = np.empty((n, Hq, d), np.float64)
    rc = _load(lib).oracle_decode(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt), _ptr(cl), float(scale),
        S, Hq, Hkv, d, B, bt.shape[1] if bt.ndim == 2 else 0, N, _CODE[dtype], _ptr(sl), n)
    _check(rc, "decode")
    return out


def prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, dtype: str,
            lib: str | None = None) -> np.ndarray:
    """Causal multi-query attention in float64, shape [num_q_tokens, Hq, d].

    Query rows query_start[s] .. query_start[s+1]-1 are the last n_s tokens of sequence s
    (n_s <= context_lens[s]); query i of the sequence attends to positions 0 .. T-n_s+i."""
    for name, a in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _need(a, dtype, name)
    Nq, Hq, d = q.shape
    N, Hkv, B, d2 = k_cache.shape
    if d2 != d or v_cache.shape != k_cache.shape:
        raise ValueError("shape mismatch")
    bt = np.ascontiguousarray(block_tables, np.int32)
    cl = np.ascontiguousarray(context_lens, np.int32)
    qs = np.ascontiguousarray(query_start, np.int32)
    S = len(cl)
    if len(qs) != S + 1:
        raise ValueError("query_start must have num_seqs + 1 entries")
    out = np.zeros((Nq, Hq, d), np.float64)
    rc = _load(lib).oracle_prefill(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(bt), _ptr(cl), _ptr(qs),
        float(scale), S, Nq, Hq, Hkv, d, B, bt.shape[1] if bt.ndim == 2 else 0, N,
        _CODE[dtype])
    _check(rc, "prefill")
    return out


def write_kv(k_cache, v_cache, k_new, v_new, slot_mapping, dtype: str, lib: str | None = None):
    """In-place slot-mapped write of new keys/values into the pools."""
    for name, a in (("k_cache", k_cache), ("v_cache", v_cache), ("k_new", k_new),
                    ("v_new", v_new)):
        _need(a, dtype, name)
    N, Hkv, B, d = k_cache.shape
    sm = np.ascontiguousarray(slot_mapping, np.int32)
    rc = _load(lib).oracle_write_kv(_ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new),
                                    _ptr(sm), len(sm), Hkv, d, B, N, k_cache.itemsize)
    _check(rc, "write_kv")


def copy_blocks(k_cache, v_cache, pairs, dtype: str, lib: str | None = None):
    """In-place whole-block copies (src, dst)."""
    _need(k_cache, dtype, "k_cache")
    _need(v_cache, dtype, "v_cache")
    N, Hkv, B, d = k_cache.shape
    pr = np.ascontiguousarray(pairs, np.int32).reshape(-1, 2)
    rc = _load(lib).oracle_copy_blocks(_ptr(k_cache), _ptr(v_cache), _ptr(pr), len(pr), Hkv, d,
                                       B, N, k_cache.itemsize)
    _check(rc, "copy_blocks")


def swap_blocks(dst_k, dst_v, src_k, src_v, pairs, dtype: str, lib: str | None = None):
    """In-place whole-block moves between two pools: dst[pair[1]] = src[pair[0]]."""
    for name, a in (("dst_k", dst_k), ("dst_v", dst_v), ("src_k", src_k), ("src_v", src_v)):
        _need(a, dtype, name)
    Nd, Hkv, B, d = dst_k.shape
    if src_k.shape[1:] != dst_k.shape[1:]:
        raise ValueError("pools differ in block shape")
    pr = np.ascontiguousarray(pairs, np.int32).reshape(-1, 2)
    rc = _load(lib).oracle_swap_blocks(_ptr(dst_k), _ptr(dst_v), Nd, _ptr(src_k), _ptr(src_v),
                                       src_k.shape[0], _ptr(pr), len(pr), Hkv, d, B,
                                       dst_k.itemsize)
    _check(rc, "swap_blocks")


def run_prefill_step(step, in_place: bool = False, lib: str | None = None):
    """Apply a PrefillStep's KV writes (the chunk's new tokens) to the pools, then run causal
    multi-query attention. Returns (out64, k_cache, v_cache)."""
    kc = step.k_cache if in_place else step.k_cache.copy()
    vc = step.v_cache if in_place else step.v_cache.copy()
    for w in step.writes:
        write_kv(kc, vc, w.k_new, w.v_new, w.slot_mapping, step.dtype, lib)
    out = prefill(step.q, kc, vc, step.block_tables, step.context_lens, step.query_start,
                  step.scale, step.dtype, lib)
    return out, kc, vc


def run_step(step, seq_list=None, in_place: bool = False, lib: str | None = None):
    """Apply a DecodeStep's copies and writes to the pools, then decode.

    Returns (out64, k_cache, v_cache): outputs in float64 and the pools after the step."""
    kc = step.k_cache if in_place else step.k_cache.copy()
    vc = step.v_cache if in_place else step.v_cache.copy()
    if len(step.copies):
        copy_blocks(kc, vc, step.copies, step.dtype, lib)
    for w in step.writes:
        write_kv(kc, vc, w.k_new, w.v_new, w.slot_mapping, step.dtype, lib)
    out = decode(step.q, kc, vc, step.block_tables, step.context_lens, step.scale, step.dtype,
                 seq_list, lib)
    return out, kc, vc
