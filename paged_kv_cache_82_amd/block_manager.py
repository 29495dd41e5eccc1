"""Binding of libpa's host block manager (C ABI in include/pa_block_manager.h).

Argument marshalling only: every decision (free list, reference counts, on-demand allocation,
copy-on-write, moves between pools) is made by the native manager. Arrays come back as numpy
int32 arrays, ready to be copied to the device for pa_write_kv, pa_copy_blocks,
pa_swap_blocks, pa_decode and pa_prefill.
"""
from __future__ import annotations

import ctypes

import numpy as np

from ._binding import PAError, load

PA_OK = 0
PA_ERR_NO_BLOCKS = 5


class _Stats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "num_blocks", "free_blocks", "used_blocks", "shared_blocks", "logical_blocks",
        "num_seqs", "tokens", "filled_slots", "reserved_slots")]


class NoFreeBlocks(PAError):
    """The free list cannot cover the request; the manager is unchanged."""


_declared = False


def _lib():
    global _declared
    lib = load()
    if not _declared:
        P, I, I64, I32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int32
        sig = {
            "pa_bm_create": ([I64, I, P, P], I),
            "pa_bm_destroy": ([P], None),
            "pa_bm_add": ([P, I64], I),
            "pa_bm_fork": ([P, I64, I64], I),
            "pa_bm_blocks_needed": ([P, I64, I], I64),
            "pa_bm_append": ([P, I64, I, P, P, I, P], I),
            "pa_bm_release": ([P, I64], I),
            "pa_bm_move": ([P, P, I64, P, I, P], I),
            "pa_bm_length": ([P, I64], I64),
            "pa_bm_num_seq_blocks": ([P, I64], I),
            "pa_bm_tables": ([P, P, I, P, I, I32], I),
            "pa_bm_refcount": ([P, I64], I32),
            "pa_bm_get_stats": ([P, P], I),
            "pa_bm_prefix_groups": ([P, P, I, P, P, P], I),
        }
        for name, (args, res) in sig.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = res
        _declared = True
    return lib


def _check(fn: str, status: int) -> None:
    if status == PA_ERR_NO_BLOCKS:
        raise NoFreeBlocks(fn, status)
    if status != PA_OK:
        raise PAError(fn, status)


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


class BlockManager:
    """Free list and reference counts over `num_blocks` physical blocks of `block_size` slots.

    free_order: None (blocks handed out 0, 1, 2, ...) or a permutation of the block ids."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self._lib = _lib()
        self.block_size = int(block_size)
        self.num_blocks = int(num_blocks)
        h = ctypes.c_void_p()
        order = None
        if free_order is not None:
            order = np.ascontiguousarray(free_order, np.int32)
            if order.shape != (num_blocks,):
                raise ValueError("free_order must hold num_blocks ids")
        _check("pa_bm_create", self._lib.pa_bm_create(
            num_blocks, block_size, None if order is None else _p(order), ctypes.byref(h)))
        self._h = h

    def close(self) -> None:
        if getattr(self, "_h", None) and self._h.value:
            self._lib.pa_bm_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def add(self, seq: int) -> None:
        _check("pa_bm_add", self._lib.pa_bm_add(self._h, seq))

    def fork(self, parent: int, child: int) -> None:
        _check("pa_bm_fork", self._lib.pa_bm_fork(self._h, parent, child))

    def blocks_needed(self, seq: int, n_tokens: int) -> int:
        r = int(self._lib.pa_bm_blocks_needed(self._h, seq, n_tokens))
        if r < 0:
            raise KeyError(seq)
        return r

    def append(self, seq: int, n_tokens: int):
        """Slots (int32 [n_tokens]) and copy-on-write pairs (int32 [k, 2]) of the next
        n_tokens tokens of `seq`; the pairs must be copied before the tokens are written."""
        slots = np.empty(max(n_tokens, 1), np.int32)
        pairs = np.empty((2, 2), np.int32)  # an append copies at most one block
        n = ctypes.c_int(0)
        _check("pa_bm_append", self._lib.pa_bm_append(
            self._h, seq, n_tokens, _p(slots), _p(pairs), 2, ctypes.byref(n)))
        return slots[:n_tokens].copy(), pairs[: n.value].copy()

    def release(self, seq: int) -> None:
        _check("pa_bm_release", self._lib.pa_bm_release(self._h, seq))

    def move_to(self, other: "BlockManager", seq: int) -> np.ndarray:
        """Move `seq` into `other` (e.g. device pool -> host pool); returns the (src, dst)
        pairs for pa_swap_blocks."""
        nb = max(self.num_seq_blocks(seq), 1)
        pairs = np.empty((nb, 2), np.int32)
        n = ctypes.c_int(0)
        _check("pa_bm_move", self._lib.pa_bm_move(self._h, other._h, seq, _p(pairs), nb,
                                                  ctypes.byref(n)))
        return pairs[: n.value].copy()

    def length(self, seq: int) -> int:
        r = int(self._lib.pa_bm_length(self._h, seq))
        if r < 0:
            raise KeyError(seq)
        return r

    def num_seq_blocks(self, seq: int) -> int:
        r = int(self._lib.pa_bm_num_seq_blocks(self._h, seq))
        if r < 0:
            raise KeyError(seq)
        return r

    def tables(self, seqs, width: int | None = None, pad: int = -1) -> np.ndarray:
        """Dense int32 [len(seqs), width] block tables (pad beyond each table)."""
        ids = np.ascontiguousarray(seqs, np.int64)
        if width is None:
            width = max([self.num_seq_blocks(int(s)) for s in ids] + [1])
        out = np.empty((len(ids), width), np.int32)
        _check("pa_bm_tables", self._lib.pa_bm_tables(self._h, _p(ids), len(ids), _p(out),
                                                      width, pad))
        return out

    def prefix_groups(self, seqs):
        """(group_start int32 [G + 1], prefix_lens int32 [len(seqs)]): consecutive sequences
        whose tables start with the same block, and the tokens each shares with its group (the
        inputs of pa_decode_shared_prefix)."""
        ids = np.ascontiguousarray(seqs, np.int64)
        gs = np.empty(len(ids) + 1, np.int32)
        pl = np.empty(len(ids), np.int32)
        ng = ctypes.c_int(0)
        _check("pa_bm_prefix_groups", self._lib.pa_bm_prefix_groups(
            self._h, _p(ids), len(ids), _p(gs), ctypes.byref(ng), _p(pl)))
        return gs[: ng.value + 1].copy(), pl

    def refcount(self, block: int) -> int:
        return int(self._lib.pa_bm_refcount(self._h, block))

    def stats(self) -> dict:
        st = _Stats()
        _check("pa_bm_get_stats", self._lib.pa_bm_get_stats(self._h, ctypes.byref(st)))
        return {name: int(getattr(st, name)) for name, _ in _Stats._fields_}
