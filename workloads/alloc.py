"""Host toy block manager that builds block tables, slot mappings and copy-on-write pairs.

Its semantics are those of the block manager the pages describe (the structure is this
project's own: batched requests checked against the pool before anything changes, as the
native manager does):
  - [PA-summary] azimuth.plus, "Efficient Memory Management for Large Language Model Serving
    with PagedAttention", sections "Key idea: virtual memory for the KV cache" (blocks are
    allocated one at a time, on demand, as tokens are generated), "vLLM" (the block manager
    keeps the free physical blocks and reference counts of shared blocks) and "Memory sharing:
    copy-on-write" (a write into a shared block first copies that block only);
  - [PA-tutorial] un.csdn.net, "PagedAttention实战：如何用Python手搓一个高效KV缓存管理器",
    §2.2 BlockManager (a free list popped from the end; allocation fails when it is empty),
    §3.1 append_kv (page = pos // page_size, offset = pos % page_size) and §5.1 clone_sequence
    (a fork shares every page and raises its reference count).

Reading where the pages leave the step open: when a shared block (reference count r > 1) is
written, the writer copies it and the count drops by one; the last holder (r == 1) writes in
place. The allocator is host logic for tests and benchmarks; the GPU library only consumes the
tables, slots and pairs it produces.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


class PoolExhausted(MemoryError):
    """No free physical block is left."""


class InOrder:
    """Stands in for a Generator in BlockAllocator: hands out block ids in increasing order
    (contiguous placement; used to measure what scattering costs)."""

    @staticmethod
    def permutation(n):
        return np.arange(n)


class BlockAllocator:
    """Reference counts and a stack of free block ids over `num_blocks` physical blocks.

    Blocks are handed out from the top of the stack. It starts as the seeded permutation
    (first element on top), so consecutive requests land at scattered physical positions, and a
    block whose count falls to zero goes back on top (the last freed is the next handed out)."""

    def __init__(self, num_blocks: int, rng: np.random.Generator | None = None):
        if num_blocks < 0:
            raise ValueError("num_blocks must be >= 0")
        self.num_blocks = int(num_blocks)
        order = np.arange(num_blocks) if rng is None else np.asarray(rng.permutation(num_blocks))
        self._stack = np.asarray(order[::-1], dtype=np.int64).copy()  # top = last element
        self._top = self.num_blocks
        self.ref = np.zeros(num_blocks, dtype=np.int64)

    @property
    def num_free(self) -> int:
        return self._top

    def take(self, count: int) -> np.ndarray:
        """`count` blocks off the top of the stack, in hand-out order, each with count 1."""
        if count > self._top:
            raise PoolExhausted("no free physical blocks")
        got = self._stack[self._top - count: self._top][::-1].copy()
        self._top -= count
        assert (self.ref[got] == 0).all()
        self.ref[got] = 1
        return got

    def share(self, blocks) -> None:
        """One more holder for each of `blocks`."""
        b = np.asarray(blocks, dtype=np.int64)
        assert (self.ref[b] > 0).all()
        np.add.at(self.ref, b, 1)

    def drop(self, blocks) -> None:
        """One holder less for each of `blocks`, in order; blocks left with none go back on the
        stack in that order."""
        for b in (int(x) for x in blocks):
            assert self.ref[b] > 0
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self._stack[self._top] = b
                self._top += 1


@dataclass
class Sequence:
    """Logical-to-physical block map and current length of one sequence."""

    block_size: int
    table: list = field(default_factory=list)
    length: int = 0


def append_tokens(alloc: BlockAllocator, seq: Sequence, n: int):
    """Reserve slots for `n` new tokens of `seq` ([PA-summary] "Key idea": a block is taken when
    a token starts it; "Memory sharing: copy-on-write": a write into a block that other
    sequences still hold goes to a private copy of that block alone).

    What the request needs is worked out first: a copy of the partly filled last block when
    others hold it too, and the blocks that the new length adds. It is taken from the pool in
    one step (PoolExhausted, with nothing changed, if the pool cannot cover it). Returns (slots,
    cow_pairs): slots[i] = physical block * B + offset of token seq.length + i; cow_pairs are
    the (src, dst) whole-block copies that must run before the tokens are written."""
    B = seq.block_size
    if n <= 0:
        return [], []
    last = seq.length // B
    copy_last = seq.length % B != 0 and alloc.ref[seq.table[last]] > 1
    grow = -(-(seq.length + n) // B) - len(seq.table)
    got = alloc.take(int(copy_last) + grow)
    pairs = []
    if copy_last:  # the writer repoints to its copy; the others keep the original
        old = seq.table[last]
        seq.table[last] = int(got[0])
        alloc.drop([old])
        pairs.append((old, int(got[0])))
    seq.table.extend(int(b) for b in got[int(copy_last):])
    pos = seq.length + np.arange(n)
    slots = (np.asarray(seq.table, dtype=np.int64)[pos // B] * B + pos % B).tolist()
    seq.length += n
    return slots, pairs


def fork(alloc: BlockAllocator, seq: Sequence) -> Sequence:
    """A child that shares every block of `seq` ([PA-tutorial] §5.1: the page table is copied
    and every page gains a holder)."""
    alloc.share(seq.table)
    return Sequence(seq.block_size, list(seq.table), seq.length)


def release(alloc: BlockAllocator, seq: Sequence) -> None:
    alloc.drop(seq.table)
    seq.table.clear()
    seq.length = 0


def block_tables_array(seqs, pad: int = -1, min_width: int = 1) -> np.ndarray:
    """Dense int32 [S, max_blocks] table, unused entries set to `pad`."""
    width = max([len(s.table) for s in seqs] + [min_width])
    out = np.full((len(seqs), width), pad, dtype=np.int32)
    for i, s in enumerate(seqs):
        out[i, : len(s.table)] = s.table
    return out


def wasted_slots(seq: Sequence) -> int:
    """Reserved-but-unused token slots of one sequence (internal fragmentation)."""
    return len(seq.table) * seq.block_size - seq.length


def prefix_groups(block_tables, context_lens, block_size):
    """The sharing structure of a batch, read off its block tables: runs of consecutive
    sequences whose tables start with the same physical block form a group; a group's shared
    tokens are its members' common leading table entries times the block size, capped by its
    shortest member (0 for a group of one). Returns (group_start int32 [G + 1], prefix_lens
    int32 [S]), the description pa_decode_shared_prefix takes."""
    S = len(context_lens)
    nblk = [-(-int(t) // block_size) for t in context_lens]
    starts, pl, i = [], np.zeros(S, np.int32), 0
    while i < S:
        j = i + 1
        while (j < S and nblk[i] > 0 and nblk[j] > 0
               and block_tables[j, 0] == block_tables[i, 0]):
            j += 1
        if j - i > 1:
            c = 0
            while all(c < nblk[k] and block_tables[k, c] == block_tables[i, c]
                      for k in range(i, j)):
                c += 1
            pl[i:j] = min(c * block_size, int(min(context_lens[i:j])))
        starts.append(i)
        i = j
    starts.append(S)
    return np.asarray(starts, np.int32), pl
