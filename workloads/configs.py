"""Seeded synthetic decode-step workloads for paged attention (numpy only).

A DecodeStep is one decode iteration of a batch: the block pool as it stands before the step,
the copy-on-write pairs and KV writes the step performs (in that order), then one query per
sequence and query head to attend over the updated cache. The GPU library and the CPU oracle
consume the same arrays; nothing here computes attention.

Content recipe (identical for both sides):
  - keys and values are drawn per logical token, N(0,1) in float32, then rounded to the element
    type; chunk k (4096 tokens) of sequence s comes from SeedSequence(seed, spawn_key=(0|1, s,
    k)) so content does not depend on physical placement, threading or pool size;
  - queries come from SeedSequence(seed, spawn_key=(2, s));
  - structure (context lengths, placement) comes from default_rng(seed);
  - physical blocks are handed out by the toy BlockAllocator, whose free list is a seeded
    permutation of the pool, so tables point at scattered blocks;
  - every sequence's last token arrives through the step's KV write (slot mapping);
  - with poison=True, every slot not holding a token (unused blocks, tails of last blocks) is
    NaN, and table entries past a sequence's blocks are -1.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

from .alloc import BlockAllocator, Sequence, append_tokens, block_tables_array, fork
from .numfmt import ELEM_BYTES, STORAGE, check_dtype, full, nan_value, to_storage

CHUNK = 4096


@dataclass
class KVWrite:
    k_new: np.ndarray  # [n, Hkv, d]
    v_new: np.ndarray  # [n, Hkv, d]
    slot_mapping: np.ndarray  # int32 [n]


@dataclass
class DecodeStep:
    name: str
    seed: int
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    k_cache: np.ndarray  # [N, Hkv, B, d], state before the step
    v_cache: np.ndarray
    q: np.ndarray  # [S, Hq, d]
    block_tables: np.ndarray  # int32 [S, max_blocks]
    context_lens: np.ndarray  # int32 [S], after the step's writes
    copies: np.ndarray  # int32 [n_pairs, 2], applied first
    writes: list = field(default_factory=list)  # KVWrite, applied in order after the copies
    scale: np.float32 = np.float32(0)
    logical_k: list | None = None  # per sequence [T, Hkv, d] (small cases only)
    logical_v: list | None = None
    notes: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.size else 0

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.dtype]


def _normal(seed: int, key: tuple, shape) -> np.ndarray:
    rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=key))
    return rng.standard_normal(shape, dtype=np.float32)


def logical_kv(seed: int, s: int, T: int, Hkv: int, d: int, dtype: str, which: int):
    """Keys (which=0) or values (which=1) of tokens 0..T-1 of content stream s."""
    out = np.empty((T, Hkv, d), dtype=STORAGE[dtype])
    for k in range(0, (T + CHUNK - 1) // CHUNK):
        lo, hi = k * CHUNK, min(T, (k + 1) * CHUNK)
        out[lo:hi] = to_storage(_normal(seed, (which, s, k), (hi - lo, Hkv, d)), dtype)
    return out


def _scatter(pool: np.ndarray, table, data: np.ndarray, start: int, B: int) -> None:
    """Place tokens start..start+len(data)-1 of a sequence into pool via its table."""
    n = data.shape[0]
    t = 0
    while t < n:
        pos = start + t
        j, off = divmod(pos, B)
        take = min(B - off, n - t)
        pool[table[j], :, off : off + take, :] = np.swapaxes(data[t : t + take], 0, 1)
        t += take


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def make_step(name: str, seed: int, lengths, num_q_heads: int, num_kv_heads: int, head_dim: int,
              block_size: int, dtype: str, num_blocks: int | None = None,
              pool_factor: float = 1.2, poison: bool = True, keep_logical: bool = False,
              alloc_rng: np.random.Generator | None = None,
              scale: float | None = None) -> DecodeStep:
    """General decode step: each sequence holds T-1 prefilled tokens and its T-th token is
    written by the step (a sequence with T == 0 gets no token)."""
    check_dtype(dtype)
    lengths = [int(t) for t in lengths]
    S, Hkv, d, B = len(lengths), num_kv_heads, head_dim, block_size
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    need = sum(math.ceil(t / B) for t in lengths)
    if num_blocks is None:
        num_blocks = max(1, math.ceil(pool_factor * need))
    if alloc_rng is None:
        alloc_rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(3,)))
    alloc = BlockAllocator(num_blocks, alloc_rng)

    fill = nan_value(dtype) if poison else 0
    k_cache = full((num_blocks, Hkv, B, d), fill, dtype)
    v_cache = full((num_blocks, Hkv, B, d), fill, dtype)

    seqs = [Sequence(B) for _ in range(S)]
    for s, T in enumerate(lengths):
        if T > 0:
            append_tokens(alloc, seqs[s], T - 1)

    def prefill(s):
        T = lengths[s]
        if T == 0:
            return None
        kk = logical_kv(seed, s, T, Hkv, d, dtype, 0)
        vv = logical_kv(seed, s, T, Hkv, d, dtype, 1)
        _scatter(k_cache, seqs[s].table, kk[: T - 1], 0, B)
        _scatter(v_cache, seqs[s].table, vv[: T - 1], 0, B)
        last = (kk[T - 1].copy(), vv[T - 1].copy())
        return (kk, vv, last) if keep_logical else (None, None, last)

    with ThreadPoolExecutor(_workers()) as ex:
        res = list(ex.map(prefill, range(S)))

    # The step: one new token per sequence through the slot mapping.
    k_new, v_new, slots = [], [], []
    for s, T in enumerate(lengths):
        if T == 0:
            continue
        sl, pairs = append_tokens(alloc, seqs[s], 1)
        assert not pairs
        slots.extend(sl)
        k_new.append(res[s][2][0])
        v_new.append(res[s][2][1])
    shape = (0, Hkv, d)
    write = KVWrite(
        np.stack(k_new) if k_new else np.empty(shape, STORAGE[dtype]),
        np.stack(v_new) if v_new else np.empty(shape, STORAGE[dtype]),
        np.asarray(slots, dtype=np.int32),
    )
    qs = np.stack([to_storage(_normal(seed, (2, s), (num_q_heads, d)), dtype) for s in range(S)])
    step = DecodeStep(
        name=name, seed=seed, dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=Hkv,
        head_dim=d, block_size=B, k_cache=k_cache, v_cache=v_cache, q=qs,
        block_tables=block_tables_array(seqs), context_lens=np.asarray(lengths, np.int32),
        copies=np.zeros((0, 2), np.int32), writes=[write],
        scale=np.float32(1.0 / math.sqrt(d) if scale is None else scale),
    )
    if keep_logical:
        step.logical_k = [r[0] if r else np.empty(shape, STORAGE[dtype]) for r in res]
        step.logical_v = [r[1] if r else np.empty(shape, STORAGE[dtype]) for r in res]
    step.notes["blocks_needed"] = need
    return step


# ---- multi-query (prefill / chunked-prefill) steps --------------------------------------------


@dataclass
class PrefillStep:
    """One chunked-prefill iteration: sequence s already holds its first T_s - n_s tokens; the
    step writes its next n_s tokens through the slot mapping and runs causal attention for
    those n_s query tokens (query i of s sees positions 0 .. T_s - n_s + i)."""

    name: str
    seed: int
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    k_cache: np.ndarray  # [N, Hkv, B, d], state before the step
    v_cache: np.ndarray
    q: np.ndarray  # [num_q_tokens, Hq, d], sequences one after another
    block_tables: np.ndarray  # int32 [S, max_blocks]
    context_lens: np.ndarray  # int32 [S], T_s after the step's write
    query_start: np.ndarray  # int32 [S + 1]
    writes: list = field(default_factory=list)
    scale: np.float32 = np.float32(0)
    logical_k: list | None = None
    logical_v: list | None = None
    notes: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def num_q_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def query_lens(self) -> np.ndarray:
        return np.diff(self.query_start)

    @property
    def max_query_len(self) -> int:
        return int(self.query_lens.max()) if self.num_seqs else 0

    @property
    def num_blocks(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def max_context_len(self) -> int:
        return int(self.context_lens.max()) if self.context_lens.size else 0

    @property
    def elem_bytes(self) -> int:
        return ELEM_BYTES[self.dtype]


def make_prefill_step(name: str, seed: int, context_lens, query_lens, num_q_heads: int,
                      num_kv_heads: int, head_dim: int, block_size: int, dtype: str,
                      num_blocks: int | None = None, pool_factor: float = 1.2,
                      poison: bool = True, keep_logical: bool = False,
                      alloc_rng: np.random.Generator | None = None,
                      scale: float | None = None) -> PrefillStep:
    """Sequence s ends with T_s = context_lens[s] tokens of which the last n_s = query_lens[s]
    arrive in this step (keys/values written through the slot mapping, queries in q)."""
    check_dtype(dtype)
    T_all = [int(t) for t in context_lens]
    n_all = [int(n) for n in query_lens]
    if len(T_all) != len(n_all) or any(n < 0 or n > t for t, n in zip(T_all, n_all)):
        raise ValueError("need 0 <= query_lens[s] <= context_lens[s]")
    S, Hkv, d, B = len(T_all), num_kv_heads, head_dim, block_size
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    need = sum(math.ceil(t / B) for t in T_all)
    if num_blocks is None:
        num_blocks = max(1, math.ceil(pool_factor * need))
    if alloc_rng is None:
        alloc_rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(3,)))
    alloc = BlockAllocator(num_blocks, alloc_rng)
    fill = nan_value(dtype) if poison else 0
    k_cache = full((num_blocks, Hkv, B, d), fill, dtype)
    v_cache = full((num_blocks, Hkv, B, d), fill, dtype)

    seqs = [Sequence(B) for _ in range(S)]
    for s in range(S):
        append_tokens(alloc, seqs[s], T_all[s] - n_all[s])

    def prior(s):
        T, n = T_all[s], n_all[s]
        kk = logical_kv(seed, s, T, Hkv, d, dtype, 0)
        vv = logical_kv(seed, s, T, Hkv, d, dtype, 1)
        _scatter(k_cache, seqs[s].table, kk[: T - n], 0, B)
        _scatter(v_cache, seqs[s].table, vv[: T - n], 0, B)
        return kk, vv

    with ThreadPoolExecutor(_workers()) as ex:
        res = list(ex.map(prior, range(S)))

    k_new, v_new, slots = [], [], []
    for s in range(S):
        T, n = T_all[s], n_all[s]
        sl, pairs = append_tokens(alloc, seqs[s], n)
        assert not pairs
        slots.extend(sl)
        k_new.append(res[s][0][T - n:])
        v_new.append(res[s][1][T - n:])
    shape = (0, Hkv, d)
    write = KVWrite(
        np.concatenate(k_new) if k_new else np.empty(shape, STORAGE[dtype]),
        np.concatenate(v_new) if v_new else np.empty(shape, STORAGE[dtype]),
        np.asarray(slots, dtype=np.int32),
    )
    qs = [to_storage(_normal(seed, (4, s), (n_all[s], num_q_heads, d)), dtype) for s in range(S)]
    q = np.concatenate(qs) if qs else np.empty((0, num_q_heads, d), STORAGE[dtype])
    step = PrefillStep(
        name=name, seed=seed, dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=Hkv,
        head_dim=d, block_size=B, k_cache=k_cache, v_cache=v_cache,
        q=np.ascontiguousarray(q), block_tables=block_tables_array(seqs),
        context_lens=np.asarray(T_all, np.int32),
        query_start=np.concatenate([[0], np.cumsum(n_all)]).astype(np.int32),
        writes=[write],
        scale=np.float32(1.0 / math.sqrt(d) if scale is None else scale),
    )
    if keep_logical:
        step.logical_k = [r[0] for r in res]
        step.logical_v = [r[1] for r in res]
    step.notes["blocks_needed"] = need
    return step


def prefill_mha13b(**kw) -> PrefillStep:
    """Chunked prefill, 13B shape, fp16 MHA: 16 sequences, 40 heads, d=128, B=16; each appends a
    512-token chunk to a cached prefix of lognormal length (median 512, sigma 1) clipped to
    [0, 1536], so T <= 2048."""
    rng = np.random.default_rng(6)
    prefix = np.clip(np.rint(rng.lognormal(math.log(512.0), 1.0, size=16)), 0, 1536)
    n = np.full(16, 512)
    return make_prefill_step("prefill-mha13b-f16", 6, prefix + n, n, 40, 40, 128, 16, "f16", **kw)


def prefill_mha13b_f32(**kw) -> PrefillStep:
    """Chunked prefill in fp32 (the vector-ALU prefill kernel), 13B shape: 16 sequences, 40
    heads, d=128, B=16; each appends a 64-token chunk to the same lognormal prefixes as the fp16
    workload."""
    rng = np.random.default_rng(6)
    prefix = np.clip(np.rint(rng.lognormal(math.log(512.0), 1.0, size=16)), 0, 1536)
    n = np.full(16, 64)
    return make_prefill_step("prefill-mha13b-f32", 6, prefix + n, n, 40, 40, 128, 16, "f32", **kw)


def prefill_gqa(**kw) -> PrefillStep:
    """Chunked prefill, GQA bf16: 16 sequences, 64 query heads over 8 KV heads, d=128, B=16;
    each appends a 1024-token chunk to a cached prefix of length uniform in [0, 3072]."""
    prefix = np.random.default_rng(7).integers(0, 3072 + 1, size=16)
    n = np.full(16, 1024)
    return make_prefill_step("prefill-gqa-bf16", 7, prefix + n, n, 64, 8, 128, 16, "bf16", **kw)


# ---- the decode workloads ---------------------------------------------------------------------


def tiny_f32(**kw) -> DecodeStep:
    """Tiny fp32: 4 sequences of lengths 7, 16, 33, 50; 8 heads, d=64, B=16, 64-block pool."""
    return make_step("tiny-f32", 1, [7, 16, 33, 50], 8, 8, 64, 16, "f32", num_blocks=64, **kw)


def mha13b_lengths(seed: int = 2, S: int = 64) -> np.ndarray:
    rng = np.random.default_rng(seed)
    t = np.rint(rng.lognormal(mean=math.log(512.0), sigma=1.0, size=S))
    return np.clip(t, 16, 2048).astype(np.int64)


def mha13b_f16(**kw) -> DecodeStep:
    """13B-shape fp16 MHA: 64 sequences, 40 heads, d=128, B=16, lengths lognormal (median
    512, sigma 1) clipped to [16, 2048], pool 1.2x the blocks needed."""
    return make_step("mha13b-f16", 2, mha13b_lengths(), 40, 40, 128, 16, "f16", **kw)


def gqa_lengths(seed: int = 3, S: int = 256) -> np.ndarray:
    return np.random.default_rng(seed).integers(128, 4096 + 1, size=S)


def gqa_bf16(**kw) -> DecodeStep:
    """GQA bf16: 256 sequences, 64 query heads over 8 KV heads, d=128, B=16, lengths uniform
    in [128, 4096]."""
    return make_step("gqa-bf16", 3, gqa_lengths(), 64, 8, 128, 16, "bf16", **kw)


def gqa32_bf16(**kw) -> DecodeStep:
    """Wide-group GQA bf16 (32 query heads per KV head, two 16-head MFMA tiles): 128 sequences,
    64 query heads over 2 KV heads, d=128, B=16, lengths uniform in [128, 4096] (a measurement
    of K/V re-reads across head tiles, not one of the headline workloads)."""
    return make_step("gqa32-bf16", 8, gqa_lengths(8, 128), 64, 2, 128, 16, "bf16", **kw)


def long_lengths(seed: int = 4, S: int = 8) -> np.ndarray:
    return np.random.default_rng(seed).integers(32768, 131072 + 1, size=S)


def long_bf16(**kw) -> DecodeStep:
    """Long-context bf16: 8 sequences, 32 heads, d=128, B=16, lengths uniform in
    [32768, 131072]; the split-K partition-and-merge path."""
    return make_step("long-bf16", 4, long_lengths(), 32, 32, 128, 16, "bf16", **kw)


def shared_prefix_f16(private: bool = False, prompts: int = 16, samples: int = 4,
                      prompt_len: int = 1040, tail_len: int = 256, heads: int = 32,
                      head_dim: int = 128, block_size: int = 32, dtype: str = "f16",
                      seed: int = 5, poison: bool = True,
                      keep_logical: bool = False) -> DecodeStep:
    """Shared-prefix sampling: each prompt's blocks are shared by reference count across its
    samples (fork); the first write into the shared, partially filled last prompt block copies
    it (copy-on-write) for every sample but the last holder; then each sample's private tail
    and one new token are written, and all sequences are decoded.

    With private=True every sample instead owns a full private copy of its prompt's blocks
    (no sharing, no copy-on-write); the tokens, and hence the attention results, are the same.
    The step is: copies (CoW pairs), write 1 (all tails), write 2 (one new token per sample)."""
    B, H, d = block_size, heads, head_dim
    S = prompts * samples
    per_prompt = math.ceil(prompt_len / B)
    per_sample = math.ceil((prompt_len + tail_len + 1) / B)
    if private:
        need = S * per_sample
    else:
        need = prompts * (prompt_len // B) + S * (per_sample - prompt_len // B)
    num_blocks = math.ceil(1.2 * need)
    alloc = BlockAllocator(num_blocks, np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(3,))))
    fill = nan_value(dtype) if poison else 0
    k_cache = full((num_blocks, H, B, d), fill, dtype)
    v_cache = full((num_blocks, H, B, d), fill, dtype)

    # Prompt content: stream p; sample tails: stream prompts + s.
    pk = [logical_kv(seed, p, prompt_len, H, d, dtype, 0) for p in range(prompts)]
    pv = [logical_kv(seed, p, prompt_len, H, d, dtype, 1) for p in range(prompts)]
    seqs = []
    for p in range(prompts):
        root = Sequence(B)
        if private:
            group = []
            for _ in range(samples):
                sq = Sequence(B)
                append_tokens(alloc, sq, prompt_len)
                _scatter(k_cache, sq.table, pk[p], 0, B)
                _scatter(v_cache, sq.table, pv[p], 0, B)
                group.append(sq)
        else:
            append_tokens(alloc, root, prompt_len)
            _scatter(k_cache, root.table, pk[p], 0, B)
            _scatter(v_cache, root.table, pv[p], 0, B)
            group = [root] + [fork(alloc, root) for _ in range(samples - 1)]
        seqs.extend(group)
    assert all(len(sq.table) == per_prompt for sq in seqs)

    # Write 1: each sample's private tail (copy-on-write of the shared partial block first).
    tails_k, tails_v, lastk, lastv = [], [], [], []
    slots1, pairs = [], []
    for s, sq in enumerate(seqs):
        tk = logical_kv(seed, prompts + s, tail_len + 1, H, d, dtype, 0)
        tv = logical_kv(seed, prompts + s, tail_len + 1, H, d, dtype, 1)
        sl, pr = append_tokens(alloc, sq, tail_len)
        slots1.extend(sl)
        pairs.extend(pr)
        tails_k.append(tk[:tail_len])
        tails_v.append(tv[:tail_len])
        lastk.append(tk[tail_len])
        lastv.append(tv[tail_len])
    w1 = KVWrite(np.concatenate(tails_k), np.concatenate(tails_v), np.asarray(slots1, np.int32))
    # Write 2: one new token per sequence.
    slots2 = []
    for sq in seqs:
        sl, pr = append_tokens(alloc, sq, 1)
        assert not pr
        slots2.extend(sl)
    w2 = KVWrite(np.stack(lastk), np.stack(lastv), np.asarray(slots2, np.int32))

    q = np.stack([to_storage(_normal(seed, (2, s), (H, d)), dtype) for s in range(S)])
    T = prompt_len + tail_len + 1
    step = DecodeStep(
        name="shared-prefix-f16" + ("-private" if private else ""), seed=seed, dtype=dtype,
        num_q_heads=H, num_kv_heads=H, head_dim=d, block_size=B, k_cache=k_cache,
        v_cache=v_cache, q=q, block_tables=block_tables_array(seqs),
        context_lens=np.full(S, T, np.int32),
        copies=np.asarray(pairs, np.int32).reshape(-1, 2), writes=[w1, w2],
        scale=np.float32(1.0 / math.sqrt(d)),
    )
    if keep_logical:
        step.logical_k = [np.concatenate([pk[s // samples], tails_k[s], lastk[s][None]]) for s in range(S)]
        step.logical_v = [np.concatenate([pv[s // samples], tails_v[s], lastv[s][None]]) for s in range(S)]
    step.notes.update(blocks_needed=need, unique_blocks=need,
                      logical_blocks=S * per_sample, refcounts=alloc.ref.copy())
    return step

