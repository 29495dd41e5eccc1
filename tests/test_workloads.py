"""Host logic: seeded generators and the toy block manager (no GPU, no oracle arithmetic)."""
import math

import numpy as np
import pytest

from workloads import (BlockAllocator, PoolExhausted, Sequence, append_tokens, tiny_f32,
                       shared_prefix_f16, fork, make_step, release, wasted_slots)
from workloads.configs import (mha13b_f16, mha13b_lengths, gqa_bf16, gqa_lengths,
                               long_lengths)


def test_generators_are_deterministic():
    a = tiny_f32()
    b = tiny_f32()
    for x, y in ((a.k_cache, b.k_cache), (a.v_cache, b.v_cache), (a.q, b.q),
                 (a.block_tables, b.block_tables), (a.writes[0].slot_mapping, b.writes[0].slot_mapping)):
        assert np.array_equal(x.view(np.uint8), y.view(np.uint8))


def test_tiny_shape():
    st = tiny_f32()
    assert st.k_cache.shape == (64, 8, 16, 64) and st.dtype == "f32"
    assert list(st.context_lens) == [7, 16, 33, 50]
    assert st.block_tables.shape == (4, 4)
    assert [int((row >= 0).sum()) for row in st.block_tables] == [1, 1, 3, 4]
    w = st.writes[0]
    assert w.k_new.shape == (4, 8, 64) and len(w.slot_mapping) == 4
    # the slot of the written token is in the last block of each sequence
    for s, T in enumerate(st.context_lens):
        j, off = divmod(T - 1, 16)
        assert w.slot_mapping[s] == st.block_tables[s, j] * 16 + off
        # and that slot is still poison before the write
        assert np.isnan(st.k_cache[st.block_tables[s, j], :, off, :]).all()
    assert np.isclose(st.scale, 1 / 8)


def test_length_distributions():
    t2 = mha13b_lengths()
    assert t2.min() >= 16 and t2.max() <= 2048 and len(t2) == 64
    assert 300 < np.median(t2) < 900
    t3 = gqa_lengths()
    assert t3.min() >= 128 and t3.max() <= 4096 and len(t3) == 256
    t4 = long_lengths()
    assert t4.min() >= 32768 and t4.max() <= 131072 and len(t4) == 8


def test_pool_sizing_and_scatter():
    st = make_step("x", 3, [5, 40, 17], 4, 2, 8, 4, "bf16")
    need = sum(math.ceil(t / 4) for t in (5, 40, 17))
    assert st.num_blocks == math.ceil(1.2 * need)
    used = st.block_tables[st.block_tables >= 0]
    assert len(set(used.tolist())) == len(used) == need


def test_allocator_exhaustion_and_reuse():
    al = BlockAllocator(3)
    s = Sequence(2)
    append_tokens(al, s, 6)
    with pytest.raises(PoolExhausted):
        append_tokens(al, s, 1)
    release(al, s)
    assert al.num_free == 3
    t = Sequence(2)
    append_tokens(al, t, 5)
    assert wasted_slots(t) == 1


def test_fork_and_copy_on_write():
    al = BlockAllocator(16, np.random.default_rng(0))
    root = Sequence(4)
    append_tokens(al, root, 6)  # 2 blocks, the second half full
    kids = [fork(al, root) for _ in range(2)]
    assert all(al.ref[b] == 3 for b in root.table)
    # writer with refcount > 1 copies; the last holder writes in place
    s0, p0 = append_tokens(al, root, 1)
    s1, p1 = append_tokens(al, kids[0], 1)
    s2, p2 = append_tokens(al, kids[1], 1)
    assert len(p0) == 1 and len(p1) == 1 and p2 == []
    assert p0[0][0] == p1[0][0] == kids[1].table[1]
    assert len({s0[0], s1[0], s2[0]}) == 3
    # full shared blocks stay shared
    assert root.table[0] == kids[0].table[0] == kids[1].table[0] and al.ref[root.table[0]] == 3


def test_shared_prefix_structure():
    st = shared_prefix_f16(poison=False)
    assert st.num_seqs == 64 and st.block_size == 32 and st.dtype == "f16"
    assert len(st.copies) == 48
    assert (st.context_lens == 1297).all()
    assert st.block_tables.shape == (64, 41)
    assert st.num_blocks == math.ceil(1.2 * 1088)
    assert len(st.writes[0].slot_mapping) == 64 * 256 and len(st.writes[1].slot_mapping) == 64
    # the first 32 blocks of each prompt's 4 samples are shared
    for p in range(16):
        rows = st.block_tables[4 * p: 4 * p + 4, :32]
        assert (rows == rows[0]).all()
    assert len(np.unique(st.block_tables)) == 1088
    src, dst = st.copies[:, 0], st.copies[:, 1]
    assert len(set(dst.tolist())) == 48 and not set(dst.tolist()) & set(src.tolist())


def test_mha13b_gqa_metadata_small():
    # structure only (pools are big): block counts agree with the lengths
    for fn, H in ((mha13b_f16, 40), (gqa_bf16, 8)):
        st = fn(poison=False)
        assert st.k_cache.shape[1] == H
        nblk = (st.block_tables >= 0).sum(axis=1)
        assert (nblk == (st.context_lens + 15) // 16).all()


def test_prefill_step_layout():
    from workloads import make_prefill_step

    st = make_prefill_step("p", 9, [7, 16, 33, 5], [7, 3, 16, 0], 4, 2, 8, 8, "f16")
    assert list(st.query_start) == [0, 7, 10, 26, 26]
    assert st.q.shape == (26, 4, 8) and st.num_q_tokens == 26 and st.max_query_len == 16
    w = st.writes[0]
    assert len(w.slot_mapping) == 26 and len(set(w.slot_mapping.tolist())) == 26
    # the chunk's tokens go to positions T-n .. T-1 of each sequence, still poison before
    k = 0
    for s, (T, n) in enumerate(zip(st.context_lens, st.query_lens)):
        for i in range(n):
            j, off = divmod(int(T - n + i), 8)
            assert w.slot_mapping[k] == st.block_tables[s, j] * 8 + off
            assert np.isnan(st.k_cache[st.block_tables[s, j], :, off, :].astype(np.float32)).all()
            k += 1
    with pytest.raises(ValueError):
        make_prefill_step("bad", 9, [4], [5], 2, 2, 8, 8, "f16")


def test_prefill_workloads_shapes():
    from workloads.configs import prefill_gqa, prefill_mha13b

    a = prefill_mha13b(poison=False)
    assert a.num_seqs == 16 and a.num_q_tokens == 16 * 512 and a.max_context_len <= 2048
    assert (a.context_lens >= 512).all() and a.dtype == "f16" and a.num_q_heads == 40
    b = prefill_gqa(poison=False)
    assert b.num_q_tokens == 16 * 1024 and b.max_context_len <= 4096
    assert (b.num_q_heads, b.num_kv_heads, b.dtype) == (64, 8, "bf16")
