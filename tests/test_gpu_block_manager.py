"""The native host block manager driving the GPU calls end to end (through the C ABI).

Parallel sampling ([PA-summary] "Memory sharing: copy-on-write"): a prompt is appended, forked
into samples that share its blocks, each sample appends its own tokens (copy-on-write pairs
applied with pa_copy_blocks first), and pa_decode over the manager's tables matches the CPU
oracle on the same pool. Preemption ([PA-summary] "vLLM"): a sequence moves to a pinned host
pool and back to other device blocks (pa_bm_move + pa_swap_blocks) and decodes bit-identically.
A serving loop: decode steps through pa_decode_append over the manager's slots, with a fork and
a finished sequence inside the loop.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import paged_kv_cache_82_amd as pa
from gpu_harness import assert_attention_close, to_dev, to_host
from paged_kv_cache_82_amd.block_manager import BlockManager
from workloads import full, nan_value, to_float64, to_storage

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-test] {request.node.name}", flush=True)
    yield


def _kv(rng, n, H, d, dt):
    return (to_storage(rng.standard_normal((n, H, d)).astype(np.float32), dt),
            to_storage(rng.standard_normal((n, H, d)).astype(np.float32), dt))


def test_sampling_and_swap_driven_by_the_native_manager():
    rng = np.random.default_rng(900)
    N, B, H, d, dt = 48, 16, 8, 128, "f16"
    bm = BlockManager(N, B, rng.permutation(N))
    kc = full((N, H, B, d), nan_value(dt), dt)
    vc = kc.copy()
    dk, dv = to_dev(kc, dt), to_dev(vc, dt)

    def write(seq, n):
        slots, pairs = bm.append(seq, n)
        if len(pairs):
            oracle.copy_blocks(kc, vc, pairs, dt)
            pa.pa_copy_blocks(dk, dv, to_dev(pairs))
        kn, vn = _kv(rng, n, H, d, dt)
        oracle.write_kv(kc, vc, kn, vn, slots, dt)
        pa.pa_write_kv(dk, dv, to_dev(kn, dt), to_dev(vn, dt), to_dev(slots))
        return pairs

    bm.add(0)
    write(0, 70)  # 5 blocks, the last one partly filled
    for c in (1, 2, 3):
        bm.fork(0, c)
    copies = [len(write(s, 40)) for s in (1, 2, 3, 0)]
    assert copies == [1, 1, 1, 0]  # the last holder of the shared block writes in place
    seqs = [0, 1, 2, 3]
    st = bm.stats()
    assert st["shared_blocks"] == 4 and st["used_blocks"] == 4 + 4 * 3

    def decode(tables, lens, q):
        out = torch.empty_like(q)
        pa.pa_decode(out, q, dk, dv, to_dev(tables), to_dev(lens), 1 / np.sqrt(d),
                     int(lens.max()))
        torch.cuda.synchronize()
        return to_host(out, dt)

    q = to_storage(rng.standard_normal((4, H, d)).astype(np.float32), dt)
    tables = bm.tables(seqs)
    lens = np.array([bm.length(s) for s in seqs], np.int32)
    got = decode(tables, lens, to_dev(q, dt))
    assert np.array_equal(to_host(dk, dt).view(np.uint16), kc.view(np.uint16))
    ref = oracle.decode(q, kc, vc, tables, lens, np.float32(1 / np.sqrt(d)), dt)
    assert_attention_close(got, ref, dt, "sampling")

    # preempt sample 2: out to a pinned host pool, its device blocks reused, then back in
    host = BlockManager(16, B)
    hk = torch.empty((16, H, B, d), dtype=torch.float16, pin_memory=True)
    hv = torch.empty((16, H, B, d), dtype=torch.float16, pin_memory=True)
    out_pairs = bm.move_to(host, 2)
    pa.pa_swap_blocks(hk, hv, dk, dv, to_dev(out_pairs))
    torch.cuda.synchronize()
    bm.add(9)
    write(9, 5 * B)  # takes the freed blocks and overwrites them
    in_pairs = host.move_to(bm, 2)
    pa.pa_swap_blocks(dk, dv, hk, hv, to_dev(in_pairs))
    torch.cuda.synchronize()
    assert bm.tables([2])[0].tolist() != tables[2, :bm.num_seq_blocks(2)].tolist()
    again = decode(bm.tables([2]), np.array([bm.length(2)], np.int32), to_dev(q[2:3], dt))
    assert np.array_equal(again.view(np.uint16), got[2:3].view(np.uint16))


def test_chunked_prefill_fork_and_decode_driven_by_the_native_manager():
    # Two prompts prefilled in chunks of different lengths, batched into the same calls
    # ([PA-summary] "vLLM": new requests join each iteration), blocks allocated on demand by
    # the native manager; then prompt 0 forks into two samples (copy-on-write of its partly
    # filled last block) and every sequence takes one decode step, through pa_prefill (n = 1)
    # and pa_decode alike. Each call is checked against the oracle on the same pool.
    rng = np.random.default_rng(910)
    N, B, Hq, Hkv, d, dt = 96, 16, 16, 2, 128, "bf16"
    scale = np.float32(1 / np.sqrt(d))
    bm = BlockManager(N, B, rng.permutation(N))
    kc = full((N, Hkv, B, d), nan_value(dt), dt)
    vc = kc.copy()
    dk, dv = to_dev(kc, dt), to_dev(vc, dt)

    def step(seqs, counts):
        """Append counts[i] tokens to seqs[i], write them, attend with their queries."""
        slots, kn, vn = [], [], []
        for s, n in zip(seqs, counts):
            sl, pairs = bm.append(s, n)
            if len(pairs):
                oracle.copy_blocks(kc, vc, pairs, dt)
                pa.pa_copy_blocks(dk, dv, to_dev(pairs))
            k1, v1 = _kv(rng, n, Hkv, d, dt)
            slots.append(sl)
            kn.append(k1)
            vn.append(v1)
        slots, kn, vn = np.concatenate(slots), np.concatenate(kn), np.concatenate(vn)
        oracle.write_kv(kc, vc, kn, vn, slots, dt)
        pa.pa_write_kv(dk, dv, to_dev(kn, dt), to_dev(vn, dt), to_dev(slots))
        q = to_storage(rng.standard_normal((int(sum(counts)), Hq, d)).astype(np.float32), dt)
        qs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
        tables = bm.tables(seqs)
        lens = np.array([bm.length(s) for s in seqs], np.int32)
        out = torch.empty_like(to_dev(q, dt))
        pa.pa_prefill(out, to_dev(q, dt), dk, dv, to_dev(tables), to_dev(lens), to_dev(qs),
                      float(scale), int(max(counts)), int(lens.max()))
        torch.cuda.synchronize()
        got = to_host(out, dt)
        ref = oracle.prefill(q, kc, vc, tables, lens, qs, scale, dt)
        assert_attention_close(got, ref, dt, f"chunks {counts}")
        return q, tables, lens, got

    bm.add(0)
    bm.add(1)
    for counts in ([128, 50], [100, 200], [77, 1]):  # prompt 0: 305 tokens, prompt 1: 251
        step([0, 1], counts)
    assert np.array_equal(to_host(dk, dt).view(np.uint16), kc.view(np.uint16))
    for c in (2, 3):
        bm.fork(0, c)
    seqs = [0, 1, 2, 3]
    q, tables, lens, got = step(seqs, [1, 1, 1, 1])
    assert bm.stats()["shared_blocks"] == 305 // B  # the full prompt blocks stay shared
    out = torch.empty_like(to_dev(q, dt))
    ws = torch.empty(max(1, pa.pa_decode_workspace_size(4, Hq, Hkv, d, B, int(lens.max()), 0,
                                                        torch.bfloat16)),
                     dtype=torch.uint8, device="cuda")
    pa.pa_decode(out, to_dev(q, dt), dk, dv, to_dev(tables), to_dev(lens), float(scale),
                 int(lens.max()), ws)
    torch.cuda.synchronize()
    assert_attention_close(to_host(out, dt), oracle.decode(q, kc, vc, tables, lens, scale, dt),
                           dt, "decode after fork")
    assert_attention_close(got, to_float64(to_host(out, dt), dt), dt, "prefill n=1 vs decode")


def test_decode_loop_with_fused_append_driven_by_the_native_manager():
    # A serving loop ([PA-summary] "vLLM": each iteration, every running sequence generates one
    # token): prompts of mixed lengths are written, then 12 decode steps run through
    # pa_decode_append, each sequence's new token attended to directly and stored at the slot
    # the manager reserved for it. Sequence 0 forks into a second sample before step 3 (the
    # loop then copies its partly filled last block, copy-on-write, before the fused call) and
    # sequence 1 finishes before step 6 (its blocks return to the free list and are taken
    # again). Every step matches the oracle's write-then-decode on the same pool, and the pools
    # match bit for bit at the end.
    rng = np.random.default_rng(930)
    N, B, Hq, Hkv, d, dt = 160, 16, 16, 2, 128, "f16"
    scale = np.float32(1 / np.sqrt(d))
    bm = BlockManager(N, B, rng.permutation(N))
    kc = full((N, Hkv, B, d), nan_value(dt), dt)
    vc = kc.copy()
    dk, dv = to_dev(kc, dt), to_dev(vc, dt)
    running = []
    for s, T in enumerate([37, 200, 1, 16, 95]):
        bm.add(s)
        slots, pairs = bm.append(s, T)
        assert len(pairs) == 0
        k1, v1 = _kv(rng, T, Hkv, d, dt)
        oracle.write_kv(kc, vc, k1, v1, slots, dt)
        pa.pa_write_kv(dk, dv, to_dev(k1, dt), to_dev(v1, dt), to_dev(slots))
        running.append(s)
    copies = 0
    for it in range(12):
        if it == 3:
            bm.fork(0, 5)
            running.append(5)
        if it == 6:
            bm.release(1)
            running.remove(1)
        slots = []
        for s in running:
            sl, pairs = bm.append(s, 1)
            if len(pairs):
                copies += len(pairs)
                oracle.copy_blocks(kc, vc, pairs, dt)
                pa.pa_copy_blocks(dk, dv, to_dev(pairs))
            slots.append(int(sl[0]))
        slots = np.asarray(slots, np.int32)
        S = len(running)
        kn, vn = _kv(rng, S, Hkv, d, dt)
        q = to_storage(rng.standard_normal((S, Hq, d)).astype(np.float32), dt)
        tables = bm.tables(running)
        lens = np.array([bm.length(s) for s in running], np.int32)
        oracle.write_kv(kc, vc, kn, vn, slots, dt)
        ref = oracle.decode(q, kc, vc, tables, lens, scale, dt)
        dq = to_dev(q, dt)
        out = torch.empty_like(dq)
        ws = torch.empty(max(1, pa.pa_decode_workspace_size(S, Hq, Hkv, d, B, int(lens.max()), 0,
                                                            torch.float16)),
                         dtype=torch.uint8, device="cuda")
        pa.pa_decode_append(out, dq, dk, dv, to_dev(kn, dt), to_dev(vn, dt), to_dev(slots),
                            to_dev(tables), to_dev(lens), float(scale), int(lens.max()), ws)
        torch.cuda.synchronize()
        assert_attention_close(to_host(out, dt), ref, dt, f"decode step {it} ({S} sequences)")
    assert copies >= 1, "the fork's first write must copy the shared last block"
    assert np.array_equal(to_host(dk, dt).view(np.uint16), kc.view(np.uint16))
    assert np.array_equal(to_host(dv, dt).view(np.uint16), vc.view(np.uint16))
