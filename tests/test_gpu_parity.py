"""GPU parity of the C ABI (pa_write_kv, pa_copy_blocks, pa_decode) against the CPU oracle on
small and edge-case inputs. Bit-exact for the indexing kernels; attention within max-abs 1e-5
for fp32 and |gpu - ref| <= 2e-2 + 1e-2 |ref| for fp16/bf16 (fp32 accumulation)."""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
from gpu_harness import (DevStep, assert_attention_close, check_full_size, make_dominant_token,
                         to_host, uses_mfma_decode)
from workloads import tiny_f32, shared_prefix_f16, make_step, to_float64, to_storage

pytestmark = pytest.mark.gpu


def _bits(a):
    return a.view(np.uint8)


def _run_and_check(step, partition_tokens=0, check_pools=True, what=""):
    ref, kc, vc = oracle.run_step(step)
    dev = DevStep(step, partition_tokens)
    got = dev.run()
    if check_pools:
        assert np.array_equal(_bits(to_host(dev.k_cache, step.dtype)), _bits(kc)), what
        assert np.array_equal(_bits(to_host(dev.v_cache, step.dtype)), _bits(vc)), what
    assert_attention_close(got, ref, step.dtype, what)
    return got, ref


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-test] {request.node.name}", flush=True)
    yield


def test_tiny_f32():
    got, ref = _run_and_check(tiny_f32(), what="tiny_f32")
    assert np.abs(got.astype(np.float64) - ref).max() <= 1e-5


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B", [8, 16, 32, 64])
def test_shapes_mha(dt, d, B):
    step = make_step("mha", 31 + B + d, [1, 7, B, B + 1, 3 * B - 1, 200], 4, 4, d, B, dt)
    _run_and_check(step, what=f"mha {dt} d{d} B{B}")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("g", [2, 4, 8, 16, 32])
@pytest.mark.parametrize("d,B", [(128, 16), (64, 8), (128, 32), (128, 64), (64, 64)])
def test_shapes_gqa(dt, g, d, B):
    step = make_step("gqa", 41 + g, [1, 5, 16, 33, 130, 257], 2 * g, 2, d, B, dt)
    _run_and_check(step, what=f"gqa {dt} g{g} d{d} B{B}")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("Hq,Hkv,d", [(24, 1, 128), (48, 1, 128), (64, 1, 128), (96, 2, 64),
                                      (34, 2, 128)])
@pytest.mark.parametrize("P", [0, 64])
def test_wide_groups(dt, Hq, Hkv, d, P):
    # more than 16 query heads per KV head: workgroups of 32 heads (two MFMA column tiles), the
    # last one part-empty for g = 24, 48, 17; single-KV-head (multi-query) batches; whole and
    # split sequences, empty and one-token sequences among them
    step = make_step("wide", 90 + Hq + d, [0, 1, 31, 33, 200, 700], Hq, Hkv, d, 16, dt)
    _run_and_check(step, partition_tokens=P, what=f"wide {dt} {Hq}/{Hkv} d{d} P{P}")


FEW_UNIT_CASES = [
    # (Hq, Hkv, d, B, lengths): small grouped-query batches with very uneven lengths
    (16, 2, 128, 16, [4000] + [1] * 30 + [0] * 5),     # one long sequence, many tiny and empty
    (64, 2, 128, 16, [0, 1, 33, 64, 65, 500, 1025, 2047]),  # 32-head units
    (48, 1, 128, 32, [17, 900, 3000, 0, 64]),          # 2 head tiles of 32, the second part-empty
    (8, 2, 64, 8, [257, 1, 31, 2500, 96]),
    (32, 4, 128, 64, [130, 4095, 7, 640]),
]


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("case", range(len(FEW_UNIT_CASES)))
def test_few_unit_batches(dt, case):
    # few (sequence, head tile) units: the automatic plan splits the long sequences into
    # partitions and leaves the short ones whole
    Hq, Hkv, d, B, lens = FEW_UNIT_CASES[case]
    step = make_step("few", 500 + case, lens, Hq, Hkv, d, B, dt)
    _run_and_check(step, what=f"few units {dt} case {case}")


def test_workspace_reused_with_other_lengths():
    # partial states are rewritten by every call: a second call with other lengths (other
    # splits) on the same workspace must not see the first call's
    shared_ws = None
    for lens in ([3000, 5, 700, 0, 64], [10, 2990, 0, 650, 1]):
        step = make_step("reuse", 520, lens, 16, 2, 128, 16, "bf16")
        ref, _, _ = oracle.run_step(step)
        dev = DevStep(step)
        if shared_ws is None:
            shared_ws = dev.workspace
        assert dev.workspace.numel() <= shared_ws.numel()
        dev.workspace = shared_ws
        assert_attention_close(dev.run(), ref, step.dtype, f"reused workspace {lens}")


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("Hq,B", [(8, 16), (32, 8), (64, 32), (8, 64)])
def test_mfma_ring_tails(dt, Hq, B, decode_kernel):
    # A wave of an MFMA workgroup takes every 4th 32-token step of its partition through a ring
    # of 3 slots: whole rounds of 3 in a loop, then the last 1 or 2 steps on their own, with
    # counted waits of their own. Lengths 32 s - 5 (s = 1 .. 28 steps, whole sequences) give the
    # waves 0 to 7 steps each, so every remainder follows 0, 1 and 2 whole rounds; 16- and
    # 32-head workgroups, every block-size path of the loads.
    decode_kernel("mfma")
    lens = [32 * s - 5 for s in range(1, 29)]
    step = make_step("ring", 700 + Hq + B, lens, Hq, 2, 128, B, dt)
    _run_and_check(step, partition_tokens=1024, what=f"ring tails {dt} Hq{Hq} B{B}")


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("d,B", [(128, 8), (64, 16), (128, 16)])
def test_valu_ring_tails(dt, d, B, decode_kernel):
    # The vector-ALU kernel's register ring is 8 deep for units of one or two loads per tensor
    # (8-token blocks, 64-dim heads at 16-bit) and 3 or 4 deep otherwise. Lengths 32 k + 5
    # (k = 0 .. 39, whole sequences) give the waves up to 39 units each: several whole rounds of
    # every ring depth, then every remainder.
    decode_kernel("valu")
    lens = [32 * k + 5 for k in range(40)]
    step = make_step("vring", 740 + d + B, lens, 4, 4, d, B, dt)
    _run_and_check(step, partition_tokens=2048, what=f"valu ring tails {dt} d{d} B{B}")


def _rising_scores(step, rise_log2, rng):
    """Rewrite the single sequence of a decode step so that its scores climb by about
    rise_log2 (base-2 exponent, times 1 + h/16 for query head h) from one 32-token step to the
    next, with small noise inside each step: the running maximum keeps rising, in jumps below
    and above any fixed slack. K dim 0 carries the ramp, the other dims and V are random."""
    from workloads import to_storage

    dt, B, d, Hkv = step.dtype, step.block_size, step.head_dim, step.num_kv_heads
    T = int(step.context_lens[0])
    n_new = sum(w.k_new.shape[0] for w in step.writes)
    prefix = T - n_new
    unit = 1.0 / (4.0 * float(step.scale) * np.log2(np.e))  # K dim 0 per unit of log2 score
    k = 0.3 * rng.standard_normal((T, Hkv, d))
    k[:, :, 0] = rise_log2 * unit * (np.arange(T) // 32)[:, None]
    v = rng.standard_normal((T, Hkv, d))
    table = step.block_tables[0]
    for t in range(prefix):
        step.k_cache[table[t // B], :, t % B, :] = to_storage(k[t], dt)
        step.v_cache[table[t // B], :, t % B, :] = to_storage(v[t], dt)
    at = prefix
    for w in step.writes:
        m = w.k_new.shape[0]
        w.k_new[...] = to_storage(k[at:at + m], dt)
        w.v_new[...] = to_storage(v[at:at + m], dt)
        at += m
    Hq = step.q.shape[1]
    q = 0.3 * rng.standard_normal(step.q.shape)
    q[..., 0] = 4.0 * (1.0 + np.arange(Hq) / 16.0)
    step.q[...] = to_storage(q, dt)
    return step


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("Hq", [16, 64])
@pytest.mark.parametrize("rise", [0.5, 1.9, 2.1, 8.5])
@pytest.mark.parametrize("P", [0, 256])
def test_mfma_rising_maximum(dt, Hq, rise, P, decode_kernel):
    # The MFMA kernels take weights against a reference maximum that is raised only when a
    # score passes it by more than a slack (2^8 in weight). Scores that climb from step to step
    # (a wave sees every 4th step, so 4 x rise per wave step: 2, 7.6, 8.4 and 34 in the base-2
    # exponent, more for the later heads) raise it never, sometimes or at every step; whole
    # sequences and 256-token partitions (the merge then combines partials with different
    # references).
    decode_kernel("mfma")
    rng = np.random.default_rng(int(rise * 10) + Hq)
    step = _rising_scores(make_step("rise", 760 + Hq, [1000], Hq, 2, 128, 16, dt), rise, rng)
    _run_and_check(step, partition_tokens=P, what=f"rising maximum {dt} Hq{Hq} rise {rise} P{P}")


@pytest.mark.parametrize("path", ["valu", "mfma"])
def test_both_decode_paths_on_gqa(path, decode_kernel):
    decode_kernel(path)
    step = make_step("paths", 50, [3, 64, 100, 511, 700], 16, 2, 128, 16, "bf16")
    _run_and_check(step, what=path)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("g,path", [(1, "valu"), (4, "valu"), (4, "mfma")])
def test_small_weights_below_fp16_normal(dt, g, path, decode_kernel):
    # one token outweighs 3999 others by 2^15: their weights are below fp16's smallest normal
    # number and together add 12% to the row sum; both kernels, whole and split
    decode_kernel(path)
    for P in (0, 512):
        step = make_dominant_token(make_step("ddom", 481, [4000], 2 * g, 2, 128, 16, dt))
        _run_and_check(step, partition_tokens=P, what=f"dominant token {dt} g{g} {path} P{P}")


@pytest.mark.parametrize("P", [32, 64, 96, 512])
def test_forced_split_k(P):
    step = make_step("split", 60, [1, 31, 32, 33, 95, 400, 1000], 8, 8, 128, 16, "f16")
    got, ref = _run_and_check(step, partition_tokens=P, what=f"P={P}")
    single, _ = _run_and_check(step, partition_tokens=1024, check_pools=False)
    assert_attention_close(got, to_float64(single, step.dtype), step.dtype, "split vs single")


@pytest.mark.parametrize("P", [32, 128])
def test_forced_split_k_gqa(P):
    step = make_step("splitg", 61, [2, 40, 300, 900], 32, 4, 128, 16, "bf16")
    _run_and_check(step, partition_tokens=P, what=f"gqa P={P}")


def test_tiny_split_k_every_partition_size():
    for P in (32, 64, 96, 128, 512):
        _run_and_check(tiny_f32(), partition_tokens=P, what=f"tiny_f32 P={P}")


def test_empty_and_single_token_sequences():
    step = make_step("edge", 70, [0, 1, 0, 2, 16, 17], 8, 2, 128, 16, "bf16")
    got, ref = _run_and_check(step, what="edges")
    assert np.array_equal(got[0].view(np.uint16), np.zeros_like(got[0].view(np.uint16)))
    # T = 1 returns V_0 exactly (weight 1, sum 1)
    step1 = make_step("t1", 71, [1, 1, 1], 4, 4, 64, 16, "f32")
    dev = DevStep(step1)
    got1 = dev.run()
    v = step1.writes[0].v_new  # the only token of each sequence
    assert np.array_equal(got1, v)


def test_table_filled_to_the_last_entry():
    # T = max_blocks_per_seq * B: the last 32-token step ends exactly at the table's end
    step = make_step("full", 72, [48, 16], 8, 2, 128, 16, "f16")
    assert step.block_tables.shape[1] == 3
    _run_and_check(step, partition_tokens=32, what="full table")


def test_large_scores_stay_finite():
    step = make_step("big", 73, [50, 700], 8, 2, 128, 16, "bf16")
    step.q[...] = to_storage(to_float64(step.q, "bf16") * 30.0, "bf16")
    _run_and_check(step, what="large scores")


def test_placement_invariance_bit_exact():
    outs = []
    for r in range(3):
        step = make_step("pl", 80, [50, 7, 300, 129], 16, 2, 128, 16, "bf16",
                         alloc_rng=np.random.default_rng(500 + r), pool_factor=2.0)
        outs.append(DevStep(step).run())
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    outs = []
    for r in range(3):
        step = make_step("pl", 81, [50, 7, 300, 129], 8, 8, 128, 16, "f16",
                         alloc_rng=np.random.default_rng(600 + r), pool_factor=2.0)
        outs.append(DevStep(step).run())
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


@pytest.mark.parametrize("Hq,Hkv,dt", [(8, 8, "f16"), (16, 2, "bf16"), (4, 4, "f32")])
def test_block_size_change_within_tolerance(Hq, Hkv, dt):
    # the same tokens cut into blocks of 8, 16, 32 and 64 (both decode kernels and fp32)
    ref = None
    for B in (8, 16, 32, 64):
        step = make_step("bs", 82, [50, 7, 300, 64, 65], Hq, Hkv, 128, B, dt)
        got = DevStep(step).run()
        if ref is None:
            ref = oracle.run_step(step)[0]
        assert_attention_close(got, ref, dt, f"B={B}")


@pytest.mark.parametrize("Hq,Hkv,dt", [(8, 8, "f16"), (16, 2, "bf16"), (4, 4, "f32")])
@pytest.mark.parametrize("P", [32, 64, 96, 0])
def test_block_size_64_split(Hq, Hkv, dt, P):
    # 64-token blocks split into partitions of 32..96 tokens (partition edges inside blocks)
    step = make_step("b64", 83, [1, 63, 64, 65, 200, 1000], Hq, Hkv, 128, 64, dt)
    _run_and_check(step, partition_tokens=P, what=f"B=64 {dt} g{Hq // Hkv} P={P}")


def test_repeated_calls_reuse_workspace():
    step = make_step("rep", 83, [700, 1500, 33], 8, 8, 128, 16, "f16")
    dev = DevStep(step, partition_tokens=128)
    first = dev.run()
    for _ in range(3):
        # poison the output first: a call whose merge never ran would leave it NaN
        dev.out.fill_(float("nan"))
        dev.decode()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(dev.out, "f16"), first)


def test_nondefault_stream():
    step = make_step("strm", 84, [100, 200], 8, 2, 128, 16, "bf16")
    ref = oracle.run_step(step)[0]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dev = DevStep(step)
        dev.apply_updates()
        dev.decode()
    s.synchronize()
    assert_attention_close(to_host(dev.out, "bf16"), ref, "bf16", "stream")


def test_shared_prefix_small_shared_vs_private():
    kw = dict(prompts=3, samples=4, prompt_len=70, tail_len=20, heads=4, head_dim=128,
              block_size=32, dtype="f16")
    shared = shared_prefix_f16(**kw)
    private = shared_prefix_f16(private=True, **kw)
    a, _ = _run_and_check(shared, what="shared")
    b, _ = _run_and_check(private, what="private")
    assert np.array_equal(a, b)


def test_shared_prefix_full():
    shared = shared_prefix_f16()
    a, ref = _run_and_check(shared, what="shared_prefix_f16 shared")
    check_full_size(a, ref, shared.dtype, shared.context_lens, uses_mfma_decode(shared),
                    shared.name)
    b = DevStep(shared_prefix_f16(private=True)).run()
    assert np.array_equal(a, b)


def test_copy_blocks_and_write_leave_rest_untouched():
    rng = np.random.default_rng(90)
    step = make_step("cw", 90, [40, 70], 4, 4, 128, 16, "bf16", pool_factor=3.0)
    # add copies of used blocks into free ones
    used = set(step.block_tables[step.block_tables >= 0].tolist())
    free = [b for b in range(step.num_blocks) if b not in used]
    src = sorted(used)[:3]
    dst = rng.choice(free, size=3, replace=False)
    step.copies = np.stack([src, dst], axis=1).astype(np.int32)
    _run_and_check(step, what="copy+write")


def test_swap_out_and_in_restores_attention():
    """Preempt a sequence: its blocks go to a pinned host pool, the device blocks are reused
    (clobbered), the blocks come back at new device positions, the table is repointed, and the
    attention output is bit-identical to the one before the swap."""
    step = make_step("swap", 95, [70, 300, 45], 8, 8, 128, 16, "f16", pool_factor=2.5)
    dev = DevStep(step)
    before = dev.run()
    s = 1
    nblk = (int(step.context_lens[s]) + 15) // 16
    blocks = step.block_tables[s, :nblk].astype(np.int32)
    H, B, d = 8, 16, 128
    host_k = torch.empty((nblk + 3, H, B, d), dtype=torch.float16).pin_memory()
    host_v = torch.empty_like(host_k).pin_memory()
    host_k.fill_(float("nan"))
    host_v.fill_(float("nan"))
    out_pairs = np.stack([blocks, np.arange(nblk, dtype=np.int32) + 2], 1).astype(np.int32)
    import paged_kv_cache_82_amd as pa
    pa.pa_swap_blocks(host_k, host_v, dev.k_cache, dev.v_cache,
                      torch.from_numpy(out_pairs).cuda())
    torch.cuda.synchronize()
    # host side against the oracle's move from the same device pool
    kc, vc = to_host(dev.k_cache, "f16"), to_host(dev.v_cache, "f16")
    ek = np.full((nblk + 3, H, B, d), np.nan, np.float16)
    ev = ek.copy()
    oracle.swap_blocks(ek, ev, kc, vc, out_pairs, "f16")
    assert np.array_equal(host_k.numpy().view(np.uint16), ek.view(np.uint16))
    assert np.array_equal(host_v.numpy().view(np.uint16), ev.view(np.uint16))
    # the device blocks are reused by someone else
    idx = torch.from_numpy(blocks.astype(np.int64)).cuda()
    dev.k_cache.index_fill_(0, idx, float("nan"))
    dev.v_cache.index_fill_(0, idx, float("nan"))
    # swap back into free blocks
    used = set(step.block_tables[step.block_tables >= 0].tolist())
    free = np.array([b for b in range(step.num_blocks) if b not in used][:nblk], np.int32)
    in_pairs = np.stack([np.arange(nblk, dtype=np.int32) + 2, free], 1).astype(np.int32)
    pa.pa_swap_blocks(dev.k_cache, dev.v_cache, host_k, host_v,
                      torch.from_numpy(in_pairs).cuda())
    bt = step.block_tables.copy()
    bt[s, :nblk] = free
    dev.block_tables.copy_(torch.from_numpy(bt))
    dev.decode()
    torch.cuda.synchronize()
    after = to_host(dev.out, "f16")
    assert np.array_equal(after.view(np.uint16), before.view(np.uint16))


def test_swap_between_device_pools_vs_oracle():
    rng = np.random.default_rng(96)
    for dt in ("bf16", "f32"):
        src = make_step("sw2", 96, [100, 50], 4, 4, 64, 32, dt, poison=False)
        dev = DevStep(src)
        dst_k = torch.zeros((7,) + tuple(dev.k_cache.shape[1:]), dtype=dev.k_cache.dtype,
                            device="cuda")
        dst_v = torch.zeros_like(dst_k)
        pairs = np.array([[1, 6], [0, 0], [3, 2], [99, 1], [2, 77]], np.int32)  # 2 skipped
        import paged_kv_cache_82_amd as pa
        pa.pa_swap_blocks(dst_k, dst_v, dev.k_cache, dev.v_cache, torch.from_numpy(pairs).cuda())
        torch.cuda.synchronize()
        ek = to_host(dst_k, dt).copy()
        ev = to_host(dst_v, dt).copy()
        ek[...] = 0
        ev[...] = 0
        oracle.swap_blocks(ek, ev, src.k_cache, src.v_cache, pairs, dt)
        assert np.array_equal(to_host(dst_k, dt).view(np.uint8), ek.view(np.uint8))
        assert np.array_equal(to_host(dst_v, dt).view(np.uint8), ev.view(np.uint8))
