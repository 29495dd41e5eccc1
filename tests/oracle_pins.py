"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each pin is a function `pin_xxx(lib)` that raises AssertionError on failure; `lib` is the path
of the oracle library to check (the real one, or a build with a planted mistake in the
mutation test). What pins what:

  widening       all 65536 fp16 / bf16 patterns vs numpy's float16 and torch's bfloat16
  rounding       vs numpy's correctly rounded float64 -> float16 / float32 casts, torch's
                 float32 -> bfloat16 cast, and hand-built ties where double rounding would
                 differ from direct rounding
  decode         vs torch's scaled_dot_product_attention (float64, CPU) on the logical,
                 contiguous K/V the workload generated before scattering it into the pool
                 ([PA-summary] "The PagedAttention algorithm": the block-wise result equals
                 standard attention); closed forms (T = 1 gives V_0; q = 0, scale = 0 or equal
                 keys give the mean of V; a dominant key selects its value; two tokens whose
                 scores differ by ln 3 weigh 1/4 and 3/4); large scores stay finite; T = 0 gives
                 0 ([PA-tutorial] §3.2); invariance under physical placement (all placements of
                 a tiny pool, brute force), block size and poison in unused slots; shared
                 prefix blocks vs private copies ([PA-summary] "Memory sharing: copy-on-write")
  write / copy   vs numpy fancy-index assignment, everything else untouched, invalid inputs
                 rejected
  swap           moves between two pools vs numpy assignment, a round trip out and back in
                 restores the contents ([PA-summary] "vLLM": preemption by swapping to CPU)
  prefill        causal multi-query attention ([PA-summary] "The PagedAttention algorithm" runs
                 the block-table walk for each query vector) vs torch SDPA (float64, CPU) with
                 an explicit mask (query i of a chunk of n sees positions <= T-n+i), and with
                 is_causal=True when the chunk is the whole context; the last query of a chunk
                 equals the decode oracle; keys/values after a query's position never change
                 it while its own position's do; placement and block-size invariance
"""
from __future__ import annotations

import itertools
import math

import numpy as np
import torch

import oracle
from workloads import (BlockAllocator, Sequence, append_tokens, block_tables_array, shared_prefix_f16,
                       make_prefill_step, make_step, to_float64, to_storage)
from oracle import blockwise

RTOL = 1e-12


def _sdpa_ref(step, s):
    """Standard attention (torch SDPA, float64 CPU) of sequence s on its logical K/V."""
    q = torch.from_numpy(to_float64(step.q[s], step.dtype))  # [Hq, d]
    k = torch.from_numpy(to_float64(step.logical_k[s], step.dtype))  # [T, Hkv, d]
    v = torch.from_numpy(to_float64(step.logical_v[s], step.dtype))
    g = step.num_q_heads // step.num_kv_heads
    T = k.shape[0]
    if T == 0:
        return np.zeros(q.shape)
    k = k.repeat_interleave(g, dim=1).permute(1, 0, 2).contiguous()  # [Hq, T, d]
    v = v.repeat_interleave(g, dim=1).permute(1, 0, 2).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(
        q[:, None, :], k, v, scale=float(step.scale))
    return o[:, 0, :].numpy()


def _run(step, lib, **kw):
    return oracle.run_step(step, lib=lib, **kw)[0]


def _close(a, b, rtol=RTOL, atol=1e-13, what=""):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    ok = np.allclose(a, b, rtol=rtol, atol=atol, equal_nan=False)
    if not ok:
        err = np.nanmax(np.abs(a - b)) if a.size else 0
        raise AssertionError(f"{what}: max abs diff {err}")


# ---- element formats -----------------------------------------------------------------------


def pin_widen_f16(lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    h = bits.view(np.float16)
    got = oracle.widen(h, "f16", lib=lib)
    ref = h.astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(got[m], ref[m])


def pin_widen_bf16(lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.widen(bits, "bf16", lib=lib)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    m = ~np.isnan(ref)
    assert np.array_equal(got[m], ref[m])


def _round_samples():
    rng = np.random.default_rng(11)
    parts = [
        rng.standard_normal(20000),
        rng.standard_normal(5000) * 1e-5,  # fp16 subnormals
        rng.standard_normal(5000) * 6e4,  # around fp16 overflow
        rng.standard_normal(2000) * 1e-40,  # fp32/bf16 subnormals
        rng.standard_normal(2000) * 3e38,  # around fp32/bf16 overflow
        np.array([0.0, -0.0, 65504.0, 65520.0, 65519.99, -65520.0, 2.0 ** -25, 2.0 ** -24,
                  3 * 2.0 ** -26, 1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, np.inf, -np.inf]),
    ]
    return np.concatenate(parts)


def pin_round_f16(lib):
    x = _round_samples()
    got = oracle.round_to(x, "f16", lib=lib)
    ref = x.astype(np.float16)
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))


def pin_round_f32(lib):
    x = _round_samples()
    got = oracle.round_to(x, "f32", lib=lib)
    ref = x.astype(np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def pin_round_bf16(lib):
    # (a) float32-representable inputs: no double rounding, torch's cast is the reference.
    x = _round_samples().astype(np.float32)
    x = x[np.isfinite(x)].astype(np.float64)
    got = oracle.round_to(x, "bf16", lib=lib)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(got.view(np.int16), ref)
    # (b) hand-built cases (value -> expected bf16 value).
    cases = [
        (1 + 2.0 ** -8, 1.0),  # tie between 1 and 1+2^-7: even is 1
        (1 + 3 * 2.0 ** -8, 1 + 2.0 ** -6),  # tie: even mantissa is 1+2^-6
        (1 + 2.0 ** -8 + 2.0 ** -30, 1 + 2.0 ** -7),  # above the tie (float32 would lose it)
        (-(1 + 2.0 ** -8 + 2.0 ** -30), -(1 + 2.0 ** -7)),
    ]
    vals = np.array([c[0] for c in cases])
    exp = np.array([c[1] for c in cases])
    got = oracle.round_to(vals, "bf16", lib=lib)
    back = (got.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(back, exp), (back, exp)


# ---- decode: library routine, closed forms, invariants ---------------------------------------

TINY = [
    # (lengths, Hq, Hkv, d, B, dtype)
    ([7, 16, 33, 50], 8, 8, 64, 16, "f32"),
    ([1, 2, 9, 5], 2, 1, 8, 3, "f16"),
    ([9, 4, 1], 4, 2, 8, 4, "bf16"),
    ([5, 17, 0, 31], 4, 4, 16, 8, "f32"),
    ([3, 8], 2, 2, 4, 1, "f32"),
    ([40, 2, 64], 16, 2, 64, 32, "bf16"),
]


def pin_decode_vs_sdpa(lib):
    for i, (lengths, Hq, Hkv, d, B, dt) in enumerate(TINY):
        step = make_step("tiny", 100 + i, lengths, Hq, Hkv, d, B, dt, keep_logical=True)
        out = _run(step, lib)
        for s in range(len(lengths)):
            _close(out[s], _sdpa_ref(step, s), what=f"case {i} seq {s}")


def pin_blockwise_forms_agree(lib):
    for i, (lengths, Hq, Hkv, d, B, dt) in enumerate(TINY):
        step = make_step("tiny", 200 + i, lengths, Hq, Hkv, d, B, dt, poison=False)
        out, kc, vc = oracle.run_step(step, lib=lib)
        args = (to_float64(step.q, dt), to_float64(kc, dt), to_float64(vc, dt),
                step.block_tables, step.context_lens, step.scale)
        for form in (blockwise.equation_form, blockwise.running_form):
            _close(out, blockwise.decode_all(form, *args), what=form.__name__)


def pin_single_token_returns_v0(lib):
    for dt in ("f32", "f16", "bf16"):
        step = make_step("t1", 7, [1, 1, 1], 4, 2, 16, 16, dt, keep_logical=True)
        out = _run(step, lib)
        for s in range(3):
            v0 = to_float64(step.logical_v[s][0], dt)  # [Hkv, d]
            assert np.array_equal(out[s], np.repeat(v0, 2, axis=0)), dt


def _mean_v(step, s):
    v = to_float64(step.logical_v[s], step.dtype).mean(axis=0)
    return np.repeat(v, step.num_q_heads // step.num_kv_heads, axis=0)


def pin_uniform_scores_give_mean(lib):
    # q = 0
    step = make_step("q0", 8, [5, 13, 32], 4, 2, 8, 4, "f32", keep_logical=True)
    step.q[...] = 0
    out = _run(step, lib)
    for s in range(3):
        _close(out[s], _mean_v(step, s), what="q=0")
    # scale = 0
    step = make_step("s0", 9, [6, 11], 2, 2, 8, 4, "bf16", keep_logical=True, scale=0.0)
    out = _run(step, lib)
    for s in range(2):
        _close(out[s], _mean_v(step, s), what="scale=0")
    # equal keys: overwrite every stored key (pool and new token) with one vector per head
    step = make_step("ek", 10, [9, 4], 4, 4, 8, 2, "f16", keep_logical=True)
    kvec = to_storage(np.linspace(-1, 1, 8, dtype=np.float32), "f16")
    step.k_cache[...] = kvec
    step.writes[0].k_new[...] = kvec
    out = _run(step, lib)
    for s in range(2):
        _close(out[s], _mean_v(step, s), what="equal keys")


def pin_two_token_closed_form(lib):
    # Scores s_0 = 0 and s_1 = scale * a; with scale*a = ln 3 the weights are 1/4 and 3/4.
    d = 4
    step = make_step("two", 12, [2], 1, 1, d, 4, "f32", keep_logical=True, scale=1.0)
    a = np.float32(math.log(3.0))
    q = np.zeros(d, np.float32)
    q[0] = 1.0
    step.q[0, 0] = q
    k0 = np.zeros(d, np.float32)
    k1 = np.zeros(d, np.float32)
    k1[0] = a
    phys = step.block_tables[0, 0]
    step.k_cache[phys, 0, 0] = k0
    step.writes[0].k_new[0, 0] = k1
    out = _run(step, lib)
    v = to_float64(step.logical_v[0], "f32")[:, 0, :]
    r = math.exp(float(a))  # = 3 up to the float32 rounding of ln 3
    expect = (v[0] + r * v[1]) / (1.0 + r)
    _close(out[0, 0], expect, what="two tokens")
    assert abs(r - 3.0) < 1e-6
    _close(out[0, 0], 0.25 * v[0] + 0.75 * v[1], rtol=1e-6, atol=1e-6, what="1/4, 3/4")


def pin_dominant_key(lib):
    step = make_step("dom", 13, [24], 2, 1, 16, 8, "f32", keep_logical=True)
    q64 = to_float64(step.q[0], "f32")
    # token 10 gets key = 40 * q_0, the others are small
    tstar = 10
    phys = step.block_tables[0, tstar // 8]
    step.k_cache[:, :, :, :] *= np.float32(0.01)
    step.writes[0].k_new *= np.float32(0.01)
    step.k_cache[phys, 0, tstar % 8] = (40.0 * q64[0]).astype(np.float32)
    out = _run(step, lib)
    v = to_float64(step.logical_v[0], "f32")[tstar, 0]
    _close(out[0, 0], v, rtol=1e-6, atol=1e-6, what="dominant key")


def pin_large_scores_finite(lib):
    step = make_step("big", 14, [50, 33], 4, 2, 64, 16, "f32", keep_logical=True)
    step.q *= np.float32(100.0)  # scores of order 1e3: exp would overflow without the max shift
    out = _run(step, lib)
    assert np.isfinite(out).all()
    for s in range(2):
        _close(out[s], _sdpa_ref(step, s), rtol=1e-10, what="large scores")


def pin_empty_context_is_zero(lib):
    step = make_step("t0", 15, [0, 3, 0], 2, 2, 8, 4, "f16", keep_logical=True)
    out = _run(step, lib)
    assert np.array_equal(out[0], np.zeros((2, 8))) and np.array_equal(out[2], np.zeros((2, 8)))
    _close(out[1], _sdpa_ref(step, 1), what="T=3 next to empty ones")


def pin_placement_invariance_bruteforce(lib):
    # All 5! placements of a 3-block sequence (T = 9, B = 4) in a 5-block pool.
    base = make_step("pl", 16, [9], 2, 1, 8, 4, "f32", num_blocks=5, keep_logical=True)
    ref = None
    for perm in itertools.permutations(range(5)):
        step = make_step("pl", 16, [9], 2, 1, 8, 4, "f32", num_blocks=5,
                         alloc_rng=_FixedOrder(perm))
        out = _run(step, lib)
        if ref is None:
            ref = out
            _close(ref[0], _sdpa_ref(base, 0), what="placement base")
        assert np.array_equal(out, ref), perm


class _FixedOrder:
    """Stands in for a Generator: its permutation() returns a fixed order."""

    def __init__(self, order):
        self.order = np.asarray(order)

    def permutation(self, n):
        assert n == len(self.order)
        return self.order.copy()


def pin_placement_invariance_random(lib):
    outs = []
    for r in range(4):
        step = make_step("pr", 17, [50, 7, 33, 16], 8, 2, 64, 16, "bf16",
                         alloc_rng=np.random.default_rng(1000 + r), pool_factor=3.0)
        outs.append(_run(step, lib))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


def pin_block_size_invariance(lib):
    outs = []
    for B in (1, 3, 8, 16, 32, 64):
        step = make_step("bs", 18, [50, 7, 33], 4, 2, 16, B, "f16")
        outs.append(_run(step, lib))
    for o in outs[1:]:
        _close(o, outs[0], what="block size")


def pin_poison_invariance(lib):
    clean = _run(make_step("pz", 19, [7, 16, 33, 50], 4, 4, 32, 16, "f32", poison=False), lib)
    nan = _run(make_step("pz", 19, [7, 16, 33, 50], 4, 4, 32, 16, "f32", poison=True), lib)
    step = make_step("pz", 19, [7, 16, 33, 50], 4, 4, 32, 16, "f32", poison=False)
    used = np.zeros(step.num_blocks, bool)
    used[step.block_tables[step.block_tables >= 0]] = True
    step.k_cache[~used] = np.float32(1e30)
    step.v_cache[~used] = np.float32(-1e30)
    big = _run(step, lib)
    assert np.array_equal(clean, nan) and np.array_equal(clean, big)
    assert np.isfinite(nan).all()


def pin_shared_prefix_matches_private(lib):
    kw = dict(prompts=2, samples=3, prompt_len=21, tail_len=9, heads=2, head_dim=8,
              block_size=4, dtype="f16", keep_logical=True)
    shared = shared_prefix_f16(**kw)
    private = shared_prefix_f16(private=True, **kw)
    assert len(shared.copies) == 2 * 2 and len(private.copies) == 0
    a = _run(shared, lib)
    b = _run(private, lib)
    assert np.array_equal(a, b)
    for s in range(shared.num_seqs):
        _close(a[s], _sdpa_ref(shared, s), what=f"shared seq {s}")


# ---- KV write and block copy ---------------------------------------------------------------


def pin_write_kv_vs_numpy(lib):
    rng = np.random.default_rng(20)
    for dt in ("f32", "f16", "bf16"):
        N, H, B, d = 6, 3, 4, 8
        kc = to_storage(rng.standard_normal((N, H, B, d)), dt)
        vc = to_storage(rng.standard_normal((N, H, B, d)), dt)
        n = 7
        slots = rng.choice(N * B, size=n, replace=False).astype(np.int32)
        slots[2] = -1  # skipped
        slots[5] = N * B + 3  # outside the pool: skipped
        kn = to_storage(rng.standard_normal((n, H, d)), dt)
        vn = to_storage(rng.standard_normal((n, H, d)), dt)
        ek, ev = kc.copy(), vc.copy()
        for i, sl in enumerate(slots):
            if 0 <= sl < N * B:
                ek[sl // B, :, sl % B, :] = kn[i]
                ev[sl // B, :, sl % B, :] = vn[i]
        oracle.write_kv(kc, vc, kn, vn, slots, dt, lib=lib)
        assert np.array_equal(kc.view(np.uint8), ek.view(np.uint8))
        assert np.array_equal(vc.view(np.uint8), ev.view(np.uint8))
    dup = np.array([3, 5, 3], np.int32)
    try:
        oracle.write_kv(kc, vc, kn[:3], vn[:3], dup, dt, lib=lib)
    except ValueError:
        pass
    else:
        raise AssertionError("duplicate slots accepted")


def pin_copy_blocks_vs_numpy(lib):
    rng = np.random.default_rng(21)
    for dt in ("f32", "bf16"):
        N, H, B, d = 8, 2, 4, 8
        kc = to_storage(rng.standard_normal((N, H, B, d)), dt)
        vc = to_storage(rng.standard_normal((N, H, B, d)), dt)
        pairs = np.array([[0, 5], [3, 6], [0, 7], [1, 99]], np.int32)  # last one skipped
        ek, ev = kc.copy(), vc.copy()
        for s, t in pairs[:3]:
            ek[t] = ek[s]
            ev[t] = ev[s]
        oracle.copy_blocks(kc, vc, pairs, dt, lib=lib)
        assert np.array_equal(kc.view(np.uint8), ek.view(np.uint8))
        assert np.array_equal(vc.view(np.uint8), ev.view(np.uint8))
    for bad in ([[0, 5], [5, 6]], [[0, 5], [1, 5]]):
        try:
            oracle.copy_blocks(kc, vc, np.array(bad, np.int32), dt, lib=lib)
        except ValueError:
            continue
        raise AssertionError(f"overlapping pairs accepted: {bad}")


def pin_swap_blocks_vs_numpy(lib):
    rng = np.random.default_rng(23)
    for dt in ("f16", "f32"):
        H, B, d = 2, 4, 8
        dev_k = to_storage(rng.standard_normal((9, H, B, d)), dt)
        dev_v = to_storage(rng.standard_normal((9, H, B, d)), dt)
        host_k = to_storage(rng.standard_normal((5, H, B, d)), dt)
        host_v = to_storage(rng.standard_normal((5, H, B, d)), dt)
        out_pairs = np.array([[3, 0], [8, 4], [1, 2], [2, 77]], np.int32)  # last one skipped
        ek, ev = host_k.copy(), host_v.copy()
        for s_, t in out_pairs[:3]:
            ek[t] = dev_k[s_]
            ev[t] = dev_v[s_]
        oracle.swap_blocks(host_k, host_v, dev_k, dev_v, out_pairs, dt, lib=lib)
        assert np.array_equal(host_k.view(np.uint8), ek.view(np.uint8))
        assert np.array_equal(host_v.view(np.uint8), ev.view(np.uint8))
        # and back into other device blocks: the round trip restores the contents
        back = np.array([[0, 5], [4, 6], [2, 7]], np.int32)
        oracle.swap_blocks(dev_k, dev_v, host_k, host_v, back, dt, lib=lib)
        for (s_, _), (_, t) in zip(out_pairs[:3], back):
            assert np.array_equal(dev_k[t].view(np.uint8), dev_k[s_].view(np.uint8)) or s_ == t
    try:
        oracle.swap_blocks(host_k, host_v, dev_k, dev_v, np.array([[0, 1], [2, 1]], np.int32),
                           dt, lib=lib)
    except ValueError:
        pass
    else:
        raise AssertionError("repeated destination accepted")


def pin_allocator_tables(lib):
    """The toy block manager gives ceil(T/B) blocks per sequence, never shares a block between
    unrelated sequences, and wastes at most B-1 slots per sequence ([PA-summary] "Results":
    the only waste left is internal fragmentation of each sequence's last block)."""
    alloc = BlockAllocator(40, np.random.default_rng(22))
    seqs = [Sequence(4) for _ in range(5)]
    for s, T in zip(seqs, (1, 4, 5, 16, 17)):
        append_tokens(alloc, s, T)
        assert len(s.table) == math.ceil(T / 4)
        assert 0 <= len(s.table) * 4 - T < 4
    used = [b for s in seqs for b in s.table]
    assert len(used) == len(set(used))
    bt = block_tables_array(seqs)
    assert bt.shape == (5, 5) and (bt[0, 1:] == -1).all()


# ---- multi-query (prefill / chunked-prefill) attention ----------------------------------------

PREFILL_TINY = [
    # (context lengths, query lengths, Hq, Hkv, d, B, dtype)
    ([7, 16, 33, 50, 5], [7, 3, 16, 1, 0], 4, 2, 16, 8, "f16"),
    ([9, 12], [9, 12], 2, 2, 8, 4, "f32"),
    ([20, 1, 6], [5, 1, 2], 8, 2, 8, 3, "bf16"),
    ([40, 17], [40, 9], 4, 1, 16, 16, "f32"),
    ([3, 8], [2, 8], 2, 2, 4, 1, "f16"),
]


def _sdpa_prefill_ref(step, s, is_causal=False):
    """Standard attention (torch SDPA, float64 CPU) of the query chunk of sequence s on its
    logical K/V, query i seeing positions 0 .. T-n+i."""
    T = int(step.context_lens[s])
    a, b = int(step.query_start[s]), int(step.query_start[s + 1])
    n = b - a
    q = torch.from_numpy(to_float64(step.q[a:b], step.dtype)).permute(1, 0, 2)  # [Hq, n, d]
    k = torch.from_numpy(to_float64(step.logical_k[s], step.dtype))  # [T, Hkv, d]
    v = torch.from_numpy(to_float64(step.logical_v[s], step.dtype))
    g = step.num_q_heads // step.num_kv_heads
    k = k.repeat_interleave(g, dim=1).permute(1, 0, 2).contiguous()  # [Hq, T, d]
    v = v.repeat_interleave(g, dim=1).permute(1, 0, 2).contiguous()
    if is_causal:
        assert n == T
        o = torch.nn.functional.scaled_dot_product_attention(
            q.contiguous(), k, v, is_causal=True, scale=float(step.scale))
    else:
        mask = torch.arange(T)[None, :] <= (T - n + torch.arange(n))[:, None]  # True = attend
        o = torch.nn.functional.scaled_dot_product_attention(
            q.contiguous(), k, v, attn_mask=mask, scale=float(step.scale))
    return o.permute(1, 0, 2).numpy()  # [n, Hq, d]


def _prefill(step, lib):
    return oracle.run_prefill_step(step, lib=lib)[0]


def pin_prefill_vs_sdpa_masked(lib):
    for i, (T, n, Hq, Hkv, d, B, dt) in enumerate(PREFILL_TINY):
        step = make_prefill_step("pf", 300 + i, T, n, Hq, Hkv, d, B, dt, keep_logical=True)
        out = _prefill(step, lib)
        for s in range(len(T)):
            a, b = step.query_start[s], step.query_start[s + 1]
            if b > a:
                _close(out[a:b], _sdpa_prefill_ref(step, s), what=f"prefill case {i} seq {s}")


def pin_prefill_whole_prompt_is_causal(lib):
    # n == T: the chunk is the whole context; SDPA's own causal mask (top-left aligned, which
    # equals bottom-right alignment when n == T) is the reference
    for i, (T, Hq, Hkv, d, B, dt) in enumerate([([9, 12, 1], 2, 2, 8, 4, "f32"),
                                                  ([33, 16], 8, 2, 16, 16, "bf16")]):
        step = make_prefill_step("pc", 320 + i, T, T, Hq, Hkv, d, B, dt, keep_logical=True)
        out = _prefill(step, lib)
        for s in range(len(T)):
            a, b = step.query_start[s], step.query_start[s + 1]
            _close(out[a:b], _sdpa_prefill_ref(step, s, is_causal=True), what=f"causal {i}/{s}")


def pin_prefill_last_query_is_decode(lib):
    step = make_prefill_step("pd", 330, [7, 16, 33, 50], [7, 3, 16, 1], 8, 2, 16, 8, "f16")
    out, kc, vc = oracle.run_prefill_step(step, lib=lib)
    last = step.query_start[1:] - 1
    q_dec = np.ascontiguousarray(step.q[last])  # [S, Hq, d]
    dec = oracle.decode(q_dec, kc, vc, step.block_tables, step.context_lens, step.scale,
                        step.dtype, lib=lib)
    _close(out[last], dec, what="last query vs decode")


def pin_prefill_future_tokens_ignored(lib):
    # Sequence 0: T = 20 with a chunk of n = 6 (positions 14..19). Changing the stored key and
    # value at position 16 must leave queries 0, 1 (positions 14, 15) bit-identical and change
    # queries 2.. (positions 16..19).
    step = make_prefill_step("pfut", 340, [20, 9], [6, 4], 2, 1, 8, 4, "f32")
    out, kc, vc = oracle.run_prefill_step(step, lib=lib)
    pos = 16
    phys = step.block_tables[0, pos // 4]
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[phys, :, pos % 4] += np.float32(3.0)
    vc2[phys, :, pos % 4] -= np.float32(5.0)
    out2 = oracle.prefill(step.q, kc2, vc2, step.block_tables, step.context_lens,
                          step.query_start, step.scale, step.dtype, lib=lib)
    assert np.array_equal(out2[0:2], out[0:2]), "a query saw a later position"
    assert np.array_equal(out2[6:], out[6:]), "another sequence changed"
    for i in range(2, 6):
        assert np.abs(out2[i] - out[i]).max() > 1e-6, f"query {i} did not see position {pos}"


def pin_prefill_placement_and_block_size(lib):
    outs = []
    for r in range(3):
        step = make_prefill_step("ppl", 350, [50, 7, 33], [20, 7, 1], 8, 2, 16, 8, "bf16",
                                 alloc_rng=np.random.default_rng(2000 + r), pool_factor=2.5)
        outs.append(_prefill(step, lib))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    for B in (1, 3, 16, 64):
        step = make_prefill_step("ppl", 350, [50, 7, 33], [20, 7, 1], 8, 2, 16, B, "bf16")
        _close(_prefill(step, lib), outs[0], what=f"prefill block size {B}")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
