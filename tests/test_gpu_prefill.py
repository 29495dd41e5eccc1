"""GPU parity of pa_prefill (causal multi-query attention over the paged pool) against the CPU
oracle, through the C ABI: |gpu - ref| <= 2e-2 + 1e-2 |ref| elementwise for 16-bit inputs (fp32
accumulation, 16-bit MFMA kernel) and max-abs 1e-5 for fp32 inputs (fp32 MFMA kernel), the
chunk's KV write bit-exact. Shapes span several row tiles with ragged
tails, contexts that need more than one register of block ids, every supported head size,
block size and group size, empty chunks, whole prompts and single-token chunks."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
from gpu_harness import (DevPrefill, DevStep, assert_attention_close, check_full_size,
                         make_dominant_token, prefill_rows_reference, to_host)
from workloads import make_prefill_step, make_step, to_float64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-test] {request.node.name}", flush=True)
    yield


def _bits(a):
    return a.view(np.uint8)


def _check(step, what="", f32_score_factor=1.0):
    """f32_score_factor: how many times larger than N(0,1) data at scale 1/sqrt(d) the scores
    are. An fp32 score's rounding error grows with the products it sums, and an output moves by
    about that error times the spread of V, so the fp32 bound (1e-5) is scaled by the factor;
    a numpy fp32 evaluation of the scale-3 case below (4-term fp32 sums, fp32 softmax) is off
    by 4.0e-5, for example."""
    ref, kc, vc = oracle.run_prefill_step(step)
    dev = DevPrefill(step)
    got = dev.run()
    assert np.array_equal(_bits(to_host(dev.k_cache, step.dtype)), _bits(kc)), what
    assert np.array_equal(_bits(to_host(dev.v_cache, step.dtype)), _bits(vc)), what
    owned = np.zeros(step.num_q_tokens, bool)
    owned[step.query_start[0]:step.query_start[-1]] = True
    if step.dtype == "f32" and f32_score_factor > 1.0:
        assert np.isfinite(got[owned]).all(), what
        err = float(np.abs(got[owned].astype(np.float64) - ref[owned]).max())
        assert err <= f32_score_factor * 1e-5, (what, err)
    else:
        assert_attention_close(got[owned], ref[owned], step.dtype, what)
    return got, ref


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B", [8, 16, 32, 64])
def test_prefill_shapes_mha(dt, d, B):
    # whole prompts, chunks after a cached prefix, a single-token chunk, an empty chunk; 300
    # query rows span three row tiles of 128 with a ragged tail
    T = [40, 300, 77, 1, 65, 9]
    n = [40, 300, 20, 1, 1, 0]
    step = make_prefill_step("pmha", 400 + B + d, T, n, 4, 4, d, B, dt)
    _check(step, f"mha {dt} d{d} B{B}")


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("g", [2, 4, 8, 16])
@pytest.mark.parametrize("d,B", [(128, 16), (64, 8), (128, 32), (128, 64)])
def test_prefill_shapes_gqa(dt, g, d, B):
    T = [33, 130, 257, 5]
    n = [33, 50, 17, 5]
    step = make_prefill_step("pgqa", 420 + g, T, n, 2 * g, 2, d, B, dt)
    _check(step, f"gqa {dt} g{g} d{d} B{B}")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_prefill_long_context_rotates_block_ids(dt):
    # positions past 64 and 128 stages of 32 tokens: both kernels load block ids 64 stages at a
    # time, and rows of one wave straddle a 32-token stage boundary
    T = [4500, 2100, 70]
    n = [100, 37, 70]
    step = make_prefill_step("plong", 430, T, n, 8, 2, 128, 16, dt)
    _check(step, f"long {dt}")


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
def test_prefill_bulk_loop_boundaries(dt):
    # prefixes of 0 .. 700 tokens in steps that move the end of the leading fully visible
    # stages (whole 32-token stages before a workgroup's first row, rounded down to the stage
    # unroll) through every stage and buffer phase, for chunks of one and of several row tiles
    T = [p + n for p in range(0, 701, 37) for n in (48, 200)]
    n = [n for p in range(0, 701, 37) for n in (48, 200)]
    step = make_prefill_step("pbulk", 475, T, n, 4, 4, 128, 16, dt)
    _check(step, f"bulk boundaries {dt}")


def test_prefill_single_token_matches_decode():
    # n = 1 for every sequence is a decode step: both kernels against the oracle, and each other
    lengths = [1, 7, 100, 513, 1500]
    pstep = make_prefill_step("p1", 440, lengths, [1] * len(lengths), 16, 2, 128, 16, "f16")
    got_p, _ = _check(pstep, "prefill n=1")
    dstep = make_step("d1", 440, lengths, 16, 2, 128, 16, "f16")
    dstep.q[...] = pstep.q  # same query vectors
    dref, _, _ = oracle.run_step(dstep)
    got_d = DevStep(dstep).run()
    assert_attention_close(got_d, dref, "f16", "decode")
    assert_attention_close(got_p, to_float64(got_d, "f16"), "f16", "prefill vs decode")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_prefill_placement_invariance_bit_exact(dt):
    outs = []
    for r in range(3):
        step = make_prefill_step("ppl", 450, [300, 41, 129], [200, 41, 3], 16, 2, 128, 16,
                                 dt, alloc_rng=np.random.default_rng(700 + r),
                                 pool_factor=2.0)
        outs.append(DevPrefill(step).run())
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_prefill_large_scores_stay_finite(dt):
    step = make_prefill_step("pbig", 460, [90, 300], [90, 64], 8, 2, 128, 16, dt)
    from workloads import to_storage

    step.q[...] = to_storage(to_float64(step.q, dt) * 30.0, dt)
    _check(step, f"large scores {dt}", f32_score_factor=30.0)


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("g", [1, 4])
def test_prefill_small_weights_below_fp16_normal(dt, g):
    # one token outweighs 3999 others by 2^15: their 16-bit weights are fp16 subnormals that
    # together add 12% to the row sum; the weighted sum and the row sum must both keep them
    step = make_dominant_token(make_prefill_step("pdom", 480, [4000], [4], 2 * g, 2, 128, 16, dt))
    _check(step, f"dominant token {dt} g{g}")


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("g", [1, 8])
@pytest.mark.parametrize("rise", [2.0, 7.9, 8.1, 20.0])
def test_prefill_rising_maximum(dt, g, rise):
    # The prefill kernels take weights against a reference maximum raised only past a slack of
    # 2^8. Scores that climb by about `rise` in the base-2 exponent (times 1 + h/16 for query
    # head h) from one 32-token stage to the next, prefix and chunk alike, raise it never,
    # sometimes or at every stage. fp32 scores this large (up to about 2e3) carry rounding
    # errors of their own, hence the scaled fp32 bound.
    from workloads import to_storage

    Hkv, d, B = 2, 128, 16
    prefix, n = 700, 300
    step = make_prefill_step("rise", 780 + g, [prefix + n], [n], g * Hkv, Hkv, d, B, dt)
    rng = np.random.default_rng(int(rise * 10) + g)
    T = prefix + n
    unit = 1.0 / (4.0 * float(step.scale) * np.log2(np.e))
    k = 0.3 * rng.standard_normal((T, Hkv, d))
    k[:, :, 0] = rise * unit * (np.arange(T) // 32)[:, None]
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
    q = 0.3 * rng.standard_normal(step.q.shape)
    q[..., 0] = 4.0 * (1.0 + np.arange(g * Hkv) / 16.0)
    step.q[...] = to_storage(q, dt)
    _check(step, f"rising maximum {dt} g{g} rise {rise}", f32_score_factor=1000.0)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("scale", [0.0, -1.0 / 128 ** 0.5, 3.0])
def test_prefill_scale_zero_negative_large(dt, scale):
    # scale 0 weighs every visible token equally (the mean of V over the causal prefix); a
    # negative scale reverses the score order; both are taken exactly by the kernels
    step = make_prefill_step("pscale", 465, [90, 300, 17], [90, 64, 17], 8, 2, 128, 16, dt,
                             scale=scale)
    _check(step, f"scale {scale} {dt}", f32_score_factor=abs(scale) * 128 ** 0.5)


@pytest.mark.parametrize("dt", ["f16", "f32"])
def test_prefill_rows_outside_sequences_untouched(dt):
    # query_start need not start at 0 nor end at num_q_tokens: rows no sequence owns keep
    # their contents
    step = make_prefill_step("pown", 470, [20, 30], [8, 12], 4, 4, 64, 16, dt)
    pad = 3
    Nq = step.num_q_tokens
    q = np.zeros((Nq + 2 * pad,) + step.q.shape[1:], step.q.dtype)
    q[pad:pad + Nq] = step.q
    step.q = q
    step.query_start = step.query_start + pad
    dev = DevPrefill(step)
    dev.out.fill_(7.0)
    got = dev.run()
    assert (got[:pad] == 7.0).all() and (got[pad + Nq:] == 7.0).all()
    ref, _, _ = oracle.run_prefill_step(step)
    assert_attention_close(got[pad:pad + Nq], ref[pad:pad + Nq], dt, "offset rows")


@pytest.mark.parametrize("name", ["prefill_mha13b", "prefill_gqa", "prefill_mha13b_f32"])
def test_prefill_full_size_sampled_rows(name):
    # the benchmark's workloads at full size, in the benchmark's launch configuration; the
    # oracle checks 96 sampled rows (first, last and random rows of every sequence)
    import workloads.configs as cfg

    step = getattr(cfg, name)()
    dev = DevPrefill(step)
    got = dev.run()
    kc = to_host(dev.k_cache, step.dtype)
    vc = to_host(dev.v_cache, step.dtype)
    ref_pool = step.k_cache.copy(), step.v_cache.copy()
    for w in step.writes:
        oracle.write_kv(ref_pool[0], ref_pool[1], w.k_new, w.v_new, w.slot_mapping, step.dtype)
    assert np.array_equal(_bits(kc), _bits(ref_pool[0])) and np.array_equal(_bits(vc), _bits(ref_pool[1]))
    rng = np.random.default_rng(480)
    qs = step.query_start
    rows = set()
    for s in range(step.num_seqs):
        if qs[s + 1] > qs[s]:
            rows.update({int(qs[s]), int(qs[s + 1] - 1)})
    rows.update(rng.integers(0, step.num_q_tokens, size=96 - len(rows)).tolist())
    rows = np.array(sorted(rows))
    ref = prefill_rows_reference(step, kc, vc, rows)
    seq = np.searchsorted(qs, rows, side="right") - 1
    visible = step.context_lens[seq] - (qs[seq + 1] - qs[seq]) + (rows - qs[seq]) + 1
    check_full_size(got[rows], ref, step.dtype, visible, True, f"{step.name} (96 rows)")
    assert np.isfinite(to_float64(got, step.dtype)).all()
