"""GPU parity of pa_decode_shared_prefix (groups of sequences sharing the blocks of a common
prefix; the prefix is scored once per group on MFMA) against the CPU oracle, through the C ABI.
The oracle reads every sequence through its own table, so sharing is invisible to it: the
result must be plain decode attention, within the attention tolerance. Also compared with
pa_decode on the same step. Cases: the shared-prefix workload at full size (its groups read off
the tables, as pa_bm_prefix_groups gives them), grouped heads, every block size, prefixes that
end inside a 32-token step, members with no tokens of their own, groups of one, groups wider
than one 16-column tile, forced partitions of both passes, and fp32 (pa_decode's path)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import paged_kv_cache_82_amd as pa
from gpu_harness import (TORCH_DT, DevStep, assert_attention_close, check_full_size,
                         groups_from_tables, share_prefixes, to_dev, to_host)
from workloads import make_step, shared_prefix_f16, to_float64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-test] {request.node.name}", flush=True)
    yield


def _run_shared(step, group_start, prefix_lens, P=0, max_group=None):
    dev = DevStep(step)
    dev.apply_updates()
    gs = to_dev(np.asarray(group_start, np.int32))
    pl = to_dev(np.asarray(prefix_lens, np.int32))
    sizes = np.diff(group_start)
    mg = int(max_group or (sizes.max() if len(sizes) else 1))
    mp = int(np.max(prefix_lens)) if len(prefix_lens) else 0
    nbytes = pa.pa_decode_shared_prefix_workspace_size(
        step.num_seqs, len(group_start) - 1, step.num_q_heads, step.num_kv_heads, step.head_dim,
        step.block_size, step.max_context_len, mp, mg, P, TORCH_DT[step.dtype])
    ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    out = torch.full_like(dev.q, float("nan"))
    pa.pa_decode_shared_prefix(out, dev.q, dev.k_cache, dev.v_cache, dev.block_tables,
                               dev.context_lens, pl, gs, float(step.scale), step.max_context_len,
                               mp, mg, ws, P)
    dev.decode()  # pa_decode on the same pools, for comparison
    torch.cuda.synchronize()
    return to_host(out, step.dtype), to_host(dev.out, step.dtype)


def _check(step, group_start, prefix_lens, what, **kw):
    got, plain = _run_shared(step, group_start, prefix_lens, **kw)
    ref, _, _ = oracle.run_step(step)
    err = assert_attention_close(got, ref, step.dtype, what)
    assert_attention_close(got, to_float64(plain, step.dtype), step.dtype, what + " vs pa_decode")
    return got, ref, err


@pytest.mark.parametrize("dt", ["f16", "bf16"])
@pytest.mark.parametrize("B", [8, 16, 32, 64])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (16, 2)])
def test_groups_every_block_size(dt, B, Hq, Hkv):
    # three groups (4, 3 and 2 members) and two sequences on their own; prefixes of whole
    # 32-token steps and prefixes that end inside a step (the rest goes with the own tokens)
    lens = [300, 310, 299, 400, 90, 75, 96, 50, 1, 0, 260, 261]
    step = make_step("shp", 900 + B + Hq, lens, Hq, Hkv, 128, B, dt)
    k1 = 64 // B          # 64 tokens: two whole steps
    k2 = max(1, 40 // B)  # 40 (or 32, 64) tokens: inside a step for B = 8
    gs, pl = share_prefixes(step, [(0, 4, 280 // B), (4, 3, k1), (10, 2, k2)])
    _check(step, gs, pl, f"groups {dt} B{B} g{Hq // Hkv}")


@pytest.mark.parametrize("P", [32, 64, 96, 256, 0])
def test_forced_partitions(P):
    # a group's list (a 640-token prefix, then 60-65 own tokens per member) cut into partitions
    # of 32 .. 256 tokens, the merge kernel combining them; partition edges between the prefix
    # and the own tokens and inside either
    lens = [700, 701, 705, 703, 64, 33]
    step = make_step("shpP", 930, lens, 16, 2, 128, 16, "bf16")
    gs, pl = share_prefixes(step, [(0, 4, 40)])
    _check(step, gs, pl, f"P={P}", P=P)


def test_members_without_own_tokens_and_wide_groups():
    # a prefix that reaches each member's last block (no own tokens beyond the last step of
    # the prefix but the written token), 20 MHA members (two column tiles) and 5 members x 8
    # query heads (three column tiles)
    lens = [129] * 20 + [65] * 5
    step = make_step("shpW", 931, lens, 8, 8, 64, 32, "f16")
    gs, pl = share_prefixes(step, [(0, 20, 4), (20, 5, 2)])
    _check(step, gs, pl, "wide MHA groups")
    step = make_step("shpW2", 932, [65] * 5 + [200], 16, 2, 128, 16, "bf16")
    gs, pl = share_prefixes(step, [(0, 5, 4)])
    _check(step, gs, pl, "wide GQA group")


def test_no_groups_and_fp32():
    step = make_step("shp0", 933, [10, 0, 300, 1], 8, 8, 128, 16, "f16")
    _check(step, np.array([0, 1, 2, 3, 4], np.int32), np.zeros(4, np.int32), "groups of one")
    step = make_step("shpf", 934, [100, 101, 300], 4, 4, 128, 16, "f32")
    gs, pl = share_prefixes(step, [(0, 2, 6)])
    got, ref, err = _check(step, gs, pl, "fp32")
    assert err <= 1e-5


def test_shared_prefix_workload_full():
    # the 16 prompts x 4 samples workload: groups read off its tables (32 shared blocks of 32
    # tokens per prompt after the copy-on-write of the partial one)
    step = shared_prefix_f16()
    gs, pl = groups_from_tables(step.block_tables, step.context_lens, step.block_size)
    assert len(gs) - 1 == 16 and (pl == 1024).all()
    got, plain = _run_shared(step, gs, pl)
    ref, _, _ = oracle.run_step(step)
    check_full_size(got, ref, step.dtype, step.context_lens, True, "shared-prefix-f16 grouped")
    assert_attention_close(got, to_float64(plain, step.dtype), step.dtype, "vs pa_decode")


@pytest.mark.parametrize("P", [0, 64])
def test_prefix_is_the_whole_context(P):
    # every member's table is the leader's and the prefix is the whole context (no own tokens):
    # with one partition the workgroup writes the final outputs, with two the merge kernel
    # combines them
    step = make_step("shpA", 935, [128] * 4 + [40], 8, 8, 128, 32, "bf16")
    for m in range(1, 4):
        step.block_tables[m] = step.block_tables[0]
    w = step.writes[0]
    w.slot_mapping[1:4] = -1  # the leader's write is every member's last token
    gs = np.array([0, 4, 5], np.int32)
    pl = np.array([128] * 4 + [0], np.int32)
    _check(step, gs, pl, f"whole-context prefix P={P}", P=P)
