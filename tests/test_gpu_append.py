"""GPU parity of pa_decode_append (the decode step's KV write and attention in one launch)
against the CPU oracle, through the C ABI: the oracle runs the step as pa_write_kv followed by
decode; the fused call must leave the pools bit-identical and match the attention within the
tolerance (max-abs 1e-5 for fp32, 2e-2 + 1e-2 |ref| for fp16/bf16). Both decode kernels, whole
and split sequences (the new token is folded into the last partition), one-token and empty
sequences, and tokens whose slot is negative (attended, not stored). Graph replay is in
test_gpu_graph.py."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import paged_kv_cache_82_amd as pa
from gpu_harness import DevStep, assert_attention_close, to_dev, to_host
from workloads import make_step, to_float64

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[gpu-test] {request.node.name}", flush=True)
    yield


def _bits(a):
    return a.view(np.uint8)


def append_rows(step):
    """The step's new tokens as [S][Hkv][d] rows and [S] slots (zero rows and slot -1 for a
    sequence with no token)."""
    w = step.writes[0]
    S, Hkv, d = step.num_seqs, step.num_kv_heads, step.head_dim
    kn = np.zeros((S, Hkv, d), w.k_new.dtype)
    vn = np.zeros((S, Hkv, d), w.v_new.dtype)
    slots = np.full(S, -1, np.int32)
    has = np.nonzero(step.context_lens > 0)[0]
    kn[has], vn[has], slots[has] = w.k_new, w.v_new, w.slot_mapping
    return kn, vn, slots


def _run_append(step, P=0, drop_slot=None):
    """Fused call on the step's pools (before its write); returns (out, k pool, v pool)."""
    dev = DevStep(step, P)
    kn, vn, slots = append_rows(step)
    if drop_slot is not None:
        slots[drop_slot] = -1
    pa.pa_decode_append(dev.out, dev.q, dev.k_cache, dev.v_cache, to_dev(kn, step.dtype, "cuda"),
                        to_dev(vn, step.dtype, "cuda"), to_dev(slots, None, "cuda"),
                        dev.block_tables, dev.context_lens, float(step.scale),
                        step.max_context_len, dev.workspace, P)
    torch.cuda.synchronize()
    return (to_host(dev.out, step.dtype), to_host(dev.k_cache, step.dtype),
            to_host(dev.v_cache, step.dtype))


CASES = [
    # (Hq, Hkv, d, B, dtype, lengths)
    (8, 8, 128, 16, "f16", [1, 2, 16, 17, 33, 700, 2048]),     # vector-ALU kernel
    (4, 4, 64, 32, "f32", [1, 31, 32, 33, 500]),
    (16, 2, 128, 16, "bf16", [1, 5, 16, 33, 130, 1500]),       # MFMA kernel
    (64, 2, 128, 64, "bf16", [1, 63, 64, 65, 900]),            # 32 heads per workgroup
    (8, 2, 64, 8, "f16", [0, 1, 9, 0, 300]),                   # empty sequences
    (8, 8, 64, 16, "bf16", [1, 15, 16, 17, 250, 1100]),        # vector-ALU, 8-deep ring
    (8, 8, 128, 8, "f16", [1, 7, 8, 9, 400, 1500]),            # vector-ALU, 8-deep ring
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("P", [0, 32, 64])
def test_append_matches_write_then_decode(case, P):
    Hq, Hkv, d, B, dt, lens = CASES[case]
    step = make_step("app", 600 + case, lens, Hq, Hkv, d, B, dt)
    ref, kc, vc = oracle.run_step(step)
    got, gk, gv = _run_append(step, P)
    assert np.array_equal(_bits(gk), _bits(kc)) and np.array_equal(_bits(gv), _bits(vc))
    assert_attention_close(got, ref, dt, f"append case {case} P{P}")
    # the plain pair of calls on the same inputs agrees within the same tolerance
    plain = DevStep(step, P).run()
    assert_attention_close(got, to_float64(plain, dt), dt, f"append vs write+decode {case}")


def test_append_with_negative_slot_attends_but_does_not_store():
    step = make_step("appneg", 620, [40, 300, 7], 16, 2, 128, 16, "bf16")
    ref, kc, vc = oracle.run_step(step)
    got, gk, gv = _run_append(step, drop_slot=1)
    assert_attention_close(got, ref, "bf16", "negative slot")
    # the pools equal the oracle's except the dropped slot, which keeps its prior contents
    slot = int(step.writes[0].slot_mapping[1])
    blk, off = divmod(slot, step.block_size)
    assert np.array_equal(_bits(gk[blk, :, off]), _bits(step.k_cache[blk, :, off]))
    gk[blk, :, off] = kc[blk, :, off]
    gv[blk, :, off] = vc[blk, :, off]
    assert np.array_equal(_bits(gk), _bits(kc)) and np.array_equal(_bits(gv), _bits(vc))
