"""pa_decode_noalloc (split-K partials in the library's static per-GPU scratch array) against
pa_decode with a caller workspace, through the C ABI: the same kernels and partition choice, so
the outputs must agree bit for bit, and both must match the oracle within the attention
tolerance. Two calls in a row share the scratch array; the second is smaller (fewer sequences,
shorter contexts, other partitions), so stale partials from the first call would show."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import paged_kv_cache_82_amd as pa
from gpu_harness import DevStep, assert_attention_close, to_host
from workloads import make_step

pytestmark = pytest.mark.gpu


def _both(step, P):
    dev = DevStep(step, partition_tokens=P)
    dev.apply_updates()
    dev.decode()
    ref_out = dev.out.clone()
    out2 = torch.full_like(dev.out, float("nan"))
    pa.pa_decode_noalloc(out2, dev.q, dev.k_cache, dev.v_cache, dev.block_tables,
                         dev.context_lens, float(step.scale), step.max_context_len, P)
    torch.cuda.synchronize()
    got = to_host(out2, step.dtype)
    want = to_host(ref_out, step.dtype)
    assert got.view(np.uint8).tobytes() == want.view(np.uint8).tobytes(), "noalloc != pa_decode"
    ref, _, _ = oracle.run_step(step)
    return assert_attention_close(got, ref, step.dtype, f"{step.name} P={P}")


@pytest.mark.parametrize("dt,Hq,Hkv", [("bf16", 32, 4), ("f16", 8, 8), ("f32", 4, 4)])
def test_noalloc_matches_decode_twice(dt, Hq, Hkv):
    print(f"\n[gpu-test] noalloc {dt} Hq={Hq} Hkv={Hkv}", flush=True)
    big = make_step("noalloc-big", 90, [3000, 17, 0, 1, 4096, 2049, 640, 33], Hq, Hkv, 128, 16, dt)
    e1 = _both(big, 128)
    small = make_step("noalloc-small", 91, [700, 5, 96], Hq, Hkv, 128, 16, dt)
    e2 = _both(small, 64)
    # the automatic partition choice (these batches are small: the sequences split)
    e3 = _both(small, 0)
    print(f"noalloc {dt} max abs err {e1:.3g} / {e2:.3g} / {e3:.3g}", flush=True)


def test_noalloc_long_context_plan_fits():
    """The long-context shape's automatic plan (8 sequences x 32 heads, 2048-token partitions of
    up to 128k tokens) fits the scratch array; a few sequences of that length, decoded."""
    need = pa.pa_decode_workspace_size(8, 32, 32, 128, 16, 131072, 0, torch.bfloat16)
    assert 0 < need <= pa.SCRATCH_BYTES
    print("\n[gpu-test] noalloc long", flush=True)
    step = make_step("noalloc-long", 92, [40000, 9000], 32, 32, 128, 16, "bf16")
    err = _both(step, 0)
    print(f"noalloc long max abs err {err:.3g}", flush=True)


def test_noalloc_rejects_plans_beyond_the_scratch_array():
    step = make_step("noalloc-reject", 93, [4096] * 4, 64, 64, 128, 16, "f16", poison=False)
    dev = DevStep(step, partition_tokens=32)
    # 4 x 64 heads x 128 partitions x 130 floats: 17 MB > 16 MiB; nothing is launched
    assert (pa.pa_decode_workspace_size(4, 64, 64, 128, 16, 4096, 32, torch.float16)
            > pa.SCRATCH_BYTES)
    with pytest.raises(pa.PAError) as e:
        pa.pa_decode_noalloc(dev.out, dev.q, dev.k_cache, dev.v_cache, dev.block_tables,
                             dev.context_lens, float(step.scale), step.max_context_len, 32)
    assert e.value.status == 3  # PA_ERR_WORKSPACE
