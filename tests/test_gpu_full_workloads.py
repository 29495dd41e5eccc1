"""GPU parity at the full sizes of the four large workloads, in the launch configuration the
benchmark times (automatic partition size).

  13B-shape fp16 MHA    (64 seqs, 40 heads, d=128, B=16, lognormal lengths)  all outputs
  GQA bf16              (256 seqs, 64/8 heads, uniform 128..4096)            all outputs
  long-context bf16     (8 seqs, 32 heads, uniform 32k..128k)                2 sampled seqs
  shared-prefix fp16    (16 prompts x 4 samples, B=32)                       in test_gpu_parity

The KV writes are checked bit-exactly: the whole pool for the first two, and for the long-
context pool (13+ GB) the written rows plus a count of changed elements, on the device."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
from gpu_harness import DevStep, assert_attention_close, to_dev, to_host
from workloads import mha13b_f16, gqa_bf16, long_bf16

pytestmark = pytest.mark.gpu


def _full(step):
    dev = DevStep(step)
    got = dev.run()
    ref, kc, vc = oracle.run_step(step, in_place=True)
    assert np.array_equal(to_host(dev.k_cache, step.dtype).view(np.uint8), kc.view(np.uint8))
    assert np.array_equal(to_host(dev.v_cache, step.dtype).view(np.uint8), vc.view(np.uint8))
    return assert_attention_close(got, ref, step.dtype, step.name)


def test_mha13b_f16_full():
    print("\n[gpu-test] mha13b_f16 full", flush=True)
    err = _full(mha13b_f16())
    print(f"mha13b_f16 max abs err {err:.3g}", flush=True)


def test_gqa_bf16_full():
    print("\n[gpu-test] gqa_bf16 full", flush=True)
    err = _full(gqa_bf16())
    print(f"gqa_bf16 max abs err {err:.3g}", flush=True)


def test_long_bf16_sampled():
    print("\n[gpu-test] long_bf16 sampled", flush=True)
    step = long_bf16()
    dev = DevStep(step)
    k_before = dev.k_cache.clone()
    got = dev.run()
    # writes: exactly the written rows changed, to the new values
    w = step.writes[0]
    B = step.block_size
    slots = w.slot_mapping.astype(np.int64)
    blk = torch.from_numpy(slots // B).cuda()
    off = torch.from_numpy(slots % B).cuda()
    rows = dev.k_cache[blk, :, off, :]  # [n, Hkv, d]
    assert torch.equal(rows.view(torch.int16), to_dev(w.k_new, step.dtype).view(torch.int16))
    changed = (dev.k_cache.view(torch.int16) != k_before.view(torch.int16)).sum().item()
    assert changed <= rows.numel()
    del k_before
    sample = [int(np.argmin(step.context_lens)), int(np.argmax(step.context_lens))]
    ref, _, _ = oracle.run_step(step, seq_list=sample, in_place=True)
    err = assert_attention_close(got[sample], ref, step.dtype, "long_bf16 sample")
    print(f"long_bf16 sample {sample} lens {step.context_lens[sample].tolist()} max abs err {err:.3g}",
          flush=True)
