"""Benchmark of the paged decode hot path on one MI355X.

One step = pa_write_kv of every sequence's new token, then pa_decode of the whole batch (the
decode kernel, and the merge kernel when a sequence is split), on seeded synthetic inputs
already resident in HBM. The timed steps replay a captured HIP graph of consecutive steps, as a
serving loop would (--no-graph times eager launches; the eager rate is reported too). The
default workload is the 13B-shape fp16 MHA decode batch: 64 sequences, 40 heads, head dim
128, block size 16, context lengths lognormal (median 512, sigma 1) clipped to [16, 2048],
blocks scattered over a pool 1.2x the need. Other workloads (--workload) are for profiling.

Prints one JSON line: value = algorithmic HBM bytes of the step / step time (GB/s), plus
decode seq-tokens/s, the decode kernel's roofline (HIP-event duration on the launch stream,
vs 8 TB/s) and the CPU oracle timed on this host.

Cache honesty: the KV pools are replicated (--pool-copies, default 4, about 4.8 GB for the
default workload) and consecutive steps use different copies, so no step finds the previous
step's blocks in the 256 MB last-level cache.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E peak, vendor figure
PEAK_MFMA_TFLOPS_16 = 2500.0  # MI355X dense fp16/bf16 matrix peak, vendor figure
PEAK_MFMA_TFLOPS_32 = 157.3  # MI355X dense fp32 matrix peak, vendor figure

WORKLOADS = {
    "mha13b": ("mha13b_f16", "13B-shape fp16 MHA decode: 64 seqs, 40 heads, d=128, B=16, "
               "lognormal lengths (median 512) clipped to [16,2048]"),
    "gqa": ("gqa_bf16", "GQA bf16 decode: 256 seqs, 64 query / 8 KV heads, d=128, B=16, "
            "lengths uniform in [128,4096]"),
    "gqa32": ("gqa32_bf16", "wide-group GQA bf16 decode: 128 seqs, 64 query / 2 KV heads (32 per "
              "KV head), d=128, B=16, lengths uniform in [128,4096]"),
    "long": ("long_bf16", "long-context bf16 split-K decode: 8 seqs, 32 heads, d=128, B=16, "
             "lengths uniform in [32768,131072]"),
    "shared": ("shared_prefix_f16", "shared-prefix fp16 decode: 16 prompts x 4 samples, 32 heads, "
               "d=128, B=32, 1297 tokens each"),
    "tiny": ("tiny_f32", "tiny fp32 decode: 4 seqs (7,16,33,50), 8 heads, d=64, B=16"),
    "prefill-mha13b": ("prefill_mha13b", "chunked prefill, 13B shape fp16 MHA: 16 seqs, 40 heads, "
                       "d=128, B=16, 512-token chunks after lognormal (median 512) prefixes "
                       "clipped to [0,1536]"),
    "prefill-gqa": ("prefill_gqa", "chunked prefill, GQA bf16: 16 seqs, 64 query / 8 KV heads, "
                    "d=128, B=16, 1024-token chunks after prefixes uniform in [0,3072]"),
    "prefill-f32": ("prefill_mha13b_f32", "chunked prefill, 13B shape fp32 (vector-ALU kernel): "
                    "16 seqs, 40 heads, d=128, B=16, 64-token chunks after lognormal (median "
                    "512) prefixes clipped to [0,1536]"),
    "copy": (None, "plain copy calibration: pa_copy_blocks of 4096 blocks of 256 KiB"),
    "sharing": (None, "KV memory accounting on the host block manager (no GPU): prompt sharing "
                "in parallel sampling and beam search, paged vs contiguous waste"),
    "kvwrite": (None, "pa_write_kv of an 8192-token chunk (40 KV heads, d=128, fp16) into "
                "scattered slots"),
    "cow": (None, "pa_copy_blocks of 4096 random block pairs (40 heads, B=16, d=128, fp16)"),
    "swap": (None, "preemption swap: pa_swap_blocks of 2048 blocks of 160 KiB (40 heads, B=16, "
             "d=128, fp16) device -> pinned host and back"),
}

# The sources each kernel family is built from: a committed counter summary is used only while
# their code (comments and spacing aside) is unchanged since the counters were taken.
KERNEL_SOURCES = {
    "decode": ["paged_kv_cache_82_amd/csrc/pa_decode.hip",
               "paged_kv_cache_82_amd/csrc/pa_device.h",
               "paged_kv_cache_82_amd/csrc/pa_mfma.h",
               "paged_kv_cache_82_amd/csrc/pa_internal.h"],
    "prefill": ["paged_kv_cache_82_amd/csrc/pa_prefill.hip",
                "paged_kv_cache_82_amd/csrc/pa_device.h",
                "paged_kv_cache_82_amd/csrc/pa_mfma.h",
                "paged_kv_cache_82_amd/csrc/pa_internal.h"],
}


def code_only(text: str) -> str:
    """C/C++ source without its comments, whitespace runs collapsed to one space (string and
    character literals kept as they are)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return re.sub(r"\s+", " ", "".join(out)).strip()


def source_hash(kind: str) -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[kind]:
        h.update(code_only(open(os.path.join(ROOT, p)).read()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def measured_traffic(kind: str, workload: str):
    """HBM bytes (read + written) per launch of the `kind` kernel from the committed rocprofv3
    counter summary, if it was taken on the current sources of that kernel family; else None."""
    path = os.path.join(ROOT, "profiles", f"pa_{kind}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    src = re.search(r"source_sha256_16:\s*(\w+)", text)
    val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not src or not val or src.group(1) != source_hash(kind):
        return None
    return float(val.group(1))


def algorithmic_bytes(step) -> dict:
    """Bytes the method itself must move (per decode launch and per KV write)."""
    e = step.elem_bytes
    S, Hq, Hkv, d, B = (step.num_seqs, step.num_q_heads, step.num_kv_heads, step.head_dim,
                        step.block_size)
    T = step.context_lens.astype(float)
    kv = float(T.sum()) * 2 * Hkv * d * e
    qo = 2.0 * S * Hq * d * e
    idx = 4.0 * (float(sum(math.ceil(t / B) for t in T)) + S)
    n_new = sum(len(w.slot_mapping) for w in step.writes)
    write = 2.0 * n_new * Hkv * d * e * 2 + 4.0 * n_new
    # What must come from HBM: each distinct physical block once, at the most tokens any
    # sequence uses of it. Equal to the logical count unless sequences share blocks (the
    # shared-prefix step, whose samples re-read their prompt's blocks).
    used = {}
    for s in range(S):
        t = int(step.context_lens[s])
        for j in range(-(-t // B)):
            p = int(step.block_tables[s, j])
            used[p] = max(used.get(p, 0), min(B, t - j * B))
    kv_unique = float(sum(used.values())) * 2 * Hkv * d * e
    return {"decode": kv_unique + qo + idx, "decode_logical": kv + qo + idx, "write": write,
            "tokens": float(T.sum())}


def make_workload(name: str, poison: bool, placement: str = "random"):
    import workloads

    cfg = WORKLOADS[name][0]
    kw = {"poison": poison}
    if placement == "contiguous" and cfg != "shared_prefix_f16":
        kw["alloc_rng"] = workloads.InOrder()
    return getattr(workloads, cfg)(**kw)


def cpu_baseline(step, budget_s: float = 12.0) -> dict:
    """The oracle (test infrastructure, plain C, fp64) on this host: the whole step (KV write and
    decode of every sequence) repeated until about `budget_s` of CPU time; a bounded sample."""
    import numpy as np

    import oracle

    nb = algorithmic_bytes(step)
    # Bound the sample: whole sequences, in order, until about 1/4 of the budget per pass.
    S = step.num_seqs
    seqs = list(range(S))
    t0 = time.perf_counter()
    oracle.decode(step.q, step.k_cache, step.v_cache, step.block_tables, step.context_lens,
                  step.scale, step.dtype, seq_list=np.asarray(seqs[:1], np.int32))
    one = time.perf_counter() - t0
    per_seq_est = max(one, 1e-4)
    n = max(1, min(S, int((budget_s / 4) / per_seq_est)))
    sample = np.asarray(seqs[:n], np.int32)
    reps, elapsed = 0, 0.0
    t0 = time.perf_counter()
    while elapsed < budget_s and reps < 1000:
        oracle.decode(step.q, step.k_cache, step.v_cache, step.block_tables, step.context_lens,
                      step.scale, step.dtype, seq_list=sample)
        reps += 1
        elapsed = time.perf_counter() - t0
    tok = float(step.context_lens[sample].sum()) * reps
    frac = float(step.context_lens[sample].sum()) / nb["tokens"]
    gbs = nb["decode"] * frac * reps / elapsed / 1e9
    res = {"value": round(gbs, 4), "unit": "GB/s", "cores": oracle.num_threads(),
           "kind": "oracle",
           "sample": f"decode of sequences 0..{n - 1} of {S} ({int(step.context_lens[sample].sum())} "
                     f"of {int(nb['tokens'])} context tokens), fp64 oracle, {reps} passes in "
                     f"{elapsed:.1f} s",
           "seq_tokens_per_s": round(tok / elapsed, 1), "cpu_model": cpu_model()}
    # The same oracle on one thread, on the first sequence(s) for about a quarter of the budget.
    threads = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        one = np.asarray(seqs[:max(1, n // threads)], np.int32)
        reps1, t0 = 0, time.perf_counter()
        while reps1 == 0 or (time.perf_counter() - t0 < budget_s / 4 and reps1 < 1000):
            oracle.decode(step.q, step.k_cache, step.v_cache, step.block_tables,
                          step.context_lens, step.scale, step.dtype, seq_list=one)
            reps1 += 1
        el1 = time.perf_counter() - t0
    finally:
        oracle.set_num_threads(threads)
    t1 = float(step.context_lens[one].sum())
    res["single_thread"] = {
        "value": round(nb["decode"] * (t1 / nb["tokens"]) * reps1 / el1 / 1e9, 4), "unit": "GB/s",
        "seq_tokens_per_s": round(t1 * reps1 / el1, 1),
        "sample": f"decode of sequences 0..{len(one) - 1} ({int(t1)} context tokens), "
                  f"{reps1} passes in {el1:.1f} s on 1 thread"}
    return res


def cpu_model() -> str:
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def prefill_flops(step) -> float:
    """Algorithmic flops of one pa_prefill launch: every (query row, query head, visible token)
    costs 2d for q.K and 2d for p.V."""
    qs = step.query_start
    total = 0
    for s in range(step.num_seqs):
        n = int(qs[s + 1] - qs[s])
        T = int(step.context_lens[s])
        total += n * (T - n) + n * (n + 1) // 2  # sum over i of (T - n + i + 1)
    return float(total) * step.num_q_heads * 4.0 * step.head_dim


def prefill_bytes(step) -> float:
    """HBM bytes one pa_prefill launch must move: each sequence's K and V once per KV head, the
    q rows read and the out rows written, the block tables and lengths."""
    e = step.elem_bytes
    T = step.context_lens.astype(float)
    B = step.block_size
    kv = float(T.sum()) * 2 * step.num_kv_heads * step.head_dim * e
    qo = 2.0 * step.num_q_tokens * step.num_q_heads * step.head_dim * e
    idx = 4.0 * (float(sum(math.ceil(t / B) for t in T)) + 2 * step.num_seqs + 1)
    return kv + qo + idx


def prefill_cpu_baseline(step, budget_s: float = 12.0) -> dict:
    """The oracle on this host, on a bounded sample: the chunks of the first sequences, as many
    as fit about a quarter of the budget per pass, repeated until the budget is spent."""
    import numpy as np

    import oracle
    from workloads.configs import PrefillStep

    def sub(nseq):
        qs = step.query_start
        return PrefillStep(
            name=step.name, seed=step.seed, dtype=step.dtype, num_q_heads=step.num_q_heads,
            num_kv_heads=step.num_kv_heads, head_dim=step.head_dim, block_size=step.block_size,
            k_cache=step.k_cache, v_cache=step.v_cache, q=step.q[: qs[nseq]],
            block_tables=step.block_tables[:nseq], context_lens=step.context_lens[:nseq],
            query_start=qs[: nseq + 1], scale=step.scale)

    def run(st):
        return oracle.prefill(st.q, st.k_cache, st.v_cache, st.block_tables, st.context_lens,
                              st.query_start, st.scale, st.dtype)

    t0 = time.perf_counter()
    run(sub(1))
    one = max(time.perf_counter() - t0, 1e-4)
    n = max(1, min(step.num_seqs, int((budget_s / 4) / one)))
    st = sub(n)
    reps, elapsed = 0, 0.0
    t0 = time.perf_counter()
    while elapsed < budget_s and reps < 1000:
        run(st)
        reps += 1
        elapsed = time.perf_counter() - t0
    fl = prefill_flops(st) * reps
    return {"value": round(fl / elapsed / 1e12, 6), "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"causal attention of the chunks of sequences 0..{n - 1} of "
                      f"{step.num_seqs} ({int(st.query_start[-1])} of {step.num_q_tokens} query "
                      f"tokens), fp64 oracle, {reps} passes in {elapsed:.1f} s"}


def measure_prefill(workload: str, args, cpu: bool) -> dict:
    """One step = pa_write_kv of every sequence's chunk, then pa_prefill. The bound is the
    matrix cores (about 2d flops per byte of K/V per query row): the roofline is the dense
    fp16/bf16 MFMA peak."""
    import numpy as np
    import torch

    import paged_kv_cache_82_amd as pa
    import workloads

    t_gen = time.perf_counter()
    step = getattr(workloads, WORKLOADS[workload][0])(poison=False)
    t_gen = time.perf_counter() - t_gen
    dev = torch.device("cuda")

    def up(a, dt=None):
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    ncopy = max(1, args.pool_copies)
    kc0, vc0 = up(step.k_cache, step.dtype), up(step.v_cache, step.dtype)
    pools = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(ncopy - 1)]
    q = up(step.q, step.dtype)
    bt, cl, qs = up(step.block_tables), up(step.context_lens), up(step.query_start)
    writes = [(up(w.k_new, step.dtype), up(w.v_new, step.dtype), up(w.slot_mapping))
              for w in step.writes]
    out = torch.empty_like(q)
    scale, maxn, maxT = float(step.scale), step.max_query_len, step.max_context_len

    def attend(i):
        kc, vc = pools[i % ncopy]
        pa.pa_prefill(out, q, kc, vc, bt, cl, qs, scale, maxn, maxT)

    def one_step(i):
        kc, vc = pools[i % ncopy]
        for kn, vn, sm in writes:
            pa.pa_write_kv(kc, vc, kn, vn, sm)
        attend(i)

    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < args.prewarm_s:
        for i in range(4):
            one_step(i)
        torch.cuda.synchronize()
    for i in range(args.warmup):
        one_step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(args.warmup + i)
    torch.cuda.synchronize()
    eager_wall = time.perf_counter() - t0
    if args.no_graph:
        wall = eager_wall
    else:  # as for decode: a captured graph of ncopy steps, replayed; the rest eagerly
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(ncopy):
                one_step(i)
        graph.replay()
        torch.cuda.synchronize()
        reps, rest = divmod(args.steps, ncopy)
        t0 = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        for i in range(rest):
            one_step(i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    n_roof = max(args.steps, 100)  # as for decode: enough launches for a stable average
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n_roof):
        attend(i)
    e1.record()
    torch.cuda.synchronize()
    att_s = e0.elapsed_time(e1) / 1e3 / n_roof
    fl = prefill_flops(step)
    n_new = step.num_q_tokens
    f32 = step.dtype == "f32"
    peak = PEAK_MFMA_TFLOPS_32 if f32 else PEAK_MFMA_TFLOPS_16
    res = {
        "metric": "paged prefill attention: achieved TFLOP/s (% of MFMA peak) + query tokens/s",
        "value": round(fl / (wall / args.steps) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": step.dtype, "accumulate": "f32",
        "data": "synthetic (seeded N(0,1) K/V/q; lengths and placement as described)",
        "config": {
            "workload": WORKLOADS[workload][1],
            "num_seqs": step.num_seqs, "num_q_heads": step.num_q_heads,
            "num_kv_heads": step.num_kv_heads, "head_dim": step.head_dim,
            "block_size": step.block_size, "num_blocks": step.num_blocks,
            "query_tokens": n_new, "context_tokens": int(step.context_lens.sum()),
            "max_context_len": maxT, "pool_copies": ncopy, "parallelism": "single GPU",
        },
        "query_tokens_per_s": round(n_new / (wall / args.steps), 1),
        "execution": "eager" if args.no_graph else f"HIP graph of {ncopy} steps, replayed",
        "eager_ms_per_step": round(eager_wall / args.steps * 1e3, 5),
        "roofline": {
            "kernel": ("pa_prefill: prefill_f32_kernel" if f32 else
                       "pa_prefill: prefill_mfma_kernel"),
            "bound": "mfma",
            "achieved": round(fl / att_s / 1e12, 3),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(fl / att_s / 1e12 / peak, 4),
            "traffic": measured_traffic("prefill", workload[len("prefill-"):]),
            "algorithmic_flops_per_launch": fl,
            "algorithmic_bytes_per_launch": prefill_bytes(step),
            "avg_launch_us": round(att_s * 1e6, 3),
        },
        "input_generation_s": round(t_gen, 2),
    }
    if cpu:
        res["cpu_baseline"] = prefill_cpu_baseline(step)
    del pools, kc0, vc0, q, bt, cl, qs, writes, out
    if not args.no_graph:
        del graph
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def run_prefill(args):
    print(json.dumps(measure_prefill(args.workload, args, cpu=not args.no_cpu_baseline)))


def run_copy_calibration(args):
    import torch

    import paged_kv_cache_82_amd as pa

    dev = torch.device("cuda")
    nblk, H, B, d = 8192, 32, 32, 128  # 256 KiB blocks, 2 GiB pools
    k = torch.zeros((nblk, H, B, d), dtype=torch.float16, device=dev)
    v = torch.zeros_like(k)
    pairs = torch.stack([torch.arange(0, 4096), torch.arange(4096, 8192)], 1).int().to(dev)
    for _ in range(args.warmup):
        pa.pa_copy_blocks(k, v, pairs)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        pa.pa_copy_blocks(k, v, pairs)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    nbytes = 2 * 2 * 4096 * H * B * d * 2
    print(json.dumps({"metric": "copy calibration", "bytes_read_per_launch": nbytes // 2,
                      "bytes_written_per_launch": nbytes // 2, "GB_per_s": nbytes / dt / 1e9}))


def run_kv_bandwidth(args):
    """Secondary measurements of the indexing kernels at a serving shape (40 KV heads, d=128,
    B=16, fp16; a pool of 16,384 blocks = 2.5 GiB per tensor):
      kvwrite: pa_write_kv of one 8,192-token chunk (the 13B-shape prefill chunk) to slots
               scattered over the pool by a seeded permutation of its blocks;
      cow:     pa_copy_blocks of 4,096 (src, dst) pairs drawn from a seeded permutation.
    Bytes are the algorithmic ones (read + written); time is the HIP-event average of K
    back-to-back launches on the launch stream."""
    import numpy as np
    import torch

    import paged_kv_cache_82_amd as pa

    dev = torch.device("cuda")
    N, H, B, d = 16384, 40, 16, 128
    k = torch.zeros((N, H, B, d), dtype=torch.float16, device=dev)
    v = torch.zeros_like(k)
    rng = np.random.default_rng(11)
    if args.workload == "kvwrite":
        n = 8192
        blocks = rng.permutation(N)[: n // B]
        slots = (blocks[:, None] * B + np.arange(B)[None, :]).reshape(-1).astype(np.int32)
        kn = torch.randn((n, H, d), device=dev).half()
        vn = torch.randn_like(kn)
        sm = torch.from_numpy(slots).to(dev)
        launch = lambda: pa.pa_write_kv(k, v, kn, vn, sm)  # noqa: E731
        nbytes = 2 * (2 * n * H * d * 2) + 4 * n
        what = "pa_write_kv: 8192 tokens x 40 KV heads x d=128 fp16 into scattered slots"
    else:
        n = 4096
        perm = rng.permutation(N)
        pairs = torch.from_numpy(np.stack([perm[:n], perm[n:2 * n]], 1).astype(np.int32)).to(dev)
        launch = lambda: pa.pa_copy_blocks(k, v, pairs)  # noqa: E731
        nbytes = 2 * (2 * n * H * B * d * 2) + 8 * n
        what = "pa_copy_blocks: 4096 random (src, dst) pairs of 40x16x128 fp16 blocks, K and V"
    for _ in range(args.warmup):
        launch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        launch()
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / args.steps
    gbs = nbytes / sec / 1e9
    print(json.dumps({
        "metric": f"{args.workload} bandwidth: algorithmic bytes read + written per second",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(sec * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": what, "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": nbytes,
                     "avg_launch_us": round(sec * 1e6, 3)},
    }))


def run_swap(args):
    """Swap-out (device -> pinned host) and swap-in (host -> device) rates of pa_swap_blocks.
    The bound is the host link, not HBM."""
    import torch

    import paged_kv_cache_82_amd as pa

    dev = torch.device("cuda")
    n, H, B, d = 2048, 40, 16, 128
    k = torch.randn((n, H, B, d), device=dev).half()
    v = torch.randn((n, H, B, d), device=dev).half()
    hk = torch.empty((n, H, B, d), dtype=torch.float16).pin_memory()
    hv = torch.empty_like(hk).pin_memory()
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(0))
    out_pairs = torch.stack([perm, torch.arange(n)], 1).int().to(dev)
    in_pairs = torch.stack([torch.arange(n), perm], 1).int().to(dev)
    nbytes = 2 * n * H * B * d * 2
    res = {}
    for name, fn in (("out", lambda: pa.pa_swap_blocks(hk, hv, k, v, out_pairs)),
                     ("in", lambda: pa.pa_swap_blocks(k, v, hk, hv, in_pairs))):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        dt = e0.elapsed_time(e1) / 1e3 / args.steps
        res[f"swap_{name}_GB_per_s"] = round(nbytes / dt / 1e9, 2)
        res[f"swap_{name}_ms"] = round(dt * 1e3, 4)
    print(json.dumps({"metric": "pa_swap_blocks device<->pinned host", "bytes_per_call": nbytes,
                      **res}))


def run_sharing(args):
    """Block-manager accounting only (host code, no GPU): synthetic lognormal lengths."""
    from paged_kv_cache_82_amd import sharing

    t0 = time.perf_counter()
    res = {
        "metric": "KV memory saved by block sharing / wasted by allocation (host block manager)",
        "block_size": 16,
        "parallel_sampling": [sharing.parallel_sampling(n) for n in (2, 4, 6)],
        "beam_search": [sharing.beam_search(k) for k in (2, 4, 6)],
        "waste": sharing.waste(),
        "data": "synthetic lognormal lengths (prompt median 160, output median 300 / 200 for "
                "beams, sigma 0.8; waste: median 400, sigma 0.9, max 2048); random beam parents",
    }
    res["seconds"] = round(time.perf_counter() - t0, 2)
    print(json.dumps(res))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mha13b", choices=sorted(WORKLOADS))
    ap.add_argument("--pool-copies", type=int, default=4)
    ap.add_argument("--prewarm-s", type=float, default=0.5,
                    help="untimed seconds of steps before the warmup steps (GPU clock ramp)")
    ap.add_argument("--partition-tokens", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="time the default (13B-shape) workload only, not the other decode "
                         "and prefill workloads after it")
    ap.add_argument("--separate-write", action="store_true",
                    help="decode steps: pa_write_kv then pa_decode, not pa_decode_append")
    ap.add_argument("--no-graph", action="store_true",
                    help="time eager launches instead of replays of a captured step graph")
    ap.add_argument("--placement", default="random", choices=["random", "contiguous"],
                    help="block placement; 'contiguous' is a diagnostic of what scattering costs")
    args = ap.parse_args()

    if args.workload == "sharing":
        return run_sharing(args)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(sequences and KV heads would shard with no exchange; see the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import paged_kv_cache_82_amd as pa

    if not os.path.exists(pa.lib_path()):
        from paged_kv_cache_82_amd import build as pa_build

        pa_build.build()
    pa.load()
    if args.workload == "copy":
        return run_copy_calibration(args)
    if args.workload == "swap":
        return run_swap(args)
    if args.workload in ("kvwrite", "cow"):
        return run_kv_bandwidth(args)
    if args.workload.startswith("prefill"):
        return run_prefill(args)

    res = measure_decode(args.workload, args, cpu=not args.no_cpu_baseline)
    if args.workload == "mha13b" and not args.no_extra:
        # The other decode workloads in the same process, each under its own key: the GQA batch
        # is the second bandwidth target; long-context and shared-prefix run the split-K merge
        # and shared blocks. Same step, graph replay and event timing; no CPU baseline.
        res["workloads"] = {"mha13b": summary(res)}
        for name in EXTRA_WORKLOADS:
            t0 = time.perf_counter()
            res["workloads"][name] = summary(measure_decode(name, args, cpu=False,
                                                            compare_plain=True))
            print(f"bench: {name} measured in {time.perf_counter() - t0:.1f} s", file=sys.stderr,
                  flush=True)
        # The chunked-prefill workloads (the matrix-core-bound path), same contract, under
        # their own keys; their roofline is the MFMA peak of their dtype.
        for name in EXTRA_PREFILL:
            t0 = time.perf_counter()
            res["workloads"][name] = prefill_summary(measure_prefill(name, args, cpu=False))
            print(f"bench: {name} measured in {time.perf_counter() - t0:.1f} s", file=sys.stderr,
                  flush=True)
    print(json.dumps(res))


EXTRA_WORKLOADS = ("gqa", "long", "shared")
EXTRA_PREFILL = ("prefill-mha13b", "prefill-gqa", "prefill-f32")


def prefill_summary(res: dict) -> dict:
    """The per-workload figures of one prefill measurement."""
    r = res["roofline"]
    return {"workload": res["config"]["workload"], "dtype": res["dtype"], "value": res["value"],
            "unit": res["unit"], "ms_per_step": res["ms_per_step"],
            "query_tokens_per_s": res["query_tokens_per_s"],
            "roofline": {k: r[k] for k in ("kernel", "bound", "achieved", "peak", "unit", "frac",
                                           "traffic", "algorithmic_flops_per_launch",
                                           "algorithmic_bytes_per_launch", "avg_launch_us")}}


def summary(res: dict) -> dict:
    """The per-workload figures of one decode measurement."""
    r = res["roofline"]
    out = {"workload": res["config"]["workload"], "dtype": res["dtype"],
           "value": res["value"], "unit": res["unit"], "ms_per_step": res["ms_per_step"],
           "seq_tokens_per_s": res["seq_tokens_per_s"],
           "decode_seq_tokens_per_s": res["decode_seq_tokens_per_s"],
           "roofline": {k: r[k] for k in ("kernel", "bound", "achieved", "peak", "unit", "frac",
                                          "traffic", "algorithmic_bytes_per_launch",
                                          "avg_launch_us")}}
    for k in ("logical_bytes_per_launch", "logical_GB_per_s", "pa_decode_avg_launch_us",
              "pa_decode_GB_per_s"):
        if k in r:
            out["roofline"][k] = r[k]
    return out


def measure_decode(workload: str, args, cpu: bool, compare_plain: bool = False) -> dict:
    """One decode workload: inputs generated and uploaded, W warmup steps, K timed steps (graph
    replay unless --no-graph), then back-to-back decode launches between HIP events on the
    launch stream for the roofline. The shared-prefix workload decodes with
    pa_decode_shared_prefix, its groups read off the step's tables (compare_plain: plain
    pa_decode timed the same way beside it). Frees its device memory before returning."""
    import numpy as np
    import torch

    import paged_kv_cache_82_amd as pa

    t_gen = time.perf_counter()
    step = make_workload(workload, poison=False, placement=args.placement)
    t_gen = time.perf_counter() - t_gen
    dev = torch.device("cuda")
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[step.dtype]

    def up(a, dt=None):
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    ncopy = max(1, args.pool_copies)
    kc0, vc0 = up(step.k_cache, step.dtype), up(step.v_cache, step.dtype)
    pools = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(ncopy - 1)]
    q = up(step.q, step.dtype)
    bt, cl = up(step.block_tables), up(step.context_lens)
    copies = up(step.copies)
    writes = [(up(w.k_new, step.dtype), up(w.v_new, step.dtype), up(w.slot_mapping))
              for w in step.writes]
    out = torch.empty_like(q)
    P = args.partition_tokens
    ws_bytes = pa.pa_decode_workspace_size(step.num_seqs, step.num_q_heads, step.num_kv_heads,
                                           step.head_dim, step.block_size, step.max_context_len,
                                           P, tdt)
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    split = ws_bytes > 0  # partial states are needed only when some sequence splits
    scale = float(step.scale)
    maxT = step.max_context_len
    shared_api = workload == "shared"
    if shared_api:
        # the sharing structure as the block manager reports it (pa_bm_prefix_groups): runs of
        # consecutive sequences holding the same leading blocks
        from workloads import prefix_groups

        gs_np, pl_np = prefix_groups(step.block_tables, step.context_lens, step.block_size)
        gs, pl = up(gs_np), up(pl_np)
        max_group, max_prefix = int(np.diff(gs_np).max()), int(pl_np.max())
        ws_sh_bytes = pa.pa_decode_shared_prefix_workspace_size(
            step.num_seqs, len(gs_np) - 1, step.num_q_heads, step.num_kv_heads, step.head_dim,
            step.block_size, maxT, max_prefix, max_group, P, tdt)
        ws_sh = torch.zeros(max(ws_sh_bytes, 256), dtype=torch.uint8, device=dev)

    def decode(kc, vc):
        if shared_api:
            pa.pa_decode_shared_prefix(out, q, kc, vc, bt, cl, pl, gs, scale, maxT, max_prefix,
                                       max_group, ws_sh, P)
        else:
            pa.pa_decode(out, q, kc, vc, bt, cl, scale, maxT, ws, P)

    torch.cuda.synchronize()

    # The step's KV write and decode in one launch (pa_decode_append) when the step writes
    # exactly one new token per sequence, in sequence order, and copies nothing; otherwise (and
    # with --separate-write) pa_write_kv, then the decode.
    fused = (not args.separate_write and not shared_api and len(step.copies) == 0
             and len(step.writes) == 1 and step.writes[0].k_new.shape[0] == step.num_seqs
             and bool((step.context_lens > 0).all()))

    def one_step(i, ev=None):
        kc, vc = pools[i % ncopy]
        if len(step.copies):
            pa.pa_copy_blocks(kc, vc, copies)
        if fused:
            kn, vn, sm = writes[0]
            if ev is not None:
                ev[0].record()
            pa.pa_decode_append(out, q, kc, vc, kn, vn, sm, bt, cl, scale, maxT, ws, P)
            if ev is not None:
                ev[1].record()
            return
        for kn, vn, sm in writes:
            pa.pa_write_kv(kc, vc, kn, vn, sm)
        if ev is not None:
            ev[0].record()
        decode(kc, vc)
        if ev is not None:
            ev[1].record()

    # Untimed: bring the GPU to its working clocks (a fresh process on an idle GPU starts low),
    # then the W warmup steps of the contract.
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < args.prewarm_s:
        for i in range(10):
            one_step(i)
        torch.cuda.synchronize()
    for i in range(args.warmup):
        one_step(i)
    torch.cuda.synchronize()
    # Diagnostic (untimed for `value`): K eager steps with events around each decode launch.
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        one_step(args.warmup + i, events[i])
    torch.cuda.synchronize()
    eager_wall = time.perf_counter() - t0
    step_event_us = float(np.mean([a.elapsed_time(b) for a, b in events])) * 1e3
    # Timed region: exactly K steps. By default a serving loop's step is captured once as a
    # HIP graph of `ncopy` consecutive steps (one per pool copy) and replayed, which removes
    # the host launch gaps between the kernels; steps that do not fill a whole graph run eagerly.
    if args.no_graph:
        wall = eager_wall
    else:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(ncopy):
                one_step(i)
        graph.replay()  # untimed first replay
        torch.cuda.synchronize()
        reps, rest = divmod(args.steps, ncopy)
        t0 = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        for i in range(rest):
            one_step(i)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    # Part 2: K decode launches back to back (rotating pool copies) between two events on the
    # launch stream; the average is the decode kernel's launch duration for the roofline (an
    # event right before each launch would also time the dispatch gap after the KV write).
    # At least 100 launches: with 20 a short batch (7 ms for the GQA step) read a few percent
    # slow.
    n_roof = max(args.steps, 100)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n_roof):
        kc, vc = pools[i % ncopy]
        decode(kc, vc)
    e1.record()
    torch.cuda.synchronize()
    dec_s = e0.elapsed_time(e1) / 1e3 / n_roof
    plain_s = None
    if shared_api and compare_plain:  # the same launches without the sharing description
        e0.record()
        for i in range(n_roof):
            kc, vc = pools[i % ncopy]
            pa.pa_decode(out, q, kc, vc, bt, cl, scale, maxT, ws, P)
        e1.record()
        torch.cuda.synchronize()
        plain_s = e0.elapsed_time(e1) / 1e3 / n_roof

    nb = algorithmic_bytes(step)
    ms_per_step = wall / args.steps * 1e3
    step_bytes = nb["decode"] + nb["write"]
    value = step_bytes / (wall / args.steps) / 1e9
    achieved = nb["decode"] / dec_s / 1e9
    traffic = measured_traffic("decode", workload)
    res = {
        "metric": "paged decode attention: achieved HBM GB/s (% of peak) + seq-tokens/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": step.dtype,
        "accumulate": "f32",
        "data": "synthetic (seeded N(0,1) K/V/q; lengths and placement as described)",
        "config": {
            "workload": WORKLOADS[workload][1],
            "num_seqs": step.num_seqs, "num_q_heads": step.num_q_heads,
            "num_kv_heads": step.num_kv_heads, "head_dim": step.head_dim,
            "block_size": step.block_size, "num_blocks": step.num_blocks,
            "context_tokens": int(nb["tokens"]), "max_context_len": maxT,
            "partition_tokens": P or "auto", "pool_copies": ncopy,
            "placement": args.placement,
            "parallelism": "single GPU",
        },
        "execution": "eager" if args.no_graph else f"HIP graph of {ncopy} steps, replayed",
        "step_calls": ("pa_decode_append (the KV write and the decode in one launch)" if fused
                       else ("pa_copy_blocks + " if len(step.copies) else "")
                       + "pa_write_kv + " + ("pa_decode_shared_prefix" if shared_api
                                             else "pa_decode")),
        "eager_ms_per_step": round(eager_wall / args.steps * 1e3, 5),
        "frac_of_peak": round(value / PEAK_HBM_GBS, 4),
        "seq_tokens_per_s": round(nb["tokens"] / (wall / args.steps), 1),
        "decode_seq_tokens_per_s": round(nb["tokens"] / dec_s, 1),
        "roofline": {
            "kernel": ("pa_decode_shared_prefix: group kernel (each shared tile scored once "
                       "for all samples, then their own tokens; one launch)" if shared_api else
                       "pa_decode: decode kernel (every sequence in one partition, no merge)"
                       if not split else
                       "pa_decode: decode kernel + partition-merge kernel (split sequences)"),
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": nb["decode"],
            "avg_launch_us": round(dec_s * 1e6, 3),
            "step_event_decode_us": round(step_event_us, 3),
        },
        "bytes_per_step": step_bytes,
        "input_generation_s": round(t_gen, 2),
    }
    if nb["decode_logical"] != nb["decode"]:
        # shared blocks: `value` and `achieved` count each block once; the logical bytes (every
        # sequence's tokens, shared prefixes once per sequence) beside them
        res["roofline"]["logical_bytes_per_launch"] = nb["decode_logical"]
        res["roofline"]["logical_GB_per_s"] = round(nb["decode_logical"] / dec_s / 1e9, 2)
    if plain_s is not None:
        res["roofline"]["pa_decode_avg_launch_us"] = round(plain_s * 1e6, 3)
        res["roofline"]["pa_decode_GB_per_s"] = round(nb["decode"] / plain_s / 1e9, 2)
    if cpu:
        res["cpu_baseline"] = cpu_baseline(step)
    del pools, kc0, vc0, q, bt, cl, copies, writes, out, ws
    if not args.no_graph:
        del graph
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    main()
