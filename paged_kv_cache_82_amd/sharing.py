"""KV-memory accounting of paged allocation with sharing, on synthetic request streams.

The native block manager (libpa, include/pa_block_manager.h) runs the allocation; this module
only drives it and counts blocks. It measures the kind of figures [PA-summary] reports in
"Memory sharing: copy-on-write" and "Results" on synthetic inputs (the pages' datasets and
models are not used):
  - parallel sampling: n samples forked from one prompt share its blocks; the saving is the
    time-averaged fraction of blocks that private copies of the prompt would have needed
    beyond what the shared pool holds;
  - beam search: k beams, each step every new beam forks from a surviving parent (chosen at
    random here, a stand-in for scores) and appends one token; dead beams are released, so
    the shared prefix forms a tree;
  - waste: reserved-but-unused slots of paged allocation (at most the unfilled tail of each
    sequence's last block) against a contiguous allocator that reserves the maximum length
    for every request up front.
Lengths are drawn from lognormal distributions (seeded) as a stand-in for conversation
traces; the recipe is in each function's arguments.
"""
from __future__ import annotations

import math

import numpy as np

from .block_manager import BlockManager


def parallel_sampling(n: int, requests: int = 64, block_size: int = 16, seed: int = 0,
                      prompt_median: float = 160.0, output_median: float = 300.0,
                      sigma: float = 0.8) -> dict:
    """Time-averaged KV blocks with the prompt shared by `n` samples vs private copies."""
    rng = np.random.default_rng(seed)
    prompts = np.maximum(1, np.rint(rng.lognormal(math.log(prompt_median), sigma, requests)))
    outs = np.maximum(1, np.rint(rng.lognormal(math.log(output_median), sigma, (requests, n))))
    B = block_size
    need = int(sum(math.ceil((p + o.max()) / B) * n for p, o in zip(prompts, outs))) + 1
    bm = BlockManager(need, B)
    shared_sum, private_sum = 0, 0
    sid = 0
    for p, o in zip(prompts.astype(int), outs.astype(int)):
        root = sid
        bm.add(root)
        bm.append(root, int(p))
        ids = [root] + list(range(root + 1, root + n))
        for c in ids[1:]:
            bm.fork(root, c)
        sid += n
        lens = {c: int(p) for c in ids}
        alive = dict(zip(ids, o))
        for _step in range(int(o.max())):
            for c in list(alive):
                bm.append(c, 1)
                lens[c] += 1
                if lens[c] - p >= alive[c]:
                    del alive[c]  # finished: keeps its blocks until the request ends
            shared_sum += bm.stats()["used_blocks"]
            private_sum += sum(math.ceil(L / B) for L in lens.values())
        for c in ids:
            bm.release(c)
    return {"n": n, "shared_block_steps": shared_sum, "private_block_steps": private_sum,
            "saving": 1.0 - shared_sum / private_sum}


def beam_search(k: int, requests: int = 32, block_size: int = 16, seed: int = 0,
                prompt_median: float = 160.0, output_median: float = 200.0,
                sigma: float = 0.8) -> dict:
    """Time-averaged KV blocks of a k-beam search tree with shared prefixes vs every beam
    holding a private copy of its whole history."""
    rng = np.random.default_rng(seed)
    prompts = np.maximum(1, np.rint(rng.lognormal(math.log(prompt_median), sigma, requests)))
    outs = np.maximum(1, np.rint(rng.lognormal(math.log(output_median), sigma, requests)))
    B = block_size
    need = int(sum(math.ceil((p + o) / B) * (2 * k + 1) for p, o in zip(prompts, outs))) + 1
    bm = BlockManager(need, B)
    shared_sum, private_sum = 0, 0
    next_id = 0
    for p, o in zip(prompts.astype(int), outs.astype(int)):
        bm.add(next_id)
        bm.append(next_id, int(p))
        beams = [next_id]
        next_id += 1
        for _step in range(int(o)):
            parents = rng.integers(0, len(beams), size=k)
            new = []
            for par in parents:
                bm.fork(beams[int(par)], next_id)
                bm.append(next_id, 1)
                new.append(next_id)
                next_id += 1
            for b in beams:
                bm.release(b)
            beams = new
            shared_sum += bm.stats()["used_blocks"]
            private_sum += sum(math.ceil(bm.length(b) / B) for b in beams)
        for b in beams:
            bm.release(b)
    return {"k": k, "shared_block_steps": shared_sum, "private_block_steps": private_sum,
            "saving": 1.0 - shared_sum / private_sum}


def waste(requests: int = 256, block_size: int = 16, max_len: int = 2048, seed: int = 0,
          median: float = 400.0, sigma: float = 0.9) -> dict:
    """Fraction of reserved KV slots that hold no token: paged (blocks on demand) against a
    contiguous allocator that reserves max_len slots per request."""
    rng = np.random.default_rng(seed)
    lens = np.clip(np.rint(rng.lognormal(math.log(median), sigma, requests)), 1, max_len)
    bm = BlockManager(int(sum(math.ceil(L / block_size) for L in lens)), block_size)
    for i, L in enumerate(lens.astype(int)):
        bm.add(i)
        bm.append(i, int(L))
    st = bm.stats()
    paged = 1.0 - st["filled_slots"] / st["reserved_slots"]
    contiguous = 1.0 - float(lens.sum()) / (requests * max_len)
    return {"requests": requests, "tokens": int(lens.sum()), "paged_waste": paged,
            "contiguous_waste": contiguous, "paged_waste_bound": (block_size - 1) * requests /
            st["reserved_slots"]}
