"""Fixtures under tests/golden/ that hold facts printed on the pages (each file cites its page).

The pages print no numeric attention outputs; the tutorial's workflow example prints shapes and
when pages are allocated, which pins the host allocator and the oracle's output shape."""
import json
import os

import numpy as np

import oracle
from workloads import BlockAllocator, Sequence, append_tokens, to_storage

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_tutorial_workflow(oracle_lib):
    fx = json.load(open(os.path.join(GOLDEN, "tutorial_workflow.json")))
    P, B, H, d = fx["total_pages"], fx["page_size"], fx["num_heads"], fx["head_dim"]
    rng = np.random.default_rng(0)
    alloc = BlockAllocator(P)
    seq = Sequence(B)
    kc = np.full((P, H, B, d), np.nan, np.float32)
    vc = np.full((P, H, B, d), np.nan, np.float32)
    for step in range(fx["steps"]):
        slots, pairs = append_tokens(alloc, seq, 1)
        assert not pairs
        kn = to_storage(rng.standard_normal((1, H, d)), "f32")
        vn = to_storage(rng.standard_normal((1, H, d)), "f32")
        oracle.write_kv(kc, vc, kn, vn, np.asarray(slots, np.int32), "f32", lib=oracle_lib)
        q = to_storage(rng.standard_normal((1, H, d)), "f32")
        table = np.asarray([seq.table], np.int32)
        out = oracle.decode(q, kc, vc, table, np.asarray([seq.length], np.int32),
                            1 / np.sqrt(d), "f32", lib=oracle_lib)
        assert list(out.shape) == fx["output_shape"]
        assert np.isfinite(out).all()
        if str(step) in fx["pages_in_use_after_step"]:
            assert len(seq.table) == fx["pages_in_use_after_step"][str(step)]
