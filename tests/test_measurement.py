"""Host-side measurement logic (no GPU): the comment-insensitive source hash that gates the
committed HBM counter figures, the algorithmic byte count of a decode step against a count by
hand, and the SQ counter summary of rocprof_summary.py on a synthetic counter file."""
import csv
import math
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import rocprof_summary  # noqa: E402
from workloads import tiny_f32  # noqa: E402


def test_code_only_ignores_comments_and_spacing():
    a = 'int f(int x) {  // doubled\n  return 2 * x; /* no overflow here */\n}\n'
    b = 'int f(int x) {\n\n    return 2 * x;\n}'
    assert bench.code_only(a) == bench.code_only(b)
    assert bench.code_only(a) != bench.code_only(a.replace("2 * x", "3 * x"))
    # comment markers inside literals are code
    s = 'const char* p = "// not a comment"; char c = \'/\';'
    assert bench.code_only(s) == s


def test_code_only_keeps_escaped_quotes():
    s = 'const char* p = "a \\" // b"; int y = 1; // trailing'
    assert bench.code_only(s) == 'const char* p = "a \\" // b"; int y = 1;'


def test_source_hash_is_stable():
    for kind in bench.KERNEL_SOURCES:
        h = bench.source_hash(kind)
        assert len(h) == 16 and h == bench.source_hash(kind)


def test_algorithmic_bytes_tiny_by_hand():
    step = tiny_f32(poison=False)
    nb = bench.algorithmic_bytes(step)
    e, Hq, Hkv, d, B = 4, step.num_q_heads, step.num_kv_heads, step.head_dim, step.block_size
    T = [int(t) for t in step.context_lens]
    kv = sum(T) * 2 * Hkv * d * e  # every token's K and V row once (no shared blocks)
    qo = 2 * len(T) * Hq * d * e  # q read, out written
    idx = 4 * (sum(math.ceil(t / B) for t in T) + len(T))  # table entries and lengths
    assert nb["decode"] == nb["decode_logical"] == kv + qo + idx
    n_new = sum(len(w.slot_mapping) for w in step.writes)
    assert nb["write"] == 2 * n_new * Hkv * d * e * 2 + 4 * n_new


def test_unique_bytes_count_shared_blocks_once():
    step = tiny_f32(poison=False)
    base = bench.algorithmic_bytes(step)
    # point sequence 3's first block at sequence 2's first block: that block is now read by
    # both sequences but stored once, with at most B tokens used of it
    B, Hkv, d = step.block_size, step.num_kv_heads, step.head_dim
    assert step.context_lens[2] >= B and step.context_lens[3] >= B
    step.block_tables[3, 0] = step.block_tables[2, 0]
    shared = bench.algorithmic_bytes(step)
    assert shared["decode_logical"] == base["decode_logical"]
    assert base["decode"] - shared["decode"] == B * 2 * Hkv * d * 4


def _write_counters(path, kernel, values):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for dispatch in range(2):
            for k, v in values.items():
                w.writerow({"Kernel_Name": kernel, "Counter_Name": k,
                            "Counter_Value": v * (1 + dispatch)})
            w.writerow({"Kernel_Name": "other_kernel", "Counter_Name": "SQ_WAVE_CYCLES",
                        "Counter_Value": 1})


def test_sq_summary(tmp_path):
    k = "void pa::prefill_mfma_kernel<...>(pa::PrefillArgs)"
    p1, p2 = tmp_path / "p1.csv", tmp_path / "p2.csv"
    _write_counters(p1, k, {"SQ_WAVE_CYCLES": 1000, "SQ_ACTIVE_INST_ANY": 300,
                            "SQ_WAIT_ANY": 250, "SQ_WAIT_INST_ANY": 450})
    _write_counters(p2, k, {"SQ_INSTS_MFMA": 100, "SQ_INSTS_VALU": 325, "SQ_INSTS_SALU": 87,
                            "SQ_VALU_MFMA_BUSY_CYCLES": 800, "SQ_VALU_MFMA_COEXEC_CYCLES": 200})

    class A:
        needle, passes, command = "prefill_mfma", [str(p1), str(p2)], "cmd"

    text = rocprof_summary.do_sq(A)
    # per-dispatch averages (1x and 2x the values: 1.5x), shares and ratios are scale-free
    assert "SQ_WAVE_CYCLES: 1500" in text
    assert "issuing any instruction: 0.300" in text
    assert "waiting to issue (dependency or arbitration): 0.450" in text
    assert "SQ_INSTS_VALU: 3.250" in text and "SQ_INSTS_SALU: 0.870" in text
    assert "share of MFMA-busy cycles: 0.250" in text
    # a kernel without MFMA work gets no per-MFMA or co-execution lines
    p3 = tmp_path / "p3.csv"
    _write_counters(p3, k, {"SQ_WAVE_CYCLES": 1000, "SQ_INSTS_MFMA": 0,
                            "SQ_VALU_MFMA_BUSY_CYCLES": 0, "SQ_VALU_MFMA_COEXEC_CYCLES": 0})
    A.passes = [str(p3)]
    text = rocprof_summary.do_sq(A)
    assert "per MFMA" not in text and "co-executing" not in text
    A.needle = "no_such_kernel"
    with pytest.raises(SystemExit):
        rocprof_summary.do_sq(A)
