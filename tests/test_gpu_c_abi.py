"""libpa from a plain C caller: tests/c_abi_example.c allocates with hipMalloc, runs a
copy-on-write block copy, a slot-mapped KV write and a split-K decode on its own stream
through include/pa.h, and checks the pools (bit for bit) and the outputs (2e-2 + 1e-2 |ref|)
against the C oracle linked into the same program."""
import os
import subprocess
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import c_abi_build  # noqa: E402

pytestmark = pytest.mark.gpu


def test_c_caller_decode_step_matches_oracle():
    print("\n[gpu-test] c_abi_example", flush=True)
    exe = c_abi_build.EXE
    if not os.path.exists(exe):
        from paged_kv_cache_82_amd import build as pa_build

        if not os.path.exists(pa_build.LIB):
            pa_build.build()
        c_abi_build.build()
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(r.stdout + r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "bit-identical" in r.stdout
