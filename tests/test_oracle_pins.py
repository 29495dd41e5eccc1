"""The CPU oracle against its pins, and planted mistakes against the same pins.

The pins themselves live in oracle_pins.py. The mutation test compiles copies of the oracle
with one plausible mistake each (wrong head group, wrong offset or block index, dropped scale,
flipped exponent sign, keys used as values, no normalisation, no max shift, wrong fp16
exponent bias, wrong bf16 precision, a write or copy that misses data, a causal mask that is off
by one, starts at the chunk or is missing, the chunk's first query used for every row) and
checks that every copy fails at least one pin, so the pins would catch such a mistake in the
oracle.
"""
import os
import subprocess
import sys

import pytest

import oracle
import oracle_pins

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, oracle_lib):
    pin(oracle_lib)


MUTANTS = [
    ("kv_group", "const int kv = h / group;", "const int kv = h % num_kv_heads;"),
    ("offset", "const int off = t % B;", "const int off = (t + 1) % B;"),
    ("block_index", "const int j = t / B;", "const int j = (t + 1) / B;"),
    ("no_scale", "score[t] = scale * acc;", "score[t] = acc;"),
    ("exp_sign", "score[t] = exp(score[t] - M);", "score[t] = exp(M - score[t]);"),
    ("k_as_v", "out[c] += score[t] * vbuf", "out[c] += score[t] * kbuf"),
    ("no_normalise", "out[c] /= L;", "out[c] /= 1.0;"),
    ("no_max_shift", "if (score[t] > M) M = score[t];", "M = 0.0;"),
    ("drop_last", "for (int t = 0; t < T; ++t) {\n    score[t] = exp",
     "for (int t = 0; t < T - 1; ++t) {\n    score[t] = exp"),
    ("half_bias", "e - 25);", "e - 24);"),
    ("bf16_precision", "round_to_format(x, 8, -126", "round_to_format(x, 9, -126"),
    ("write_v_missing", "memcpy((char *)v_cache + dst, (const char *)v_new + src, row_bytes);",
     ";"),
    ("copy_v_missing", "memcpy((char *)v_cache + dst * block_bytes", "(void)(v_cache + dst * block_bytes"),
    ("swap_wrong_src", "(const char *)src_k + src * block_bytes", "(const char *)src_k + dst * block_bytes"),
    ("causal_off_by_one", "const int visible = T - n + i + 1;", "const int visible = T - n + i;"),
    ("causal_from_chunk_start", "const int visible = T - n + i + 1;", "const int visible = i + 1;"),
    ("causal_whole_context", "const int visible = T - n + i + 1;", "const int visible = T;"),
    ("prefill_first_query_row", "q, qtok, k_cache, v_cache, block_tables, visible,",
     "q, query_start[s], k_cache, v_cache, block_tables, visible,"),
]

_RUNNER = """
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle_pins
for pin in oracle_pins.ALL_PINS:
    try:
        pin({lib!r})
    except Exception as e:
        print('CAUGHT-BY', pin.__name__, type(e).__name__, str(e)[:200])
        sys.exit(1)
print('SURVIVED')
"""


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(name, old, new, tmp_path):
    src = open(oracle.core.SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
    if name == "copy_v_missing":
        # turn the whole V memcpy statement into a no-op expression
        line_start = src.index(old)
        line_end = src.index(";", line_start)
        mutated = src[:line_start] + "(void)0" + src[line_end:]
    else:
        mutated = src.replace(old, new)
    cfile = tmp_path / f"m_{name}.c"
    cfile.write_text(mutated)
    lib = oracle.build(src=str(cfile), out=str(tmp_path / f"libm_{name}.so"))
    code = _RUNNER.format(root=os.path.dirname(HERE), tests=HERE, lib=lib)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600)
    assert "SURVIVED" not in r.stdout, f"mutant {name} passed every pin:\n{r.stdout}\n{r.stderr}"
    assert r.returncode != 0
