"""Block-wise forms of paged attention in numpy float64 — the oracle's self-check.

TEST INFRASTRUCTURE ONLY. Small inputs only (Python loop over blocks).

[PA-summary] azimuth.plus, "Efficient Memory Management for Large Language Model Serving with
PagedAttention", section "The PagedAttention algorithm": a length-T context is cut into
ceil(T/B) blocks; block j holds B_j valid tokens with keys K_j and values V_j; with scores
s_ji = q.K_ji / sqrt(d), every block forms its partial numerator and denominator against its
own maximum s_j^max and the blocks are merged with the log-sum-exp rescaling. The page says the
result is the same as standard attention. The section "Inside: block-table lookup" gives the
same merge as a running accumulation (a correction factor rescales the running output and sum
whenever the running maximum grows).

Two forms are written here, both reached through the block table:
  equation_form  -- per-block (s_j^max, numerator, denominator), merged once. The equation as
                    printed multiplies by e^{s_j^max}; that overflows for large scores, so both
                    sides are scaled by e^{-M} with M = max_j s_j^max (the log-sum-exp trick the
                    section names), which leaves the ratio unchanged.
  running_form   -- one block at a time with a running maximum, sum and output.
Reading: the last block contributes only its valid tokens (B_j), never its tail slots.
"""
from __future__ import annotations

import numpy as np


def _blocks(k64, v64, table, T, B, kv):
    """Yield (K_j, V_j) for the valid tokens of each logical block j."""
    for j in range((T + B - 1) // B):
        n = min(B, T - j * B)
        phys = int(table[j])
        yield k64[phys, kv, :n, :], v64[phys, kv, :n, :]


def equation_form(q64, k64, v64, table, T, B, kv, scale):
    if T == 0:
        return np.zeros(q64.shape[-1])
    parts = []
    for K, V in _blocks(k64, v64, table, T, B, kv):
        s = scale * (K @ q64)
        m = s.max()
        w = np.exp(s - m)
        parts.append((m, w @ V, w.sum()))
    M = max(p[0] for p in parts)
    num = sum(np.exp(m - M) * a for m, a, _ in parts)
    den = sum(np.exp(m - M) * b for m, _, b in parts)
    return num / den


def running_form(q64, k64, v64, table, T, B, kv, scale):
    d = q64.shape[-1]
    out = np.zeros(d)
    total = 0.0
    run_max = -np.inf
    if T == 0:
        return out
    for K, V in _blocks(k64, v64, table, T, B, kv):
        s = scale * (K @ q64)
        new_max = max(run_max, s.max())
        correction = np.exp(run_max - new_max)
        w = np.exp(s - new_max)
        out = out * correction + w @ V
        total = total * correction + w.sum()
        run_max = new_max
    return out / total


def decode_all(form, q64, k64, v64, block_tables, context_lens, scale):
    """Apply `form` to every (sequence, query head); inputs already widened to float64."""
    S, Hq, d = q64.shape
    Hkv = k64.shape[1]
    B = k64.shape[2]
    g = Hq // Hkv
    out = np.zeros((S, Hq, d))
    for s in range(S):
        for h in range(Hq):
            out[s, h] = form(q64[s, h], k64, v64, block_tables[s], int(context_lens[s]), B,
                             h // g, float(scale))
    return out
