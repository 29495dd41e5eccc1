"""Helpers for GPU tests: move a DecodeStep to the device, run it through the C ABI binding,
compare with the oracle. Test infrastructure (imports the oracle)."""
from __future__ import annotations

import numpy as np
import torch

import paged_kv_cache_82_amd as pa
from workloads import to_float64

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
ATOL16, RTOL16, ATOL32 = 2e-2, 1e-2, 1e-5

# Unit roundoff of the 16-bit formats (half an ulp, relative): 11 and 8 significant bits.
UNIT_ROUNDOFF = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}
# Observed errors of the full-size runs, printed at the end of the session (conftest).
PARITY_LOG: list = []


def to_dev(a: np.ndarray, dtype: str | None = None, device="cuda"):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_host(t: torch.Tensor, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


class DevStep:
    """A DecodeStep's arrays on the GPU plus an output and a zeroed workspace."""

    def __init__(self, step, partition_tokens: int = 0, device="cuda"):
        self.step = step
        dt = step.dtype
        self.k_cache = to_dev(step.k_cache, dt, device)
        self.v_cache = to_dev(step.v_cache, dt, device)
        self.q = to_dev(step.q, dt, device)
        self.block_tables = to_dev(step.block_tables, None, device)
        self.context_lens = to_dev(step.context_lens, None, device)
        self.copies = to_dev(step.copies, None, device)
        self.writes = [(to_dev(w.k_new, dt, device), to_dev(w.v_new, dt, device),
                        to_dev(w.slot_mapping, None, device)) for w in step.writes]
        self.out = torch.empty_like(self.q)
        self.partition_tokens = partition_tokens
        nbytes = pa.pa_decode_workspace_size(
            step.num_seqs, step.num_q_heads, step.num_kv_heads, step.head_dim, step.block_size,
            step.max_context_len, partition_tokens, TORCH_DT[dt])
        self.workspace = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)

    def apply_updates(self):
        if len(self.step.copies):
            pa.pa_copy_blocks(self.k_cache, self.v_cache, self.copies)
        for kn, vn, sm in self.writes:
            pa.pa_write_kv(self.k_cache, self.v_cache, kn, vn, sm)

    def decode(self):
        pa.pa_decode(self.out, self.q, self.k_cache, self.v_cache, self.block_tables,
                     self.context_lens, float(self.step.scale), self.step.max_context_len,
                     self.workspace, self.partition_tokens)
        return self.out

    def run(self):
        self.apply_updates()
        self.decode()
        torch.cuda.synchronize()
        return to_host(self.out, self.step.dtype)


def assert_attention_close(gpu: np.ndarray, ref64: np.ndarray, dtype: str, what: str = ""):
    g = to_float64(gpu, dtype)
    assert g.shape == ref64.shape, (g.shape, ref64.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite outputs"
    err = np.abs(g - ref64)
    if dtype == "f32":
        bad = err > ATOL32
    else:
        bad = err > ATOL16 + RTOL16 * np.abs(ref64)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; "
                             f"max abs err {err.max():.3g}; first bad {idx.tolist()}")
    return float(err.max())


class DevPrefill:
    """A PrefillStep's arrays on the GPU plus an output; run() writes the chunk's keys/values
    (pa_write_kv) and runs pa_prefill."""

    def __init__(self, step, device="cuda"):
        self.step = step
        dt = step.dtype
        self.k_cache = to_dev(step.k_cache, dt, device)
        self.v_cache = to_dev(step.v_cache, dt, device)
        self.q = to_dev(step.q, dt, device)
        self.block_tables = to_dev(step.block_tables, None, device)
        self.context_lens = to_dev(step.context_lens, None, device)
        self.query_start = to_dev(step.query_start, None, device)
        self.writes = [(to_dev(w.k_new, dt, device), to_dev(w.v_new, dt, device),
                        to_dev(w.slot_mapping, None, device)) for w in step.writes]
        self.out = torch.zeros_like(self.q)

    def apply_updates(self):
        for kn, vn, sm in self.writes:
            pa.pa_write_kv(self.k_cache, self.v_cache, kn, vn, sm)

    def attend(self):
        st = self.step
        pa.pa_prefill(self.out, self.q, self.k_cache, self.v_cache, self.block_tables,
                      self.context_lens, self.query_start, float(st.scale), st.max_query_len,
                      st.max_context_len)
        return self.out

    def run(self):
        self.apply_updates()
        self.attend()
        torch.cuda.synchronize()
        return to_host(self.out, self.step.dtype)


def prefill_rows_reference(step, kc, vc, rows):
    """Oracle outputs (float64 [len(rows), Hq, d]) of the listed query rows, each evaluated as a
    single query over its visible prefix (positions 0 .. T-n+i) with the decode oracle on the
    pools after the chunk's write. Test infrastructure: lets full-size checks sample rows."""
    import oracle

    qs = step.query_start
    seq = np.searchsorted(qs, rows, side="right") - 1
    T = step.context_lens[seq]
    n = qs[seq + 1] - qs[seq]
    visible = (T - n + (rows - qs[seq]) + 1).astype(np.int32)
    q_rows = np.ascontiguousarray(step.q[rows])
    tables = np.ascontiguousarray(step.block_tables[seq])
    return oracle.decode(q_rows, kc, vc, tables, visible, step.scale, step.dtype)


def make_dominant_token(step, gap_log2: float = 15.0):
    """Rewrite sequence 0 of a decode or prefill step so that token 0 outscores every other
    token by gap_log2 in the base-2 exponent: every other token then weighs 2^-gap_log2 of it
    (for 15, below fp16's smallest normal number, 2^-14, yet 3999 of them add 12% to the row
    sum). Keys are big * e_0 for token 0 and 0 otherwise; queries are 4 e_0 (scale 1/sqrt(d));
    V of KV head 0 is all ones (expected output exactly 1) and V of KV head 1 is ones except
    token 0, which is 0 (expected N w / (1 + N w) with N = T - 1 small weights w). A kernel
    that flushed the small weights in the weighted sum, or only in the row sum, misses either
    head by more than the 16-bit tolerance."""
    from workloads import to_storage

    dt, B, d, Hkv = step.dtype, step.block_size, step.head_dim, step.num_kv_heads
    assert Hkv >= 2 and step.num_seqs == 1
    T = int(step.context_lens[0])
    n_new = sum(w.k_new.shape[0] for w in step.writes)
    prefix = T - n_new
    scale = float(step.scale)
    big = gap_log2 / (4.0 * scale * np.log2(np.e))
    k = np.zeros((T, Hkv, d))
    k[0, :, 0] = big
    v = np.ones((T, Hkv, d))
    v[0, 1, :] = 0.0
    table = step.block_tables[0]
    for t in range(prefix):
        step.k_cache[table[t // B], :, t % B, :] = to_storage(k[t], dt)
        step.v_cache[table[t // B], :, t % B, :] = to_storage(v[t], dt)
    at = prefix
    for w in step.writes:
        m = w.k_new.shape[0]
        w.k_new[...] = to_storage(k[at:at + m], dt)
        w.v_new[...] = to_storage(v[at:at + m], dt)
        at += m
    q = np.zeros(step.q.shape)
    q[..., 0] = 4.0
    step.q[...] = to_storage(q, dt)
    return step


def uses_mfma_decode(step) -> bool:
    """Whether pa_decode's automatic choice takes the MFMA kernel (16-bit weights) here."""
    return step.dtype != "f32" and step.num_q_heads // step.num_kv_heads >= 2


def tight_bound(ref64: np.ndarray, dtype: str, visible: np.ndarray, weights16: bool):
    """A regression bound for 16-bit outputs over N(0,1) keys, values and queries, per element,
    far below the pass rule (2e-2 + 1e-2 |ref|) and derived from where the kernels round:
      - the output is rounded once to the 16-bit format: at most u |ref| (u the unit roundoff);
        twice that allows for the fp32 result itself sitting off the exact value;
      - with 16-bit softmax weights (the MFMA kernels), each weight carries a relative rounding
        error of at most u, and the numerator and the row sum see the same rounded weights, so
        the output moves by sum_t w_t d_t (v_t - out) / W. With independent errors uniform in
        [-u, u] its standard deviation is (u / sqrt 3) sqrt(sum_t w_t^2 (v_t - out)^2) / W,
        about (u / sqrt 3) sqrt(e / T) for N(0,1) scores and values (the weights' effective
        count is T / e); eight of those are allowed;
      - 1e-5 absolute for the fp32 accumulation and exp2.
    visible: visible tokens per output row (broadcast over heads and dims)."""
    u = UNIT_ROUNDOFF[dtype]
    T = np.maximum(np.asarray(visible, np.float64), 1.0).reshape(-1, *([1] * (ref64.ndim - 1)))
    b = 2.0 * u * np.abs(ref64) + 1e-5
    if weights16:
        b = b + 8.0 * (u / np.sqrt(3.0)) * np.sqrt(np.e / T)
    return b


def check_full_size(gpu: np.ndarray, ref64: np.ndarray, dtype: str, visible, weights16: bool,
                    what: str) -> float:
    """The pass rule (spec tolerance) and, for 16-bit outputs, the tight regression bound;
    logs the observed maximum error and its ratio to each bound."""
    err = assert_attention_close(gpu, ref64, dtype, what)
    g = to_float64(gpu, dtype)
    e = np.abs(g - ref64)
    if dtype == "f32":
        PARITY_LOG.append(f"{what}: max|err| {err:.2e} (pass rule 1e-05: {err / ATOL32:.3f}x)")
        return err
    loose = float((e / (ATOL16 + RTOL16 * np.abs(ref64))).max())
    bound = tight_bound(ref64, dtype, visible, weights16)
    ratio = e / bound
    tight = float(ratio.max())
    PARITY_LOG.append(f"{what}: max|err| {err:.2e} (pass rule {loose:.3f}x, tight bound "
                      f"{tight:.3f}x)")
    if tight > 1.0:
        idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        raise AssertionError(f"{what}: outside the tight bound, {int((ratio > 1).sum())} of "
                             f"{ratio.size}; worst {idx}: err {e[idx]:.3g} > {bound[idx]:.3g}")
    return err


def tight_failures(gpu: np.ndarray, ref64: np.ndarray, dtype: str, visible, weights16: bool):
    """(elements outside the tight bound, elements outside the pass rule)."""
    g = to_float64(gpu, dtype)
    e = np.abs(g - ref64)
    bound = tight_bound(ref64, dtype, visible, weights16)
    loose = ATOL16 + RTOL16 * np.abs(ref64)
    return int((e > bound).sum()), int((e > loose).sum())


def pools_equal(dev_pool: torch.Tensor, host_pool: np.ndarray, dtype: str,
                chunk_bytes: int = 1 << 30) -> bool:
    """Bit-exact comparison of a device pool with a host array, a chunk of blocks at a time on
    the device (for pools too large to copy back whole)."""
    n = host_pool.shape[0]
    per = max(1, chunk_bytes // max(1, host_pool[0].nbytes))
    ity = torch.int32 if dtype == "f32" else torch.int16
    for i in range(0, n, per):
        want = to_dev(host_pool[i:i + per], dtype, dev_pool.device)
        if not torch.equal(dev_pool[i:i + per].view(ity), want.view(ity)):
            return False
    return True


def share_prefixes(step, groups):
    """Make runs of consecutive sequences of a DecodeStep share leading blocks: groups is a list
    of (first, count, blocks); members first+1 .. first+count-1 point their first `blocks` table
    entries at the first member's blocks (so their first blocks*B tokens become the first
    member's). The shared blocks must end before every member's last token (which the step
    writes). Returns (group_start, prefix_lens) covering every sequence (a sequence in no listed
    group is a group of one with prefix 0). Test infrastructure."""
    S, B = step.num_seqs, step.block_size
    pl = np.zeros(S, np.int32)
    starts, covered = [], np.zeros(S, bool)
    spec = {first: (count, blocks) for first, count, blocks in groups}
    s = 0
    while s < S:
        starts.append(s)
        if s in spec:
            count, blocks = spec[s]
            T = step.context_lens[s:s + count]
            assert blocks * B <= int(T.min()) - 1, "shared blocks must end before every last token"
            for m in range(s + 1, s + count):
                step.block_tables[m, :blocks] = step.block_tables[s, :blocks]
            pl[s:s + count] = blocks * B
            covered[s:s + count] = True
            s += count
        else:
            s += 1
    starts.append(S)
    return np.asarray(starts, np.int32), pl



def groups_from_tables(block_tables, context_lens, B):
    from workloads import prefix_groups

    return prefix_groups(block_tables, context_lens, B)
