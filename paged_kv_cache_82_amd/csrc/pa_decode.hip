// pa_decode.hip — paged decode attention kernels for gfx950 (CDNA4, wave64).
//
// Method: [PA-summary] azimuth.plus, "Efficient Memory Management for Large Language Model
// Serving with PagedAttention", section "The PagedAttention algorithm" and its block-wise
// attention equation: for each query vector the kernel walks the block table, fetches the
// keys and values of each logical block from wherever its physical block sits, scores the
// block's tokens, and folds them into a running (maximum, sum, output) state with the
// log-sum-exp rescaling; the result equals standard softmax attention. The last block of a
// sequence contributes only its valid tokens (B_j in the equation).
//
// Work decomposition (not on the pages; chosen for MI355X):
//   - a workgroup of NW waves owns one (sequence, head unit, partition of P tokens);
//     waves take blocks (VALU path) or 32-token steps (MFMA path) of the partition in turn;
//   - every wave keeps its own running state; states are merged across lanes, then across
//     waves through LDS, with the same rescaling as the equation;
//   - when a sequence needs more than one partition, each workgroup stores its partial
//     (max, sum, unnormalised output) and a second, small kernel merges the partials of each
//     (sequence, query head) with the same rescaling (split-K). Merging across workgroups in
//     the same launch would need device-scope release/acquire fences, which on gfx950 write
//     back and invalidate the whole L2 of an XCD; the kernel boundary is far cheaper.
//   - each wave's physical block ids are read once into one register (lane k = k-th block)
//     and broadcast with readlane; the K/V loads of the next blocks (steps) are issued before
//     the current one is consumed, through a ring of buffers; K/V bytes are read once per
//     launch, with non-temporal loads.
// Scores are kept in the base-2 exponent domain: s' = s * log2(e), exp(s - m) = 2^(s' - m').
//
// Two kernels:
//   decode_valu_kernel: one query head per workgroup; 16-byte coalesced loads, q.K on the
//     vector ALU with a DPP all-reduce across the lanes of a token row; p.V accumulated per
//     lane. Used for single-head groups (MHA) and for fp32.
//   decode_mfma_kernel: one KV head and up to 16 query heads per workgroup (grouped-query
//     attention); each K/V tile is read once for all heads of the group and both products run
//     on 16x16x32 MFMA: S^T = K Q^T (tokens x heads) and O^T += V^T P^T (dims x heads).
//     K reaches its operand layout through a per-wave LDS ring (whole-line DMA loads); V is
//     read with 16-byte row loads straight into registers, the transposition the p.V product
//     needs being absorbed by pairing M-tile row r with head dimension (D/16)*r + mt.
#include "pa_device.h"
#include "pa_internal.h"
#include "pa_mfma.h"

namespace pa {

// ---- shared pieces ----------------------------------------------------------------------

// Context length of sequence s, clamped into what the table and grid can address.
__device__ __forceinline__ int seq_len(const DecodeArgs& a, int s, int BS) {
  int T = a.context_lens[s];
  const int64_t cap64 = (int64_t)a.max_blocks_per_seq * BS;
  const int cap = (int)(cap64 < (int64_t)a.max_context_len ? cap64 : (int64_t)a.max_context_len);
  return T < 0 ? 0 : (T > cap ? cap : T);
}

// After a workgroup has merged its partition into (fm, fl, fo[nh][D]) in LDS: store the final
// output when the sequence has a single partition, otherwise the partial state for the merge
// kernel.
template <DT dt, int D, int NT>
__device__ void finish_partition(const DecodeArgs& a, int s, int h0, int nh, int p, int nparts,
                                 const float* fm, const float* fl, const float* fo) {
  const int tid = threadIdx.x;
  const int Hq = a.num_q_heads;
  if (nparts == 1) {
    for (int idx = tid; idx < nh * D; idx += NT) {
      const int hh = idx / D, dim = idx % D;
      store_elem<dt>(a.out, ((int64_t)s * Hq + h0 + hh) * D + dim, fo[idx] / fl[hh]);
    }
    return;
  }
  const int MP = a.max_parts;
  for (int idx = tid; idx < nh * D; idx += NT) {
    const int hh = idx / D, dim = idx % D;
    a.part_o[(((int64_t)s * Hq + h0 + hh) * MP + p) * D + dim] = fo[idx];
  }
  if (tid < nh) {
    a.part_m[((int64_t)s * Hq + h0 + tid) * MP + p] = fm[tid];
    a.part_l[((int64_t)s * Hq + h0 + tid) * MP + p] = fl[tid];
  }
}

template <DT dt, int D, int NT>
__device__ void store_zeros(const DecodeArgs& a, int s, int h0, int nh) {
  for (int idx = threadIdx.x; idx < nh * D; idx += NT)
    store_elem<dt>(a.out, ((int64_t)s * a.num_q_heads + h0) * D + idx, 0.0f);
}

// Merge kernel: one workgroup of D threads per (query head, sequence) whose context spans more
// than one partition. With M = max_p m_p and w_p = 2^(m_p - M):
//   out = sum_p w_p o_p / sum_p w_p l_p          (the equation's rescaling, over partitions)
template <DT dt, int D, int BS>
__global__ __launch_bounds__(D) void merge_partitions_kernel(const DecodeArgs a) {
  const int h = blockIdx.x, s = blockIdx.y;
  const int T = seq_len(a, s, BS);
  const int nparts = (T + a.partition_tokens - 1) / a.partition_tokens;
  if (nparts <= 1) return;
  const int64_t base = ((int64_t)s * a.num_q_heads + h) * a.max_parts;
  // Partitions are read 8 at a time, so that their loads are in flight together (one at a
  // time, each waiting for the last, 64 partitions took 19 us).
  constexpr int U = 8;
  float M = kNegInf;
  int p = 0;
  for (; p + U <= nparts; p += U) {
    float mv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) mv[u] = a.part_m[base + p + u];
#pragma unroll
    for (int u = 0; u < U; ++u) M = fmaxf(M, mv[u]);
  }
  for (; p < nparts; ++p) M = fmaxf(M, a.part_m[base + p]);
  float acc = 0.0f, L = 0.0f;
  const int dim = threadIdx.x;
  p = 0;
  for (; p + U <= nparts; p += U) {
    float mv[U], lv[U], ov[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      mv[u] = a.part_m[base + p + u];
      lv[u] = a.part_l[base + p + u];
      ov[u] = a.part_o[(base + p + u) * D + dim];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float wgt = rescale(mv[u], M);
      acc = fmaf(wgt, ov[u], acc);
      L = fmaf(wgt, lv[u], L);
    }
  }
  for (; p < nparts; ++p) {
    const float wgt = rescale(a.part_m[base + p], M);
    acc = fmaf(wgt, a.part_o[(base + p) * D + dim], acc);
    L = fmaf(wgt, a.part_l[base + p], L);
  }
  store_elem<dt>(a.out, ((int64_t)s * a.num_q_heads + h) * D + dim, acc / L);
}

// ---- VALU kernel ------------------------------------------------------------------------

// Tokens a wave of the VALU kernels takes at once (a "unit"): the whole block up to 32 tokens;
// 16 tokens of a larger block, so that a unit's registers stay those of a 16-token block.
template <int BS>
constexpr int valu_unit_tokens() {
  return BS > 32 ? 16 : BS;
}

template <DT dt, int D, int SB, int NW>
struct ValuCfg {
  static constexpr int E = Elem<dt>::bytes;
  static constexpr int VEC = 16 / E;    // elements per 16-byte chunk
  static constexpr int R = D / VEC;     // lanes that share one token row
  static constexpr int TPI = 64 / R;    // token rows covered by one wave-wide load
  static constexpr int NL = SB / TPI;   // loads per unit per tensor
  static constexpr int NT = NW * 64;
  static_assert(64 % R == 0 && R >= 1, "row must split evenly over the wave");
  static_assert(SB % TPI == 0, "a unit must cover whole wave loads");
  static_assert(D <= NT, "one thread per head dimension in the merge");
};

// One unit (SB tokens) of one wave: scores, running-state update and p.V accumulation. Lane
// (c, r) holds head dimensions c*VEC.. of token rows i*TPI + r. TAIL masks tokens at or beyond
// t_end.
template <DT dt, int D, int SB, int NW, bool TAIL>
__device__ __forceinline__ void valu_block(const float (&qf)[ValuCfg<dt, D, SB, NW>::VEC],
                                           const u32x4* kr, const u32x4* vr, int tok0,
                                           int t_end, int r, float& m, float& l,
                                           float (&o)[ValuCfg<dt, D, SB, NW>::VEC]) {
  using C = ValuCfg<dt, D, SB, NW>;
  float sc[C::NL];
#pragma unroll
  for (int i = 0; i < C::NL; ++i) {
    const uint32_t w[4] = {kr[i][0], kr[i][1], kr[i][2], kr[i][3]};
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < C::VEC; ++e) acc = fmaf(qf[e], elem_of<dt>(w, e), acc);
    sc[i] = group_sum<C::R>(acc);
    if (TAIL && tok0 + i * C::TPI + r >= t_end) sc[i] = kNegInf;
  }
  float bm = sc[0];
#pragma unroll
  for (int i = 1; i < C::NL; ++i) bm = fmaxf(bm, sc[i]);
  const float mn = fmaxf(m, bm);
  const bool empty = (mn == kNegInf);  // no valid token seen yet by this lane row
  const float corr = empty ? 1.0f : fast_exp2(m - mn);
  float ps = 0.0f;
  float pr[C::NL];
#pragma unroll
  for (int i = 0; i < C::NL; ++i) {
    pr[i] = empty ? 0.0f : fast_exp2(sc[i] - mn);
    ps += pr[i];
  }
  l = fmaf(l, corr, ps);
#pragma unroll
  for (int e = 0; e < C::VEC; ++e) o[e] *= corr;
#pragma unroll
  for (int i = 0; i < C::NL; ++i) {
    const uint32_t w[4] = {vr[i][0], vr[i][1], vr[i][2], vr[i][3]};
    const bool ok = !TAIL || (tok0 + i * C::TPI + r < t_end);
#pragma unroll
    for (int e = 0; e < C::VEC; ++e) {
      float v = elem_of<dt>(w, e);
      if (TAIL) v = ok ? v : 0.0f;  // select, never multiply: tail slots may hold NaN
      o[e] = fmaf(pr[i], v, o[e]);
    }
  }
  m = mn;
}

// Maximum units (VALU) or 32-token steps (MFMA) one wave handles in one partition: their
// physical ids sit one per lane of a single register.
constexpr int kMaxPerWave = 64;

template <DT dt, int D, int BS, int NW, int NBUF>
__global__ __launch_bounds__(NW * 64) void decode_valu_kernel(const DecodeArgs a) {
  constexpr int SB = valu_unit_tokens<BS>();  // tokens per unit; a block holds NSUB units
  constexpr int NSUB = BS / SB;
  using C = ValuCfg<dt, D, SB, NW>;
  constexpr int E = C::E, VEC = C::VEC, R = C::R, TPI = C::TPI, NL = C::NL, NT = C::NT;
  __shared__ float lds_o[NW][D];
  __shared__ float lds_m[NW], lds_l[NW];
  __shared__ float lds_fm[1], lds_fl[1];

  const int p = blockIdx.x, h = blockIdx.y;
  const int s = blockIdx.z;
  const int P = a.partition_tokens;
  const int jb0 = p * (P / SB);  // first unit of the partition
  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int c = lane % R, r = lane / R;
  // Issued before the context length is known, so the id, query and length loads overlap:
  // lane k takes the id of the block holding this wave's k-th unit of the partition (when
  // inside the table).
  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  int my_id = 0;
  {
    const int j = (jb0 + w + lane * NW) / NSUB;
    if (lane < (P / SB + NW - 1) / NW && j < a.max_blocks_per_seq) my_id = bt[j];
  }
  const u32x4 qraw =
      load16((const char*)a.q + (((int64_t)s * a.num_q_heads + h) * D + c * VEC) * E);

  const int T = seq_len(a, s, BS);
  const int nparts = (T + P - 1) / P;
  if (T == 0) {
    if (p == 0) store_zeros<dt, D, NT>(a, s, h, 1);
    return;
  }
  if (p >= nparts) return;
  const int kvh = h / (a.num_q_heads / a.num_kv_heads);
  const int t0 = p * P;
  const int t1 = (T < t0 + P) ? T : t0 + P;
  const int jb1 = (t1 + SB - 1) / SB;

  float qf[VEC];
  {
    const uint32_t wq[4] = {qraw[0], qraw[1], qraw[2], qraw[3]};
#pragma unroll
    for (int e = 0; e < VEC; ++e) qf[e] = elem_of<dt>(wq, e) * a.scale_log2;
  }

  float m = kNegInf, l = 0.0f;
  float o[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) o[e] = 0.0f;

  // This wave takes units jb0 + w + k*NW, k < nb; lane k holds the k-th unit's physical id.
  const int nb = (jb1 - jb0 - w + NW - 1) / NW;
  const char* kbase = (const char*)a.k_cache;
  const char* vbase = (const char*)a.v_cache;
  constexpr int row_bytes = D * E;
  // Per-lane byte offset inside a (block, head) tile: loop-invariant and 32-bit, so loads take
  // the form (wave-uniform 64-bit tile base) + (per-lane 32-bit offset).
  const uint32_t lane_off = (uint32_t)(r * row_bytes + c * 16);
  // Fetch k >= nb is a prefetch past the wave's last unit, never consumed. It reads the pool's
  // first tile, which such prefetches of every workgroup share, so it stays cached; the wave's
  // own last unit would not be, since the streaming loads evict it first.
  auto fetch = [&](int k, u32x4* kr, u32x4* vr) {
    const bool live = k < nb;
    const int32_t id = __builtin_amdgcn_readlane(my_id, live ? k : 0);
    int64_t tile =
        live ? (clamp_block(id, a.num_blocks) * a.num_kv_heads + kvh) * (int64_t)(BS * row_bytes)
             : 0;
    if constexpr (NSUB > 1) {  // the unit's rows within its block
      if (live) tile += (int64_t)(((jb0 + w + k * NW) % NSUB) * SB * row_bytes);
    }
    const char* kt = kbase + tile;
    const char* vt = vbase + tile;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      kr[i] = load16_stream(kt + lane_off + i * TPI * row_bytes);
      vr[i] = load16_stream(vt + lane_off + i * TPI * row_bytes);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the consume that follows
  };
  auto consume = [&](int k, const u32x4* kr, const u32x4* vr) {
    const int tok0 = (jb0 + w + k * NW) * SB;
    if (tok0 + SB <= t1)
      valu_block<dt, D, SB, NW, false>(qf, kr, vr, tok0, t1, r, m, l, o);
    else
      valu_block<dt, D, SB, NW, true>(qf, kr, vr, tok0, t1, r, m, l, o);
  };
  // A ring of NBUF register buffers: the loads of the next NBUF-1 blocks are in flight while
  // one block is consumed. Prefetches are unconditional (past the end they read the shared
  // first tile, a cache hit) so that the compiler's wait before each consume only covers the
  // oldest buffer.
  if (nb > 0) {
    u32x4 kbuf[NBUF][NL], vbuf[NBUF][NL];
#pragma unroll
    for (int u = 0; u + 1 < NBUF; ++u) fetch(u, kbuf[u], vbuf[u]);
    for (int k = 0; k < nb; k += NBUF) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        if (k + u >= nb) break;
        fetch(k + u + NBUF - 1, kbuf[(u + NBUF - 1) % NBUF], vbuf[(u + NBUF - 1) % NBUF]);
        consume(k + u, kbuf[u], vbuf[u]);
      }
    }
  }

  // Merge the TPI row states of this wave (lanes with equal c), then the waves.
#pragma unroll
  for (int off = R; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off);
    const float l2 = __shfl_xor(l, off);
    const float M = fmaxf(m, m2);
    const float wa = rescale(m, M), wb = rescale(m2, M);
    l = wa * l + wb * l2;
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[e] = wa * o[e] + wb * __shfl_xor(o[e], off);
    m = M;
  }
  if (r == 0) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) lds_o[w][c * VEC + e] = o[e];
  }
  if (lane == 0) {
    lds_m[w] = m;
    lds_l[w] = l;
  }
  __syncthreads();
  float* fo = &lds_o[0][0];  // merged output reuses wave 0's row (read-before-write per thread)
  if (threadIdx.x < D) {
    const int dim = threadIdx.x;
    float M = kNegInf;
#pragma unroll
    for (int k = 0; k < NW; ++k) M = fmaxf(M, lds_m[k]);
    float acc = 0.0f, L = 0.0f;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      const float wgt = rescale(lds_m[k], M);
      acc = fmaf(wgt, lds_o[k][dim], acc);
      L = fmaf(wgt, lds_l[k], L);
    }
    fo[dim] = acc;
    if (dim == 0) {
      lds_fm[0] = M;
      lds_fl[0] = L;
    }
  }
  __syncthreads();
  finish_partition<dt, D, NT>(a, s, h, 1, p, nparts, lds_fm, lds_fl, fo);
}

// ---- fp32 prefill on the vector ALU ---------------------------------------------------------

// Causal multi-query attention for fp32 pools (the MFMA prefill kernel takes 16-bit data): one
// workgroup per (query row, query head) runs the decode computation over the tokens the row
// sees. [PA-summary] "The PagedAttention algorithm", applied to every query vector of a chunk:
// query i of a sequence's n new tokens sits at position T - n + i and attends to positions
// 0 .. T - n + i. Rows past the chunk (i >= n, with n = min(query rows, T, max_query_len))
// are not written, as in the MFMA kernel. Block ids come 64 per wave at a time; K/V tiles are
// double-buffered in registers. No part of the 16-bit workloads runs here.
template <DT dt, int D, int BS, int NW>
__global__ __launch_bounds__(NW * 64) void prefill_valu_kernel(const PrefillArgs a) {
  constexpr int SB = valu_unit_tokens<BS>();  // tokens per unit; a block holds NSUB units
  constexpr int NSUB = BS / SB;
  using C = ValuCfg<dt, D, SB, NW>;
  constexpr int E = C::E, VEC = C::VEC, R = C::R, TPI = C::TPI, NL = C::NL, NT = C::NT;
  __shared__ float lds_o[NW][D];
  __shared__ float lds_m[NW], lds_l[NW];

  const int Hq = a.num_q_heads;
  const int64_t L = blockIdx.x;
  const int h = (int)(L % Hq);
  const int row = (int)(L / Hq);
  const int Nq = a.num_q_tokens;
  // The sequence of this row: the last s with query_start[s] <= row (query_start ascending).
  int lo = 0, hi = a.num_seqs;  // query_start[lo] <= row holds for lo = 0 when row is in range
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.query_start[mid] <= row) lo = mid; else hi = mid;
  }
  const int s = lo;
  const int q0 = clampi(a.query_start[s], 0, Nq);
  const int q1 = clampi(a.query_start[s + 1], q0, Nq);
  const int64_t cap64 = (int64_t)a.max_blocks_per_seq * BS;
  const int cap = (int)(cap64 < (int64_t)a.max_context_len ? cap64 : (int64_t)a.max_context_len);
  const int T = clampi(a.context_lens[s], 0, cap);
  int n = q1 - q0;
  n = n < T ? n : T;
  n = n < a.max_query_len ? n : a.max_query_len;
  const int i = row - q0;
  if (i < 0 || i >= n) return;  // uniform over the workgroup
  const int t_end = T - n + i + 1;  // the row sees tokens 0 .. t_end - 1
  const int nunit = (t_end + SB - 1) / SB;
  const int kvh = h / (Hq / a.num_kv_heads);

  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int c = lane % R, r = lane / R;
  float qf[VEC];
  {
    const u32x4 qraw = load16((const char*)a.q + (((int64_t)row * Hq + h) * D + c * VEC) * E);
    const uint32_t wq[4] = {qraw[0], qraw[1], qraw[2], qraw[3]};
#pragma unroll
    for (int e = 0; e < VEC; ++e) qf[e] = elem_of<dt>(wq, e) * a.scale_log2;
  }
  float m = kNegInf, l = 0.0f;
  float o[VEC];
#pragma unroll
  for (int e = 0; e < VEC; ++e) o[e] = 0.0f;

  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  constexpr int row_bytes = D * E;
  const uint32_t lane_off = (uint32_t)(r * row_bytes + c * 16);
  const char* kbase = (const char*)a.k_cache;
  const char* vbase = (const char*)a.v_cache;
  // Chunks of 64 units per wave: wave w takes units base + w + k*NW, k < nb; lane k of
  // my_id holds the id of the block holding the k-th.
  for (int base = 0; base < nunit; base += 64 * NW) {
    const int j = base + w + lane * NW;
    const int my_id = (j < nunit) ? bt[j / NSUB] : 0;  // j / NSUB < max_blocks_per_seq
    const int left = nunit - base < 64 * NW ? nunit - base : 64 * NW;
    const int nb = (left - w + NW - 1) / NW;
    auto fetch = [&](int k, u32x4* kr, u32x4* vr) {
      const int32_t id = __builtin_amdgcn_readlane(my_id, k);
      int64_t tile =
          (clamp_block(id, a.num_blocks) * a.num_kv_heads + kvh) * (int64_t)(BS * row_bytes);
      if constexpr (NSUB > 1) tile += (int64_t)(((base + w + k * NW) % NSUB) * SB * row_bytes);
#pragma unroll
      for (int q = 0; q < NL; ++q) {
        kr[q] = load16(kbase + tile + lane_off + q * TPI * row_bytes);
        vr[q] = load16(vbase + tile + lane_off + q * TPI * row_bytes);
      }
    };
    auto consume = [&](int k, const u32x4* kr, const u32x4* vr) {
      const int tok0 = (base + w + k * NW) * SB;
      if (tok0 + SB <= t_end)
        valu_block<dt, D, SB, NW, false>(qf, kr, vr, tok0, t_end, r, m, l, o);
      else
        valu_block<dt, D, SB, NW, true>(qf, kr, vr, tok0, t_end, r, m, l, o);
    };
    if (nb <= 0) continue;  // uniform
    // Two buffers, unrolled so that both are register arrays; the fetch ahead is unconditional
    // (past the end it re-reads the wave's last block).
    u32x4 k0[NL], v0[NL], k1[NL], v1[NL];
    fetch(0, k0, v0);
    for (int k = 0; k < nb; k += 2) {
      fetch(k + 1 < nb ? k + 1 : nb - 1, k1, v1);
      consume(k, k0, v0);
      if (k + 1 >= nb) break;
      fetch(k + 2 < nb ? k + 2 : nb - 1, k0, v0);
      consume(k + 1, k1, v1);
    }
  }

  // Merge the TPI row states of this wave, then the waves (as in the decode kernel).
#pragma unroll
  for (int off = R; off < 64; off <<= 1) {
    const float m2 = __shfl_xor(m, off);
    const float l2 = __shfl_xor(l, off);
    const float M = fmaxf(m, m2);
    const float wa = rescale(m, M), wb = rescale(m2, M);
    l = wa * l + wb * l2;
#pragma unroll
    for (int e = 0; e < VEC; ++e) o[e] = wa * o[e] + wb * __shfl_xor(o[e], off);
    m = M;
  }
  if (r == 0) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) lds_o[w][c * VEC + e] = o[e];
  }
  if (lane == 0) {
    lds_m[w] = m;
    lds_l[w] = l;
  }
  __syncthreads();
  for (int dim = threadIdx.x; dim < D; dim += NT) {
    float M = kNegInf;
#pragma unroll
    for (int k = 0; k < NW; ++k) M = fmaxf(M, lds_m[k]);
    float acc = 0.0f, Lsum = 0.0f;
#pragma unroll
    for (int k = 0; k < NW; ++k) {
      const float wgt = rescale(lds_m[k], M);
      acc = fmaf(wgt, lds_o[k][dim], acc);
      Lsum = fmaf(wgt, lds_l[k], Lsum);
    }
    store_elem<dt>(a.out, ((int64_t)row * Hq + h) * D + dim, acc / Lsum);
  }
}

// ---- MFMA kernel (grouped query heads) -----------------------------------------------------

// s_waitcnt vmcnt(N) (vmcnt in bits [3:0] and [15:14]), expcnt and lgkmcnt left at their maxima.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt holds 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// K operand fragments of a 32-token step from the wave's LDS slot: t[u][kk] from ka[kk] +
// OFF + u * UOFF. One asm block that also waits for the reads: the compiler treats LDS reads
// as possibly aliasing the K DMA loads still in flight and would drain every load before them.
template <int OFF, int UOFF>
__device__ __forceinline__ void lds_read_k(u32x4 (&t)[2][4], const uint32_t (&ka)[4]) {
  asm volatile(
      "ds_read_b128 %0, %8 offset:%12\n\t"
      "ds_read_b128 %1, %9 offset:%12\n\t"
      "ds_read_b128 %2, %10 offset:%12\n\t"
      "ds_read_b128 %3, %11 offset:%12\n\t"
      "ds_read_b128 %4, %8 offset:%13\n\t"
      "ds_read_b128 %5, %9 offset:%13\n\t"
      "ds_read_b128 %6, %10 offset:%13\n\t"
      "ds_read_b128 %7, %11 offset:%13\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(t[0][0]), "=&v"(t[0][1]), "=&v"(t[0][2]), "=&v"(t[0][3]), "=&v"(t[1][0]),
        "=&v"(t[1][1]), "=&v"(t[1][2]), "=&v"(t[1][3])
      : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "i"(OFF), "i"(OFF + UOFF));
}
template <int OFF, int UOFF>
__device__ __forceinline__ void lds_read_k(u32x4 (&t)[2][2], const uint32_t (&ka)[2]) {
  asm volatile(
      "ds_read_b128 %0, %4 offset:%6\n\t"
      "ds_read_b128 %1, %5 offset:%6\n\t"
      "ds_read_b128 %2, %4 offset:%7\n\t"
      "ds_read_b128 %3, %5 offset:%7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(t[0][0]), "=&v"(t[0][1]), "=&v"(t[1][0]), "=&v"(t[1][1])
      : "v"(ka[0]), "v"(ka[1]), "i"(OFF), "i"(OFF + UOFF));
}

template <DT dt, int D, int BS, int NW, int NBUF, int MINB>
__global__ __launch_bounds__(NW * 64, MINB) void decode_mfma_kernel(const DecodeArgs a) {
  static_assert(dt != DT::F32, "MFMA path takes 16-bit inputs");
  static_assert(32 % BS == 0 || BS % 32 == 0, "a 32-token step spans whole blocks or part of one");
  using M = MfmaT<dt>;
  using vec8 = typename M::vec8;
  using VF = VFrag<D>;
  constexpr int E = 2;
  constexpr int KC = D / 32;  // q.K MFMAs per 16-token tile
  constexpr int MT = D / 16;  // p.V M-tiles; row r of tile mt is head dimension MT*r + mt
  constexpr int NBS = BS >= 32 ? 1 : 32 / BS;  // blocks a step touches
  constexpr int SPB = BS > 32 ? BS / 32 : 1;    // steps per block
  constexpr int NT = NW * 64;
  __shared__ __attribute__((aligned(1024))) char lds_k[NW][NBUF][32 * D * 2];  // K ring
  __shared__ float lds_o[NW][16][D];
  __shared__ float lds_m[NW][16], lds_l[NW][16];
  __shared__ float lds_fm[16], lds_fl[16];

  const int p = blockIdx.x, unit = blockIdx.y;
  const int s = blockIdx.z;
  const int Hq = a.num_q_heads;
  const int g = Hq / a.num_kv_heads;
  const int ntile = (g + 15) / 16;
  const int kvh = unit / ntile, ht = unit % ntile;
  const int h0 = kvh * g + ht * 16;
  const int nh = (g - ht * 16 < 16) ? g - ht * 16 : 16;
  const int P = a.partition_tokens;
  const int st0 = p * (P / 32);
  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int hh = lane & 15, gq = lane >> 4;

  // Issued before the context length is known, so the id, query and length loads overlap:
  // lane k takes the NBS block ids of this wave's k-th 32-token step (when inside the table).
  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  int my_id[NBS];
#pragma unroll
  for (int b = 0; b < NBS; ++b) {
    my_id[b] = 0;
    const int j = (st0 + w + lane * NW) * NBS / SPB + b;
    if (lane < (P / 32 + NW - 1) / NW && j < a.max_blocks_per_seq) my_id[b] = bt[j];
  }
  // Q^T operand: column hh = query head h0 + hh, k = head dims 32*kk + 8*gq + e.
  vec8 qop[KC];
#pragma unroll
  for (int kk = 0; kk < KC; ++kk) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (hh < nh)
      raw = load16((const char*)a.q +
                   (((int64_t)s * Hq + h0 + hh) * D + 32 * kk + 8 * gq) * E);
    qop[kk] = __builtin_bit_cast(vec8, raw);
  }

  const int T = seq_len(a, s, BS);
  const int nparts = (T + P - 1) / P;
  if (T == 0) {
    if (p == 0) store_zeros<dt, D, NT>(a, s, h0, nh);
    return;
  }
  if (p >= nparts) return;
  const int t1 = (T < (p + 1) * P) ? T : (p + 1) * P;
  const int st1 = (t1 + 31) / 32;
  const int jlast = (t1 - 1) / BS;  // last block of this partition

  f32x4 oacc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) oacc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = kNegInf, lsum = 0.0f;

  // This wave takes steps st0 + w + k*NW, k < ns; lane k holds the NBS physical ids of step k.
  const int ns = (st1 - st0 - w + NW - 1) / NW;
  const int64_t Hkv = a.num_kv_heads;

  constexpr int RB = D * E;  // bytes per token row
  // V: loop-invariant per-lane byte offset inside a (block, head) tile. Token tk of a step lives
  // in the step's block tk / BS at row tk % BS.
  const uint32_t voff = (uint32_t)(((4 * gq) % BS) * RB + MT * hh * E);
  const int64_t tile_bytes = (int64_t)BS * RB;
  // Tile (block p, head kvh) starts at p * blk_stride + kvh * tile_bytes in each pool; the head
  // offset is folded into the bases once.
  const int64_t blk_stride = Hkv * tile_bytes;
  const char* kbase = (const char*)a.k_cache + kvh * tile_bytes;
  const char* vbase = (const char*)a.v_cache + kvh * tile_bytes;
  const int id_max = last_block_id(a.num_blocks);

  // K goes through a ring of NBUF LDS slots per wave (no other wave touches them), V through a
  // ring of NBUF register sets. A step's K is KD DMA loads (buffer_load ... lds) of 1 KB, RPL
  // whole rows each, so every K load instruction reads whole 128-byte lines and can be
  // non-temporal. Loaded straight into registers in the MFMA operand layout, a K load
  // instruction would cover 64 bytes of each of 16 rows, with the other half of each line in the
  // next instruction; that only works with ordinary loads, which keep the line cached in between
  // (measured on MI355X: the GQA batch took 366.8 us that way). The operand is read back with
  // ds_read_b128; rows are XOR-swizzled in 16-byte chunks so that the 16 rows read at one chunk
  // hit distinct banks. V loads cover whole token rows and are non-temporal loads into
  // registers. A fetch past the wave's last step, and a block of the last step past the
  // partition's last token, read nothing: their buffer resources span no bytes (B = 8 V loads
  // excepted, see below).
  constexpr int KSTEP = 32 * RB;  // K bytes per 32-token step
  constexpr int KD = KSTEP / 1024;
  constexpr int RPL = 1024 / RB;  // rows per K load
  constexpr int CPR = RB / 16;    // 16-byte chunks per row
  constexpr int RPBL = 256 / RB;  // rows per 256-byte line of banks
  static_assert(BS % RPL == 0, "the rows of one K load lie in one block");
  auto swz = [](int r) { return (r / RPBL) % CPR; };
  // K load j: lane L fills LDS chunk L % CPR of step row j * RPL + L / CPR with the logical
  // chunk the swizzle maps there.
  uint32_t kdo[KD];
#pragma unroll
  for (int j = 0; j < KD; ++j) {
    const int r = j * RPL + lane / CPR;
    kdo[j] = (uint32_t)((r % BS) * RB + (((lane % CPR) ^ swz(r)) * 16));
  }
  // K operand of tile u, MFMA kk: lane (gq, hh) reads row 16u + hh, chunk 4kk + gq (head dims
  // 32kk + 8gq ..); swz(16u + hh) = swz(hh), so tile u is a constant offset of 16 rows.
  typedef __attribute__((address_space(3))) char lds_char;
  uint32_t ka[KC];
#pragma unroll
  for (int kk = 0; kk < KC; ++kk)
    ka[kk] = (uint32_t)(uintptr_t)(lds_char*)&lds_k[w][0][0] + hh * RB +
             (((4 * kk + gq) ^ swz(hh)) * 16);

  auto fetch = [&](int k, auto slotc, VRegs<D>& R) {
    constexpr int slot = decltype(slotc)::value;
    const bool live = k < ns;
    const int kq = live ? k : 0;
    const int step = st0 + w + k * NW;
    const int jfirst = step * NBS / SPB;  // block of the step's first token
    // Blocks larger than a step: the step's 32 rows start (step % SPB) * 32 rows into its block,
    // and its resources span those rows only.
    constexpr int span = BS > 32 ? 32 * RB : (int)(BS * RB);
    __amdgpu_buffer_rsrc_t kr[NBS];
    int64_t tile[NBS];
    bool has[NBS];
#pragma unroll
    for (int b = 0; b < NBS; ++b) {
      const int id = clamp_id(__builtin_amdgcn_readlane(my_id[b], kq), id_max);
      tile[b] = (int64_t)id * blk_stride;
      if constexpr (SPB > 1) tile[b] += (int64_t)((step % SPB) * span);
      has[b] = live && jfirst + b <= jlast;
      kr[b] = tile_rsrc(kbase + tile[b], has[b] ? span : 0);
    }
    // K first, then V: 0.7% faster on the GQA batch than the other order (measured on MI355X).
#pragma unroll
    for (int j = 0; j < KD; ++j)
      load16_tile_stream_lds(kr[(j * RPL) / BS], &lds_k[w][slot][j * 1024], kdo[j]);
    if constexpr (BS >= 16) {
      __amdgpu_buffer_rsrc_t vr[NBS];
#pragma unroll
      for (int b = 0; b < NBS; ++b) vr[b] = tile_rsrc(vbase + tile[b], has[b] ? span : 0);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          R.v[u][i] = VF::load_tile_stream(vr[(16 * u) / BS], voff + ((16 * u) % BS + i) * RB);
    } else {
      // BS == 8: lanes of one V load instruction read two different blocks, which one buffer
      // resource cannot span. Plain loads of the clamped block ids (any block id in the pool
      // is readable memory; tokens past the partition are masked); a fetch past the wave's last
      // step reads block 0 of its KV head, shared by every such fetch and so cached.
      const char* vt[NBS];
#pragma unroll
      for (int b = 0; b < NBS; ++b) vt[b] = vbase + (live ? tile[b] : 0);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)  // token 16u + 4gq + i: block 2u + gq/2, row 4*(gq&1) + i
          R.v[u][i] = VF::load_stream(vt[2 * u + (gq >> 1)] + voff + i * RB);
    }
    __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the consume that follows
  };

  auto consume = [&](int k, auto slotc, VRegs<D>& R) {
    constexpr int slot = decltype(slotc)::value;
    const int tau0 = (st0 + w + k * NW) * 32;
    // This step's K loads (and all loads issued before them) are done once at most its own 8 V
    // loads and those of the NBUF - 1 later fetches (8 V and KD K loads each) are outstanding.
    wait_vmcnt<(NBUF - 1) * (8 + KD) + 8>();
    u32x4 kf[2][KC];
    lds_read_k<slot * KSTEP, 16 * RB>(kf, ka);
    // S^T = K Q^T: sacc[u][i] = score of token tau0 + 16u + 4*gq + i for head hh.
    f32x4 sacc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      sacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KC; ++kk)
        sacc[u] = M::mma(__builtin_bit_cast(vec8, kf[u][kk]), qop[kk], sacc[u]);
    }
    const bool tail = tau0 + 32 > t1;
    float sc[8];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = sacc[u][i] * a.scale_log2;
        if (tail && tau0 + 16 * u + 4 * gq + i >= t1) x = kNegInf;
        sc[4 * u + i] = x;
      }
    float bm = sc[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) bm = fmaxf(bm, sc[e]);
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float mn = fmaxf(m, bm);
    const bool empty = (mn == kNegInf);
    const float corr = empty ? 1.0f : fast_exp2(m - mn);
    // The weights are rounded to 16 bits for the p.V MFMA; the row sum adds those same rounded
    // weights (dot2 of each packed pair with (1, 1)), so numerator and denominator agree.
    float pe[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pe[e] = empty ? 0.0f : fast_exp2(sc[e] - mn);
    const u32x4 pw = {pack2<dt>(pe[0], pe[1]), pack2<dt>(pe[2], pe[3]),
                      pack2<dt>(pe[4], pe[5]), pack2<dt>(pe[6], pe[7])};
    float ps = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) ps = sum2<dt>(pw[j], ps);
    const vec8 pop = __builtin_bit_cast(vec8, pw);
    lsum = fmaf(lsum, corr, ps);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) oacc[mt] *= corr;
    if (tail) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tau0 + 16 * u + 4 * gq + i >= t1) R.v[u][i] = typename VF::T{};  // select
    }
    // O^T += V^T P^T with k element e <-> token 16*(e/4) + 4*gq + (e%4).
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      u32x4 vw;
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        const int e0 = 2 * q2, e1 = 2 * q2 + 1;
        const uint32_t lo = vfrag_elem<D>(R.v[e0 / 4][e0 % 4], mt);
        const uint32_t hi = vfrag_elem<D>(R.v[e1 / 4][e1 % 4], mt);
        vw[q2] = lo | (hi << 16);
      }
      oacc[mt] = M::mma(__builtin_bit_cast(vec8, vw), pop, oacc[mt]);
    }
    m = mn;
  };

  if (ns > 0) {  // rings of NBUF slots, unconditional prefetch (see the VALU kernel)
    VRegs<D> rb[NBUF];
    static_for<NBUF - 1>([&](auto uc) { fetch(decltype(uc)::value, uc, rb[decltype(uc)::value]); });
    // Unrolled NBUF steps at a time so that every slot index is a constant.
    for (int k = 0; k < ns; k += NBUF) {
      static_for<NBUF>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        if (k + u >= ns) return;  // uniform
        constexpr int ahead = (u + NBUF - 1) % NBUF;
        fetch(k + u + NBUF - 1, std::integral_constant<int, ahead>{}, rb[ahead]);
        consume(k + u, uc, rb[u]);
      });
    }
  }

  // Sum the per-lane partial sums over the four lane groups of each head.
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  // oacc[mt][i] is O[head hh][dim MT*(4*gq + i) + mt].
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) lds_o[w][hh][MT * (4 * gq + i) + mt] = oacc[mt][i];
  if (gq == 0) {
    lds_m[w][hh] = m;
    lds_l[w][hh] = lsum;
  }
  __syncthreads();
  if (threadIdx.x < 16) {
    const int k = threadIdx.x;
    float Mx = kNegInf;
#pragma unroll
    for (int x = 0; x < NW; ++x) Mx = fmaxf(Mx, lds_m[x][k]);
    float L = 0.0f;
#pragma unroll
    for (int x = 0; x < NW; ++x) L = fmaf(rescale(lds_m[x][k], Mx), lds_l[x][k], L);
    lds_fm[k] = Mx;
    lds_fl[k] = L;
  }
  float* fo = &lds_o[0][0][0];  // merged output reuses wave 0's slab (read-before-write)
  for (int idx = threadIdx.x; idx < 16 * D; idx += NT) {
    const int k = idx / D, dim = idx % D;
    float Mx = kNegInf;
#pragma unroll
    for (int x = 0; x < NW; ++x) Mx = fmaxf(Mx, lds_m[x][k]);
    float acc = 0.0f;
#pragma unroll
    for (int x = 0; x < NW; ++x) acc = fmaf(rescale(lds_m[x][k], Mx), lds_o[x][k][dim], acc);
    fo[idx] = acc;
  }
  __syncthreads();
  finish_partition<dt, D, NT>(a, s, h0, nh, p, nparts, lds_fm, lds_fl, fo);
}

// ---- host launchers -----------------------------------------------------------------------

constexpr int kWaves = 4;          // waves per workgroup
// Prefetch depth and occupancy, measured on MI355X (13B-shape fp16 MHA and GQA bf16 batches):
// more blocks in flight per wave beat more waves per SIMD up to these depths.
constexpr int kValuBuffers = 4;    // VALU kernel: blocks in registers (NBUF-1 in flight)
// fp32 blocks of 8 or more loads per tensor (d = 64 with B = 32, d = 128 with B >= 16) take 3:
// four of them need more registers than a wave has and spill. The 16-bit B = 32 kernel keeps 4
// although it then runs one wave per SIMD: with 3 (two waves per SIMD) the shared-prefix step's
// decode took 174.9 against 169.9 us (measured on MI355X).
template <DT dt, int D, int BS>
constexpr int valu_buffers() {
  return (dt == DT::F32 && ValuCfg<dt, D, valu_unit_tokens<BS>(), kWaves>::NL >= 8)
             ? 3
             : kValuBuffers;
}
constexpr int kMfmaBuffers = 3;    // MFMA kernel: 32-token steps in registers
constexpr int kMfmaMinBlocks = 1;  // MFMA kernel: workgroups per CU the registers must allow

WorkspaceLayout workspace_layout(int num_seqs, int num_q_heads, int head_dim, int max_parts) {
  WorkspaceLayout L{};
  if (max_parts <= 1 || num_seqs <= 0) return L;  // a single partition needs no workspace
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t sh = (size_t)num_seqs * num_q_heads;
  L.m_off = 0;
  L.l_off = up(L.m_off + sh * max_parts * sizeof(float));
  L.o_off = up(L.l_off + sh * max_parts * sizeof(float));
  L.total = up(L.o_off + sh * max_parts * (size_t)head_dim * sizeof(float));
  return L;
}

int decode_units_per_seq(DecodePath path, int num_q_heads, int num_kv_heads) {
  if (path == DecodePath::Valu) return num_q_heads;
  const int g = num_q_heads / num_kv_heads;
  return num_kv_heads * ((g + 15) / 16);
}

template <int D, int BS>
static hipError_t launch_pf_valu_t(const PrefillArgs& a, hipStream_t stream) {
  const int64_t total = (int64_t)a.num_q_tokens * a.num_q_heads;
  if (total == 0) return hipSuccess;
  if (total > INT32_MAX) return hipErrorInvalidValue;  // the API checks this first
  PrefillArgs args_copy = a;
  void* args[] = {&args_copy};
  return hipLaunchKernel((const void*)prefill_valu_kernel<DT::F32, D, BS, kWaves>,
                         dim3((unsigned)total), dim3(kWaves * 64), args, 0, stream);
}

hipError_t launch_prefill_valu(int head_dim, int block_size, const PrefillArgs& a,
                               hipStream_t stream) {
  switch (head_dim * 100 + block_size) {
    case 6408: return launch_pf_valu_t<64, 8>(a, stream);
    case 6416: return launch_pf_valu_t<64, 16>(a, stream);
    case 6432: return launch_pf_valu_t<64, 32>(a, stream);
    case 6464: return launch_pf_valu_t<64, 64>(a, stream);
    case 12808: return launch_pf_valu_t<128, 8>(a, stream);
    case 12816: return launch_pf_valu_t<128, 16>(a, stream);
    case 12832: return launch_pf_valu_t<128, 32>(a, stream);
    case 12864: return launch_pf_valu_t<128, 64>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

int max_partition_tokens(DecodePath path, int block_size) {
  // every wave's unit (or step) ids must fit one register: kMaxPerWave per wave
  const int unit = block_size > 32 ? 16 : block_size;  // valu_unit_tokens
  return path == DecodePath::Valu ? kMaxPerWave * kWaves * unit : kMaxPerWave * kWaves * 32;
}

// Launches report their own status (hipLaunchKernel), never a stale error left by an earlier,
// unrelated runtime call.
template <DT dt, int D, int BS>
static hipError_t launch_t(DecodePath path, const DecodeArgs& a, hipStream_t stream) {
  const dim3 block(kWaves * 64);
  // Grid (partition, unit, sequence), partition fastest. Workgroups are dealt round-robin over
  // the 8 XCDs in order of their linear id p + gx * (unit + units * s), so an even gx would put
  // each partition index on a fixed subset of XCDs: with gx = 2 every sequence's first partition
  // ran on four of them, with gx = 4 on two (measured: 13B-shape batch split at 1024 / 512
  // tokens, 192 / 246 us instead of 156 us). An odd gx steps every (unit, sequence) through all
  // eight; the extra partition slot finds no work and returns at once.
  const unsigned gx = (unsigned)a.max_parts | 1u;
  const dim3 grid(gx, (unsigned)decode_units_per_seq(path, a.num_q_heads, a.num_kv_heads),
                  (unsigned)a.num_seqs);
  DecodeArgs args_copy = a;
  void* args[] = {&args_copy};
  const void* fn = nullptr;
  if (path == DecodePath::Mfma) {
    if constexpr (dt != DT::F32) {
      fn = (const void*)decode_mfma_kernel<dt, D, BS, kWaves, kMfmaBuffers, kMfmaMinBlocks>;
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    fn = (const void*)decode_valu_kernel<dt, D, BS, kWaves, valu_buffers<dt, D, BS>()>;
  }
  hipError_t e = hipLaunchKernel(fn, grid, block, args, 0, stream);
  if (e != hipSuccess || a.max_parts <= 1) return e;
  return hipLaunchKernel((const void*)merge_partitions_kernel<dt, D, BS>,
                         dim3((unsigned)a.num_q_heads, (unsigned)a.num_seqs), dim3(D), args, 0,
                         stream);
}

template <DT dt, int D>
static hipError_t launch_bs(DecodePath path, int bs, const DecodeArgs& a, hipStream_t st) {
  switch (bs) {
    case 8: return launch_t<dt, D, 8>(path, a, st);
    case 16: return launch_t<dt, D, 16>(path, a, st);
    case 32: return launch_t<dt, D, 32>(path, a, st);
    case 64: return launch_t<dt, D, 64>(path, a, st);
    default: return hipErrorInvalidValue;
  }
}

template <DT dt>
static hipError_t launch_d(DecodePath path, int d, int bs, const DecodeArgs& a, hipStream_t st) {
  switch (d) {
    case 64: return launch_bs<dt, 64>(path, bs, a, st);
    case 128: return launch_bs<dt, 128>(path, bs, a, st);
    default: return hipErrorInvalidValue;
  }
}

bool decode_supported(DecodePath path, int dt, int head_dim, int block_size) {
  if (dt < 0 || dt > 2) return false;
  if (head_dim != 64 && head_dim != 128) return false;
  if (block_size != 8 && block_size != 16 && block_size != 32 && block_size != 64) return false;
  if (path == DecodePath::Mfma && dt == 0) return false;
  return true;
}

hipError_t launch_decode(DecodePath path, int dt, int head_dim, int block_size,
                         const DecodeArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  switch (dt) {
    case 0: return launch_d<DT::F32>(path, head_dim, block_size, a, stream);
    case 1: return launch_d<DT::F16>(path, head_dim, block_size, a, stream);
    case 2: return launch_d<DT::BF16>(path, head_dim, block_size, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
