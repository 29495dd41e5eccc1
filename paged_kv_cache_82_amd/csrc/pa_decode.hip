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

// Tokens of a sequence of T (seq_len) read from the pool: all of them, or all but the newest
// when the call appends it (pa_decode_append).
__device__ __forceinline__ int pool_len(const DecodeArgs& a, int T) {
  return a.append ? (T > 0 ? T - 1 : 0) : T;
}

// Partitions of a sequence of T tokens: 0 for an empty sequence; with an appended token at
// least one, whose last partition folds the new token in.
__device__ __forceinline__ int parts_of(const DecodeArgs& a, int T) {
  const int P = a.partition_tokens;
  if (T == 0) return 0;
  const int n = (pool_len(a, T) + P - 1) / P;
  return n > 0 ? n : 1;
}

// The appended tokens' K and V rows of KV head kvh, every sequence's stored at new_slots[s]
// (as pa_write_kv would; nothing for a negative slot, one past the pool, or an empty sequence),
// in 16-byte chunks. A workgroup of the grid's last sequence slice does this: at the end of a
// decode workgroup the stores would hold it (and its CU slot) until they complete.
template <DT dt, int D, int NT>
__device__ void store_new_tokens(const DecodeArgs& a, int kvh, int BS) {
  constexpr int CH = D * Elem<dt>::bytes / 16;  // 16-byte chunks per row
  for (int64_t i = threadIdx.x; i < (int64_t)a.num_seqs * 2 * CH; i += NT) {
    const int s = (int)(i / (2 * CH));
    const int j = (int)(i % (2 * CH));
    const int slot = a.new_slots[s];
    if (slot < 0 || slot / BS >= a.num_blocks || seq_len(a, s, BS) == 0) continue;
    const bool v = j >= CH;
    const int c = v ? j - CH : j;
    const int64_t row = (((int64_t)(slot / BS) * a.num_kv_heads + kvh) * BS + slot % BS) * CH;
    const int64_t src = ((int64_t)s * a.num_kv_heads + kvh) * CH;
    const u32x4 x = reinterpret_cast<const u32x4*>(v ? a.v_new : a.k_new)[src + c];
    reinterpret_cast<u32x4*>(const_cast<void*>(v ? a.v_cache : a.k_cache))[row + c] = x;
  }
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
// Tokens of sequence s that its group's shared pass covers (shared-prefix decode): its prefix
// length within [0, T], rounded down to whole 32-token steps (the rest of the prefix is scored
// with the sequence's own tokens).
__device__ __forceinline__ int shared_len(const DecodeArgs& a, int s, int T) {
  int L = a.prefix_lens[s];
  L = L < 0 ? 0 : (L < T ? L : T);
  L = (L / 32) * 32;
  return L < a.max_shared ? L : a.max_shared;  // keeps every partial slot inside the workspace
}

// GROUP = false: sequence s is split into partitions of partition_tokens tokens. GROUP = true
// (shared-prefix decode): the partition count its workgroups recorded, kept within the
// workspace's slots.
template <DT dt, int D, int BS, bool GROUP>
__global__ __launch_bounds__(D) void merge_partitions_kernel(const DecodeArgs a) {
  const int h = blockIdx.x, s = blockIdx.y;
  int nparts;
  if constexpr (GROUP) {
    nparts = clampi(a.part_n[(int64_t)s * a.num_q_heads + h], 0, a.max_parts);
  } else {
    nparts = parts_of(a, seq_len(a, s, BS));
  }
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
  // L == 0: no partition saw a token (a column of the shared-prefix decode); the output is 0
  store_elem<dt>(a.out, ((int64_t)s * a.num_q_heads + h) * D + dim, L > 0.0f ? acc / L : 0.0f);
}

// ---- VALU kernel ------------------------------------------------------------------------

// Tokens a wave of the VALU kernels takes at once (a "unit"): the whole block up to 16 tokens;
// 16 tokens of a larger block, so that a unit's registers stay those of a 16-token block (two
// waves per SIMD for 16-bit data). Measured on MI355X with 32-token blocks, against whole-block
// units (one wave per SIMD): 13B-shape batch 154.4 against 160.6 us, unshared 64 x 1297-token
// batch 206.8 against 219.8 us.
template <int BS>
constexpr int valu_unit_tokens() {
  return BS > 16 ? 16 : BS;
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
  if (s == a.num_seqs) {  // the appended tokens' store slice (pa_decode_append only)
    const int g = a.num_q_heads / a.num_kv_heads;
    if (p == 0 && h % g == 0) store_new_tokens<dt, D, NT>(a, h / g, BS);
    return;
  }
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
  const int nparts = parts_of(a, T);
  if (T == 0) {
    if (p == 0) store_zeros<dt, D, NT>(a, s, h, 1);
    return;
  }
  if (p >= nparts) return;
  const int g = a.num_q_heads / a.num_kv_heads;
  const int kvh = h / g;
  const int Tp = pool_len(a, T);  // tokens read from the pool (an appended one is not)
  const int t0 = p * P;
  const int t1 = (Tp < t0 + P) ? Tp : t0 + P;
  const int jb1 = (t1 + SB - 1) / SB;

  float qf[VEC];
  {
    const uint32_t wq[4] = {qraw[0], qraw[1], qraw[2], qraw[3]};
#pragma unroll
    for (int e = 0; e < VEC; ++e) qf[e] = elem_of<dt>(wq, e) * a.scale_log2;
  }
  // An appended token (pa_decode_append): wave 0 of the last partition folds it into its
  // running state after its blocks, as one more token; its rows load now, in flight during the
  // loop. (The grid's last slice stores it in the pool.)
  const bool fold_new = a.append && p == nparts - 1 && w == 0;  // uniform per wave
  u32x4 kn_raw = {0u, 0u, 0u, 0u}, vn_raw = {0u, 0u, 0u, 0u};
  if (fold_new) {
    const int64_t row = (((int64_t)s * a.num_kv_heads + kvh) * D + c * VEC) * E;
    kn_raw = load16((const char*)a.k_new + row);
    vn_raw = load16((const char*)a.v_new + row);
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
  // oldest buffer. The round can stop part-way, which gives the loop a path back to its head
  // with slots still loading: the compiler waits for every load in flight there, once per
  // round. The form without that wait (whole rounds, then the last steps on their own, as in
  // the MFMA kernel) was 0.7% slower on the 13B-shape batch and no faster elsewhere (MI355X,
  // same box): at this kernel's load count the memory system is saturated, and the extra
  // requests in flight only queue.
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

  if (fold_new) {  // the appended token joins lane row 0 of wave 0
    const uint32_t wk[4] = {kn_raw[0], kn_raw[1], kn_raw[2], kn_raw[3]};
    const uint32_t wv[4] = {vn_raw[0], vn_raw[1], vn_raw[2], vn_raw[3]};
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc = fmaf(qf[e], elem_of<dt>(wk, e), acc);
    const float sn = group_sum<R>(acc);  // every lane row computes it; row 0 takes it
    if (r == 0) {
      const float mn = fmaxf(m, sn);
      const float corr = rescale(m, mn);
      const float pw = fast_exp2(sn - mn);
      l = fmaf(l, corr, pw);
#pragma unroll
      for (int e = 0; e < VEC; ++e) o[e] = fmaf(o[e], corr, pw * elem_of<dt>(wv, e));
      m = mn;
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

// One workgroup of the MFMA decode: NC tiles of 16 query columns (column 16c + hh, lane hh of
// tile c, reads its query row at qrow[c], null for an empty column) against the tokens of one
// table row `bt`, KV head kvh, in 32-token steps st0, st0 + 1, ... The block ids of at most
// max_steps steps are loaded first, with the queries; end_fn() then returns the token at which
// the workgroup's range ends, or -1 for no work (the workgroup returns; a range ending at token
// 32 * st0 has no step but still merges and stores its empty state). The workgroup's waves take
// the steps in turn, merge their (max, sum, output) states in LDS and hand the merged state of
// each column to store(fm, fl, fo) (fo: [16 NC][D]). Each K/V step is read once for all NC
// tiles.
// The LDS of one MFMA decode workgroup, declared once per kernel (a kernel may run the core
// from more than one place). A wave's output state for the merge, [16][D] floats, takes the
// place of its own K ring once its steps are done (no other wave touches that ring).
template <int D, int NW, int NBUF, int NC = 1>
struct MfmaSmem {
  __attribute__((aligned(1024))) char k[NW][NBUF][32 * D * 2];  // K ring, one per wave
  float m[NW][16 * NC], l[NW][16 * NC];
  float fm[16 * NC], fl[16 * NC];
  static_assert(16 * NC * D * sizeof(float) <= NBUF * 32 * D * 2, "an output state fits a ring");
  __device__ __forceinline__ float (*o(int w))[D] {
    return reinterpret_cast<float (*)[D]>(&k[w][0][0]);
  }
};

// One 32-token step of an MFMA decode workgroup, as its step source describes it: `index`
// (token / 32 of its first token; also its place in a block larger than a step), `valid` (the
// tokens of the step that count, from its start; past 32 all do) and the columns of the tile it
// serves, [clo, chi).
struct StepDesc {
  int index, valid, clo, chi;
};

// An appended token's K and V rows (pa_decode_append) for the workgroup's KV head, set by the
// step source's end function when this workgroup folds it in (null otherwise).
struct NewToken {
  const char* k = nullptr;
  const char* v = nullptr;
};

// Consecutive steps st0, st0 + 1, ... of one table row, up to the token end_fn() returns,
// every column; the wave takes steps st0 + w + k*NW.
template <int BS, int NW, class EndFn>
struct RangeSteps {
  static constexpr int NBS = BS >= 32 ? 1 : 32 / BS;
  static constexpr int SPB = BS > 32 ? BS / 32 : 1;
  static constexpr bool kAllColumns = true;
  const int32_t* bt;
  int st0, max_steps, max_blocks, w;
  EndFn end_fn;
  int t1 = 0, ns = 0;
  // Issued before the range's end is known, so the id, query and length loads overlap: lane k
  // takes the NBS block ids of this wave's k-th step (when inside the table).
  __device__ __forceinline__ void load_ids(int (&my_id)[NBS], int lane) const {
#pragma unroll
    for (int b = 0; b < NBS; ++b) {
      my_id[b] = 0;
      const int j = (st0 + w + lane * NW) * NBS / SPB + b;
      if (lane < (max_steps + NW - 1) / NW && j < max_blocks) my_id[b] = bt[j];
    }
  }
  // The range's end, after the id and query loads are issued; false: no work.
  __device__ __forceinline__ bool finalize() {
    // Uniform by construction; said so explicitly, because a value the callback returns past a
    // divergent loop (the zero stores of an empty sequence) is otherwise taken as per-lane, and
    // every buffer resource built from it would be loaded through a waterfall loop.
    t1 = __builtin_amdgcn_readfirstlane(end_fn());
    if (t1 < 0) return false;
    ns = t1 > 32 * st0 ? ((t1 + 31) / 32 - st0 - w + NW - 1) / NW : 0;
    if (ns < 0) ns = 0;
    return true;
  }
  __device__ __forceinline__ StepDesc step(int k) const {
    const int index = st0 + w + k * NW;
    return {index, t1 - 32 * index, 0, 16};
  }
};

// A step list given per lane: lane k describes the wave's k-th step (its table row, its token
// index, and `meta` = valid << 10 | clo << 5 | chi); ns steps.
template <int BS>
struct ListSteps {
  static constexpr int NBS = BS >= 32 ? 1 : 32 / BS;
  static constexpr int SPB = BS > 32 ? BS / 32 : 1;
  static constexpr bool kAllColumns = false;
  const int32_t* row;  // lane k: the step's table row (null past the wave's steps)
  int index, meta, ns, max_blocks;
  __device__ __forceinline__ void load_ids(int (&my_id)[NBS], int lane) const {
#pragma unroll
    for (int b = 0; b < NBS; ++b) {
      my_id[b] = 0;
      const int j = index * NBS / SPB + b;
      if (row && j < max_blocks) my_id[b] = row[j];
    }
  }
  // Never an early return: ns is per wave, and a wave with no step must still hand its empty
  // state to the workgroup's merge (the caller returns for a workgroup with no step at all).
  __device__ __forceinline__ bool finalize() const { return true; }
  __device__ __forceinline__ StepDesc step(int k) const {
    const int mk = __builtin_amdgcn_readlane(meta, k);
    return {__builtin_amdgcn_readlane(index, k), mk >> 10, (mk >> 5) & 31, mk & 31};
  }
};

template <DT dt, int D, int BS, int NW, int NBUF, int NC, class Steps, class StoreFn>
__device__ __forceinline__ void mfma_decode_run(MfmaSmem<D, NW, NBUF, NC>& sm,
                                                const DecodeArgs& a, int kvh,
                                                const char* const (&qrow)[NC], Steps& steps,
                                                StoreFn store, const NewToken& nt = NewToken{}) {
  static_assert(dt != DT::F32, "MFMA path takes 16-bit inputs");
  static_assert(NC == 1 || Steps::kAllColumns, "per-step column ranges take one tile");
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
  auto& lds_k = sm.k;
  auto& lds_m = sm.m;
  auto& lds_l = sm.l;
  auto& lds_fm = sm.fm;
  auto& lds_fl = sm.fl;

  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int hh = lane & 15, gq = lane >> 4;

  int my_id[NBS];
  steps.load_ids(my_id, lane);
  // Q^T operand of tile c: column 16c + hh, k = head dims 32*kk + 8*gq + e.
  vec8 qop[NC][KC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (qrow[c]) raw = load16(qrow[c] + (32 * kk + 8 * gq) * E);
      qop[c][kk] = __builtin_bit_cast(vec8, raw);
    }
  if (!steps.finalize()) return;  // a step source returns false for the whole workgroup only
  // An appended token: wave 0 folds it in after its steps; its rows load now. K as the Q^T
  // operand's head dims (32kk + 8gq ..), V as the output's (MT (4gq + i) .. + MT - 1).
  using VT = typename VF::T;
  const bool fold_new = nt.k != nullptr && wave_id() == 0;  // uniform per wave
  u32x4 kn[KC];
  VT vn[4];
#pragma unroll
  for (int kk = 0; kk < KC; ++kk) kn[kk] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 4; ++i) vn[i] = VT{};
  if (fold_new) {
    const int gq0 = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) kn[kk] = load16(nt.k + (32 * kk + 8 * gq0) * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      vn[i] = *reinterpret_cast<const VT*>(nt.v + (D / 16) * (4 * gq0 + i) * 2);
  }

  f32x4 oacc[NC][MT];
  // Running state per column: reference maximum m (base 2), the shift nm = -m (0 while m is
  // -inf), the row sum and the output, all relative to m.
  float m[NC], nm[NC], lsum[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) oacc[c][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[c] = kNegInf;
    nm[c] = 0.0f;
    lsum[c] = 0.0f;
  }

  // This wave's steps k < ns; lane k holds the NBS physical ids of step k.
  const int ns = steps.ns;
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
    const StepDesc sd = steps.step(kq);
    // Blocks larger than a step: the step's 32 rows start (index % SPB) * 32 rows into its block,
    // and its resources span those rows only.
    constexpr int span = BS > 32 ? 32 * RB : (int)(BS * RB);
    __amdgpu_buffer_rsrc_t kr[NBS];
    int64_t tile[NBS];
    bool has[NBS];
#pragma unroll
    for (int b = 0; b < NBS; ++b) {
      const int id = clamp_id(__builtin_amdgcn_readlane(my_id[b], kq), id_max);
      tile[b] = (int64_t)id * blk_stride;
      if constexpr (SPB > 1) tile[b] += (int64_t)((sd.index % SPB) * span);
      has[b] = live && b * BS < sd.valid;  // the block holds a token the step uses
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

  // waitc: loads that may still be in flight once this step's K loads (and every load issued
  // before them) are done: its own 8 V loads and those of the fetches issued after it (8 V and
  // KD K loads each).
  auto consume = [&](int k, auto slotc, VRegs<D>& R, auto waitc) {
    constexpr int slot = decltype(slotc)::value;
    const StepDesc sd = steps.step(k);
    // token r of the step counts for this lane's column: r < valid, and the column is served
    const bool col_ok = Steps::kAllColumns || (hh >= sd.clo && hh < sd.chi);
    wait_vmcnt<decltype(waitc)::value>();
    u32x4 kf[2][KC];
    lds_read_k<slot * KSTEP, 16 * RB>(kf, ka);
    // S^T = K Q^T: sacc[c][u][i] = score of token tau0 + 16u + 4*gq + i for column 16c + hh;
    // 2 NC independent accumulation chains.
    f32x4 sacc[NC][2];
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int u = 0; u < 2; ++u) sacc[c][u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KC; ++kk)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int c = 0; c < NC; ++c)
          sacc[c][u] = M::mma(__builtin_bit_cast(vec8, kf[u][kk]), qop[c][kk], sacc[c][u]);
    const bool tail = sd.valid < 32 || (!Steps::kAllColumns && (sd.clo > 0 || sd.chi < 16));
    // Weights are taken against a reference maximum m[c] (base 2) that is raised only when a
    // score passes it by more than kSlack: weights stay below 2^kSlack, and the running sum and
    // the output share the reference, so the normalised result is that of the exact running
    // maximum. In most steps neither the maximum's lane shuffles nor the rescale of the output
    // accumulators (held in AGPRs: a read, a multiply and a write each) run.
    float sc[NC][8], lm[NC];
    bool raise = false;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = sacc[c][u][i] * a.scale_log2;
          if (tail && (16 * u + 4 * gq + i >= sd.valid || !col_ok)) x = kNegInf;
          sc[c][4 * u + i] = x;
        }
      float x = sc[c][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) x = fmaxf(x, sc[c][e]);
      lm[c] = x;
      raise = raise || (x > m[c] + kSlack);  // m = -inf: any finite score raises
    }
    if (__builtin_amdgcn_ballot_w64(raise)) {  // uniform; rare once the maxima settle
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        float bm = fmaxf(lm[c], __shfl_xor(lm[c], 16));
        bm = fmaxf(bm, __shfl_xor(bm, 32));
        const float mn = fmaxf(m[c], bm);
        const float corr = rescale(m[c], mn);  // 0 while m is -inf (nothing accumulated yet)
        lsum[c] *= corr;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) oacc[c][mt] *= corr;
        m[c] = mn;
        // m stays -inf only while every score of the column was -inf; the shift is 0 then,
        // and the weights exp2(-inf) = 0
        nm[c] = mn == kNegInf ? 0.0f : -mn;
      }
    }
    vec8 pop[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float pe[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pe[e] = fast_exp2(sc[c][e] + nm[c]);
      const u32x4 pw = {pack2<dt>(pe[0], pe[1]), pack2<dt>(pe[2], pe[3]),
                        pack2<dt>(pe[4], pe[5]), pack2<dt>(pe[6], pe[7])};
      // The weights are rounded to 16 bits for the p.V MFMA; the row sum adds those same
      // rounded weights (dot2 of each packed pair with (1, 1)), so numerator and denominator
      // agree.
#pragma unroll
      for (int j = 0; j < 4; ++j) lsum[c] = sum2<dt>(pw[j], lsum[c]);
      pop[c] = __builtin_bit_cast(vec8, pw);
    }
    if (tail) {  // V rows past the step's valid tokens may hold anything, NaN included
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (16 * u + 4 * gq + i >= sd.valid) R.v[u][i] = typename VF::T{};  // select
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
#pragma unroll
      for (int c = 0; c < NC; ++c)
        oacc[c][mt] = M::mma(__builtin_bit_cast(vec8, vw), pop[c], oacc[c][mt]);
    }
  };

  if (ns > 0) {  // rings of NBUF slots, unconditional prefetch (see the VALU kernel)
    VRegs<D> rb[NBUF];
    static_for<NBUF - 1>([&](auto uc) { fetch(decltype(uc)::value, uc, rb[decltype(uc)::value]); });
    // Every slot index is a constant: step k uses slot k % NBUF. In whole rounds NBUF - 1
    // fetches follow a step's; in the last ns % NBUF steps (u = k % NBUF), which fetch nothing,
    // NBUF - 2 - u.
    ring_loop<NBUF>(
        ns,
        [&](int k, auto uc) {
          constexpr int u = decltype(uc)::value;
          constexpr int ahead = (u + NBUF - 1) % NBUF;
          fetch(k + NBUF - 1, std::integral_constant<int, ahead>{}, rb[ahead]);
          consume(k, uc, rb[u], std::integral_constant<int, (NBUF - 1) * (8 + KD) + 8>{});
        },
        [&](int k, auto uc) {
          constexpr int u = decltype(uc)::value;
          consume(k, uc, rb[u], std::integral_constant<int, (NBUF - 2 - u) * (8 + KD) + 8>{});
        });
  }

  if (fold_new) {  // the appended token, one more token of every column of wave 0
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float part = 0.0f;
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) {
        const u32x4 qw = __builtin_bit_cast(u32x4, qop[c][kk]);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          part = fmaf(widen16<dt>(qw[e / 2], e & 1), widen16<dt>(kn[kk][e / 2], e & 1), part);
      }
      part += __shfl_xor(part, 16);
      part += __shfl_xor(part, 32);
      const float sn = part * a.scale_log2;
      const float mn = fmaxf(m[c], sn);
      const float corr = rescale(m[c], mn);
      const float pw = fast_exp2(sn - mn);
      lsum[c] = fmaf(lsum[c], corr, gq == 0 ? pw : 0.0f);  // lsum is summed over gq below
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          oacc[c][mt][i] = fmaf(oacc[c][mt][i], corr,
                                pw * widen16<dt>(vfrag_elem<D>(vn[i], mt), 0));
      m[c] = mn;
    }
  }

  // Sum the per-lane partial sums over the four lane groups of each head.
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    lsum[c] += __shfl_xor(lsum[c], 16);
    lsum[c] += __shfl_xor(lsum[c], 32);
  }
  // oacc[c][mt][i] is O[column 16c + hh][dim MT*(4*gq + i) + mt]. It goes where this wave's K
  // ring was: first every load the wave issued must have landed (prefetches past its last step
  // included, whose LDS loads write zeros).
  wait_vmcnt<0>();
  float (*const my_o)[D] = sm.o(w);
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) my_o[16 * c + hh][MT * (4 * gq + i) + mt] = oacc[c][mt][i];
  if (gq == 0) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      lds_m[w][16 * c + hh] = m[c];
      lds_l[w][16 * c + hh] = lsum[c];
    }
  }
  __syncthreads();
  if (threadIdx.x < 16 * NC) {
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
  float* fo = &sm.o(0)[0][0];  // merged output reuses wave 0's slab (read-before-write)
  for (int idx = threadIdx.x; idx < 16 * NC * D; idx += NT) {
    const int k = idx / D, dim = idx % D;
    float Mx = kNegInf;
#pragma unroll
    for (int x = 0; x < NW; ++x) Mx = fmaxf(Mx, lds_m[x][k]);
    float acc = 0.0f;
#pragma unroll
    for (int x = 0; x < NW; ++x) acc = fmaf(rescale(lds_m[x][k], Mx), sm.o(x)[k][dim], acc);
    fo[idx] = acc;
  }
  __syncthreads();
  store(lds_fm, lds_fl, fo);
}

// NC = 2 (groups of more than 16 query heads): a workgroup takes 32 heads of one KV head, two
// column tiles fed by each K/V step.
template <DT dt, int D, int BS, int NW, int NBUF, int MINB, int NC>
__global__ __launch_bounds__(NW * 64, MINB) void decode_mfma_kernel(const DecodeArgs a) {
  constexpr int NT = NW * 64;
  constexpr int CW = 16 * NC;  // query heads per workgroup
  int p = blockIdx.x, unit = blockIdx.y;
  int s = blockIdx.z;
  const int Hq = a.num_q_heads;
  const int g = Hq / a.num_kv_heads;
  const int ntile = (g + CW - 1) / CW;
  if (s == a.num_seqs) {  // the appended tokens' store slice (pa_decode_append only)
    if (p == 0 && unit % ntile == 0) store_new_tokens<dt, D, NT>(a, unit / ntile, BS);
    return;
  }
  if (ntile > 1) {
    // More query heads per KV head than one workgroup takes: the ntile head tiles of one
    // (partition, KV head, sequence) read the same K/V tiles. The hardware deals workgroups
    // round-robin over the 8 XCDs by linear id, so the tiles take consecutive slots on one XCD:
    // they run side by side and the second reader finds the lines in that XCD's L2. Ids past
    // the last whole round of 8 * ntile keep a plain order.
    const int64_t gx = gridDim.x, units = gridDim.y;
    const int64_t L = blockIdx.x + gx * (blockIdx.y + units * blockIdx.z);
    const int64_t span = 8 * (int64_t)ntile;
    const int64_t full = gx * units * a.num_seqs / span * span;
    int64_t W;  // work index over (partition, KV head, sequence)
    int ht;
    if (L < full) {
      const int64_t slot = L / 8;
      ht = (int)(slot % ntile);
      W = (slot / ntile) * 8 + L % 8;
    } else {
      ht = (int)((L - full) % ntile);
      W = full / ntile + (L - full) / ntile;
    }
    p = (int)(W % gx);
    const int64_t rest = W / gx;
    const int Hkv = a.num_kv_heads;
    unit = (int)(rest % Hkv) * ntile + ht;
    s = (int)(rest / Hkv);
  }
  const int kvh = unit / ntile, ht = unit % ntile;
  const int h0 = kvh * g + ht * CW;
  const int nh = (g - ht * CW < CW) ? g - ht * CW : CW;
  const int P = a.partition_tokens;
  const int hh = threadIdx.x & 15;
  // column 16c + hh = query head h0 + 16c + hh of sequence s
  const char* qrow[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c)
    qrow[c] = 16 * c + hh < nh
                  ? (const char*)a.q + ((int64_t)s * Hq + h0 + 16 * c + hh) * D * 2
                  : nullptr;
  int nparts = 0;
  __shared__ MfmaSmem<D, NW, NBUF, NC> sm;
  NewToken nt;
  auto end_fn = [&]() -> int {
    const int T = seq_len(a, s, BS);
    nparts = parts_of(a, T);
    if (T == 0) {
      if (p == 0) store_zeros<dt, D, NT>(a, s, h0, nh);
      return -1;
    }
    if (p >= nparts) return -1;
    if (a.append && p == nparts - 1) {  // the last partition takes the appended token
      const int64_t row = ((int64_t)s * a.num_kv_heads + kvh) * D * 2;
      nt.k = (const char*)a.k_new + row;
      nt.v = (const char*)a.v_new + row;
    }
    const int Tp = pool_len(a, T);  // the pool part; an appended token is folded in after it
    return (Tp < (p + 1) * P) ? Tp : (p + 1) * P;
  };
  RangeSteps<BS, NW, decltype(end_fn)> steps{a.block_tables + (int64_t)s * a.max_blocks_per_seq,
                                             p * (P / 32), P / 32, a.max_blocks_per_seq,
                                             wave_id(), end_fn};
  mfma_decode_run<dt, D, BS, NW, NBUF, NC>(
      sm, a, kvh, qrow, steps, [&](float* fm, float* fl, float* fo) {
        finish_partition<dt, D, NT>(a, s, h0, nh, p, nparts, fm, fl, fo);
      }, nt);

}

// ---- shared-prefix decode ------------------------------------------------------------------
// [PA-summary] "Memory sharing: copy-on-write for parallel decoding": the samples of one prompt
// hold the prompt's blocks by reference, so the same K/V tiles serve every sample. Against one
// such tile the members' query heads form a dense [members*g x d] . [d x B] contraction: one
// MFMA column per (member, query head). A workgroup serves one (group, KV head, 16-column tile)
// and walks a list of 32-token steps: the group's shared prefix through the first member's table
// (every column), then each member's own tokens through its own table (that member's columns
// only; the others take -inf scores and are left unchanged by the rescaled update). Every
// column's running (max, sum, output) state simply continues from one part of the list to the
// next, so a list that fits one workgroup needs no partials and no merge. Longer lists are cut
// into partitions whose partials the merge kernel combines.

// The merged state of a group workgroup: column k is (member c / g, query head c % g of KV head
// kvh), c = 16*ct + k. With one partition the final output (0 for a column that saw no token);
// otherwise a partial in slot p. Partition 0 records the partition count for the merge.
template <DT dt, int D, int NT>
__device__ void finish_group(const DecodeArgs& a, int s0, int ncols, int ct, int kvh, int p,
                             int nparts, const float* fm, const float* fl, const float* fo) {
  const int Hq = a.num_q_heads, g = Hq / a.num_kv_heads;
  const int nk = ncols - 16 * ct < 16 ? ncols - 16 * ct : 16;
  const int tid = threadIdx.x;
  const int MP = a.max_parts;
  for (int idx = tid; idx < nk * D; idx += NT) {
    const int k = idx / D, dim = idx % D;
    const int c = 16 * ct + k;
    const int64_t row = (int64_t)(s0 + c / g) * Hq + kvh * g + c % g;
    if (nparts == 1)
      store_elem<dt>(a.out, row * D + dim, fl[k] > 0.0f ? fo[idx] / fl[k] : 0.0f);
    else
      a.part_o[(row * MP + p) * D + dim] = fo[idx];
  }
  if (tid < nk) {
    const int c = 16 * ct + tid;
    const int64_t row = (int64_t)(s0 + c / g) * Hq + kvh * g + c % g;
    if (nparts > 1) {
      a.part_m[row * MP + p] = fm[tid];
      a.part_l[row * MP + p] = fl[tid];
    }
    if (p == 0 && a.part_n) a.part_n[row] = nparts;
  }
}

template <DT dt, int D, int BS, int NW, int NBUF, int MINB>
__global__ __launch_bounds__(NW * 64, MINB) void decode_group_kernel(const DecodeArgs a) {
  constexpr int NT = NW * 64;
  __shared__ MfmaSmem<D, NW, NBUF> sm;
  // grid: (partition, KV head x column tile, group), partition fastest, with an odd partition
  // count in the grid (the launcher's npg; see launch_t): slot p == np finds no work
  const int64_t L = blockIdx.x;
  const int np = a.group_parts;
  const int npg = np > 1 ? (np | 1) : 1;
  const int p = (int)(L % npg);
  if (p >= np) return;  // uniform
  const int64_t rest = L / npg;
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  const int g = Hq / Hkv;
  const int units = Hkv * a.shared_ctiles;
  const int unit = (int)(rest % units);
  const int gi = (int)(rest / units);
  const int kvh = unit / a.shared_ctiles, ct = unit % a.shared_ctiles;
  const int S = a.num_seqs;
  const int s0 = clampi(a.group_start[gi], 0, S);
  const int s1 = clampi(a.group_start[gi + 1], s0, S);
  const int ncols = (s1 - s0) * g;
  if (16 * ct >= ncols) return;  // uniform: the tile serves no column
  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int hh = lane & 15;
  // Members with a column in this tile: m0 .. m1 - 1, at most 16.
  const int m0 = (16 * ct) / g;
  const int m1 = (s1 - s0) < (16 * ct + 15) / g + 1 ? (s1 - s0) : (16 * ct + 15) / g + 1;
  const int nm = m1 - m0;
  // Lane j < nm: member m0 + j's length and its own steps; the shared prefix from the first
  // member (whole 32-token steps).
  const int Tj = lane < nm ? seq_len(a, s0 + m0 + lane, BS) : 0;
  const int Lg = shared_len(a, s0, seq_len(a, s0, BS));
  const int nS = Lg / 32;
  const int nPj = (lane < nm && Tj > Lg) ? (Tj - Lg + 31) / 32 : 0;
  // offj: first step of member j's own tokens in the list (lane j); total: the list's length
  int offj = nS, total = nS;
  for (int j = 0; j < nm; ++j) {  // uniform, at most 16
    const int nj = __builtin_amdgcn_readlane(nPj, j);
    if (lane == j) offj = total;
    total += nj;
  }
  // Uniform by construction; said so, because the loop that sums it also takes a per-lane
  // branch, after which the compiler takes it as per-lane (and would load every buffer
  // resource built from it through a waterfall loop).
  total = __builtin_amdgcn_readfirstlane(total);
  const int SP = a.group_steps;
  const int nparts = (total + SP - 1) / SP < np ? (total + SP - 1) / SP : np;
  const int c = 16 * ct + hh;
  if (total == 0) {  // no token in the whole tile (every member empty): zero outputs
    if (p == 0) {
      const int nk = ncols - 16 * ct < 16 ? ncols - 16 * ct : 16;
      for (int idx = threadIdx.x; idx < nk * D; idx += NT) {
        const int k = idx / D, cc = 16 * ct + k;
        store_elem<dt>(a.out, ((int64_t)(s0 + cc / g) * Hq + kvh * g + cc % g) * D + idx % D,
                       0.0f);
      }
      if (threadIdx.x < nk && a.part_n) {
        const int cc = 16 * ct + threadIdx.x;
        a.part_n[(int64_t)(s0 + cc / g) * Hq + kvh * g + cc % g] = 1;
      }
    }
    return;
  }
  const int pbeg = p * SP;
  const int pend = total < pbeg + SP ? total : pbeg + SP;
  if (pbeg >= pend) return;  // uniform: a partition past the list
  // Lane k: the wave's k-th step of this partition, list position pbeg + w + k*NW.
  const int gs = pbeg + w + lane * NW;
  const int M = a.max_blocks_per_seq;
  // The member whose own tokens hold list position gs (the last one starting at or before it;
  // members with no own tokens share their start with the next), found by every lane in uniform
  // control flow so that the lane shuffle reads only active lanes.
  int jj = 0, off = nS;
  for (int j = 0; j < nm; ++j) {  // uniform loop, per-lane choice
    const int oj = __builtin_amdgcn_readlane(offj, j);
    if (gs >= oj) {
      jj = j;
      off = oj;
    }
  }
  const int Tjj = __shfl(Tj, jj);
  const int32_t* row = nullptr;
  int index = 0, meta = 0;
  if (gs < pend) {
    if (gs < nS) {  // the shared prefix: every column
      row = a.block_tables + (int64_t)s0 * M;
      index = gs;
      meta = (32 << 10) | (0 << 5) | 16;
    } else {  // member jj's own tokens: its columns only
      const int tau0 = Lg + 32 * (gs - off);
      const int valid = Tjj - tau0 < 32 ? Tjj - tau0 : 32;
      const int lo = (m0 + jj) * g - 16 * ct, hi = lo + g;
      row = a.block_tables + (int64_t)(s0 + m0 + jj) * M;
      index = tau0 / 32;
      meta = (valid << 10) | ((lo > 0 ? lo : 0) << 5) | (hi < 16 ? hi : 16);
    }
  }
  ListSteps<BS> steps{row, index, meta, (pend - pbeg - w + NW - 1) / NW, M};
  if (steps.ns < 0) steps.ns = 0;
  const char* const qrow[1] = {
      c < ncols ? (const char*)a.q + ((int64_t)(s0 + c / g) * Hq + kvh * g + c % g) * D * 2
                : nullptr};
  mfma_decode_run<dt, D, BS, NW, NBUF, 1>(
      sm, a, kvh, qrow, steps, [&](float* fm, float* fl, float* fo) {
        finish_group<dt, D, NT>(a, s0, ncols, ct, kvh, p, nparts, fm, fl, fo);
      });
}

// ---- host launchers -----------------------------------------------------------------------

constexpr int kWaves = 4;          // waves per workgroup
// Prefetch depth and occupancy, measured on MI355X (13B-shape fp16 MHA and GQA bf16 batches):
// more blocks in flight per wave beat more waves per SIMD up to these depths.
constexpr int kValuBuffers = 4;    // VALU kernel: blocks in registers (NBUF-1 in flight)
// fp32 units of 8 or more loads per tensor (d = 128) take 3: four of them need more registers
// than a wave has and spill. Units of one or two loads per tensor (8-token blocks, or d = 64 at
// 16-bit) take 8, so that a wave keeps about as many bytes in flight as with 4-load units:
// measured on MI355X, the 13B-shape batch with 8-token blocks went from 168.5 to 157.7 us, and
// 64-dim batches by 1.5% (10 or 12 buffers were slower).
template <DT dt, int D, int BS>
constexpr int valu_buffers() {
  constexpr int NL = ValuCfg<dt, D, valu_unit_tokens<BS>(), kWaves>::NL;
  return (dt == DT::F32 && NL >= 8) ? 3 : NL <= 2 ? 8 : kValuBuffers;
}
constexpr int kMfmaBuffers = 3;    // MFMA kernel: 32-token steps in registers
constexpr int kMfmaMinBlocks = 1;  // MFMA kernel: workgroups per CU the registers must allow
// The shared-prefix (group) kernel runs two workgroups per CU with two steps per wave in its
// rings (66 KB of LDS, 188 VGPRs): its workgroups are fewer and shorter, and a second one on the
// CU covers a first one's start and merge. Measured on MI355X, shared-prefix step (16 prompts x
// 4 samples): 89.9 against 95.2 us with the MFMA kernel's three steps and one workgroup per CU.
// The same change made the GQA batch's MFMA kernel slower (364.6 against 352.2 us).
constexpr int kGroupBuffers = 2;
constexpr int kGroupMinBlocks = 2;

WorkspaceLayout workspace_layout(int num_seqs, int num_q_heads, int head_dim, int max_parts,
                                 bool with_counts) {
  WorkspaceLayout L{};
  if (max_parts <= 1 || num_seqs <= 0) return L;  // a single partition needs no workspace
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t sh = (size_t)num_seqs * num_q_heads;
  L.m_off = 0;
  L.l_off = up(L.m_off + sh * max_parts * sizeof(float));
  L.o_off = up(L.l_off + sh * max_parts * sizeof(float));
  L.n_off = up(L.o_off + sh * max_parts * (size_t)head_dim * sizeof(float));
  L.total = with_counts ? up(L.n_off + sh * sizeof(int32_t)) : L.n_off;
  return L;
}

// Query heads one MFMA workgroup takes: 16 (one column tile), or 32 (two tiles fed by each K/V
// step) when a KV head has more than 16.
static int mfma_heads_per_workgroup(int g) { return g > 16 ? 32 : 16; }

int decode_units_per_seq(DecodePath path, int num_q_heads, int num_kv_heads) {
  if (path == DecodePath::Valu) return num_q_heads;
  const int g = num_q_heads / num_kv_heads;
  const int cw = mfma_heads_per_workgroup(g);
  return num_kv_heads * ((g + cw - 1) / cw);
}

int max_partition_tokens(DecodePath path, int block_size) {
  // every wave's unit (or step) ids must fit one register: kMaxPerWave per wave
  const int unit = block_size > 16 ? 16 : block_size;  // valu_unit_tokens
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
  // pa_decode_append: one more sequence slice, dispatched last, stores the appended tokens
  const dim3 grid(gx, (unsigned)decode_units_per_seq(path, a.num_q_heads, a.num_kv_heads),
                  (unsigned)(a.num_seqs + (a.append ? 1 : 0)));
  DecodeArgs args_copy = a;
  void* args[] = {&args_copy};
  const void* fn = nullptr;
  if (path == DecodePath::Mfma) {
    if constexpr (dt != DT::F32) {
      fn = mfma_heads_per_workgroup(a.num_q_heads / a.num_kv_heads) == 32
               ? (const void*)decode_mfma_kernel<dt, D, BS, kWaves, kMfmaBuffers, kMfmaMinBlocks, 2>
               : (const void*)decode_mfma_kernel<dt, D, BS, kWaves, kMfmaBuffers, kMfmaMinBlocks, 1>;
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    fn = (const void*)decode_valu_kernel<dt, D, BS, kWaves, valu_buffers<dt, D, BS>()>;
  }
  hipError_t e = hipLaunchKernel(fn, grid, block, args, 0, stream);
  if (e != hipSuccess || a.max_parts <= 1) return e;
  return hipLaunchKernel((const void*)merge_partitions_kernel<dt, D, BS, false>,
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

template <DT dt, int D, int BS>
static hipError_t launch_shared_t(const DecodeArgs& a, hipStream_t stream) {
  // An odd partition count per (group, KV head, column tile) in the grid, as launch_t pads
  // it, so that one partition index does not land on a fixed subset of the XCDs (measured on
  // MI355X, shared-prefix step forced to 2048-token partitions: 210.8 us with two).
  const int64_t npg = a.group_parts > 1 ? (a.group_parts | 1) : 1;
  const int64_t total = (int64_t)a.num_groups * a.num_kv_heads * a.shared_ctiles * npg;
  if (total == 0) return hipSuccess;
  if (total > 0xffffffffLL) return hipErrorInvalidValue;  // the API checks this first
  DecodeArgs args_copy = a;
  void* args[] = {&args_copy};
  hipError_t e = hipLaunchKernel(
      (const void*)decode_group_kernel<dt, D, BS, kWaves, kGroupBuffers, kGroupMinBlocks>,
      dim3((unsigned)total), dim3(kWaves * 64), args, 0, stream);
  if (e != hipSuccess || a.max_parts <= 1) return e;
  return hipLaunchKernel((const void*)merge_partitions_kernel<dt, D, BS, true>,
                         dim3((unsigned)a.num_q_heads, (unsigned)a.num_seqs), dim3(D), args, 0,
                         stream);
}

template <DT dt, int D>
static hipError_t launch_shared_bs(int bs, const DecodeArgs& a, hipStream_t st) {
  switch (bs) {
    case 8: return launch_shared_t<dt, D, 8>(a, st);
    case 16: return launch_shared_t<dt, D, 16>(a, st);
    case 32: return launch_shared_t<dt, D, 32>(a, st);
    case 64: return launch_shared_t<dt, D, 64>(a, st);
    default: return hipErrorInvalidValue;
  }
}

template <DT dt>
static hipError_t launch_shared_d(int d, int bs, const DecodeArgs& a, hipStream_t st) {
  switch (d) {
    case 64: return launch_shared_bs<dt, 64>(bs, a, st);
    case 128: return launch_shared_bs<dt, 128>(bs, a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_shared(int dt, int head_dim, int block_size, const DecodeArgs& a,
                                hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  switch (dt) {
    case 1: return launch_shared_d<DT::F16>(head_dim, block_size, a, stream);
    case 2: return launch_shared_d<DT::BF16>(head_dim, block_size, a, stream);
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
