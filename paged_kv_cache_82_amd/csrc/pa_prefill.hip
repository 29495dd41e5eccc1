// pa_prefill.hip — causal multi-query (prefill / chunked-prefill) paged attention for gfx950.
//
// Method: [PA-summary] azimuth.plus, "Efficient Memory Management for Large Language Model
// Serving with PagedAttention", section "The PagedAttention algorithm": for each query vector
// the kernel walks the block table, fetches each logical block's keys and values from wherever
// its physical block sits and folds them into a running (maximum, sum, output) state with the
// log-sum-exp rescaling of the block-wise equation. Here a sequence brings n new tokens at once
// (a prompt, or a chunk of one); they are the last n of its T cached tokens and each is a query
// vector. Query i sits at position T - n + i and attends to positions 0 .. T - n + i (the
// causal rule; a decode step is the case n = 1).
//
// With many query vectors per KV head the scores of a 32-token step are a dense contraction, so
// both products run on 16x16x32 MFMA, in the transposed form the decode kernel uses
// (pa_mfma.h): S^T = K Q^T with tokens on rows and query rows on columns, then
// O^T += V^T P^T. Work decomposition (chosen for MI355X, not on the pages):
//   - query rows are (query token, grouped head) pairs, head fastest, so one KV tile feeds all
//     query heads of its group; a workgroup of NW waves covers NW * NCT * 16 consecutive rows,
//     each wave NCT adjacent 16-row column tiles, so that a wave's rows span few positions and
//     few of its stages need the causal mask;
//   - the workgroup walks its context in 32-token stages: each wave loads 8 rows of the
//     stage's K and V (rows of one block, found through the block table) straight from HBM
//     into LDS (buffer loads into LDS), with two stages in flight while one is consumed; one
//     barrier per stage;
//   - LDS rows are XOR-swizzled in 16-byte chunks so that the MFMA operand reads (16 rows at
//     one column for K, one row for V) hit distinct banks;
//   - each wave reads a stage's K and V fragments once from LDS and uses them for all its
//     column tiles (their MFMA chains interleave); only stages that reach past the first
//     position of one of the wave's tiles (the causal diagonal, and the workgroup's tail) take
//     the masked path, every other stage runs without any per-score test;
//   - a wave's physical block ids come 64 stages at a time into one register (lane k = stage
//     k) and are broadcast with readlane;
//   - workgroups are dealt round-robin over the 8 XCDs; (sequence, KV head) groups are spread
//     over the XCDs so that each gets a share of every sequence, and the row tiles of one group
//     run on one XCD, heaviest (latest) first, sharing its L2.
// Scores are kept in the base-2 exponent domain: s' = s * log2(e), exp(s - m) = 2^(s' - m').
#include <utility>

#include "pa_device.h"
#include "pa_internal.h"
#include "pa_mfma.h"

namespace pa {

namespace {

constexpr int kPrefillWaves = 4;     // waves per workgroup
constexpr int kPrefillColTiles = 2;  // 16-row column tiles per wave
constexpr int kPrefillStages = 3;    // LDS stage buffers (stages in flight + the one consumed)
constexpr int kXcds = 8;             // MI355X: workgroups are dealt round-robin over 8 XCDs

// The V^T operand of the p.V product comes from ds_read_b64_tr_b16: inside each aligned group
// of 16 lanes, lane 4q + p receives element p of the 8-byte chunks addressed by lanes q,
// q + 4, q + 8 and q + 12 (in that order). The reads are issued from one asm block that also
// waits for them: the compiler treats the intrinsic as possibly reading the LDS that the
// stage loads (LDS DMA) are still writing and would drain every load in flight before it.
// va[mt] is the lane's LDS byte address for M-tile mt (of the half of the head dimension being
// read) and token tile u = 0 of stage buffer 0; OFF0 / OFF1 are the byte offsets of the stage
// buffer's token tiles 0 and 1.
template <int OFF0, int OFF1>
__device__ __forceinline__ void lds_read_vt(u32x2 (&t)[4][2], const uint32_t (&va)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8 offset:%12\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:%13\n\t"
      "ds_read_b64_tr_b16 %2, %9 offset:%12\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:%13\n\t"
      "ds_read_b64_tr_b16 %4, %10 offset:%12\n\t"
      "ds_read_b64_tr_b16 %5, %10 offset:%13\n\t"
      "ds_read_b64_tr_b16 %6, %11 offset:%12\n\t"
      "ds_read_b64_tr_b16 %7, %11 offset:%13\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(t[0][0]), "=&v"(t[0][1]), "=&v"(t[1][0]), "=&v"(t[1][1]), "=&v"(t[2][0]),
        "=&v"(t[2][1]), "=&v"(t[3][0]), "=&v"(t[3][1])
      : "v"(va[0]), "v"(va[1]), "v"(va[2]), "v"(va[3]), "i"(OFF0), "i"(OFF1));
}

template <int OFF0, int OFF1>
__device__ __forceinline__ void lds_read_vt(u32x2 (&t)[2][2], const uint32_t (&va)[2]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4 offset:%6\n\t"
      "ds_read_b64_tr_b16 %1, %4 offset:%7\n\t"
      "ds_read_b64_tr_b16 %2, %5 offset:%6\n\t"
      "ds_read_b64_tr_b16 %3, %5 offset:%7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(t[0][0]), "=&v"(t[0][1]), "=&v"(t[1][0]), "=&v"(t[1][1])
      : "v"(va[0]), "v"(va[1]), "i"(OFF0), "i"(OFF1));
}

// One 16-byte-per-lane DMA load through a buffer resource straight into LDS (default cache
// policy: other row tiles of the group read the same rows); lane L writes LDS bytes
// [lds + 16 L, lds + 16 L + 16).
__device__ __forceinline__ void load16_tile_lds(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           off, 0, 0, 0);
}

// The lane id, recomputed where it is used (two instructions) rather than kept in a register
// across the stage loop: used on paths that run once per 64 stages or on the last stage.
__device__ __forceinline__ int fresh_lane() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// The largest of eight scores without the NaN-quieting copies the compiler puts in front of
// fmaxf (two of its six instructions per eight scores): v_max3_f32 takes three at a time. One
// asm block, so that the hazard padding the compiler adds around inline asm comes once, not
// after each of the four instructions. A NaN score can only come from a NaN key or query
// element and makes that row's output NaN either way.
__device__ __forceinline__ float max8f(const f32x4& x, const f32x4& y) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3\n\t"
      "v_max3_f32 %0, %0, %4, %5\n\t"
      "v_max3_f32 %0, %0, %6, %7\n\t"
      "v_max_f32 %0, %0, %8"
      : "=&v"(r)
      : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]), "v"(y[0]), "v"(y[1]), "v"(y[2]), "v"(y[3]));
  return r;
}
}  // namespace

// The work of one prefill workgroup: row tile `tile` of KV head kvh of sequence s, whose n
// query tokens (rows q0 .. q0 + n - 1 of q and out) are the last n of its T cached tokens.
struct PrefillTile {
  int tile, kvh, s, q0, T, n;
};

template <int BS>
__device__ __forceinline__ PrefillTile prefill_tile(const PrefillArgs& a) {
  PrefillTile w;
  // Workgroup -> (row tile, KV head, sequence). Linear id L runs on XCD L % 8. The (sequence,
  // KV head) groups G = kvh + Hkv * s are dealt round-robin over the XCDs, so every XCD gets
  // its share of every sequence (handing each XCD a contiguous range of groups gave it whole
  // sequences, and its work followed their lengths); on its XCD a group's row tiles run one
  // after the other, heaviest (latest) first, and share that XCD's L2. Groups past the last
  // multiple of 8 follow in order.
  const int Hkv = a.num_kv_heads;
  const int rt = a.row_tiles;
  const int64_t groups = (int64_t)Hkv * a.num_seqs;
  const int64_t dealt = groups / kXcds * kXcds;
  const int64_t L = blockIdx.x;
  int64_t G;
  int t_idx;
  if (L < dealt * rt) {
    const int64_t k = L / kXcds;  // the k-th workgroup on XCD L % 8
    G = L % kXcds + kXcds * (k / rt);
    t_idx = (int)(k % rt);
  } else {
    const int64_t r = L - dealt * rt;
    G = dealt + r / rt;
    t_idx = (int)(r % rt);
  }
  w.tile = rt - 1 - t_idx;
  w.kvh = (int)(G % Hkv);
  // Extent of a sequence, clamped into the buffers the sizes describe.
  const int Nq = a.num_q_tokens;
  const int64_t cap64 = (int64_t)a.max_blocks_per_seq * BS;
  const int cap = (int)(cap64 < (int64_t)a.max_context_len ? cap64 : (int64_t)a.max_context_len);
  auto extent = [&](int i, int& qa, int& qb, int& t) {
    qa = clampi(a.query_start[i], 0, Nq);
    qb = clampi(a.query_start[i + 1], qa, Nq);
    t = clampi(a.context_lens[i], 0, cap);
  };
  // G / Hkv is a rank. With at most 64 sequences (one per lane) the ranks follow the
  // sequences' work, heaviest first, so that each XCD also runs its share longest first: lane
  // i weighs sequence i by its visible (row, token) pairs n (2T - n) and counts the sequences
  // ahead of it (heavier, or as heavy with a smaller index), which makes the ranks a
  // permutation. With more sequences the rank is the sequence index.
  const int rank = (int)(G / Hkv);
  int s = rank, q0, q1, T;
  if (a.num_seqs <= 64) {  // uniform
    const int ln = threadIdx.x & 63;
    int qa = 0, qb = 0, Tr = 0;
    float wv = -1.0f;
    if (ln < a.num_seqs) {
      extent(ln, qa, qb, Tr);
      int nr = qb - qa;
      nr = nr < Tr ? nr : Tr;
      nr = nr < a.max_query_len ? nr : a.max_query_len;
      wv = (float)nr * (2.0f * (float)Tr - (float)nr);
    }
    int ahead = 0;
    for (int j = 0; j < a.num_seqs; ++j) {
      const float wj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                     __builtin_bit_cast(int, wv), j));
      ahead += (wj > wv || (wj == wv && j < ln)) ? 1 : 0;
    }
    const uint64_t hit = __builtin_amdgcn_ballot_w64(ln < a.num_seqs && ahead == rank);
    s = __builtin_ctzll(hit);
    // the chosen sequence's extent as its lane loaded it: no second round trip to memory
    q0 = __builtin_amdgcn_readlane(qa, s);
    q1 = __builtin_amdgcn_readlane(qb, s);
    T = __builtin_amdgcn_readlane(Tr, s);
  } else {
    extent(s, q0, q1, T);
  }
  int n = q1 - q0;
  n = n < T ? n : T;
  n = n < a.max_query_len ? n : a.max_query_len;
  w.s = s;
  w.q0 = q0;
  w.T = T;
  w.n = n;
  return w;
}

// Three workgroups per CU (12 waves, 144 KB of LDS at d = 128): the kernel fits 168 VGPRs by
// reading K and V from LDS half a head dimension at a time and recomputing the few
// lane-derived values that rare paths need; five values spill, each stored and reloaded once
// per workgroup, outside both stage loops.
template <DT dt, int D, int BS, int NW, int NCT, int NBUF>
__global__ __launch_bounds__(NW * 64, 3) void prefill_mfma_kernel(const PrefillArgs a) {
  static_assert(dt != DT::F32, "MFMA path takes 16-bit inputs");
  using M = MfmaT<dt>;
  using vec8 = typename M::vec8;
  constexpr int E = 2;
  constexpr int KC = D / 32;        // q.K MFMAs per 16-token tile
  constexpr int MT = D / 16;        // p.V M-tiles; row r of tile mt is head dimension MT*r + mt
  constexpr int RB = D * E;         // bytes per token row
  constexpr int CPR = RB / 16;      // 16-byte chunks per row
  constexpr int KT = 32;            // tokens per stage
  constexpr int RPL = 1024 / RB;    // rows one wave-wide 16-byte-per-lane load covers
  constexpr int WLW = KT * RB / 1024 / NW;  // wave-wide loads per wave per tensor per stage
  constexpr int RPW = KT / NW;      // rows of a stage one wave loads: [RPW*w, RPW*(w+1))
  constexpr int ROWS_W = 16 * NCT;
  constexpr int ROWS = NW * ROWS_W;
  constexpr int TILE = KT * RB;     // LDS bytes per tensor per stage
  static_assert(KT * RB % (1024 * NW) == 0 && WLW * RPL == RPW, "a stage splits over the waves");
  static_assert(BS % RPW == 0, "the rows one wave loads lie in one block");
  __shared__ __attribute__((aligned(1024))) char lds[NBUF][2][TILE];  // [stage][K, V]

  const PrefillTile wk = prefill_tile<BS>(a);
  const int tile = wk.tile, kvh = wk.kvh, s = wk.s, q0 = wk.q0, T = wk.T, n = wk.n;
  const int Hkv = a.num_kv_heads;
  const int Hq = a.num_q_heads;
  const int g = Hq / Hkv;
  const int nrows = n * g;
  const int W0 = tile * ROWS;  // first row of the workgroup
  if (W0 >= nrows) return;     // uniform over the workgroup: no barrier is skipped
  const int base_pos = T - n;  // position of the chunk's first query token
  const int p_hi_wg = base_pos + ((W0 + ROWS < nrows ? W0 + ROWS : nrows) - 1) / g;
  const int nstages = (p_hi_wg + KT) / KT;  // stages covering positions 0 .. p_hi_wg
  const int jlast = p_hi_wg / BS;           // last block the workgroup reads

  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int hh = lane & 15, gq = lane >> 4;

  // The scores are scaled by cs > 0, so that the largest raw score gives the largest scaled
  // one: a negative scale is applied as |scale| to the negated query, and a zero scale as 1
  // to a zero query (every score 0, as with scale 0); both are exact.
  const float cs = a.scale_log2 == 0.0f ? 1.0f : __builtin_fabsf(a.scale_log2);
  const uint32_t qflip = a.scale_log2 < 0.0f ? 0x80008000u : 0u;
  const uint32_t qkeep = a.scale_log2 == 0.0f ? 0u : 0xffffffffu;

  // Column tiles of this wave: tile c is workgroup column tile NCT*w + c.
  int pos[NCT];                // position of this lane's query row; -1 past the chunk
  int t_lo[NCT];               // first position of the tile's rows (uniform); -1 if empty
  vec8 qop[NCT][KC];
  int p_hi_w = -1;             // last position any tile of this wave needs
  int t_lo_w = 0x7fffffff;     // first position any tile of this wave starts at
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    const int Rt = W0 + 16 * (NCT * w + c);  // first row of the tile
    const int R = Rt + hh;
    const bool valid = R < nrows;
    const int i = valid ? R / g : 0;
    const int head = kvh * g + (valid ? R % g : 0);
    pos[c] = valid ? base_pos + i : -1;
    t_lo[c] = Rt < nrows ? base_pos + Rt / g : -1;
    const int t_hi = Rt < nrows ? base_pos + ((Rt + 16 < nrows ? Rt + 16 : nrows) - 1) / g : -1;
    p_hi_w = t_hi > p_hi_w ? t_hi : p_hi_w;
    t_lo_w = t_lo[c] < t_lo_w ? t_lo[c] : t_lo_w;
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (valid)
        raw = load16((const char*)a.q +
                     (((int64_t)(q0 + i) * Hq + head) * D + 32 * kk + 8 * gq) * E);
      raw = (raw ^ qflip) & qkeep;
      qop[c][kk] = __builtin_bit_cast(vec8, raw);
    }
  }

  f32x4 oacc[NCT][MT];
  // Running state per column tile: the reference maximum m (scaled, base 2) is kept as the
  // shift nm = -m applied to every score (0 while m is -inf) and as the raw-score threshold
  // thr = (m + kSlack) / cs (-inf while m is).
  float nm[NCT], lsum[NCT], thr[NCT];
  const float rcs = 1.0f / cs;
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    nm[c] = 0.0f;
    thr[c] = kNegInf;
    lsum[c] = 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) oacc[c][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Block ids: the rows a wave loads in stage st lie in block (KT*st + RPW*w) / BS. Lane k of
  // `ids` holds that id for stage 64*(st/64) + k (clamped to the workgroup's last block:
  // stages past it load stand-in rows that are masked later). The next 64 are loaded when the
  // first of them is issued and used at once: one wait for the loads in flight per 64 stages,
  // and no load of `ids` is ever outstanding across stages. Ids are clamped into the pool as
  // they are loaded, 64 at a time, so a stage only scales its id.
  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  const int id_max = last_block_id(a.num_blocks);
  auto load_ids = [&](int chunk) {
    const int j = (KT * (64 * chunk + fresh_lane()) + RPW * w) / BS;
    return clamp_id(bt[j < jlast ? j : jlast], id_max);  // jlast < max_blocks_per_seq: T <= cap
  };
  int ids = load_ids(0);

  // LDS rows are swizzled in 16-byte chunks: chunk cc of row r sits at physical chunk
  // cc ^ swz(r). K (read as 16 rows at one chunk): swz runs over the rows that share one
  // 256-byte line of banks. V (read transposed: 16 rows, two adjacent chunks each, per 32
  // lanes): rows of a line take even offsets, so the two chunks of eight consecutive rows
  // land on sixteen distinct chunk positions.
  constexpr int RPBL = 256 / RB;  // rows per 256-byte line of banks
  auto swz_k = [](int r) { return (r / RPBL) % CPR; };
  auto swz_v = [](int r) { return (2 * ((r / RPBL) % (CPR / 2)) + (r / RPBL / (CPR / 2)) % 2); };
  auto koff = [&](int r, int cc) { return r * RB + ((cc ^ swz_k(r)) * 16); };
  auto voff = [&](int r, int cc) { return r * RB + ((cc ^ swz_v(r)) * 16); };
  // Transposed V reads: lane (gq, s) addresses row 16u + 4gq + s/4, head dims
  // 16mt + 4(s%4) .. +3 (swz_v repeats every 16 rows, so token tile u adds 16 rows).
  typedef __attribute__((address_space(3))) char lds_char;
  const uint32_t lds_v0 = (uint32_t)(uintptr_t)(lds_char*)&lds[0][1][0];
  // The address for M-tile mt is va0 ^ 32 mt: the swizzle moves a row's 16-byte chunks only
  // within the bits that the M-tile's 32-byte offset occupies, and the row and buffer bits
  // above them are unaffected. One XOR per read instead of a register per M-tile.
  const uint32_t va0 = lds_v0 + voff(4 * gq + (hh >> 2), (8 * (hh & 3)) >> 4) + ((8 * (hh & 3)) & 15);

  // Stage loads go straight from global memory into LDS (buffer_load_dwordx4 ... lds): lane L
  // of a wave-wide load writes LDS bytes [base + 16L, base + 16L + 16), so one load fills
  // 1 KB = RPL whole rows. Lane L carries physical chunk L % CPR of row L / CPR and fetches
  // the logical chunk the swizzle maps there. No registers hold data in flight, so NBUF - 1
  // stages can be in flight while one is consumed.
  const int64_t tile_bytes = (int64_t)BS * RB;
  const uint64_t blk_bytes = (uint64_t)Hkv * tile_bytes;  // one physical block, all KV heads
  const char* kbase = (const char*)a.k_cache + kvh * tile_bytes;  // this KV head's tile of block 0
  const char* vbase = (const char*)a.v_cache + kvh * tile_bytes;
  const int row_in_load = lane / CPR;
  const int pchunk = lane % CPR;
  uint32_t ko[WLW], vo[WLW];  // byte offsets in the block's tile of the chunks this lane moves
#pragma unroll
  for (int k = 0; k < WLW; ++k) {
    const int r = (w * WLW + k) * RPL + row_in_load;  // row within the stage
    ko[k] = (uint32_t)((r % BS) * RB + (pchunk ^ swz_k(r)) * 16);
    vo[k] = (uint32_t)((r % BS) * RB + (pchunk ^ swz_v(r)) * 16);
  }
  auto issue_stage = [&](int st, int buf) {
    if (st > 0 && (st & 63) == 0) {  // uniform
      ids = load_ids(st >> 6);
      __builtin_amdgcn_s_waitcnt(0x0F70 & ~0x0F);  // vmcnt(0): ids is never pending past here
    }
    uint64_t t = (uint64_t)(uint32_t)__builtin_amdgcn_readlane(ids, st & 63) * blk_bytes;
    // Blocks larger than a stage: the stage's rows start (st % (BS / KT)) * KT rows into the
    // block, and the resources span those KT rows only.
    if constexpr (BS > KT) t += (uint64_t)((st % (BS / KT)) * TILE);
    constexpr int span = BS > KT ? TILE : (int)(BS * RB);
    const __amdgpu_buffer_rsrc_t kr = tile_rsrc(kbase + t, span);
    const __amdgpu_buffer_rsrc_t vr = tile_rsrc(vbase + t, span);
#pragma unroll
    for (int k = 0; k < WLW; ++k) {
      const int mload = w * WLW + k;  // wave-wide load index within the tensor
      load16_tile_lds(kr, &lds[buf][0][mload * 1024], ko[k]);
      load16_tile_lds(vr, &lds[buf][1][mload * 1024], vo[k]);
    }
  };
  // This wave's loads of stage st are done once at most `later` stages' loads are outstanding.
  auto wait_stage = [&](int later) {
    // s_waitcnt: vmcnt in bits [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] left at max
    constexpr int per = 2 * WLW;
    switch (later) {
#define PA_WAIT_CASE(n) \
  case n: __builtin_amdgcn_s_waitcnt(((n * per) & 15) | (((n * per) >> 4) << 14) | 0x0F70); break;
      PA_WAIT_CASE(0)
      PA_WAIT_CASE(1)
      PA_WAIT_CASE(2)
      PA_WAIT_CASE(3)
#undef PA_WAIT_CASE
      default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    }
  };

  // One 32-token stage in LDS buffer `buf` for every column tile of this wave. `mask`
  // (uniform): some token of the stage lies past some row's position, or past the
  // workgroup's last position (stand-in or unused tail rows, possibly NaN); then hidden scores
  // are set to -inf and V rows past the workgroup's last position to 0, both by select.
  // Otherwise every token is visible to every row and no score is tested.
  auto consume = [&](int tau0, auto bufc, bool mask, bool tail) {
    constexpr int buf = decltype(bufc)::value;
    // S^T = K Q^T for every column tile: 2*NCT independent accumulation chains. K comes from
    // LDS in two halves of the head dimension, so that only half of it is held at a time.
    f32x4 sacc[NCT][2];
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
      for (int u = 0; u < 2; ++u) sacc[c][u] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int KH = KC / 2;
    static_for<2>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      u32x4 kf[2][KH];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < KH; ++j)
          kf[u][j] = *reinterpret_cast<const u32x4*>(&lds[buf][0][koff(16 * u + hh, 4 * (h * KH + j) + gq)]);
      // The MFMA blocks run at raised wave priority, so that a wave holding matrix work issues
      // it ahead of the other waves' vector work on the same SIMD.
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int j = 0; j < KH; ++j)
#pragma unroll
        for (int c = 0; c < NCT; ++c)
#pragma unroll
          for (int u = 0; u < 2; ++u)
            sacc[c][u] = M::mma(__builtin_bit_cast(vec8, kf[u][j]), qop[c][h * KH + j], sacc[c][u]);
      __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
    });
    // V^T operand of M-tile mt (head dims 16mt .. 16mt+15), k element e <-> token
    // 16*(e/4) + 4*gq + (e%4): the transposed read hands lane (gq, 4q + p) dim 16mt + 4q + p
    // of tokens 16u + 4gq + 0..3.
    // (issued once the scores' MFMAs are: their latency overlaps the matrix cores)
    __builtin_amdgcn_sched_barrier(0);
    constexpr int MH = MT / 2;
    u32x4 vw[MH];
    auto read_v = [&](auto hc) {
      constexpr int h = decltype(hc)::value;
      u32x2 tv[MH][2];
      uint32_t vah[MH];
#pragma unroll
      for (int mt = 0; mt < MH; ++mt) vah[mt] = va0 ^ (uint32_t)(32 * (h * MH + mt));
      lds_read_vt<buf * 2 * TILE, buf * 2 * TILE + 16 * RB>(tv, vah);
#pragma unroll
      for (int mt = 0; mt < MH; ++mt) vw[mt] = u32x4{tv[mt][0][0], tv[mt][0][1], tv[mt][1][0], tv[mt][1][1]};
      if (tail && tau0 + KT - 1 > p_hi_wg) {  // uniform: V of tokens past the last position is 0
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int t0 = tau0 + 16 * u + 4 * (fresh_lane() >> 4);  // token of element 4u
          const uint32_t keep0 = (t0 > p_hi_wg ? 0u : 0xffffu) | (t0 + 1 > p_hi_wg ? 0u : 0xffff0000u);
          const uint32_t keep1 = (t0 + 2 > p_hi_wg ? 0u : 0xffffu) | (t0 + 3 > p_hi_wg ? 0u : 0xffff0000u);
#pragma unroll
          for (int mt = 0; mt < MH; ++mt) {
            vw[mt][2 * u] &= keep0;
            vw[mt][2 * u + 1] &= keep1;
          }
        }
      }
    };
    read_v(std::integral_constant<int, 0>{});
    if (mask) {  // uniform; token 16u + 4gq + i is hidden from the lane's row past its position
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        const int lim = pos[c] - tau0 - 4 * gq;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (16 * u + i > lim) sacc[c][u][i] = kNegInf;  // select
      }
    }
    // Weights are taken against a reference maximum m (scaled, base 2) that is raised only
    // when some score exceeds it by more than kSlack: weights stay below 2^kSlack, and the
    // running sum and output use the same reference, so the normalised result is the same as
    // with the exact running maximum. The test runs on raw scores against thr[c] =
    // (m + kSlack) / cs, which changes only when m does. The scaled, shifted score
    // cs * s + nm[c] = cs * s - m is one FMA.
    float lr[NCT];  // largest raw score of the lane's 8
    bool raise = false;
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      lr[c] = max8f(sacc[c][0], sacc[c][1]);
      raise = raise || (lr[c] > thr[c]);
    }
    if (__builtin_amdgcn_ballot_w64(raise)) {  // uniform; rare once the maxima settle
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        const float lm = lr[c] * cs;
        float bm = fmaxf(lm, __shfl_xor(lm, 16));
        bm = fmaxf(bm, __shfl_xor(bm, 32));
        // m is -inf exactly when thr is -inf and the shift is 0 (a finite m of 0 has a
        // positive threshold; a threshold that overflowed to -inf has a large shift)
        const float mo = (thr[c] == kNegInf && nm[c] == 0.0f) ? kNegInf : -nm[c];
        const float mn = fmaxf(mo, bm);
        const float corr = (mo == kNegInf) ? (mn == kNegInf ? 1.0f : 0.0f) : fast_exp2(mo - mn);
        lsum[c] *= corr;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) oacc[c][mt] *= corr;
        // m is -inf only while every row of the column has all its tokens hidden (all its
        // scores -inf): the shift is 0 then, so the weights are exp2(-inf) = 0
        nm[c] = mn == kNegInf ? 0.0f : -mn;
        thr[c] = (mn + kSlack) * rcs;
      }
    }
    vec8 pop[NCT];
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      float pe[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pe[e] = fast_exp2(__builtin_fmaf(sacc[c][e / 4][e % 4], cs, nm[c]));
      const u32x4 pw = {pack2<dt>(pe[0], pe[1]), pack2<dt>(pe[2], pe[3]),
                        pack2<dt>(pe[4], pe[5]), pack2<dt>(pe[6], pe[7])};
      // The row sum takes the weights as the p.V product does, rounded to 16 bits: one dot2
      // with (1, 1) per packed pair, accumulated in fp32.
#pragma unroll
      for (int j = 0; j < 4; ++j) lsum[c] = sum2<dt>(pw[j], lsum[c]);
      pop[c] = __builtin_bit_cast(vec8, pw);
    }
    // O^T += V^T P^T: MT * NCT independent MFMAs
    static_for<2>([&](auto hc) {
      constexpr int h = decltype(hc)::value;
      if constexpr (h == 1) read_v(hc);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int mt = 0; mt < MH; ++mt)
#pragma unroll
        for (int c = 0; c < NCT; ++c)
          oacc[c][h * MH + mt] = M::mma(__builtin_bit_cast(vec8, vw[mt]), pop[c], oacc[c][h * MH + mt]);
      __builtin_amdgcn_s_setprio(0);
    });
  };

  const int prolog = nstages < NBUF - 1 ? nstages : NBUF - 1;
  for (int st = 0; st < prolog; ++st) issue_stage(st, st);

  // One stage: wait for its loads, then a bare barrier (every wave's loads of stage st have
  // landed and stage st-1 is consumed; a fence here would also wait for the later stages'
  // loads still in flight; the empty asm keeps the compiler from moving LDS accesses across
  // it), then the loads of stage st + NBUF - 1 into the buffer stage st - 1 used.
  auto enter_stage = [&](int st, int later, auto bc, bool issue) {
    constexpr int b = decltype(bc)::value;
    wait_stage(later);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (issue) issue_stage(st + NBUF - 1, (b + NBUF - 1) % NBUF);
  };

  // Leading stages in bulk: every row of the workgroup sees all their tokens (the first row
  // sits at position t_lo_wg), and a later stage remains to be loaded. No test for the causal
  // mask, the tail or the end of the loop is needed there; nbulk is a multiple of NBUF and the
  // same for every wave.
  const int t_lo_wg = base_pos + W0 / g;
  int nbulk = (t_lo_wg + 1) / KT;  // stages ending at or before position t_lo_wg
  nbulk = nbulk < nstages - (NBUF - 1) ? nbulk : nstages - (NBUF - 1);
  nbulk = nbulk > 0 ? nbulk / NBUF * NBUF : 0;
  int st0 = 0;
  for (; st0 < nbulk; st0 += NBUF) {
    static_for<NBUF>([&](auto bc) {
      const int st = st0 + decltype(bc)::value;
      enter_stage(st, NBUF - 2, bc, true);
      consume(st * KT, bc, false, false);
    });
  }
  // The remaining stages, with every test. Stages are unrolled NBUF at a time so that every
  // LDS buffer offset is a constant.
  for (; st0 < nstages; st0 += NBUF) {
    static_for<NBUF>([&](auto bc) {
      constexpr int b = decltype(bc)::value;
      const int st = st0 + b;  // st % NBUF == b
      if (st >= nstages) return;  // uniform
      const int later = (nstages - 1 - st) < (NBUF - 2) ? (nstages - 1 - st) : (NBUF - 2);
      enter_stage(st, later, bc, st + NBUF - 1 < nstages);
      const int tau0 = st * KT;
      if (tau0 > p_hi_w) return;  // uniform: every tile of this wave is done
      consume(tau0, bc, tau0 + KT - 1 > t_lo_w, true);  // t_lo_w is -1 when a tile is empty
    });
  }

  // Normalise and store. oacc[c][mt][i] is O[column hh][dim 16mt + 4gq + i]: four
  // consecutive dimensions, one 8-byte store per M-tile.
  const int lane_e = fresh_lane();
  const int hh_e = lane_e & 15, gq_e = lane_e >> 4;
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    float l = lsum[c];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (pos[c] < 0) continue;
    const int R = W0 + 16 * (NCT * w + c) + hh_e;
    const int i = R / g;
    const int head = kvh * g + R % g;
    char* orow = (char*)a.out + ((int64_t)(q0 + i) * Hq + head) * D * E;
    const float rl = 1.0f / l;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const u32x2 packed = {pack2<dt>(oacc[c][mt][0] * rl, oacc[c][mt][1] * rl),
                            pack2<dt>(oacc[c][mt][2] * rl, oacc[c][mt][3] * rl)};
      *reinterpret_cast<u32x2*>(orow + (16 * mt + 4 * gq_e) * E) = packed;
    }
  }
}

// ---- fp32 prefill on fp32 MFMA ---------------------------------------------------------------
// The same attention with fp32 inputs, computed on v_mfma_f32_16x16x4_f32 (fp32 products and
// sums throughout). Work decomposition as in the 16-bit kernel: a workgroup takes NW * NCT * 16
// rows (query token, grouped head) of one (sequence, KV head), each wave NCT adjacent 16-row
// column tiles, and walks the visible context in 32-token stages that come from HBM straight
// into LDS (two stage buffers, one stage in flight while one is consumed), so each K/V row is
// read once per workgroup instead of once per query row.
//
// Layouts of v_mfma_f32_16x16x4_f32, lane l = 16 j + r:
//   A (16 x 4): lane l holds row r, k = j;   B (4 x 16): lane l holds column r, k = j;
//   C (16 x 16): lane l holds rows 4 j .. 4 j + 3 of column r.
// S^T = K Q^T: MFMA m of token tile u pairs k index j with head dimension (D/4) j + m, so lane
// l reads D/4 consecutive floats of K row 16u + r and holds D/4 consecutive query floats.
// O^T += V^T P^T: k-step (u, i) pairs k index j with token 16u + 4j + i, which makes the
// lane's own weight for that token its P^T element. M-tile mt's row r is head dimension
// 8r + 4((r >> 3) ^ (mt >> 2)) + (mt & 3) for D = 128 (4r + mt for D = 64): a lane reads its
// V operands as two 16-byte chunks of one row, the first at chunk 2r + (r >> 3), so that the
// 16 lanes reading one row hit 16 different bank groups.
// K rows sit in LDS with their 16-byte chunks XOR-swizzled by the row's index mod 16 (the 16
// lanes of a K read take 16 rows at one chunk); V rows are stored plain.
template <int D, int BS, int NW, int NCT, int NBUF>
__global__ __launch_bounds__(NW * 64, 2) void prefill_f32_kernel(const PrefillArgs a) {
  constexpr int E = 4;
  constexpr int KM = D / 4;         // q.K MFMAs per 16-token tile
  constexpr int MT = D / 16;        // p.V M-tiles
  constexpr int RB = D * E;         // bytes per token row
  constexpr int CPR = RB / 16;      // 16-byte chunks per row
  constexpr int KCH = D / 16;       // K chunks a lane reads per row (D/4 floats)
  constexpr int KT = 32;            // tokens per stage
  constexpr int RPL = 1024 / RB;    // rows one wave-wide 16-byte-per-lane load covers
  constexpr int WLW = KT * RB / 1024 / NW;  // wave-wide loads per wave per tensor per stage
  constexpr int RPW = KT / NW;      // rows of a stage one wave loads
  constexpr int ROWS = NW * 16 * NCT;
  constexpr int TILE = KT * RB;     // LDS bytes per tensor per stage
  static_assert(D == 64 || D == 128, "head dims 64 and 128");
  static_assert(KT * RB % (1024 * NW) == 0 && WLW * RPL == RPW, "a stage splits over the waves");
  static_assert(BS % RPW == 0, "the rows one wave loads lie in one block");
  static_assert(NBUF == 2, "one stage in flight while one is consumed");
  __shared__ __attribute__((aligned(1024))) char lds[NBUF][2][TILE];  // [stage][K, V]

  const PrefillTile wk = prefill_tile<BS>(a);
  const int kvh = wk.kvh, s = wk.s, q0 = wk.q0, T = wk.T, n = wk.n;
  const int Hkv = a.num_kv_heads;
  const int Hq = a.num_q_heads;
  const int g = Hq / Hkv;
  const int nrows = n * g;
  const int W0 = wk.tile * ROWS;  // first row of the workgroup
  if (W0 >= nrows) return;        // uniform over the workgroup: no barrier is skipped
  const int base_pos = T - n;     // position of the chunk's first query token
  const int p_hi_wg = base_pos + ((W0 + ROWS < nrows ? W0 + ROWS : nrows) - 1) / g;
  const int nstages = (p_hi_wg + KT) / KT;  // stages covering positions 0 .. p_hi_wg
  const int jlast = p_hi_wg / BS;           // last block the workgroup reads

  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int r = lane & 15, j = lane >> 4;

  // Scores are scaled by cs > 0 (see the 16-bit kernel): a negative scale is applied as
  // |scale| to the negated query, a zero scale as 1 to a zero query; both are exact.
  const float cs = a.scale_log2 == 0.0f ? 1.0f : __builtin_fabsf(a.scale_log2);
  const uint32_t qflip = a.scale_log2 < 0.0f ? 0x80000000u : 0u;
  const uint32_t qkeep = a.scale_log2 == 0.0f ? 0u : 0xffffffffu;

  int pos[NCT];       // position of this lane's query row; -1 past the chunk
  float qop[NCT][KM]; // Q^T operand: query row of column r, head dims (D/4) j + m
  int p_hi_w = -1;    // last position any tile of this wave needs
  int t_lo_w = 0x7fffffff;  // first position any tile of this wave starts at
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    const int Rt = W0 + 16 * (NCT * w + c);  // first row of the tile
    const int R = Rt + r;
    const bool valid = R < nrows;
    const int i = valid ? R / g : 0;
    const int head = kvh * g + (valid ? R % g : 0);
    pos[c] = valid ? base_pos + i : -1;
    const int t_lo = Rt < nrows ? base_pos + Rt / g : -1;
    const int t_hi = Rt < nrows ? base_pos + ((Rt + 16 < nrows ? Rt + 16 : nrows) - 1) / g : -1;
    p_hi_w = t_hi > p_hi_w ? t_hi : p_hi_w;
    t_lo_w = t_lo < t_lo_w ? t_lo : t_lo_w;
    const char* qp = (const char*)a.q + (((int64_t)(q0 + i) * Hq + head) * D + KM * j) * E;
#pragma unroll
    for (int x = 0; x < KM / 4; ++x) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (valid) raw = load16(qp + 16 * x);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        qop[c][4 * x + e] = __builtin_bit_cast(float, (raw[e] ^ qflip) & qkeep);
    }
  }

  f32x4 oacc[NCT][MT];
  float nm[NCT], lsum[NCT], thr[NCT];  // running state, as in the 16-bit kernel
  const float rcs = 1.0f / cs;
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    nm[c] = 0.0f;
    thr[c] = kNegInf;
    lsum[c] = 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) oacc[c][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Block ids, 64 stages at a time (lane k = stage 64 * chunk + k), clamped into the pool.
  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  const int id_max = last_block_id(a.num_blocks);
  auto load_ids = [&](int chunk) {
    const int jb = (KT * (64 * chunk + fresh_lane()) + RPW * w) / BS;
    return clamp_id(bt[jb < jlast ? jb : jlast], id_max);  // jlast < max_blocks_per_seq
  };
  int ids = load_ids(0);

  auto kswz = [](int row) { return row & 15; };
  // DMA offsets: lane L of wave-wide load k fills physical chunk L % CPR of stage row
  // (w * WLW + k) * RPL + L / CPR.
  const int64_t tile_bytes = (int64_t)BS * RB;
  const uint64_t blk_bytes = (uint64_t)Hkv * tile_bytes;
  const char* kbase = (const char*)a.k_cache + kvh * tile_bytes;
  const char* vbase = (const char*)a.v_cache + kvh * tile_bytes;
  uint32_t ko[WLW], vo[WLW];
#pragma unroll
  for (int k = 0; k < WLW; ++k) {
    const int row = (w * WLW + k) * RPL + lane / CPR;
    ko[k] = (uint32_t)((row % BS) * RB + ((lane % CPR) ^ kswz(row)) * 16);
    vo[k] = (uint32_t)((row % BS) * RB + (lane % CPR) * 16);
  }
  auto issue_stage = [&](int st, int buf) {
    if (st > 0 && (st & 63) == 0) {  // uniform
      ids = load_ids(st >> 6);
      __builtin_amdgcn_s_waitcnt(0x0F70 & ~0x0F);  // vmcnt(0): ids is never pending past here
    }
    uint64_t t = (uint64_t)(uint32_t)__builtin_amdgcn_readlane(ids, st & 63) * blk_bytes;
    if constexpr (BS > KT) t += (uint64_t)((st % (BS / KT)) * TILE);
    constexpr int span = BS > KT ? TILE : (int)(BS * RB);
    const __amdgpu_buffer_rsrc_t kr = tile_rsrc(kbase + t, span);
    const __amdgpu_buffer_rsrc_t vr = tile_rsrc(vbase + t, span);
#pragma unroll
    for (int k = 0; k < WLW; ++k) {
      const int mload = w * WLW + k;
      load16_tile_lds(kr, &lds[buf][0][mload * 1024], ko[k]);
      load16_tile_lds(vr, &lds[buf][1][mload * 1024], vo[k]);
    }
  };

  // LDS addresses this lane reads: K row 16u + r, logical chunk KCH j + x; V row 16u + 4j + i,
  // chunks c0 = 2r + (r >> 3) and c1 = 2r + 1 - (r >> 3) (D = 128) or r (D = 64).
  const int kc0 = KCH * j;
  const int vc0 = D == 128 ? 2 * r + (r >> 3) : r;
  const int vc1 = D == 128 ? 2 * r + 1 - (r >> 3) : r;

  auto consume = [&](int tau0, auto bufc, bool mask, bool tail) {
    constexpr int buf = decltype(bufc)::value;
    const char* lk = &lds[buf][0][0];
    const char* lv = &lds[buf][1][0];
    // S^T = K Q^T: sacc[c][u][e] = score of token tau0 + 16u + 4j + e for column r; the two
    // token tiles (and the column tiles) are independent accumulation chains, interleaved.
    f32x4 sacc[NCT][2];
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
      for (int u = 0; u < 2; ++u) sacc[c][u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int x = 0; x < KCH; ++x) {
      f32x4 kf[2];
#pragma unroll
      for (int u = 0; u < 2; ++u)  // K row 16u + r: its swizzle is r
        kf[u] = *reinterpret_cast<const f32x4*>(lk + (16 * u + r) * RB + ((kc0 + x) ^ r) * 16);
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int c = 0; c < NCT; ++c)
            sacc[c][u] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[u][e], qop[c][4 * x + e],
                                                               sacc[c][u], 0, 0, 0);
    }
    if (mask) {  // uniform; token tau0 + 16u + 4j + e is hidden from the lane's row past its position
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        const int lim = pos[c] - tau0 - 4 * j;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (16 * u + e > lim) sacc[c][u][e] = kNegInf;  // select
      }
    }
    // Reference maximum raised only when a score exceeds it by more than kSlack (base 2), as
    // in the 16-bit kernel.
    float lr[NCT];
    bool raise = false;
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      lr[c] = max8f(sacc[c][0], sacc[c][1]);
      raise = raise || (lr[c] > thr[c]);
    }
    if (__builtin_amdgcn_ballot_w64(raise)) {  // uniform
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        const float lm = lr[c] * cs;
        float bm = fmaxf(lm, __shfl_xor(lm, 16));
        bm = fmaxf(bm, __shfl_xor(bm, 32));
        const float mo = (thr[c] == kNegInf && nm[c] == 0.0f) ? kNegInf : -nm[c];
        const float mn = fmaxf(mo, bm);
        const float corr = (mo == kNegInf) ? (mn == kNegInf ? 1.0f : 0.0f) : fast_exp2(mo - mn);
        lsum[c] *= corr;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) oacc[c][mt] *= corr;
        nm[c] = mn == kNegInf ? 0.0f : -mn;
        thr[c] = (mn + kSlack) * rcs;
      }
    }
    float pw[NCT][2][4];
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pw[c][u][e] = fast_exp2(__builtin_fmaf(sacc[c][u][e], cs, nm[c]));
          lsum[c] += pw[c][u][e];
        }
    // O^T += V^T P^T, k-step (u, e): V row 16u + 4j + e.
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * u + 4 * j + e;
        f32x4 va = *reinterpret_cast<const f32x4*>(lv + row * RB + vc0 * 16);
        f32x4 vb = va;
        if constexpr (D == 128) vb = *reinterpret_cast<const f32x4*>(lv + row * RB + vc1 * 16);
        if (tail && tau0 + row > p_hi_wg) {  // stand-in or unused rows may hold anything
          va = f32x4{0.f, 0.f, 0.f, 0.f};
          vb = va;
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const float av = mt < 4 ? va[mt & 3] : vb[mt & 3];
#pragma unroll
          for (int c = 0; c < NCT; ++c)
            oacc[c][mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, pw[c][u][e], oacc[c][mt],
                                                                0, 0, 0);
        }
      }
  };

  issue_stage(0, 0);
  // One stage: wait for its loads (this wave's, then every wave's at the barrier, which also
  // says the buffer the next loads go to has been consumed), issue the next stage's loads,
  // consume. Unrolled two at a time so that buffer offsets are constants.
  for (int st0 = 0; st0 < nstages; st0 += 2) {
    static_for<2>([&](auto bc) {
      constexpr int b = decltype(bc)::value;
      const int st = st0 + b;
      if (st >= nstages) return;  // uniform
      __builtin_amdgcn_s_waitcnt(0x0F70 & ~0x0F);  // vmcnt(0): this wave's loads of stage st
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (st + 1 < nstages) issue_stage(st + 1, b ^ 1);
      const int tau0 = st * KT;
      if (tau0 > p_hi_w) return;  // uniform: every tile of this wave is done
      consume(tau0, bc, tau0 + KT - 1 > t_lo_w, tau0 + KT - 1 > p_hi_wg);
    });
  }

  // Normalise and store. oacc[c][mt][v] is O[column r][head dim of M-tile mt, row 4j + v].
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    float l = lsum[c];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (pos[c] < 0) continue;
    const int R = W0 + 16 * (NCT * w + c) + r;
    const int i = R / g;
    const int head = kvh * g + R % g;
    float* orow = (float*)a.out + ((int64_t)(q0 + i) * Hq + head) * D;
    const float rl = 1.0f / l;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 4 * j + v;
      if constexpr (D == 128) {
        // head dims 8m .. 8m + 7: M-tiles 0..3 hold the first four unless m >= 8 (j >= 2)
        const bool swap = j >= 2;
        f32x4 lo, hi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = oacc[c][e][v] * rl, x1 = oacc[c][4 + e][v] * rl;
          lo[e] = swap ? x1 : x0;
          hi[e] = swap ? x0 : x1;
        }
        *reinterpret_cast<f32x4*>(orow + 8 * m) = lo;
        *reinterpret_cast<f32x4*>(orow + 8 * m + 4) = hi;
      } else {
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = oacc[c][e][v] * rl;
        *reinterpret_cast<f32x4*>(orow + 4 * m) = o;
      }
    }
  }
}

// ---- host side ------------------------------------------------------------------------------

// fp32 workgroups take one 16-row column tile per wave: 64 rows, so that a 64-token MHA chunk
// (64 rows per sequence and head) keeps all four waves busy. Measured on MI355X, 13B-shape fp32
// chunks of 64 tokens: 215.3 us against 338.4 us with two tiles per wave (128-row workgroups,
// half of whose waves had no row).
constexpr int kPrefillF32ColTiles = 1;

int prefill_rows_per_workgroup(int dt) {
  return kPrefillWaves * (dt == 0 ? kPrefillF32ColTiles : kPrefillColTiles) * 16;
}

bool prefill_supported(int dt, int head_dim, int block_size) {
  if (dt < 0 || dt > 2) return false;  // fp32, fp16 and bf16, each on its own MFMA kernel
  if (head_dim != 64 && head_dim != 128) return false;
  return block_size == 8 || block_size == 16 || block_size == 32 || block_size == 64;
}

template <DT dt, int D, int BS>
static hipError_t launch_pf(const PrefillArgs& a, hipStream_t stream) {
  const int64_t total = (int64_t)a.row_tiles * a.num_kv_heads * a.num_seqs;
  if (total == 0) return hipSuccess;
  PrefillArgs args_copy = a;
  void* args[] = {&args_copy};
  return hipLaunchKernel(
      (const void*)prefill_mfma_kernel<dt, D, BS, kPrefillWaves, kPrefillColTiles,
                                       kPrefillStages>,
      dim3((unsigned)total), dim3(kPrefillWaves * 64), args, 0, stream);
}

template <DT dt, int D>
static hipError_t launch_pf_bs(int bs, const PrefillArgs& a, hipStream_t st) {
  switch (bs) {
    case 8: return launch_pf<dt, D, 8>(a, st);
    case 16: return launch_pf<dt, D, 16>(a, st);
    case 32: return launch_pf<dt, D, 32>(a, st);
    case 64: return launch_pf<dt, D, 64>(a, st);
    default: return hipErrorInvalidValue;
  }
}

template <int D, int BS>
static hipError_t launch_pf32(const PrefillArgs& a, hipStream_t stream) {
  const int64_t total = (int64_t)a.row_tiles * a.num_kv_heads * a.num_seqs;
  if (total == 0) return hipSuccess;
  PrefillArgs args_copy = a;
  void* args[] = {&args_copy};
  return hipLaunchKernel(
      (const void*)prefill_f32_kernel<D, BS, kPrefillWaves, kPrefillF32ColTiles, 2>,
      dim3((unsigned)total), dim3(kPrefillWaves * 64), args, 0, stream);
}

template <int D>
static hipError_t launch_pf32_bs(int bs, const PrefillArgs& a, hipStream_t st) {
  switch (bs) {
    case 8: return launch_pf32<D, 8>(a, st);
    case 16: return launch_pf32<D, 16>(a, st);
    case 32: return launch_pf32<D, 32>(a, st);
    case 64: return launch_pf32<D, 64>(a, st);
    default: return hipErrorInvalidValue;
  }
}

static hipError_t launch_pf32_d(int d, int bs, const PrefillArgs& a, hipStream_t st) {
  switch (d) {
    case 64: return launch_pf32_bs<64>(bs, a, st);
    case 128: return launch_pf32_bs<128>(bs, a, st);
    default: return hipErrorInvalidValue;
  }
}

template <DT dt>
static hipError_t launch_pf_d(int d, int bs, const PrefillArgs& a, hipStream_t st) {
  switch (d) {
    case 64: return launch_pf_bs<dt, 64>(bs, a, st);
    case 128: return launch_pf_bs<dt, 128>(bs, a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill(int dt, int head_dim, int block_size, const PrefillArgs& a,
                          hipStream_t stream) {
  switch (dt) {
    case 0: return launch_pf32_d(head_dim, block_size, a, stream);
    case 1: return launch_pf_d<DT::F16>(head_dim, block_size, a, stream);
    case 2: return launch_pf_d<DT::BF16>(head_dim, block_size, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
