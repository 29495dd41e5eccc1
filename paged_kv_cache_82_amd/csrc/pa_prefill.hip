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
//     query heads of its group; a wave owns NCT tiles of 16 rows and reuses every K/V step it
//     loads for all of them; a workgroup of NW waves covers NW * NCT * 16 consecutive rows;
//   - a wave walks the 32-token steps of positions 0 .. (its last row's position), keeping a
//     ring of NBUF steps of K/V in registers (the loads of the next step are in flight while
//     one is consumed); only steps that reach past the wave's first position apply the mask;
//   - physical block ids come 64 steps at a time into one register (lane k = step k) and are
//     broadcast with readlane; the next 64 are loaded while the current ones are used;
//   - workgroups are ordered so that the row tiles of one (sequence, KV head) run on one XCD
//     (workgroups are dealt round-robin over the 8 XCDs) and share that XCD's L2, heaviest
//     (latest) tiles first.
// Scores are kept in the base-2 exponent domain: s' = s * log2(e), exp(s - m) = 2^(s' - m').
#include "pa_device.h"
#include "pa_internal.h"
#include "pa_mfma.h"

namespace pa {

namespace {

constexpr int kPrefillWaves = 4;     // waves per workgroup
constexpr int kPrefillColTiles = 2;  // 16-row column tiles per wave
constexpr int kPrefillBuffers = 2;   // 32-token K/V steps held in registers
constexpr int kXcds = 8;             // MI355X: workgroups are dealt round-robin over 8 XCDs

__device__ __forceinline__ int clampi(int x, int lo, int hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

}  // namespace

template <DT dt, int D, int BS, int NW, int NCT, int NBUF>
__global__ __launch_bounds__(NW * 64, 1) void prefill_mfma_kernel(const PrefillArgs a) {
  static_assert(dt != DT::F32, "MFMA path takes 16-bit inputs");
  static_assert(BS <= 32 && 32 % BS == 0, "a 32-token step spans whole blocks");
  using M = MfmaT<dt>;
  using vec8 = typename M::vec8;
  using VF = VFrag<D>;
  constexpr int E = 2;
  constexpr int KC = D / 32;  // q.K MFMAs per 16-token tile
  constexpr int MT = D / 16;  // p.V M-tiles; row r of tile mt is head dimension MT*r + mt
  constexpr int NBS = 32 / BS;
  constexpr int ROWS_W = 16 * NCT;
  constexpr int ROWS = NW * ROWS_W;

  // Workgroup -> (row tile, KV head, sequence). Linear id L runs on XCD L % 8; renumber so
  // that each XCD takes a contiguous range of tiles (whole (sequence, KV head) groups).
  const int Hkv = a.num_kv_heads;
  const int64_t total = (int64_t)a.row_tiles * Hkv * a.num_seqs;
  int64_t L = blockIdx.x;
  const int64_t per = total / kXcds;
  if (L < per * kXcds) L = (L % kXcds) * per + L / kXcds;
  const int tile = a.row_tiles - 1 - (int)(L % a.row_tiles);
  const int64_t rest = L / a.row_tiles;
  const int kvh = (int)(rest % Hkv);
  const int s = (int)(rest / Hkv);

  // Extent of the sequence, clamped into the buffers the sizes describe.
  const int Nq = a.num_q_tokens;
  const int q0 = clampi(a.query_start[s], 0, Nq);
  const int q1 = clampi(a.query_start[s + 1], q0, Nq);
  const int64_t cap64 = (int64_t)a.max_blocks_per_seq * BS;
  const int cap = (int)(cap64 < (int64_t)a.max_context_len ? cap64 : (int64_t)a.max_context_len);
  const int T = clampi(a.context_lens[s], 0, cap);
  int n = q1 - q0;
  n = n < T ? n : T;
  n = n < a.max_query_len ? n : a.max_query_len;
  const int Hq = a.num_q_heads;
  const int g = Hq / Hkv;
  const int nrows = n * g;

  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int hh = lane & 15, gq = lane >> 4;
  const int R0 = tile * ROWS + w * ROWS_W;  // first row of this wave
  if (R0 >= nrows) return;                  // no barrier below: idle waves leave at once
  const int base_pos = T - n;               // position of the chunk's first query token
  const int R_last = (R0 + ROWS_W < nrows ? R0 + ROWS_W : nrows) - 1;
  const int p_lo = base_pos + R0 / g;       // smallest position among this wave's rows
  const int p_hi = base_pos + R_last / g;   // largest
  const int ns = (p_hi + 32) / 32;          // 32-token steps covering positions 0 .. p_hi
  const int jlast = p_hi / BS;              // last block any row of this wave reads

  // Block ids: lane k of ids_cur holds the NBS ids of step 64*chunk + k.
  const int32_t* bt = a.block_tables + (int64_t)s * a.max_blocks_per_seq;
  auto load_ids = [&](int chunk, int (&ids)[NBS]) {
#pragma unroll
    for (int b = 0; b < NBS; ++b) {
      const int j = (chunk * 64 + lane) * NBS + b;
      ids[b] = (j <= jlast) ? bt[j] : 0;  // jlast < max_blocks_per_seq since T <= cap
    }
  };
  int ids_cur[NBS], ids_nxt[NBS];
  int cur_chunk = 0;
  load_ids(0, ids_cur);
  load_ids(1, ids_nxt);

  // Query columns: column hh of tile c is row R = R0 + 16c + hh = (token R / g, head R % g).
  int pos[NCT];  // position of the column's query token; -1 for rows past the chunk
  vec8 qop[NCT][KC];
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    const int R = R0 + 16 * c + hh;
    const bool valid = R < nrows;
    const int i = valid ? R / g : 0;
    const int head = kvh * g + (valid ? R % g : 0);
    pos[c] = valid ? base_pos + i : -1;
#pragma unroll
    for (int kk = 0; kk < KC; ++kk) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (valid)
        raw = load16((const char*)a.q +
                     (((int64_t)(q0 + i) * Hq + head) * D + 32 * kk + 8 * gq) * E);
      qop[c][kk] = __builtin_bit_cast(vec8, raw);
    }
  }

  f32x4 oacc[NCT][MT];
  float m[NCT], lsum[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    m[c] = kNegInf;
    lsum[c] = 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) oacc[c][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const char* kbase = (const char*)a.k_cache;
  const char* vbase = (const char*)a.v_cache;
  constexpr int RB = D * E;  // bytes per token row
  const uint32_t koff = (uint32_t)((hh % BS) * RB + 8 * gq * E);
  const uint32_t voff = (uint32_t)(((4 * gq) % BS) * RB + MT * hh * E);
  const int64_t tile_bytes = (int64_t)BS * RB;

  auto fetch = [&](int k, StepRegs<D, KC>& Rg) {
    const bool cur = (k >> 6) == cur_chunk;  // wave-uniform
    const int kl = k & 63;
    const int id0 = cur ? __builtin_amdgcn_readlane(ids_cur[0], kl)
                        : __builtin_amdgcn_readlane(ids_nxt[0], kl);
    const char* kt[NBS];
    const char* vt[NBS];
#pragma unroll
    for (int b = 0; b < NBS; ++b) {
      const int idb = cur ? __builtin_amdgcn_readlane(ids_cur[b], kl)
                          : __builtin_amdgcn_readlane(ids_nxt[b], kl);
      // a block past the last one this wave needs holds only positions no row sees: read the
      // step's first block instead (its V is zeroed and its scores masked in consume)
      const int32_t id = (k * NBS + b <= jlast) ? idb : id0;
      const int64_t t = (clamp_block(id, a.num_blocks) * Hkv + kvh) * tile_bytes;
      kt[b] = kbase + t;
      vt[b] = vbase + t;
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const char* rp;
      if constexpr (BS >= 16) {
        rp = kt[(16 * u) / BS] + koff + ((16 * u) % BS) * RB;
      } else {  // BS == 8: lanes hh < 8 and hh >= 8 read different blocks
        rp = kt[2 * u + (hh >> 3)] + koff;
      }
#pragma unroll
      for (int kk = 0; kk < KC; ++kk) Rg.k[u][kk] = load16(rp + 32 * kk * E);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const char* rp;
        if constexpr (BS >= 16) {
          rp = vt[(16 * u) / BS] + voff + ((16 * u) % BS + i) * RB;
        } else {  // token 16u + 4gq + i sits in block 2u + gq/2 at row 4*(gq&1) + i
          rp = vt[2 * u + (gq >> 1)] + voff + i * RB;
        }
        Rg.v[u][i] = VF::load(rp);
      }
    __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the consume that follows
  };

  auto consume = [&](int k, StepRegs<D, KC>& Rg) {
    const int tau0 = k * 32;
    if (tau0 + 31 > p_hi) {  // tokens after the wave's last position: zero V (select)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tau0 + 16 * u + 4 * gq + i > p_hi) Rg.v[u][i] = typename VF::T{};
    }
    const bool masked = tau0 + 31 > p_lo;
    // V^T operand of M-tile mt, k element e <-> token 16*(e/4) + 4*gq + (e%4); shared by
    // every column tile
    u32x4 vw[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int q2 = 0; q2 < 4; ++q2) {
        const int e0 = 2 * q2, e1 = 2 * q2 + 1;
        const uint32_t lo = vfrag_elem<D>(Rg.v[e0 / 4][e0 % 4], mt);
        const uint32_t hi = vfrag_elem<D>(Rg.v[e1 / 4][e1 % 4], mt);
        vw[mt][q2] = lo | (hi << 16);
      }
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      f32x4 sacc[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        sacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KC; ++kk)
          sacc[u] = M::mma(__builtin_bit_cast(vec8, Rg.k[u][kk]), qop[c][kk], sacc[u]);
      }
      float sc[8];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = sacc[u][i] * a.scale_log2;
          if (masked && tau0 + 16 * u + 4 * gq + i > pos[c]) x = kNegInf;  // select
          sc[4 * u + i] = x;
        }
      float bm = sc[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) bm = fmaxf(bm, sc[e]);
      bm = fmaxf(bm, __shfl_xor(bm, 16));
      bm = fmaxf(bm, __shfl_xor(bm, 32));
      const float mn = fmaxf(m[c], bm);
      const bool empty = (mn == kNegInf);  // no visible token yet for this column
      const float corr = empty ? 1.0f : fast_exp2(m[c] - mn);
      vec8 pop;
      float ps = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = empty ? 0.0f : fast_exp2(sc[e] - mn);
        ps += pe;
        pop[e] = (typename M::scalar)pe;
      }
      lsum[c] = fmaf(lsum[c], corr, ps);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) oacc[c][mt] *= corr;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        oacc[c][mt] = M::mma(__builtin_bit_cast(vec8, vw[mt]), pop, oacc[c][mt]);
      m[c] = mn;
    }
  };

  {  // ring of NBUF register buffers, unconditional prefetch (past the end: the last step)
    StepRegs<D, KC> rb[NBUF];
#pragma unroll
    for (int u = 0; u + 1 < NBUF; ++u) fetch(u < ns ? u : ns - 1, rb[u]);
    for (int k = 0; k < ns; k += NBUF) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        const int kk = k + u;
        if (kk >= ns) break;
        if ((kk & 63) == 0 && kk > 0) {  // next 64 steps: rotate the id registers
#pragma unroll
          for (int b = 0; b < NBS; ++b) ids_cur[b] = ids_nxt[b];
          cur_chunk = kk >> 6;
          load_ids(cur_chunk + 1, ids_nxt);
        }
        const int ahead = kk + NBUF - 1;
        fetch(ahead < ns ? ahead : ns - 1, rb[(u + NBUF - 1) % NBUF]);
        consume(kk, rb[u]);
      }
    }
  }

  // Normalise and store. oacc[c][mt][i] is O[column hh][dim MT*(4*gq + i) + mt]: for fixed i
  // the MT values are consecutive dimensions, one 16-byte (D = 128) or 8-byte (D = 64) store.
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    float l = lsum[c];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (pos[c] < 0) continue;
    const int R = R0 + 16 * c + hh;
    const int i = R / g;
    const int head = kvh * g + R % g;
    char* orow = (char*)a.out + ((int64_t)(q0 + i) * Hq + head) * D * E;
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      uint32_t packed[MT / 2];
#pragma unroll
      for (int h2 = 0; h2 < MT / 2; ++h2) {
        const uint32_t lo = narrow_bits<dt>(oacc[c][2 * h2][i4] / l);
        const uint32_t hi = narrow_bits<dt>(oacc[c][2 * h2 + 1][i4] / l);
        packed[h2] = lo | (hi << 16);
      }
      char* dst = orow + MT * (4 * gq + i4) * E;
      if constexpr (MT == 8) {
        *reinterpret_cast<u32x4*>(dst) = u32x4{packed[0], packed[1], packed[2], packed[3]};
      } else {
        *reinterpret_cast<u32x2*>(dst) = u32x2{packed[0], packed[1]};
      }
    }
  }
}

// ---- host side ------------------------------------------------------------------------------

int prefill_rows_per_workgroup() { return kPrefillWaves * kPrefillColTiles * 16; }

bool prefill_supported(int dt, int head_dim, int block_size) {
  if (dt != 1 && dt != 2) return false;  // 16-bit inputs (MFMA)
  if (head_dim != 64 && head_dim != 128) return false;
  return block_size == 8 || block_size == 16 || block_size == 32;
}

template <DT dt, int D, int BS>
static hipError_t launch_pf(const PrefillArgs& a, hipStream_t stream) {
  const int64_t total = (int64_t)a.row_tiles * a.num_kv_heads * a.num_seqs;
  if (total == 0) return hipSuccess;
  PrefillArgs args_copy = a;
  void* args[] = {&args_copy};
  return hipLaunchKernel(
      (const void*)prefill_mfma_kernel<dt, D, BS, kPrefillWaves, kPrefillColTiles,
                                       kPrefillBuffers>,
      dim3((unsigned)total), dim3(kPrefillWaves * 64), args, 0, stream);
}

template <DT dt, int D>
static hipError_t launch_pf_bs(int bs, const PrefillArgs& a, hipStream_t st) {
  switch (bs) {
    case 8: return launch_pf<dt, D, 8>(a, st);
    case 16: return launch_pf<dt, D, 16>(a, st);
    case 32: return launch_pf<dt, D, 32>(a, st);
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
    case 1: return launch_pf_d<DT::F16>(head_dim, block_size, a, stream);
    case 2: return launch_pf_d<DT::BF16>(head_dim, block_size, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
