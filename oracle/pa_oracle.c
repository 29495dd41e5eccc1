/*
 * pa_oracle.c — plain, slow CPU oracle for paged decode attention, causal multi-query (prefill)
 * attention over the same pool, KV write, block copy and block swap.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline
 * leg load this library. The product (libpa) neither links nor calls it, and the two share no
 * code, header or constant.
 *
 * Sources:
 *   [PA-summary]  azimuth.plus, "Efficient Memory Management for Large Language Model Serving
 *                 with PagedAttention" (summary of Kwon et al., SOSP 2023).
 *   [PA-tutorial] un.csdn.net, "PagedAttention实战：如何用Python手搓一个高效KV缓存管理器".
 *
 * The decode oracle is the plain definition: [PA-summary] "The PagedAttention algorithm" states
 * that block-wise attention is mathematically identical to standard attention, and only the
 * memory layout differs. So each sequence's blocks are gathered into contiguous K and V through
 * the block table ([PA-tutorial] §3.2 gathers the valid part of each page and concatenates),
 * then textbook max-subtracted softmax attention runs in double precision.
 *
 * Readings where the pages leave a step open:
 *   - the last block contributes only its first T - j*B tokens (the B_j of the equation,
 *     valid_len in [PA-tutorial] §3.2);
 *   - query head h uses KV head h / (Hq/Hkv) (grouped heads are not on the pages);
 *   - T == 0 gives a zero output ([PA-tutorial] §3.2 returns zeros without pages);
 *   - a block-table entry that the sequence needs but that is outside the pool is an error;
 *   - multi-query attention: the n query tokens of a sequence are its last n cached tokens and
 *     query i sees positions 0 .. T-n+i (the causal rule; a decode step is n = 1).
 *
 * Element types: 0 = IEEE binary32, 1 = IEEE binary16, 2 = bfloat16 (the upper half of a
 * binary32). Every input element is widened exactly to double.
 *
 * All functions return 0 on success and a negative code on invalid input:
 *   -1 bad sizes, -2 block id out of the pool or table, -3 duplicate/overlapping indices,
 *   -4 allocation failure.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- exact widening of the three element types ------------------------------------------ */

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double half_bits_to_double(uint16_t h) {
  int sign = h >> 15;
  int e = (h >> 10) & 0x1f;
  int frac = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)frac, -24); /* subnormal: frac * 2^(1-15-10) */
  else if (e == 31)
    v = frac ? NAN : INFINITY;
  else
    v = ldexp((double)(frac | 0x400), e - 25); /* (1.frac) * 2^(e-15), as an integer * 2^-10 */
  return sign ? -v : v;
}

/* bfloat16 is the upper 16 bits of an IEEE binary32. */
static double bf16_bits_to_double(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double load_elem(const void *base, int64_t idx, int dtype) {
  if (dtype == 0) return (double)((const float *)base)[idx];
  if (dtype == 1) return half_bits_to_double(((const uint16_t *)base)[idx]);
  return bf16_bits_to_double(((const uint16_t *)base)[idx]);
}

int oracle_widen(double *dst, const void *src, int64_t n, int dtype) {
  if (n < 0 || dtype < 0 || dtype > 2) return -1;
  for (int64_t i = 0; i < n; ++i) dst[i] = load_elem(src, i, dtype);
  return 0;
}

/* ---- rounding double -> element type, round to nearest, ties to even ------------------- */

/* Round x to the nearest number that has p significand bits (implicit bit included), whose
 * exponent is at least emin (below that the quantum is fixed: subnormals), ties to even;
 * magnitudes that round above max_finite become infinities. Uses the default FP environment
 * (round-to-nearest-even) for nearbyint. */
static double round_to_format(double x, int p, int emin, double max_finite) {
  if (isnan(x) || isinf(x) || x == 0.0) return x;
  int e2;
  frexp(fabs(x), &e2);   /* |x| = m * 2^e2 with m in [0.5, 1): leading bit has weight 2^(e2-1) */
  int lead = e2 - 1;
  if (lead < emin) lead = emin;
  double quantum = ldexp(1.0, lead - (p - 1));
  double r = nearbyint(x / quantum) * quantum; /* x/quantum is exact: a power-of-two scaling */
  if (fabs(r) > max_finite) return copysign(INFINITY, x);
  return r;
}

/* dtype 0: binary32 (p=24, emin=-126), 1: binary16 (p=11, emin=-14), 2: bfloat16 (p=8,
 * emin=-126). The results are doubles that the target type represents exactly. */
int oracle_round(double *dst, const double *src, int64_t n, int dtype) {
  if (n < 0 || dtype < 0 || dtype > 2) return -1;
  for (int64_t i = 0; i < n; ++i) {
    double x = src[i];
    if (dtype == 0)
      dst[i] = round_to_format(x, 24, -126, ldexp(2.0 - ldexp(1.0, -23), 127));
    else if (dtype == 1)
      dst[i] = round_to_format(x, 11, -14, 65504.0);
    else
      dst[i] = round_to_format(x, 8, -126, ldexp(2.0 - ldexp(1.0, -7), 127));
  }
  return 0;
}

/* ---- decode attention ------------------------------------------------------------------- */

/* One query vector (row `qtok` of q, query head h) attending to the first T tokens of sequence
 * s: gather, score, softmax, weighted sum. `kbuf` and `vbuf` hold at least T*d doubles.
 * Returns 0 or a negative error. */
static int attend_one(double *out, const void *q, int64_t qtok, const void *k_cache,
                      const void *v_cache, const int32_t *block_tables, int T, double scale,
                      int s, int h, int num_q_heads, int num_kv_heads, int d, int B,
                      int max_blocks_per_seq, int64_t num_blocks, int dtype, double *kbuf,
                      double *vbuf, double *score) {
  const int group = num_q_heads / num_kv_heads;
  const int kv = h / group;
  for (int c = 0; c < d; ++c) out[c] = 0.0;
  if (T == 0) return 0;

  /* Gather: logical token t lives in logical block t / B at offset t % B; the block table maps
   * the logical block to its physical block. */
  for (int t = 0; t < T; ++t) {
    const int j = t / B;
    const int off = t % B;
    if (j >= max_blocks_per_seq) return -2;
    const int64_t phys = block_tables[(int64_t)s * max_blocks_per_seq + j];
    if (phys < 0 || phys >= num_blocks) return -2;
    const int64_t row = ((phys * num_kv_heads + kv) * B + off) * (int64_t)d;
    for (int c = 0; c < d; ++c) {
      kbuf[(int64_t)t * d + c] = load_elem(k_cache, row + c, dtype);
      vbuf[(int64_t)t * d + c] = load_elem(v_cache, row + c, dtype);
    }
  }

  /* Scores s_t = scale * q . K_t. */
  const int64_t qrow = (qtok * num_q_heads + h) * d;
  for (int t = 0; t < T; ++t) {
    double acc = 0.0;
    for (int c = 0; c < d; ++c) acc += load_elem(q, qrow + c, dtype) * kbuf[(int64_t)t * d + c];
    score[t] = scale * acc;
  }

  /* Softmax with the maximum subtracted, then the weighted sum of values. */
  double M = -INFINITY;
  for (int t = 0; t < T; ++t)
    if (score[t] > M) M = score[t];
  double L = 0.0;
  for (int t = 0; t < T; ++t) {
    score[t] = exp(score[t] - M);
    L += score[t];
  }
  for (int t = 0; t < T; ++t)
    for (int c = 0; c < d; ++c)
      out[c] += score[t] * vbuf[(int64_t)t * d + c];
  for (int c = 0; c < d; ++c) out[c] /= L;
  return 0;
}

/*
 * out: double [n_list][num_q_heads][head_dim], one row block per listed sequence.
 * seq_list: the sequences to evaluate (n_list entries), or NULL for all sequences in order
 * (then n_list must equal num_seqs).
 */
int oracle_decode(double *out, const void *q, const void *k_cache, const void *v_cache,
                  const int32_t *block_tables, const int32_t *context_lens, double scale,
                  int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                  int max_blocks_per_seq, int64_t num_blocks, int dtype, const int32_t *seq_list,
                  int n_list) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || max_blocks_per_seq < 0 || num_blocks < 0 || dtype < 0 || dtype > 2 ||
      n_list < 0 || num_q_heads % num_kv_heads != 0)
    return -1;
  if (!seq_list && n_list != num_seqs) return -1;
  int max_T = 0;
  for (int i = 0; i < n_list; ++i) {
    const int s = seq_list ? seq_list[i] : i;
    if (s < 0 || s >= num_seqs || context_lens[s] < 0) return -1;
    if (context_lens[s] > max_T) max_T = context_lens[s];
  }
  const int64_t npairs = (int64_t)n_list * num_q_heads;
  int err = 0;
#pragma omp parallel
  {
    double *kbuf = (double *)malloc(sizeof(double) * ((size_t)max_T * head_dim + 1));
    double *vbuf = (double *)malloc(sizeof(double) * ((size_t)max_T * head_dim + 1));
    double *score = (double *)malloc(sizeof(double) * ((size_t)max_T + 1));
    if (!kbuf || !vbuf || !score) {
#pragma omp atomic write
      err = -4;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t p = 0; p < npairs; ++p) {
      if (!kbuf || !vbuf || !score) continue;
      const int i = (int)(p / num_q_heads);
      const int h = (int)(p % num_q_heads);
      const int s = seq_list ? seq_list[i] : i;
      int e = attend_one(out + p * head_dim, q, s, k_cache, v_cache, block_tables,
                         context_lens[s], scale, s, h, num_q_heads, num_kv_heads, head_dim,
                         block_size, max_blocks_per_seq, num_blocks, dtype, kbuf, vbuf, score);
      if (e) {
#pragma omp atomic write
        err = e;
      }
    }
    free(kbuf);
    free(vbuf);
    free(score);
  }
  return err;
}

/* ---- multi-query (prefill / chunked-prefill) attention ---------------------------------------
 *
 * [PA-summary] "The PagedAttention algorithm" runs the block-table walk for each query vector.
 * When a sequence receives n new tokens at once (a prompt, or a chunk of one), those n tokens
 * are the last n of its T cached tokens, and each of them is a query vector. Reading (the
 * pages give no mask explicitly): query i (0 <= i < n) sits at position T - n + i and attends
 * to the tokens at positions 0 .. T - n + i, itself included -- the causal rule of
 * autoregressive attention, under which a decode step is the case n = 1.
 *
 * q, out rows: query tokens of sequence s are rows query_start[s] .. query_start[s+1]-1 of
 * q [num_q_tokens][num_q_heads][head_dim]; out is double [num_q_tokens][num_q_heads][head_dim]
 * (rows no sequence owns are left untouched). query_start is non-decreasing, query_start[0]
 * >= 0, query_start[num_seqs] <= num_q_tokens, and n_s <= context_lens[s] (error -1 otherwise).
 */
int oracle_prefill(double *out, const void *q, const void *k_cache, const void *v_cache,
                   const int32_t *block_tables, const int32_t *context_lens,
                   const int32_t *query_start, double scale, int num_seqs, int num_q_tokens,
                   int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                   int max_blocks_per_seq, int64_t num_blocks, int dtype) {
  if (num_seqs < 0 || num_q_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || block_size <= 0 || max_blocks_per_seq < 0 || num_blocks < 0 ||
      dtype < 0 || dtype > 2 || num_q_heads % num_kv_heads != 0)
    return -1;
  if (num_seqs > 0 && (query_start[0] < 0 || query_start[num_seqs] > num_q_tokens)) return -1;
  int max_T = 0;
  for (int s = 0; s < num_seqs; ++s) {
    const int n = query_start[s + 1] - query_start[s];
    if (n < 0 || context_lens[s] < 0 || n > context_lens[s]) return -1;
    if (context_lens[s] > max_T) max_T = context_lens[s];
  }
  /* one work item per (sequence, query token, query head) */
  const int64_t rows = num_seqs > 0 ? (int64_t)query_start[num_seqs] - query_start[0] : 0;
  const int64_t items = rows * num_q_heads;
  int err = 0;
#pragma omp parallel
  {
    double *kbuf = (double *)malloc(sizeof(double) * ((size_t)max_T * head_dim + 1));
    double *vbuf = (double *)malloc(sizeof(double) * ((size_t)max_T * head_dim + 1));
    double *score = (double *)malloc(sizeof(double) * ((size_t)max_T + 1));
    if (!kbuf || !vbuf || !score) {
#pragma omp atomic write
      err = -4;
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t it = 0; it < items; ++it) {
      if (!kbuf || !vbuf || !score) continue;
      const int64_t qtok = query_start[0] + it / num_q_heads;
      const int h = (int)(it % num_q_heads);
      int s = 0; /* the sequence that owns row qtok */
      while (query_start[s + 1] <= qtok) ++s;
      const int T = context_lens[s];
      const int n = query_start[s + 1] - query_start[s];
      const int i = (int)(qtok - query_start[s]);
      const int visible = T - n + i + 1; /* positions 0 .. T-n+i */
      int e = attend_one(out + qtok * (int64_t)num_q_heads * head_dim + (int64_t)h * head_dim,
                         q, qtok, k_cache, v_cache, block_tables, visible, scale, s, h,
                         num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                         num_blocks, dtype, kbuf, vbuf, score);
      if (e) {
#pragma omp atomic write
        err = e;
      }
    }
    free(kbuf);
    free(vbuf);
    free(score);
  }
  return err;
}

/* ---- KV write: [PA-tutorial] §3.1 append_kv --------------------------------------------- */

/* A slot outside [0, num_blocks*B) is skipped, as is a negative slot. Two tokens with the same
 * slot are an error (the pages define no winner). */
int oracle_write_kv(void *k_cache, void *v_cache, const void *k_new, const void *v_new,
                    const int32_t *slot_mapping, int n_tokens, int num_kv_heads, int head_dim,
                    int block_size, int64_t num_blocks, int elem_bytes) {
  if (n_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks < 0 || (elem_bytes != 2 && elem_bytes != 4))
    return -1;
  const int64_t nslots = num_blocks * block_size;
  for (int i = 0; i < n_tokens; ++i)
    for (int k = i + 1; k < n_tokens; ++k)
      if (slot_mapping[i] >= 0 && slot_mapping[i] == slot_mapping[k]) return -3;
  const size_t row_bytes = (size_t)head_dim * elem_bytes;
  for (int i = 0; i < n_tokens; ++i) {
    const int64_t slot = slot_mapping[i];
    if (slot < 0 || slot >= nslots) continue;
    const int64_t blk = slot / block_size, off = slot % block_size;
    for (int h = 0; h < num_kv_heads; ++h) {
      const int64_t dst = ((blk * num_kv_heads + h) * block_size + off) * (int64_t)row_bytes;
      const int64_t src = ((int64_t)i * num_kv_heads + h) * (int64_t)row_bytes;
      memcpy((char *)k_cache + dst, (const char *)k_new + src, row_bytes);
      memcpy((char *)v_cache + dst, (const char *)v_new + src, row_bytes);
    }
  }
  return 0;
}

/* ---- block copy: [PA-summary] "Memory sharing: copy-on-write" ---------------------------- */

/* Whole-block copies. Pairs with an id outside the pool are skipped (as the library does); a
 * dst that is also a src, or a repeated dst, is an error. */
int oracle_copy_blocks(void *k_cache, void *v_cache, const int32_t *pairs, int n_pairs,
                       int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                       int elem_bytes) {
  if (n_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks < 0 ||
      (elem_bytes != 2 && elem_bytes != 4))
    return -1;
  for (int i = 0; i < n_pairs; ++i)
    for (int k = 0; k < n_pairs; ++k) {
      if (k != i && pairs[2 * i + 1] == pairs[2 * k + 1]) return -3;
      if (pairs[2 * i + 1] == pairs[2 * k]) return -3;
    }
  const size_t block_bytes = (size_t)num_kv_heads * block_size * head_dim * elem_bytes;
  for (int i = 0; i < n_pairs; ++i) {
    const int64_t src = pairs[2 * i], dst = pairs[2 * i + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) continue;
    memcpy((char *)k_cache + dst * block_bytes, (const char *)k_cache + src * block_bytes,
           block_bytes);
    memcpy((char *)v_cache + dst * block_bytes, (const char *)v_cache + src * block_bytes,
           block_bytes);
  }
  return 0;
}

/* ---- block swap between two pools: [PA-summary] "vLLM" (preemption moves a request's
 * blocks to CPU memory and back) ------------------------------------------------------------ */

/* dst_pool[dst] = src_pool[src] for K and V, whole blocks. Pairs with an id outside its pool
 * are skipped; a repeated dst is an error. */
int oracle_swap_blocks(void *dst_k, void *dst_v, int64_t dst_num_blocks, const void *src_k,
                       const void *src_v, int64_t src_num_blocks, const int32_t *pairs,
                       int n_pairs, int num_kv_heads, int head_dim, int block_size,
                       int elem_bytes) {
  if (n_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      dst_num_blocks < 0 || src_num_blocks < 0 || (elem_bytes != 2 && elem_bytes != 4))
    return -1;
  for (int i = 0; i < n_pairs; ++i)
    for (int k = i + 1; k < n_pairs; ++k)
      if (pairs[2 * i + 1] == pairs[2 * k + 1]) return -3;
  const size_t block_bytes = (size_t)num_kv_heads * block_size * head_dim * elem_bytes;
  for (int i = 0; i < n_pairs; ++i) {
    const int64_t src = pairs[2 * i], dst = pairs[2 * i + 1];
    if (src < 0 || src >= src_num_blocks || dst < 0 || dst >= dst_num_blocks) continue;
    memcpy((char *)dst_k + dst * block_bytes, (const char *)src_k + src * block_bytes,
           block_bytes);
    memcpy((char *)dst_v + dst * block_bytes, (const char *)src_v + src * block_bytes,
           block_bytes);
  }
  return 0;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Sets the number of threads the calls that follow use (n > 0); for timing the oracle on one
 * core beside all of them. The arithmetic does not depend on it. */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
  if (n > 0) omp_set_num_threads(n);
#else
  (void)n;
#endif
}
