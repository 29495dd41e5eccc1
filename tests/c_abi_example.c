/*
 * c_abi_example.c — a plain C caller of libpa (include/pa.h), checked against the C oracle.
 *
 * Test infrastructure: built next to the library (with the oracle linked in) and run by
 * tests/test_gpu_c_abi.py on a GPU. It drives the boundary the way a C serving runtime would:
 * device buffers from hipMalloc, a stream of its own, then one decode step of a batch whose
 * blocks sit at random places in the pool:
 *   1. pa_copy_blocks: sequence 1 shares sequence 0's last, partly filled block; before it
 *      writes, that block is copied to a free block and sequence 1's table is repointed
 *      ([PA-summary] "Memory sharing: copy-on-write");
 *   2. pa_write_kv: every sequence appends its new token through the slot mapping
 *      ([PA-tutorial] §3.1);
 *   3. pa_decode: attention of every query head over the sequence's tokens
 *      ([PA-summary] "The PagedAttention algorithm").
 * The pools must match the oracle's bit for bit, and the outputs within
 * |gpu - ref| <= 2e-2 + 1e-2 |ref|. Slots that hold no token are NaN.
 * Exit status 0 when everything matches.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pa.h"

int oracle_decode(double *out, const void *q, const void *k_cache, const void *v_cache,
                  const int32_t *block_tables, const int32_t *context_lens, double scale,
                  int num_seqs, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                  int max_blocks_per_seq, int64_t num_blocks, int dtype, const int32_t *seq_list,
                  int n_list);
int oracle_write_kv(void *k_cache, void *v_cache, const void *k_new, const void *v_new,
                    const int32_t *slot_mapping, int n_tokens, int num_kv_heads, int head_dim,
                    int block_size, int64_t num_blocks, int elem_bytes);
int oracle_copy_blocks(void *k_cache, void *v_cache, const int32_t *pairs, int n_pairs,
                       int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                       int elem_bytes);

#define S 6
#define HQ 8
#define HKV 2
#define D 128
#define BS 16

#define CHECK_HIP(x)                                                        \
  do {                                                                      \
    hipError_t e_ = (x);                                                    \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));        \
      return 2;                                                             \
    }                                                                       \
  } while (0)
#define CHECK_PA(x)                                                         \
  do {                                                                      \
    pa_status s_ = (x);                                                     \
    if (s_ != PA_OK) {                                                      \
      fprintf(stderr, "%s failed: %s\n", #x, pa_status_string(s_));         \
      return 3;                                                             \
    }                                                                       \
  } while (0)

/* xorshift64* stream and Box-Muller normals: test inputs only */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double uniform01(void) {
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return ((rng_state * 2685821657736338717ull) >> 11) * (1.0 / 9007199254740992.0);
}
static float normal(void) {
  const double u = uniform01() + 1e-300, v = uniform01();
  return (float)(sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v));
}
/* bfloat16 bits of a finite float, rounded to nearest even */
static uint16_t bf16(float x) {
  uint32_t b;
  memcpy(&b, &x, 4);
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}
static double bf16_value(uint16_t h) {
  uint32_t b = (uint32_t)h << 16;
  float f;
  memcpy(&f, &b, 4);
  return f;
}

int main(void) {
  /* context lengths after this step's new token (T - 1 tokens already cached) */
  const int32_t lens[S] = {1, 40, 40, 300, 64, 17};
  int nblk[S], need = 0, maxb = 0;
  for (int s = 0; s < S; ++s) {
    nblk[s] = (lens[s] + BS - 1) / BS;
    need += nblk[s];
    if (nblk[s] > maxb) maxb = nblk[s];
  }
  const int N = need + 8;  /* spare blocks, one of them the copy-on-write target */
  const size_t pool_elems = (size_t)N * HKV * BS * D;
  uint16_t *kc = malloc(pool_elems * 2), *vc = malloc(pool_elems * 2);
  int32_t *perm = malloc(sizeof(int32_t) * N), *tables = malloc(sizeof(int32_t) * S * maxb);
  if (!kc || !vc || !perm || !tables) return 4;
  for (size_t i = 0; i < pool_elems; ++i) kc[i] = vc[i] = 0x7FC0; /* NaN: no token */
  for (int i = 0; i < N; ++i) perm[i] = i;
  for (int i = N - 1; i > 0; --i) {
    const int j = (int)(uniform01() * (i + 1));
    const int32_t t = perm[i]; perm[i] = perm[j]; perm[j] = t;
  }
  int next = 0;
  for (int s = 0; s < S; ++s)
    for (int j = 0; j < maxb; ++j) tables[s * maxb + j] = j < nblk[s] ? perm[next++] : -1;
  /* sequences 1 and 2 were forked from one prompt: they share its 39 cached tokens (three
     blocks, the last one partly filled); sequence 1 writes into the shared block first */
  for (int j = 0; j < nblk[1]; ++j) tables[2 * maxb + j] = tables[1 * maxb + j];
  const int32_t cow_dst = perm[next++];
  /* the T - 1 cached tokens of every sequence */
  for (int s = 0; s < S; ++s) {
    if (s == 2) continue; /* shares sequence 1's blocks */
    for (int t = 0; t < lens[s] - 1; ++t) {
      const int32_t blk = tables[s * maxb + t / BS];
      for (int h = 0; h < HKV; ++h)
        for (int c = 0; c < D; ++c) {
          const size_t i = (((size_t)blk * HKV + h) * BS + t % BS) * D + c;
          kc[i] = bf16(normal());
          vc[i] = bf16(normal());
        }
    }
  }
  /* copy-on-write: sequence 1's last block (shared, partly filled) goes to cow_dst */
  const int32_t pairs[2] = {tables[1 * maxb + nblk[1] - 1], cow_dst};
  tables[1 * maxb + nblk[1] - 1] = cow_dst;
  /* the step's new tokens: position T - 1 of every sequence */
  uint16_t kn[S * HKV * D], vn[S * HKV * D], q[S * HQ * D];
  int32_t slots[S];
  for (int s = 0; s < S; ++s) {
    const int t = lens[s] - 1;
    slots[s] = tables[s * maxb + t / BS] * BS + t % BS;
    for (int i = 0; i < HKV * D; ++i) {
      kn[s * HKV * D + i] = bf16(normal());
      vn[s * HKV * D + i] = bf16(normal());
    }
    for (int i = 0; i < HQ * D; ++i) q[s * HQ * D + i] = bf16(normal());
  }

  /* ---- the library, on a stream of its own ---- */
  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));
  void *dk, *dv, *dkn, *dvn, *dq, *dout, *dws = NULL;
  int32_t *dtab, *dlen, *dslots, *dpairs;
  CHECK_HIP(hipMalloc(&dk, pool_elems * 2));
  CHECK_HIP(hipMalloc(&dv, pool_elems * 2));
  CHECK_HIP(hipMalloc(&dkn, sizeof(kn)));
  CHECK_HIP(hipMalloc(&dvn, sizeof(vn)));
  CHECK_HIP(hipMalloc(&dq, sizeof(q)));
  CHECK_HIP(hipMalloc(&dout, sizeof(q)));
  CHECK_HIP(hipMalloc((void **)&dtab, sizeof(int32_t) * S * maxb));
  CHECK_HIP(hipMalloc((void **)&dlen, sizeof(lens)));
  CHECK_HIP(hipMalloc((void **)&dslots, sizeof(slots)));
  CHECK_HIP(hipMalloc((void **)&dpairs, sizeof(pairs)));
  CHECK_HIP(hipMemcpy(dk, kc, pool_elems * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dv, vc, pool_elems * 2, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dkn, kn, sizeof(kn), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dvn, vn, sizeof(vn), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dq, q, sizeof(q), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dtab, tables, sizeof(int32_t) * S * maxb, hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dlen, lens, sizeof(lens), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dslots, slots, sizeof(slots), hipMemcpyHostToDevice));
  CHECK_HIP(hipMemcpy(dpairs, pairs, sizeof(pairs), hipMemcpyHostToDevice));
  int maxT = 0;
  for (int s = 0; s < S; ++s) maxT = lens[s] > maxT ? lens[s] : maxT;
  const int partition = 64; /* force several partitions and the merge kernel */
  const size_t ws = pa_decode_workspace_size(S, HQ, HKV, D, BS, maxT, partition, PA_BF16);
  if (ws) CHECK_HIP(hipMalloc(&dws, ws));
  CHECK_PA(pa_copy_blocks(dk, dv, dpairs, 1, HKV, D, BS, N, PA_BF16, stream));
  CHECK_PA(pa_write_kv(dk, dv, dkn, dvn, dslots, S, HKV, D, BS, N, PA_BF16, stream));
  const float scale = 1.0f / sqrtf((float)D);
  CHECK_PA(pa_decode(dout, dq, dk, dv, dtab, dlen, scale, S, HQ, HKV, D, BS, maxb, N, maxT,
                     partition, dws, ws, PA_BF16, stream));
  CHECK_HIP(hipStreamSynchronize(stream));
  uint16_t *gk = malloc(pool_elems * 2), *gv = malloc(pool_elems * 2), out[S * HQ * D];
  if (!gk || !gv) return 4;
  CHECK_HIP(hipMemcpy(gk, dk, pool_elems * 2, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(gv, dv, pool_elems * 2, hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(out, dout, sizeof(out), hipMemcpyDeviceToHost));

  /* ---- the oracle on the host copies ---- */
  if (oracle_copy_blocks(kc, vc, pairs, 1, HKV, D, BS, N, 2) ||
      oracle_write_kv(kc, vc, kn, vn, slots, S, HKV, D, BS, N, 2))
    return 5;
  double *ref = malloc(sizeof(double) * S * HQ * D);
  if (!ref) return 4;
  if (oracle_decode(ref, q, kc, vc, tables, lens, (double)scale, S, HQ, HKV, D, BS, maxb, N, 2,
                    NULL, S))
    return 5;
  const int pools_equal = !memcmp(gk, kc, pool_elems * 2) && !memcmp(gv, vc, pool_elems * 2);
  double worst = 0.0;
  int bad = 0;
  for (int i = 0; i < S * HQ * D; ++i) {
    const double g = bf16_value(out[i]), err = fabs(g - ref[i]);
    if (!(err <= 2e-2 + 1e-2 * fabs(ref[i]))) ++bad;
    if (err > worst) worst = err;
  }
  printf("c_abi_example: pools %s, %d of %d outputs out of tolerance, max abs err %.3g\n",
         pools_equal ? "bit-identical" : "DIFFER", bad, S * HQ * D, worst);
  hipFree(dk); hipFree(dv); hipFree(dkn); hipFree(dvn); hipFree(dq); hipFree(dout);
  hipFree(dtab); hipFree(dlen); hipFree(dslots); hipFree(dpairs);
  if (dws) hipFree(dws);
  hipStreamDestroy(stream);
  return (pools_equal && bad == 0) ? 0 : 1;
}
