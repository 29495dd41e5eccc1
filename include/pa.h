/*
 * pa.h — C ABI of libpa: paged KV-cache attention for AMD MI355X (gfx950): slot-mapped KV
 * writes, decode and causal multi-query (prefill) attention through block tables, and
 * whole-block copies (copy-on-write) and moves between pools (swap).
 *
 * Sources cited in this header (the method is defined there; nothing else is):
 *   [PA-summary]  azimuth.plus, "Efficient Memory Management for Large Language Model Serving
 *                 with PagedAttention" (an Arabic summary of Kwon et al., SOSP 2023).
 *   [PA-tutorial] un.csdn.net, "PagedAttention实战：如何用Python手搓一个高效KV缓存管理器"
 *                 ("PagedAttention in practice: a KV-cache manager built by hand in Python").
 *
 * Data layout shared by every call (all arrays dense, row-major, no padding):
 *   k_cache, v_cache   [num_blocks][num_kv_heads][block_size][head_dim]   dtype `dt`
 *                      The physical block pool. One (block, head) tile is block_size*head_dim
 *                      contiguous elements, the per-head B x d view of a block that
 *                      [PA-summary] "The PagedAttention algorithm" (K_j, V_j in R^{B x d}) uses.
 *   block_tables       int32 [num_seqs][max_blocks_per_seq]; entry j of row s is the physical
 *                      block that holds tokens j*B .. j*B+B-1 of sequence s ([PA-summary]
 *                      "Key idea: virtual memory for the KV cache"; [PA-tutorial] §2.1 PageTable).
 *                      Entries at or beyond ceil(context_lens[s]/B) never affect the result
 *                      (they may be read, never beyond max_blocks_per_seq).
 *   context_lens       int32 [num_seqs]; T_s, the number of cached tokens of sequence s.
 *   slot_mapping       int32 [n_tokens]; slot = physical_block*block_size + offset_in_block
 *                      ([PA-tutorial] §3.1 append_kv: page = pos // page_size, offset =
 *                      pos % page_size); a negative slot means "skip this token".
 *   q, out             [num_seqs][num_q_heads][head_dim]                 dtype `dt`
 *   k_new, v_new       [n_tokens][num_kv_heads][head_dim]                dtype `dt`
 *   block_pairs        int32 [n_pairs][2] = (src, dst) physical block ids.
 *
 * Query head h reads KV head h / (num_q_heads / num_kv_heads) (contiguous groups).
 *
 * Ownership and execution: every pointer except the return of pa_status_string is a DEVICE
 * pointer owned by the caller. The library allocates no memory at call time and keeps no state
 * between calls, with two stated exceptions: the process-wide kernel choice of
 * pa_set_decode_kernel, and the static per-GPU scratch array of pa_decode_noalloc (part of the
 * library's device image, PA_DECODE_SCRATCH_BYTES per GPU, held until the process ends).
 * Each call validates its scalar arguments and pointer alignment on the host, enqueues its
 * kernel(s) on `stream` (a hipStream_t; NULL = the null stream) and returns without waiting
 * for completion. q, k_cache, v_cache, k_new and v_new must be 16-byte aligned; the workspace
 * 256-byte aligned; index arrays 4-byte aligned (PA_ERR_INVALID_ARG otherwise).
 *
 * Device-resident indices (block ids, slots, context lengths) are not validated on the host.
 * The kernels clamp them into the buffers the sizes describe, so a bad index gives an undefined
 * result but never an access outside the caller's buffers: block ids are clamped to
 * [0, num_blocks), context lengths to [0, min(max_context_len, max_blocks_per_seq*block_size)],
 * and slots outside [0, num_blocks*block_size) are skipped.
 *
 * Errors: no exception crosses the ABI. PA_ERR_INVALID_ARG for a null pointer, a non-positive
 * size, num_q_heads % num_kv_heads != 0 or an element count that overflows int64;
 * PA_ERR_UNSUPPORTED for a (dtype, head_dim, block_size) the kernels are not built for;
 * PA_ERR_WORKSPACE for a workspace smaller than pa_decode_workspace_size; PA_ERR_HIP when the
 * HIP runtime reports an error at launch.
 *
 * Supported shapes: dtype f32, f16, bf16; head_dim 64 or 128; block_size 8, 16, 32 or 64.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2 } pa_dtype;

/* Decode kernel choice (pa_set_decode_kernel). */
typedef enum { PA_DECODE_AUTO = 0, PA_DECODE_VALU = 1, PA_DECODE_MFMA = 2 } pa_decode_kernel;

/* Size of the static per-GPU split-K scratch array that pa_decode_noalloc uses (16 MiB). */
#define PA_DECODE_SCRATCH_BYTES ((size_t)16 << 20)

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,
  PA_ERR_UNSUPPORTED = 2,
  PA_ERR_WORKSPACE = 3,
  PA_ERR_HIP = 4,
  PA_ERR_NO_BLOCKS = 5 /* host block manager: the free list cannot cover the request */
} pa_status;

/*
 * pa_write_kv — slot-mapped append of new keys and values into the block pool.
 * [PA-tutorial] §3.1 (SequenceManager.append_kv): a token at position pos lands in logical page
 * pos // B at offset pos % B of the physical page the page table maps it to; [PA-summary]
 * "Key idea": physical blocks are filled one at a time as tokens arrive.
 * For every i < n_tokens with 0 <= slot_mapping[i] < num_blocks*block_size and every KV head h:
 *   k_cache[slot/B][h][slot%B][:] = k_new[i][h][:]   and the same for v_cache / v_new.
 * A bit copy. Tokens with a negative or out-of-pool slot are skipped. Two tokens with the same
 * slot in one call are a caller error (which write wins is unspecified). n_tokens == 0 is a
 * valid no-op. Copy-on-write of a shared block is the caller's job (pa_copy_blocks) before
 * the write.
 */
pa_status pa_write_kv(void *k_cache, void *v_cache, const void *k_new, const void *v_new,
                      const int32_t *slot_mapping, int n_tokens, int num_kv_heads,
                      int head_dim, int block_size, int64_t num_blocks, pa_dtype dt,
                      void *stream);

/*
 * pa_decode_workspace_size — bytes of device workspace pa_decode needs for these sizes.
 * The workspace holds the per-partition partial results (running max, running sum and partial
 * output, fp32) of every (sequence, query head).
 * partition_tokens: 0 = let the library choose (the same choice pa_decode makes for the same
 * arguments); > 0 must be a multiple of 32 and at most 64*4*min(block_size, 16) tokens
 * (fp32 and single-head groups) or 8192 tokens (grouped heads).
 * Returns 0 when no workspace is needed (every sequence fits one partition) and for invalid
 * sizes.
 */
size_t pa_decode_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                int block_size, int max_context_len, int partition_tokens,
                                pa_dtype dt);

/*
 * pa_decode — single-query (decode) attention of every sequence's query heads over its cached
 * tokens, read block by block through the block table.
 * [PA-summary] "The PagedAttention algorithm": for each query vector the kernel walks the
 * block table, fetches K_j and V_j from non-contiguous physical blocks, forms partial attention
 * per block with the block's own score maximum and merges the blocks with the log-sum-exp
 * rescaling of the block-wise attention equation; the result equals standard attention.
 * For every sequence s and query head h, with T = context_lens[s] and g = H_q/H_kv:
 *   s_t  = scale * q[s][h] . K_t,   t < T,   K_t = k_cache[block_tables[s][t/B]][h/g][t%B]
 *   out[s][h] = sum_t exp(s_t - M) V_t / sum_t exp(s_t - M),  M = max_t s_t
 * computed in fp32 and rounded to nearest-even in `dt`. T == 0 gives out = 0 ([PA-tutorial]
 * §3.2 returns zeros when a sequence has no pages). Tail slots of the last block (t >= T) and
 * blocks the table does not reach never influence the result, whatever they hold.
 * Long contexts are split into partitions of partition_tokens tokens processed by separate
 * workgroups; each writes its (max, sum, partial output) to `workspace` and a second kernel
 * on the same stream merges them with the same log-sum-exp rescaling.
 * max_context_len: a host-known upper bound on context_lens (sizes the grid; no device read).
 * workspace: device buffer of >= pa_decode_workspace_size(...) bytes, 256-byte aligned, any
 * contents (may be NULL when that size is 0). One workspace serves any number of calls
 * ordered on one stream; calls that may overlap in time must not share one.
 */
pa_status pa_decode(void *out, const void *q, const void *k_cache, const void *v_cache,
                    const int32_t *block_tables, const int32_t *context_lens, float scale,
                    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                    int block_size, int max_blocks_per_seq, int64_t num_blocks,
                    int max_context_len, int partition_tokens, void *workspace,
                    size_t workspace_bytes, pa_dtype dt, void *stream);

/*
 * pa_decode_noalloc — pa_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. Same arguments, layouts,
 * result (bit for bit: the same kernels with the same partition choice) and errors as
 * pa_decode, without the workspace arguments: the split-K partials go to a static array of
 * PA_DECODE_SCRATCH_BYTES in the library's device image, one per GPU, held until the process
 * ends. The call allocates nothing (no hipMalloc, no allocating library routine).
 * Limit: a call whose partition plan needs more partial-state bytes than
 * PA_DECODE_SCRATCH_BYTES (pa_decode_workspace_size of the same arguments) returns
 * PA_ERR_WORKSPACE and launches nothing; 16 MiB holds, for example, 8 sequences x 32 heads x 64
 * partitions at head_dim 128. Nothing in the array needs clearing between calls (every partial
 * is written before it is read).
 * Every call on one GPU shares that GPU's array: calls that may overlap in time on one GPU
 * (different streams, or different host threads without ordering) race and must not be issued.
 * The array's device address is looked up once per GPU (hipGetSymbolAddress, on the first call
 * on that GPU that splits a sequence); PA_ERR_HIP if that lookup fails.
 */
pa_status pa_decode_noalloc(void *out, const void *q, const void *k_cache, const void *v_cache,
                            const int32_t *block_tables, const int32_t *context_lens,
                            float scale, int num_seqs, int num_q_heads, int num_kv_heads,
                            int head_dim, int block_size, int max_blocks_per_seq,
                            int64_t num_blocks, int max_context_len, int partition_tokens,
                            pa_dtype dt, void *stream);

/*
 * pa_decode_append — the decode step's KV write and attention in one launch: every sequence's
 * newest token is stored in the pool and attended to together with its cached tokens.
 * [PA-summary] "Key idea: virtual memory for the KV cache" (the token a step generates goes to
 * the sequence's last block, through its slot) and "The PagedAttention algorithm".
 * With T = context_lens[s] counting the new token: positions 0 .. T-2 are read from the pool
 * through block_tables[s] exactly as pa_decode reads them; position T-1 is k_new[s], v_new[s]
 * ([num_seqs][num_kv_heads][head_dim], dtype `dt`, 16-byte aligned), folded into the running
 * softmax of the sequence's last partition as one more token. The rows are also stored bit for
 * bit at slot_mapping[s] (int32 [num_seqs]; a negative slot, or one past the pool, stores
 * nothing; the token is attended to either way), as pa_write_kv would. T == 0 gives out = 0 and
 * stores nothing.
 * The result equals pa_write_kv followed by pa_decode when slot_mapping[s] is the slot of
 * position T-1 in the table (the decode step's invariant), within the attention tolerance (the
 * new token enters the sums last rather than in its block's place). Other pool rows are only
 * read; concurrent readers of the new token's slot in the same call see it masked.
 * Arguments otherwise as pa_decode (same workspace size: pa_decode_workspace_size with the
 * same sizes), same errors; k_new, v_new and slot_mapping must be non-null when num_seqs > 0.
 */
pa_status pa_decode_append(void *out, const void *q, void *k_cache, void *v_cache,
                           const void *k_new, const void *v_new, const int32_t *slot_mapping,
                           const int32_t *block_tables, const int32_t *context_lens,
                           float scale, int num_seqs, int num_q_heads, int num_kv_heads,
                           int head_dim, int block_size, int max_blocks_per_seq,
                           int64_t num_blocks, int max_context_len, int partition_tokens,
                           void *workspace, size_t workspace_bytes, pa_dtype dt, void *stream);

/*
 * pa_set_decode_kernel — which decode kernel pa_decode, pa_decode_noalloc and
 * pa_decode_workspace_size use from now on, process-wide. PA_DECODE_AUTO (the default): the
 * MFMA kernel for f16/bf16 with at least two query heads per KV head, the vector-ALU kernel
 * otherwise. PA_DECODE_VALU / PA_DECODE_MFMA force one kernel (the MFMA kernel takes no f32:
 * PA_ERR_UNSUPPORTED then). Both kernels compute the same attention; the choice moves only the
 * rounding of the intermediate weights. Change it only between calls, not between a
 * pa_decode_workspace_size call and the pa_decode it sizes. PA_ERR_INVALID_ARG for any other
 * value.
 */
pa_status pa_set_decode_kernel(pa_decode_kernel kernel);

/*
 * pa_decode_shared_prefix — pa_decode for a batch in which groups of sequences share the KV
 * blocks of a common prefix, as the samples of one prompt do after fork.
 * [PA-summary] "Memory sharing: copy-on-write for parallel decoding": the samples of a prompt
 * hold its blocks by reference (the block manager raises their counts; pa_copy_blocks splits a
 * shared block only when one of them writes into it). Every member's query heads attend to the
 * same keys and values over the shared prefix, so each of the prefix's tiles is read and scored
 * once per group (one matrix-core column per member and query head) instead of once per
 * member; each member's own tokens follow in the same pass, and the running (max, sum, output)
 * state of the block-wise attention equation carries from one to the other. The result is the
 * attention pa_decode computes (within the attention tolerance; not bit for bit, the order of
 * the sums differs).
 * Groups: sequences group_start[i] .. group_start[i+1]-1 form group i (group_start: int32
 * [num_groups + 1], device, group_start[0] = 0, non-decreasing, group_start[num_groups] =
 * num_seqs; a group of one is allowed; pa_bm_prefix_groups computes it). prefix_lens: int32
 * [num_seqs], device: the tokens each sequence shares with its group, the same value for every
 * member of a group, at most each member's context length and at most max_prefix_len; the
 * first ceil(prefix_lens[s]/B) entries of every member's block-table row must name the same
 * physical blocks (0 for a sequence that shares nothing). A violation of these rules is a caller
 * error: the result is undefined, but no access leaves the caller's buffers. The prefix is
 * scored once in whole 32-token steps; the part short of a whole step is scored with each
 * member's own tokens.
 * max_group_size, max_prefix_len: host-known bounds (grid and workspace sizing).
 * partition_tokens: 0 = automatic; > 0 (a multiple of 32, at most 8192) forces the tokens one
 * workgroup covers of its list (the prefix, then the own tokens of the members it serves).
 * workspace: >= pa_decode_shared_prefix_workspace_size(...) bytes, 256-byte aligned, any
 * contents (may be NULL when that size is 0). f16/bf16 run on MFMA; f32 (and a forced
 * vector-ALU kernel, see pa_set_decode_kernel) run pa_decode's path and ignore the groups.
 */
pa_status pa_decode_shared_prefix(void *out, const void *q, const void *k_cache,
                                  const void *v_cache, const int32_t *block_tables,
                                  const int32_t *context_lens, const int32_t *prefix_lens,
                                  const int32_t *group_start, float scale, int num_seqs,
                                  int num_groups, int num_q_heads, int num_kv_heads,
                                  int head_dim, int block_size, int max_blocks_per_seq,
                                  int64_t num_blocks, int max_context_len, int max_prefix_len,
                                  int max_group_size, int partition_tokens, void *workspace,
                                  size_t workspace_bytes, pa_dtype dt, void *stream);

/* Bytes of workspace pa_decode_shared_prefix needs for these sizes (0 when none is needed, and
 * for invalid sizes). */
size_t pa_decode_shared_prefix_workspace_size(int num_seqs, int num_groups, int num_q_heads,
                                              int num_kv_heads, int head_dim, int block_size,
                                              int max_context_len, int max_prefix_len,
                                              int max_group_size, int partition_tokens,
                                              pa_dtype dt);

/*
 * pa_prefill — causal multi-query (prefill / chunked-prefill) attention over the same block
 * pool and tables.
 * [PA-summary] "The PagedAttention algorithm": the kernel walks the block table for each query
 * vector and merges the blocks with the log-sum-exp rescaling of the block-wise equation.
 * Here sequence s brings n_s = query_start[s+1] - query_start[s] new tokens at once (a prompt
 * or a chunk of one). They must already be in the pool (pa_write_kv) as the last n_s of its
 * T_s = context_lens[s] tokens, and each is a query vector: query i (0 <= i < n_s), row
 * query_start[s] + i of q, sits at position T_s - n_s + i and attends to positions
 * 0 .. T_s - n_s + i (the causal rule; a decode step is the case n_s = 1):
 *   out[r][h] = sum_{t <= p} exp(s_t - M) V_t / sum_{t <= p} exp(s_t - M),
 *   s_t = scale * q[r][h] . K_t,  K_t = k_cache[block_tables[s][t/B]][h/g][t%B],  p = T_s-n_s+i
 * computed in fp32 (on MFMA: 16-bit operands for f16/bf16, fp32 operands for f32) and
 * rounded to nearest-even in `dt`.
 * q, out: [num_q_tokens][num_q_heads][head_dim], 16-byte aligned; rows that belong to no
 * sequence are left untouched.
 * query_start: int32 [num_seqs + 1], device, non-decreasing, within [0, num_q_tokens].
 * max_query_len: host-known bound on every n_s; max_context_len: on every T_s (they size the
 * grid; no device read on the host). n_s > T_s or n_s > max_query_len is a caller error: only
 * min(n_s, T_s, max_query_len) rows are computed.
 * Supported: dt f32, f16 or bf16, head_dim 64 or 128, block_size 8, 16, 32 or 64. No
 * workspace. Device indices are clamped as for pa_decode.
 */
pa_status pa_prefill(void *out, const void *q, const void *k_cache, const void *v_cache,
                     const int32_t *block_tables, const int32_t *context_lens,
                     const int32_t *query_start, float scale, int num_seqs, int num_q_tokens,
                     int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                     int max_blocks_per_seq, int64_t num_blocks, int max_query_len,
                     int max_context_len, pa_dtype dt, void *stream);

/*
 * pa_copy_blocks — copy-on-write of shared blocks.
 * [PA-summary] "Memory sharing: copy-on-write for parallel decoding": when a sequence must
 * write into a block it shares with others, only that block is copied to a new physical block
 * (and that sequence's table is repointed by the caller), as fork() does for pages.
 * For each pair p < n_pairs: k_cache[dst] = k_cache[src] and v_cache[dst] = v_cache[src], the
 * whole block (all KV heads, all block_size slots, including unused tail slots), bit-exact.
 * Pairs with an id outside [0, num_blocks) are skipped. A dst that is also some pair's src, or
 * a dst repeated, is a caller error (result unspecified). n_pairs == 0 is a valid no-op.
 */
pa_status pa_copy_blocks(void *k_cache, void *v_cache, const int32_t *block_pairs, int n_pairs,
                         int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                         pa_dtype dt, void *stream);

/*
 * pa_swap_blocks — move whole blocks between two block pools, e.g. out of the GPU pool into a
 * pinned host pool and back.
 * [PA-summary] "vLLM: the serving system built on PagedAttention": when GPU memory runs short
 * the scheduler can pause a lower-priority request by moving its blocks to CPU memory (or by
 * freeing them to recompute later); the blocks come back before the request resumes, at new
 * physical positions recorded in its block table.
 * For each pair p < n_pairs with src = block_pairs[p][0], dst = block_pairs[p][1]:
 *   dst_k[dst] = src_k[src] and dst_v[dst] = src_v[src], whole blocks, bit-exact.
 * The two pools share (num_kv_heads, block_size, head_dim, dt) and have their own block counts.
 * Each pool may be device memory or pinned host memory (hipHostMalloc, mapped into the device
 * address space); block_pairs must be device-accessible too. Pairs with an id outside its
 * pool are skipped; a repeated dst, or the same buffer as both src and dst pool with a dst that
 * is also a src, is a caller error. n_pairs == 0 is a valid no-op.
 */
pa_status pa_swap_blocks(void *dst_k, void *dst_v, int64_t dst_num_blocks, const void *src_k,
                         const void *src_v, int64_t src_num_blocks, const int32_t *block_pairs,
                         int n_pairs, int num_kv_heads, int head_dim, int block_size,
                         pa_dtype dt, void *stream);

/* Static, never-null description of a status code. */
const char *pa_status_string(pa_status s);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
