/*
 * pa_block_manager.h — C ABI of libpa's host block manager: the bookkeeping that produces the
 * block tables, slot mappings and copy-on-write pairs the GPU calls in pa.h consume.
 *
 * Sources (the method is defined there):
 *   [PA-summary]  azimuth.plus, "Efficient Memory Management for Large Language Model Serving
 *                 with PagedAttention": "Key idea: virtual memory for the KV cache" (a
 *                 sequence's KV cache is cut into fixed-size logical blocks mapped through a
 *                 block table to physical blocks that need not be contiguous; physical blocks
 *                 are allocated one at a time, on demand, as tokens are generated), "vLLM" (the
 *                 block manager keeps the free physical blocks and the reference counts of
 *                 shared blocks, copies on write, and can move a paused request's blocks to CPU
 *                 memory), "Memory sharing: copy-on-write" (sequences forked from one prompt
 *                 point at the same physical blocks; a write into a shared block copies only
 *                 that block and repoints the writer's table) and "Results" (the only waste
 *                 left is the unfilled tail of each sequence's last block, at most B slots).
 *   [PA-tutorial] un.csdn.net, "PagedAttention实战：如何用Python手搓一个高效KV缓存管理器":
 *                 §2.2 BlockManager (a free list popped from its end; reference counts; a page
 *                 returns to the free list when its count reaches zero; allocation fails when
 *                 the list is empty), §3.1 append_kv (position pos lives in logical page
 *                 pos // B at offset pos % B) and §5.1 clone_sequence (a fork copies the page
 *                 table and raises every page's count).
 *
 * Readings where the pages leave a step open:
 *   - which holder copies a shared block: every writer whose block still has a reference count
 *     above 1 copies it and drops the count by one; the last holder (count 1) writes in place;
 *   - an append that would need more free blocks than there are fails as a whole and changes
 *     nothing (PA_ERR_NO_BLOCKS), so a scheduler can try a smaller request or preempt;
 *   - blocks are handed out in the order of `free_order` (or 0, 1, 2, ...) and freed blocks are
 *     reused last-freed-first, as [PA-tutorial] §2.2's list does.
 *
 * Ownership: a manager is created by pa_bm_create and owned by the caller until pa_bm_destroy.
 * Every pointer argument is HOST memory owned by the caller; the manager copies what it keeps.
 * The manager is not thread-safe: calls on one manager must not overlap. It never touches the
 * GPU; the pairs it returns are applied with pa_copy_blocks / pa_swap_blocks by the caller.
 *
 * Errors: PA_ERR_INVALID_ARG for a null pointer, a bad size, an unknown or duplicate sequence
 * id, or an output array that is too small; PA_ERR_NO_BLOCKS when the free list cannot cover
 * the request. A failed call leaves the manager unchanged.
 */
#ifndef PA_BLOCK_MANAGER_H
#define PA_BLOCK_MANAGER_H

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_bm pa_bm;

/* Counters of one manager (all in blocks or token slots). */
typedef struct {
  int64_t num_blocks;      /* pool size */
  int64_t free_blocks;     /* on the free list */
  int64_t used_blocks;     /* reference count > 0 */
  int64_t shared_blocks;   /* reference count > 1 */
  int64_t logical_blocks;  /* sum over sequences of their table lengths */
  int64_t num_seqs;
  int64_t tokens;          /* sum over sequences of their lengths */
  int64_t filled_slots;    /* slots of used blocks that hold a token of some sequence */
  int64_t reserved_slots;  /* used_blocks * block_size */
} pa_bm_stats;

/*
 * Create a manager of `num_blocks` physical blocks of `block_size` token slots.
 * free_order: NULL, or a permutation of 0..num_blocks-1 (checked): the order in which blocks
 * are first handed out (a scattered order places consecutive blocks far apart).
 */
pa_status pa_bm_create(int64_t num_blocks, int block_size, const int32_t *free_order,
                       pa_bm **out);
void pa_bm_destroy(pa_bm *bm);

/* Register an empty sequence. */
pa_status pa_bm_add(pa_bm *bm, int64_t seq);

/* [PA-tutorial] §5.1 clone_sequence / [PA-summary] CoW: `child` (new id) shares every block of
 * `parent` (reference counts raised) and has its length. */
pa_status pa_bm_fork(pa_bm *bm, int64_t parent, int64_t child);

/* Free blocks the next pa_bm_append(seq, n_tokens) would take (new blocks plus copies of
 * shared blocks), or -1 for an unknown sequence or negative n_tokens. */
int64_t pa_bm_blocks_needed(const pa_bm *bm, int64_t seq, int n_tokens);

/*
 * Reserve slots for the next n_tokens tokens of `seq` ([PA-tutorial] §3.1; [PA-summary] "Key
 * idea": a block is taken from the free list when a token starts it).
 * slots: [n_tokens] out, slot = physical_block * block_size + offset (pa_write_kv's input).
 * cow_pairs: [max_pairs][2] out, (src, dst) whole-block copies that must run (pa_copy_blocks)
 * before the tokens are written; *n_pairs receives their count (at most one per block the
 * append touches). max_pairs too small for what the append needs: PA_ERR_INVALID_ARG.
 */
pa_status pa_bm_append(pa_bm *bm, int64_t seq, int n_tokens, int32_t *slots,
                       int32_t *cow_pairs, int max_pairs, int *n_pairs);

/* Drop the sequence: every block's count falls by one; blocks at zero return to the free list
 * (last freed is handed out first). */
pa_status pa_bm_release(pa_bm *bm, int64_t seq);

/*
 * Move `seq` from manager `from` to manager `to` (e.g. a device pool and a pinned host pool of
 * the same block size): every block of its table gets a block in `to`, `from` releases the
 * sequence, and `to` holds it under the same id with the same length. pairs: [max_pairs][2]
 * out, (block in `from`, block in `to`), one per table entry, for pa_swap_blocks. Blocks the
 * sequence shared with others in `from` are copied, not moved: the others keep theirs.
 * [PA-summary] "vLLM": preemption moves a paused request's blocks to CPU memory and back.
 */
pa_status pa_bm_move(pa_bm *from, pa_bm *to, int64_t seq, int32_t *pairs, int max_pairs,
                     int *n_pairs);

/* Length in tokens (-1: unknown sequence) and table length in blocks (-1: unknown). */
int64_t pa_bm_length(const pa_bm *bm, int64_t seq);
int pa_bm_num_seq_blocks(const pa_bm *bm, int64_t seq);

/* Dense block tables for pa_decode / pa_prefill: row i (of n) is the table of seqs[i], padded
 * with `pad` to `width` entries. A table longer than width: PA_ERR_INVALID_ARG. */
pa_status pa_bm_tables(const pa_bm *bm, const int64_t *seqs, int n, int32_t *out, int width,
                       int32_t pad);

/*
 * The prefix groups of a batch, for pa_decode_shared_prefix. [PA-summary] "Memory sharing:
 * copy-on-write": forked sequences hold their parent's blocks by reference until one writes.
 * Consecutive sequences of seqs[0..n) whose tables start with the same physical block form a
 * group (every sequence is in exactly one; a sequence with no block, or whose first block
 * differs from its predecessor's, starts a new group). A group's shared prefix is the number of
 * leading table entries identical in every member, times block_size, capped by its shortest
 * member's length (0 for a group of one).
 * group_start: [n + 1] out (group i = positions group_start[i] .. group_start[i+1]-1 of seqs);
 * *num_groups receives the group count; prefix_lens: [n] out, each sequence's shared tokens.
 * An unknown sequence id: PA_ERR_INVALID_ARG, outputs unchanged.
 */
pa_status pa_bm_prefix_groups(const pa_bm *bm, const int64_t *seqs, int n, int32_t *group_start,
                              int *num_groups, int32_t *prefix_lens);

/* Reference count of a physical block (-1 outside the pool). */
int32_t pa_bm_refcount(const pa_bm *bm, int64_t block);

pa_status pa_bm_get_stats(const pa_bm *bm, pa_bm_stats *out);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCK_MANAGER_H */
