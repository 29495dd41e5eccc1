// pa_internal.h — host-side launch interface between the C ABI (pa_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

// Arguments of the decode kernels (passed by value as the kernel argument block).
struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float scale_log2;  // scale * log2(e): scores are kept in the base-2 exponent domain
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int max_blocks_per_seq;
  int64_t num_blocks;
  int max_context_len;
  int partition_tokens;  // P, a multiple of 32
  int max_parts;         // ceil(max_context_len / P), at least 1
  float* part_m;         // [S][Hq][max_parts]   running maxima (base-2 domain)
  float* part_l;         // [S][Hq][max_parts]   running sums
  float* part_o;         // [S][Hq][max_parts][D] unnormalised partial outputs
  // Shared-prefix decode only (pa_decode_shared_prefix; null / 0 otherwise). Sequences
  // group_start[i] .. group_start[i+1]-1 form group i and share their first prefix_lens[s]
  // tokens. A workgroup serves one (group, KV head, 16-column tile): its steps are the group's
  // prefix (32-token steps through the first member's table, every column of the tile), then
  // each member's own tokens (through its table, its columns only), cut into partitions of
  // group_steps steps when longer.
  const int32_t* prefix_lens;  // [S]
  const int32_t* group_start;  // [num_groups + 1]
  int num_groups;
  int group_steps;       // steps per partition (at most 64 per wave)
  int group_parts;       // partitions per (group, KV head, column tile)
  int shared_ctiles;     // 16-column tiles of the largest group (members x query heads per KV head)
  int max_shared;        // host bound on the shared tokens of any sequence (a multiple of 32)
  int32_t* part_n;       // [S][Hq] partitions each (sequence, query head) was split into
  // Fused append (pa_decode_append; null / 0 otherwise): the newest token of sequence s,
  // position context_lens[s] - 1, comes from k_new / v_new ([S][Hkv][D]) instead of the pool:
  // the pool part is the first context_lens[s] - 1 tokens, the last partition folds the new
  // token into its state, and the new K/V rows are stored at new_slots[s] (not when < 0).
  const void* k_new;
  const void* v_new;
  const int32_t* new_slots;
  int append;
};

// Workspace layout for a given problem: byte offsets of each region.
struct WorkspaceLayout {
  size_t m_off, l_off, o_off, n_off, total;
};
// with_counts: a [S][Hq] int32 partition count per (sequence, query head) after the partials
// (the shared-prefix decode, whose partition counts the merge kernel cannot derive).
WorkspaceLayout workspace_layout(int num_seqs, int num_q_heads, int head_dim, int max_parts,
                                 bool with_counts = false);

enum class DecodePath : int { Valu = 0, Mfma = 1 };

// Launchers return hipSuccess or the launch error. `dt` uses pa_dtype codes.
hipError_t launch_decode(DecodePath path, int dt, int head_dim, int block_size,
                         const DecodeArgs& a, hipStream_t stream);
// Shared-prefix decode (16-bit inputs): the shared pass and every sequence's own tokens in one
// MFMA launch, then the merge of each (sequence, query head)'s partials.
hipError_t launch_decode_shared(int dt, int head_dim, int block_size, const DecodeArgs& a,
                                hipStream_t stream);
bool decode_supported(DecodePath path, int dt, int head_dim, int block_size);
int decode_units_per_seq(DecodePath path, int num_q_heads, int num_kv_heads);
// Largest partition (tokens) a launch supports: a wave keeps its block ids in one register.
int max_partition_tokens(DecodePath path, int block_size);

// Arguments of the multi-query (prefill / chunked-prefill) kernel.
struct PrefillArgs {
  void* out;                   // [num_q_tokens][Hq][D]
  const void* q;               // [num_q_tokens][Hq][D]
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* query_start;  // [num_seqs + 1]
  float scale_log2;
  int num_seqs;
  int num_q_tokens;
  int num_q_heads;
  int num_kv_heads;
  int max_blocks_per_seq;
  int64_t num_blocks;
  int max_query_len;
  int max_context_len;
  int row_tiles;               // workgroup row tiles per (sequence, KV head)
};

bool prefill_supported(int dt, int head_dim, int block_size);
// Query rows (query token x grouped head) one workgroup covers, for dtype code dt.
int prefill_rows_per_workgroup(int dt);
hipError_t launch_prefill(int dt, int head_dim, int block_size, const PrefillArgs& a,
                          hipStream_t stream);

hipError_t launch_write_kv(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                           const int32_t* slot_mapping, int n_tokens, int num_kv_heads,
                           int row_bytes, int block_size, int64_t num_blocks,
                           hipStream_t stream);
// Whole-block copies dst[pairs[p][1]] = src[pairs[p][0]] for K and V (same or separate pools).
hipError_t launch_copy_blocks(void* dst_k, void* dst_v, int64_t dst_num_blocks,
                              const void* src_k, const void* src_v, int64_t src_num_blocks,
                              const int32_t* pairs, int n_pairs, int64_t block_bytes,
                              hipStream_t stream);

}  // namespace pa
