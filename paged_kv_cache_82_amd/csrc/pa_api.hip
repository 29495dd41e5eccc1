// pa_api.hip — the C ABI of libpa (declared in include/pa.h): argument checks, path and
// partition choice, and kernel launches on the caller's stream. No allocation, no host sync.
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "pa.h"
#include "pa_internal.h"

namespace {

using pa::DecodePath;

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int elem_bytes(pa_dtype dt) { return dt == PA_F32 ? 4 : 2; }

bool valid_dtype(pa_dtype dt) { return dt == PA_F32 || dt == PA_F16 || dt == PA_BF16; }

// Pool element count num_blocks * heads * B * d, or -1 on overflow of int64.
int64_t pool_elems(int64_t num_blocks, int heads, int block_size, int head_dim) {
  const int64_t per_block = (int64_t)heads * block_size * head_dim;
  if (per_block <= 0 || num_blocks < 0) return -1;
  if (num_blocks > INT64_MAX / 4 / per_block) return -1;
  return num_blocks * per_block;
}

// Decode kernel choice, process-wide (pa_set_decode_kernel): PA_DECODE_AUTO picks the grouped-
// query MFMA kernel for 16-bit inputs with at least two query heads per KV head and the VALU
// kernel otherwise; the other values force one kernel for every later call.
std::atomic<int> g_decode_kernel{PA_DECODE_AUTO};

bool choose_path(pa_dtype dt, int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                 DecodePath* path) {
  const int g = num_q_heads / num_kv_heads;
  DecodePath p = (dt != PA_F32 && g >= 2) ? DecodePath::Mfma : DecodePath::Valu;
  const int forced = g_decode_kernel.load(std::memory_order_relaxed);
  if (forced == PA_DECODE_VALU) p = DecodePath::Valu;
  else if (forced == PA_DECODE_MFMA) p = DecodePath::Mfma;
  *path = p;
  return pa::decode_supported(p, (int)dt, head_dim, block_size);
}

// Tokens per partition. A workgroup covers P tokens of one (sequence, head unit); each extra
// partition costs a partial-state write, a read in the merge kernel and a short-lived
// workgroup, so sequences are split only when there are too few (sequence, head) units to fill
// the GPU: with at least `many` units every sequence stays whole; otherwise partitions of 2048
// tokens (halved while the grid would be smaller than `many` workgroups, down to 256). `many` is
// 1024 for the vector-ALU kernel (several workgroups per CU) and 256 for the MFMA kernel (one
// per CU, 100-132 KB of LDS). Measured on MI355X: unsplit 13B-shape and GQA batches ran 25-35%
// faster than with 512-token partitions; long contexts peaked at 2048; a batch of 256
// (sequence, 32-head) units (128 sequences, 64 query / 2 KV heads, lengths 128..4096) took 59.9
// us whole against 69.6 / 78.6 / 98.8 us with 2048 / 1024 / 512-token partitions. The halving
// counts the grid at half the longest length for the vector-ALU kernel and at the longest for
// the MFMA kernel, whose short workgroups cost more than its idle CUs: 128 (sequence, 32-head)
// units (64 sequences, 64 query / 2 KV heads, lengths 128..4096) took 37.3 us with 2048-token
// partitions against 46.4 us with 1024. 0 = automatic.
int choose_partition(int num_seqs, int units_per_seq, int max_context_len, int cap,
                     int requested, pa::DecodePath path) {
  if (requested > 0) return requested;
  const bool mfma = path == pa::DecodePath::Mfma;
  const int many = mfma ? 256 : 1024;
  const int64_t units = (int64_t)num_seqs * units_per_seq;
  const int whole = ((max_context_len + 31) / 32) * 32;
  if (whole <= 0) return 32;
  if (units >= many && whole <= cap) return whole;
  int P = 2048 < cap ? 2048 : cap;
  const int span = mfma ? max_context_len : max_context_len / 2;
  auto est = [&](int p) { return units * ((span + p - 1) / p); };
  while (P > 256 && est(P) < many) P /= 2;
  return P < whole ? P : whole;
}

int parts_for(int max_context_len, int P) {
  const int n = (max_context_len + P - 1) / P;
  return n > 1 ? n : 1;
}

// The automatic plan of a decode call: partition size, partition count and workspace.
struct DecodePlan {
  int P, max_parts;
  pa::WorkspaceLayout L;
};

DecodePlan plan_decode(DecodePath path, int num_seqs, int num_q_heads, int num_kv_heads,
                       int head_dim, int max_context_len, int partition_tokens, int cap) {
  DecodePlan pl{};
  pl.P = choose_partition(num_seqs, pa::decode_units_per_seq(path, num_q_heads, num_kv_heads),
                          max_context_len, cap, partition_tokens, path);
  pl.max_parts = parts_for(max_context_len, pl.P);
  pl.L = pa::workspace_layout(num_seqs, num_q_heads, head_dim, pl.max_parts);
  return pl;
}

pa_status from_hip(hipError_t e) { return e == hipSuccess ? PA_OK : PA_ERR_HIP; }

// ---- the allocation-free decode: split-K partials in a static device array -----------------
// `scratch` is a file-scope device array; every GPU the library runs on holds its own copy,
// at its own address, until the process ends. Host code never uses the array's name as an
// address (on the host it is only a stand-in symbol): the per-device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and only that address
// is passed to kernels. No region of it needs initialising: each partition's workgroup writes
// its (max, sum, output) before the merge kernel reads them, and the merge reads only the
// partitions that exist.
static __device__ __align__(256) unsigned char scratch[PA_DECODE_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_dev[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

pa_status scratch_ptr(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_dev[dev] = (g_scratch_err[dev] == hipSuccess) ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess || !g_scratch_dev[dev]) return PA_ERR_HIP;
  *ptr = g_scratch_dev[dev];
  return PA_OK;
}

// The newest token of each sequence, for pa_decode_append (all null otherwise).
struct AppendRows {
  const void* k_new = nullptr;
  const void* v_new = nullptr;
  const int32_t* slots = nullptr;
};

// pa_decode with the split-K partials in `workspace` (the caller's buffer), or, with
// use_scratch, in the library's static scratch array (pa_decode_noalloc; workspace ignored);
// with `app`, pa_decode_append.
pa_status decode_impl(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, float scale,
                      int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                      int block_size, int max_blocks_per_seq, int64_t num_blocks,
                      int max_context_len, int partition_tokens, void* workspace,
                      size_t workspace_bytes, bool use_scratch, pa_dtype dt, void* stream,
                      const AppendRows& app = AppendRows{}) {
  if (!valid_dtype(dt)) return PA_ERR_INVALID_ARG;
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || max_blocks_per_seq < 0 || num_blocks <= 0 || max_context_len < 0 ||
      partition_tokens < 0)
    return PA_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads) return PA_ERR_INVALID_ARG;
  if (partition_tokens % 32) return PA_ERR_INVALID_ARG;
  if (pool_elems(num_blocks, num_kv_heads, block_size, head_dim) < 0) return PA_ERR_INVALID_ARG;
  if (num_seqs > 65535 || num_q_heads > 65535) return PA_ERR_INVALID_ARG;  // grid limits
  DecodePath path;
  if (!choose_path(dt, num_q_heads, num_kv_heads, head_dim, block_size, &path))
    return PA_ERR_UNSUPPORTED;
  const int cap = pa::max_partition_tokens(path, block_size);
  if (partition_tokens > cap) return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (max_blocks_per_seq <= 0) return PA_ERR_INVALID_ARG;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return PA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(out, elem_bytes(dt)) || !aligned(block_tables, 4) || !aligned(context_lens, 4))
    return PA_ERR_INVALID_ARG;
  const bool append = app.k_new || app.v_new || app.slots;
  if (append && (!app.k_new || !app.v_new || !app.slots || !aligned(app.k_new, 16) ||
                 !aligned(app.v_new, 16) || !aligned(app.slots, 4)))
    return PA_ERR_INVALID_ARG;
  if (append && num_seqs > 65534) return PA_ERR_INVALID_ARG;  // one more grid slice stores

  const DecodePlan plan = plan_decode(path, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                      max_context_len, partition_tokens, cap);
  const pa::WorkspaceLayout& L = plan.L;
  if (use_scratch) {
    workspace = nullptr;
    workspace_bytes = PA_DECODE_SCRATCH_BYTES;
    if (L.total > workspace_bytes) return PA_ERR_WORKSPACE;
    if (L.total > 0) {
      const pa_status st = scratch_ptr(&workspace);
      if (st != PA_OK) return st;
    }
  }
  if (workspace_bytes < L.total || (L.total > 0 && !workspace)) return PA_ERR_WORKSPACE;
  if (L.total > 0 && !aligned(workspace, 256)) return PA_ERR_INVALID_ARG;

  pa::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.max_context_len = max_context_len;
  a.partition_tokens = plan.P;
  a.max_parts = plan.max_parts;
  char* ws = (char*)workspace;
  a.part_m = L.total ? (float*)(ws + L.m_off) : nullptr;
  a.part_l = L.total ? (float*)(ws + L.l_off) : nullptr;
  a.part_o = L.total ? (float*)(ws + L.o_off) : nullptr;
  if (append) {
    a.k_new = app.k_new;
    a.v_new = app.v_new;
    a.new_slots = app.slots;
    a.append = 1;
  }
  return from_hip(pa::launch_decode(path, (int)dt, head_dim, block_size, a, (hipStream_t)stream));
}


// Partition plan of pa_decode_shared_prefix (16-bit inputs, MFMA kernel). A workgroup serves
// one (group, KV head, 16-column tile) and walks that tile's list of 32-token steps: the
// group's shared prefix, then the own tokens of each member with a column in the tile. A list
// longer than a partition (at most 256 steps, 64 per wave) is split; partitions shrink (to 32
// steps) only while the grid would have fewer workgroups than the GPU has compute units.
struct SharedPlan {
  int ctiles, max_shared, steps, parts;
  int64_t wgs;
};

bool shared_plan(int num_groups, int num_q_heads, int num_kv_heads, int max_context_len,
                 int max_prefix_len, int max_group_size, int partition_tokens, SharedPlan* out) {
  constexpr int kMaxSteps = 256;  // steps per partition: 64 per wave, one register of ids
  constexpr int kCUs = 256;
  if (num_groups < 0 || max_context_len < 0 || max_prefix_len < 0 || max_group_size < 1 ||
      partition_tokens < 0 || partition_tokens % 32 || partition_tokens > 32 * kMaxSteps)
    return false;
  const int g = num_q_heads / num_kv_heads;
  if ((int64_t)max_group_size * g > 16 * 4096) return false;
  SharedPlan P{};
  P.ctiles = (max_group_size * g + 15) / 16;
  const int lmax = max_prefix_len < max_context_len ? max_prefix_len : max_context_len;
  P.max_shared = num_groups > 0 ? (lmax / 32) * 32 : 0;  // no group: nothing is shared
  // members with a column in one tile, and the longest list a tile can have
  const int per_tile = max_group_size < (15 + g - 1) / g + 1 ? max_group_size
                                                             : (15 + g - 1) / g + 1;
  const int64_t bound = P.max_shared / 32 + (int64_t)per_tile * ((max_context_len + 31) / 32);
  const int64_t units = (int64_t)num_groups * num_kv_heads * P.ctiles;
  if (partition_tokens > 0) {
    P.steps = partition_tokens / 32;
  } else {
    P.steps = kMaxSteps;
    while (P.steps > 32 && units * ((bound + P.steps - 1) / P.steps) < kCUs) P.steps /= 2;
  }
  const int64_t parts = bound > 0 ? (bound + P.steps - 1) / P.steps : 1;
  if (parts > (1 << 20)) return false;
  P.parts = (int)parts;
  P.wgs = units * (P.parts > 1 ? (P.parts | 1) : 1);  // the grid pads partitions to an odd count
  *out = P;
  return true;
}

}  // namespace

extern "C" {

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported dtype/head_dim/block_size combination";
    case PA_ERR_WORKSPACE: return "workspace too small";
    case PA_ERR_HIP: return "HIP runtime error at launch";
    case PA_ERR_NO_BLOCKS: return "not enough free blocks";
  }
  return "unknown status";
}

pa_status pa_write_kv(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                      const int32_t* slot_mapping, int n_tokens, int num_kv_heads, int head_dim,
                      int block_size, int64_t num_blocks, pa_dtype dt, void* stream) {
  if (!valid_dtype(dt)) return PA_ERR_INVALID_ARG;
  if (n_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PA_ERR_INVALID_ARG;
  if (pool_elems(num_blocks, num_kv_heads, block_size, head_dim) < 0) return PA_ERR_INVALID_ARG;
  if ((int64_t)n_tokens * num_kv_heads * head_dim > INT64_MAX / 8) return PA_ERR_INVALID_ARG;
  const int row_bytes = head_dim * elem_bytes(dt);
  if (row_bytes % 16) return PA_ERR_UNSUPPORTED;
  if (n_tokens == 0) return PA_OK;
  if (!k_cache || !v_cache || !k_new || !v_new || !slot_mapping) return PA_ERR_INVALID_ARG;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(k_new, 16) ||
      !aligned(v_new, 16) || !aligned(slot_mapping, 4))
    return PA_ERR_INVALID_ARG;
  return from_hip(pa::launch_write_kv(k_cache, v_cache, k_new, v_new, slot_mapping, n_tokens,
                                      num_kv_heads, row_bytes, block_size, num_blocks,
                                      (hipStream_t)stream));
}

size_t pa_decode_workspace_size(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                                int block_size, int max_context_len, int partition_tokens,
                                pa_dtype dt) {
  if (!valid_dtype(dt) || num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads || head_dim <= 0 || block_size <= 0 || max_context_len < 0 ||
      partition_tokens < 0 || partition_tokens % 32)
    return 0;
  DecodePath path;
  if (!choose_path(dt, num_q_heads, num_kv_heads, head_dim, block_size, &path)) return 0;
  const int cap = pa::max_partition_tokens(path, block_size);
  if (partition_tokens > cap) return 0;
  return plan_decode(path, num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                     partition_tokens, cap)
      .L.total;
}

pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens, float scale,
                    int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                    int block_size, int max_blocks_per_seq, int64_t num_blocks,
                    int max_context_len, int partition_tokens, void* workspace,
                    size_t workspace_bytes, pa_dtype dt, void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, scale, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                     num_blocks, max_context_len, partition_tokens, workspace, workspace_bytes,
                     false, dt, stream);
}

pa_status pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens,
                            float scale, int num_seqs, int num_q_heads, int num_kv_heads,
                            int head_dim, int block_size, int max_blocks_per_seq,
                            int64_t num_blocks, int max_context_len, int partition_tokens,
                            pa_dtype dt, void* stream) {
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, scale, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                     num_blocks, max_context_len, partition_tokens, nullptr, 0, true, dt,
                     stream);
}

pa_status pa_decode_append(void* out, const void* q, void* k_cache, void* v_cache,
                           const void* k_new, const void* v_new, const int32_t* slot_mapping,
                           const int32_t* block_tables, const int32_t* context_lens,
                           float scale, int num_seqs, int num_q_heads, int num_kv_heads,
                           int head_dim, int block_size, int max_blocks_per_seq,
                           int64_t num_blocks, int max_context_len, int partition_tokens,
                           void* workspace, size_t workspace_bytes, pa_dtype dt, void* stream) {
  AppendRows app;
  app.k_new = k_new;
  app.v_new = v_new;
  app.slots = slot_mapping;
  if (num_seqs > 0 && (!k_new || !v_new || !slot_mapping)) return PA_ERR_INVALID_ARG;
  return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, scale, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                     num_blocks, max_context_len, partition_tokens, workspace, workspace_bytes,
                     false, dt, stream, app);
}

pa_status pa_set_decode_kernel(pa_decode_kernel kernel) {
  if (kernel != PA_DECODE_AUTO && kernel != PA_DECODE_VALU && kernel != PA_DECODE_MFMA)
    return PA_ERR_INVALID_ARG;
  g_decode_kernel.store((int)kernel, std::memory_order_relaxed);
  return PA_OK;
}

size_t pa_decode_shared_prefix_workspace_size(int num_seqs, int num_groups, int num_q_heads,
                                              int num_kv_heads, int head_dim, int block_size,
                                              int max_context_len, int max_prefix_len,
                                              int max_group_size, int partition_tokens,
                                              pa_dtype dt) {
  if (!valid_dtype(dt) || num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      num_q_heads % num_kv_heads || head_dim <= 0 || block_size <= 0 || max_context_len < 0)
    return 0;
  DecodePath path;
  if (!choose_path(dt, num_q_heads, num_kv_heads, head_dim, block_size, &path)) return 0;
  if (dt == PA_F32 || g_decode_kernel.load(std::memory_order_relaxed) == PA_DECODE_VALU)
    return pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                    max_context_len, partition_tokens, dt);
  SharedPlan P;
  if (!shared_plan(num_groups, num_q_heads, num_kv_heads, max_context_len, max_prefix_len,
                   max_group_size, partition_tokens, &P))
    return 0;
  return pa::workspace_layout(num_seqs, num_q_heads, head_dim, P.parts, true).total;
}

pa_status pa_decode_shared_prefix(void* out, const void* q, const void* k_cache,
                                  const void* v_cache, const int32_t* block_tables,
                                  const int32_t* context_lens, const int32_t* prefix_lens,
                                  const int32_t* group_start, float scale, int num_seqs,
                                  int num_groups, int num_q_heads, int num_kv_heads,
                                  int head_dim, int block_size, int max_blocks_per_seq,
                                  int64_t num_blocks, int max_context_len, int max_prefix_len,
                                  int max_group_size, int partition_tokens, void* workspace,
                                  size_t workspace_bytes, pa_dtype dt, void* stream) {
  if (!valid_dtype(dt)) return PA_ERR_INVALID_ARG;
  if (num_seqs < 0 || num_groups < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || block_size <= 0 || max_blocks_per_seq < 0 || num_blocks <= 0 ||
      max_context_len < 0 || max_prefix_len < 0 || max_group_size < 1)
    return PA_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads) return PA_ERR_INVALID_ARG;
  if (pool_elems(num_blocks, num_kv_heads, block_size, head_dim) < 0) return PA_ERR_INVALID_ARG;
  if (num_seqs > 65535 || num_q_heads > 65535) return PA_ERR_INVALID_ARG;
  DecodePath path;
  if (!choose_path(dt, num_q_heads, num_kv_heads, head_dim, block_size, &path))
    return PA_ERR_UNSUPPORTED;
  // fp32 (and a forced vector-ALU kernel): the same attention, through pa_decode's path
  if (dt == PA_F32 || g_decode_kernel.load(std::memory_order_relaxed) == PA_DECODE_VALU)
    return decode_impl(out, q, k_cache, v_cache, block_tables, context_lens, scale, num_seqs,
                       num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                       num_blocks, max_context_len, partition_tokens, workspace,
                       workspace_bytes, false, dt, stream);
  SharedPlan P;
  if (!shared_plan(num_groups, num_q_heads, num_kv_heads, max_context_len, max_prefix_len,
                   max_group_size, partition_tokens, &P))
    return PA_ERR_INVALID_ARG;
  if (num_seqs == 0) return PA_OK;
  if (max_blocks_per_seq <= 0) return PA_ERR_INVALID_ARG;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !prefix_lens ||
      (num_groups > 0 && !group_start))
    return PA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(out, elem_bytes(dt)) || !aligned(block_tables, 4) || !aligned(context_lens, 4) ||
      !aligned(prefix_lens, 4) || !aligned(group_start, 4))
    return PA_ERR_INVALID_ARG;
  if (P.wgs > 0xffffffffLL) return PA_ERR_INVALID_ARG;  // one-dimensional grid
  const pa::WorkspaceLayout L =
      pa::workspace_layout(num_seqs, num_q_heads, head_dim, P.parts, true);
  if (workspace_bytes < L.total || (L.total > 0 && !workspace)) return PA_ERR_WORKSPACE;
  if (L.total > 0 && !aligned(workspace, 256)) return PA_ERR_INVALID_ARG;

  pa::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.max_context_len = max_context_len;
  a.partition_tokens = 32 * P.steps;
  a.max_parts = P.parts;
  char* ws = (char*)workspace;
  a.part_m = L.total ? (float*)(ws + L.m_off) : nullptr;
  a.part_l = L.total ? (float*)(ws + L.l_off) : nullptr;
  a.part_o = L.total ? (float*)(ws + L.o_off) : nullptr;
  a.part_n = L.total ? (int32_t*)(ws + L.n_off) : nullptr;
  a.prefix_lens = prefix_lens;
  a.group_start = group_start;
  a.num_groups = num_groups;
  a.group_steps = P.steps;
  a.group_parts = P.parts;
  a.shared_ctiles = P.ctiles;
  a.max_shared = P.max_shared;
  return from_hip(pa::launch_decode_shared((int)dt, head_dim, block_size, a,
                                           (hipStream_t)stream));
}

pa_status pa_prefill(void* out, const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, const int32_t* context_lens,
                     const int32_t* query_start, float scale, int num_seqs, int num_q_tokens,
                     int num_q_heads, int num_kv_heads, int head_dim, int block_size,
                     int max_blocks_per_seq, int64_t num_blocks, int max_query_len,
                     int max_context_len, pa_dtype dt, void* stream) {
  if (!valid_dtype(dt)) return PA_ERR_INVALID_ARG;
  if (num_seqs < 0 || num_q_tokens < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      head_dim <= 0 || block_size <= 0 || max_blocks_per_seq < 0 || num_blocks <= 0 ||
      max_query_len < 0 || max_context_len < 0)
    return PA_ERR_INVALID_ARG;
  if (num_q_heads % num_kv_heads) return PA_ERR_INVALID_ARG;
  if (pool_elems(num_blocks, num_kv_heads, block_size, head_dim) < 0) return PA_ERR_INVALID_ARG;
  if ((int64_t)num_q_tokens * num_q_heads * head_dim > INT64_MAX / 8) return PA_ERR_INVALID_ARG;
  if (!pa::prefill_supported((int)dt, head_dim, block_size)) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0 || num_q_tokens == 0 || max_query_len == 0 || max_context_len == 0)
    return PA_OK;
  if (max_blocks_per_seq <= 0) return PA_ERR_INVALID_ARG;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
    return PA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(query_start, 4))
    return PA_ERR_INVALID_ARG;
  const int g = num_q_heads / num_kv_heads;
  const int64_t rows = (int64_t)max_query_len * g;
  const int per_wg = pa::prefill_rows_per_workgroup((int)dt);
  const int64_t row_tiles = (rows + per_wg - 1) / per_wg;
  if (rows > INT32_MAX || row_tiles * num_kv_heads * (int64_t)num_seqs > INT32_MAX)
    return PA_ERR_INVALID_ARG;  // one-dimensional grid

  pa::PrefillArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.query_start = query_start;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.num_seqs = num_seqs;
  a.num_q_tokens = num_q_tokens;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.max_query_len = max_query_len;
  a.max_context_len = max_context_len;
  a.row_tiles = (int)row_tiles;
  return from_hip(pa::launch_prefill((int)dt, head_dim, block_size, a, (hipStream_t)stream));
}

pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* block_pairs, int n_pairs,
                         int num_kv_heads, int head_dim, int block_size, int64_t num_blocks,
                         pa_dtype dt, void* stream) {
  if (!valid_dtype(dt)) return PA_ERR_INVALID_ARG;
  if (n_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return PA_ERR_INVALID_ARG;
  if (pool_elems(num_blocks, num_kv_heads, block_size, head_dim) < 0) return PA_ERR_INVALID_ARG;
  const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * elem_bytes(dt);
  if (block_bytes % 16) return PA_ERR_UNSUPPORTED;
  if (n_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !block_pairs) return PA_ERR_INVALID_ARG;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(block_pairs, 4))
    return PA_ERR_INVALID_ARG;
  return from_hip(pa::launch_copy_blocks(k_cache, v_cache, num_blocks, k_cache, v_cache,
                                         num_blocks, block_pairs, n_pairs, block_bytes,
                                         (hipStream_t)stream));
}

pa_status pa_swap_blocks(void* dst_k, void* dst_v, int64_t dst_num_blocks, const void* src_k,
                         const void* src_v, int64_t src_num_blocks, const int32_t* block_pairs,
                         int n_pairs, int num_kv_heads, int head_dim, int block_size,
                         pa_dtype dt, void* stream) {
  if (!valid_dtype(dt)) return PA_ERR_INVALID_ARG;
  if (n_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      dst_num_blocks <= 0 || src_num_blocks <= 0)
    return PA_ERR_INVALID_ARG;
  if (pool_elems(dst_num_blocks, num_kv_heads, block_size, head_dim) < 0 ||
      pool_elems(src_num_blocks, num_kv_heads, block_size, head_dim) < 0)
    return PA_ERR_INVALID_ARG;
  const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * elem_bytes(dt);
  if (block_bytes % 16) return PA_ERR_UNSUPPORTED;
  if (n_pairs == 0) return PA_OK;
  if (!dst_k || !dst_v || !src_k || !src_v || !block_pairs) return PA_ERR_INVALID_ARG;
  if (!aligned(dst_k, 16) || !aligned(dst_v, 16) || !aligned(src_k, 16) || !aligned(src_v, 16) ||
      !aligned(block_pairs, 4))
    return PA_ERR_INVALID_ARG;
  return from_hip(pa::launch_copy_blocks(dst_k, dst_v, dst_num_blocks, src_k, src_v,
                                         src_num_blocks, block_pairs, n_pairs, block_bytes,
                                         (hipStream_t)stream));
}

}  // extern "C"
