// pa_block_manager.cpp — host block manager of libpa (C ABI in include/pa_block_manager.h).
//
// Free list, reference counts, on-demand allocation, fork, copy-on-write decision and moves
// between pools, as [PA-summary] ("Key idea", "vLLM", "Memory sharing: copy-on-write") and
// [PA-tutorial] (§2.2 BlockManager, §3.1 append_kv, §5.1 clone_sequence) describe them. Host
// code only: it produces the tables, slots and pairs the GPU calls consume.
#include "pa_block_manager.h"

#include <algorithm>
#include <new>
#include <unordered_map>
#include <vector>

struct pa_bm {
  int64_t num_blocks = 0;
  int block_size = 0;
  std::vector<int32_t> free_list;  // back() is handed out next
  std::vector<int32_t> ref;        // reference count per physical block
  struct Seq {
    std::vector<int32_t> table;  // logical block j -> physical block
    int64_t len = 0;             // tokens
  };
  std::unordered_map<int64_t, Seq> seqs;

  Seq* find(int64_t id) {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }
  const Seq* find(int64_t id) const {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }
  int32_t take() {
    const int32_t b = free_list.back();
    free_list.pop_back();
    ref[b] = 1;
    return b;
  }
  void drop(int32_t b) {
    if (--ref[b] == 0) free_list.push_back(b);
  }
  // Copies of shared blocks an append of n tokens makes: only the last block can be touched
  // among the existing ones, and only when it is partly filled.
  int64_t cow_needed(const Seq& s, int64_t n) const {
    if (n <= 0 || s.len % block_size == 0 || s.table.empty()) return 0;
    const int64_t j = s.len / block_size;
    if (j >= (int64_t)s.table.size()) return 0;
    return ref[s.table[j]] > 1 ? 1 : 0;
  }
  int64_t new_needed(const Seq& s, int64_t n) const {
    const int64_t want = (s.len + n + block_size - 1) / block_size;
    return std::max<int64_t>(0, want - (int64_t)s.table.size());
  }
};

extern "C" {

pa_status pa_bm_create(int64_t num_blocks, int block_size, const int32_t* free_order,
                       pa_bm** out) {
  // slots (block * block_size + offset) are int32 in the GPU calls
  if (!out || num_blocks < 0 || block_size <= 0 || num_blocks * (int64_t)block_size > INT32_MAX)
    return PA_ERR_INVALID_ARG;
  *out = nullptr;
  pa_bm* bm = new (std::nothrow) pa_bm();
  if (!bm) return PA_ERR_INVALID_ARG;
  try {
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->ref.assign((size_t)num_blocks, 0);
    bm->free_list.resize((size_t)num_blocks);
    if (free_order) {
      std::vector<char> seen((size_t)num_blocks, 0);
      for (int64_t i = 0; i < num_blocks; ++i) {
        const int32_t b = free_order[i];
        if (b < 0 || b >= num_blocks || seen[b]) {
          delete bm;
          return PA_ERR_INVALID_ARG;  // not a permutation
        }
        seen[b] = 1;
      }
    }
    // back() is handed out first: store the order reversed
    for (int64_t i = 0; i < num_blocks; ++i)
      bm->free_list[(size_t)(num_blocks - 1 - i)] = free_order ? free_order[i] : (int32_t)i;
  } catch (...) {
    delete bm;
    return PA_ERR_INVALID_ARG;
  }
  *out = bm;
  return PA_OK;
}

void pa_bm_destroy(pa_bm* bm) { delete bm; }

pa_status pa_bm_add(pa_bm* bm, int64_t seq) {
  if (!bm || bm->find(seq)) return PA_ERR_INVALID_ARG;
  try {
    bm->seqs.emplace(seq, pa_bm::Seq{});
  } catch (...) {
    return PA_ERR_INVALID_ARG;
  }
  return PA_OK;
}

pa_status pa_bm_fork(pa_bm* bm, int64_t parent, int64_t child) {
  if (!bm || parent == child) return PA_ERR_INVALID_ARG;
  const pa_bm::Seq* p = bm->find(parent);
  if (!p || bm->find(child)) return PA_ERR_INVALID_ARG;
  try {
    pa_bm::Seq c;
    c.table = p->table;
    c.len = p->len;
    bm->seqs.emplace(child, std::move(c));  // may throw: nothing is changed before it
  } catch (...) {
    return PA_ERR_INVALID_ARG;
  }
  for (int32_t b : bm->find(child)->table) ++bm->ref[b];
  return PA_OK;
}

int64_t pa_bm_blocks_needed(const pa_bm* bm, int64_t seq, int n_tokens) {
  if (!bm || n_tokens < 0) return -1;
  const pa_bm::Seq* s = bm->find(seq);
  if (!s) return -1;
  return bm->new_needed(*s, n_tokens) + bm->cow_needed(*s, n_tokens);
}

pa_status pa_bm_append(pa_bm* bm, int64_t seq, int n_tokens, int32_t* slots,
                       int32_t* cow_pairs, int max_pairs, int* n_pairs) {
  if (!bm || n_tokens < 0 || max_pairs < 0 || !n_pairs) return PA_ERR_INVALID_ARG;
  pa_bm::Seq* s = bm->find(seq);
  if (!s) return PA_ERR_INVALID_ARG;
  if (n_tokens > 0 && !slots) return PA_ERR_INVALID_ARG;
  const int64_t B = bm->block_size;
  const int64_t fresh = bm->new_needed(*s, n_tokens);
  const int64_t cow = bm->cow_needed(*s, n_tokens);
  if (cow > max_pairs || (cow > 0 && !cow_pairs)) return PA_ERR_INVALID_ARG;
  if (fresh + cow > (int64_t)bm->free_list.size()) return PA_ERR_NO_BLOCKS;
  try {
    s->table.reserve(s->table.size() + (size_t)fresh);
  } catch (...) {
    return PA_ERR_INVALID_ARG;
  }
  int np = 0;
  for (int i = 0; i < n_tokens; ++i) {
    const int64_t pos = s->len;
    const int64_t j = pos / B, off = pos % B;
    if (j == (int64_t)s->table.size()) {
      s->table.push_back(bm->take());  // a token that starts a block takes a free block
    } else if (bm->ref[s->table[j]] > 1) {
      const int32_t old = s->table[j];  // shared: copy this block only, repoint the writer
      const int32_t fresh_block = bm->take();
      cow_pairs[2 * np] = old;
      cow_pairs[2 * np + 1] = fresh_block;
      ++np;
      bm->drop(old);
      s->table[j] = fresh_block;
    }
    slots[i] = (int32_t)(s->table[j] * B + off);
    s->len += 1;
  }
  *n_pairs = np;
  return PA_OK;
}

pa_status pa_bm_release(pa_bm* bm, int64_t seq) {
  if (!bm) return PA_ERR_INVALID_ARG;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_ERR_INVALID_ARG;
  for (int32_t b : it->second.table) bm->drop(b);
  bm->seqs.erase(it);
  return PA_OK;
}

pa_status pa_bm_move(pa_bm* from, pa_bm* to, int64_t seq, int32_t* pairs, int max_pairs,
                     int* n_pairs) {
  if (!from || !to || from == to || !n_pairs || from->block_size != to->block_size)
    return PA_ERR_INVALID_ARG;
  const pa_bm::Seq* s = from->find(seq);
  if (!s || to->find(seq)) return PA_ERR_INVALID_ARG;
  const int64_t n = (int64_t)s->table.size();
  if (n > max_pairs || (n > 0 && !pairs)) return PA_ERR_INVALID_ARG;
  if (n > (int64_t)to->free_list.size()) return PA_ERR_NO_BLOCKS;
  pa_bm::Seq* moved = nullptr;
  try {  // the only steps that may throw come first, before anything is changed
    pa_bm::Seq fresh;
    fresh.table.reserve((size_t)n);
    moved = &to->seqs.emplace(seq, std::move(fresh)).first->second;
  } catch (...) {
    return PA_ERR_INVALID_ARG;
  }
  moved->len = s->len;
  for (int64_t j = 0; j < n; ++j) {
    const int32_t dst = to->take();
    pairs[2 * j] = s->table[(size_t)j];
    pairs[2 * j + 1] = dst;
    moved->table.push_back(dst);  // capacity reserved: no allocation
  }
  *n_pairs = (int)n;
  return pa_bm_release(from, seq);
}

int64_t pa_bm_length(const pa_bm* bm, int64_t seq) {
  const pa_bm::Seq* s = bm ? bm->find(seq) : nullptr;
  return s ? s->len : -1;
}

int pa_bm_num_seq_blocks(const pa_bm* bm, int64_t seq) {
  const pa_bm::Seq* s = bm ? bm->find(seq) : nullptr;
  return s ? (int)s->table.size() : -1;
}

pa_status pa_bm_tables(const pa_bm* bm, const int64_t* seqs, int n, int32_t* out, int width,
                       int32_t pad) {
  if (!bm || n < 0 || width < 0 || (n > 0 && (!seqs || !out))) return PA_ERR_INVALID_ARG;
  for (int i = 0; i < n; ++i) {
    const pa_bm::Seq* s = bm->find(seqs[i]);
    if (!s || (int64_t)s->table.size() > width) return PA_ERR_INVALID_ARG;
  }
  for (int i = 0; i < n; ++i) {
    const pa_bm::Seq* s = bm->find(seqs[i]);
    int32_t* row = out + (int64_t)i * width;
    const int m = (int)s->table.size();
    std::copy(s->table.begin(), s->table.end(), row);
    std::fill(row + m, row + width, pad);
  }
  return PA_OK;
}

pa_status pa_bm_prefix_groups(const pa_bm* bm, const int64_t* seqs, int n, int32_t* group_start,
                              int* num_groups, int32_t* prefix_lens) {
  if (!bm || n < 0 || !num_groups || !group_start || (n > 0 && (!seqs || !prefix_lens)))
    return PA_ERR_INVALID_ARG;
  for (int i = 0; i < n; ++i)
    if (!bm->find(seqs[i])) return PA_ERR_INVALID_ARG;
  const int64_t B = bm->block_size;
  int ng = 0;
  for (int i = 0; i < n;) {
    const pa_bm::Seq* lead = bm->find(seqs[i]);
    // the run of sequences whose tables start with the leader's first block
    int j = i + 1;
    while (j < n && !lead->table.empty()) {
      const pa_bm::Seq* t = bm->find(seqs[j]);
      if (t->table.empty() || t->table[0] != lead->table[0]) break;
      ++j;
    }
    int64_t shared = 0;
    if (j - i > 1) {
      // leading table entries common to every member, and the shortest member's length
      size_t common = lead->table.size();
      int64_t min_len = lead->len;
      for (int k = i + 1; k < j; ++k) {
        const pa_bm::Seq* t = bm->find(seqs[k]);
        size_t c = 0;
        while (c < common && c < t->table.size() && t->table[c] == lead->table[c]) ++c;
        common = c;
        min_len = std::min(min_len, t->len);
      }
      shared = std::min<int64_t>((int64_t)common * B, min_len);
    }
    group_start[ng++] = i;
    for (int k = i; k < j; ++k) prefix_lens[k] = (int32_t)shared;
    i = j;
  }
  group_start[ng] = n;
  *num_groups = ng;
  return PA_OK;
}

int32_t pa_bm_refcount(const pa_bm* bm, int64_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->ref[(size_t)block];
}

pa_status pa_bm_get_stats(const pa_bm* bm, pa_bm_stats* out) {
  if (!bm || !out) return PA_ERR_INVALID_ARG;
  pa_bm_stats st{};
  st.num_blocks = bm->num_blocks;
  st.free_blocks = (int64_t)bm->free_list.size();
  st.num_seqs = (int64_t)bm->seqs.size();
  std::vector<int32_t> fill;
  try {
    fill.assign((size_t)bm->num_blocks, 0);
  } catch (...) {
    return PA_ERR_INVALID_ARG;
  }
  const int64_t B = bm->block_size;
  for (const auto& kv : bm->seqs) {
    const pa_bm::Seq& s = kv.second;
    st.logical_blocks += (int64_t)s.table.size();
    st.tokens += s.len;
    for (size_t j = 0; j < s.table.size(); ++j) {
      const int64_t f = std::min<int64_t>(B, std::max<int64_t>(0, s.len - (int64_t)j * B));
      fill[(size_t)s.table[j]] = (int32_t)std::max<int64_t>(fill[(size_t)s.table[j]], f);
    }
  }
  for (int64_t b = 0; b < bm->num_blocks; ++b) {
    if (bm->ref[(size_t)b] > 0) ++st.used_blocks;
    if (bm->ref[(size_t)b] > 1) ++st.shared_blocks;
    st.filled_slots += fill[(size_t)b];
  }
  st.reserved_slots = st.used_blocks * B;
  *out = st;
  return PA_OK;
}

}  // extern "C"
