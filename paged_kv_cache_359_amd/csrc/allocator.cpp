// Host block allocator: the KV Cache Manager side of paged attention.
//
// One pool of fixed-size physical blocks shared by all sequences, one block table per
// sequence mapping logical page -> physical block, blocks handed out on demand as a
// sequence grows and returned when it ends ("vLLM + PagedAttention：打造高并发LLM推理引擎",
// steps 1, 2 and 4 under "它是怎么工作的？"; "PagedAttention 与 vLLM 推理加速", §2.2–§2.4;
// "LLM Systems 24: Efficient LLM Inference with PagedAttention and vLLM", §2.1.3).
// Blocks shared by several sequences (a common system prompt) carry a reference count and
// are copied before a sharer writes into them ("PagedAttention 与 vLLM 推理加速", §3.2 (3);
// "LLM Systems 24", §3 Conclusion).  Running out of blocks is reported, never partially
// applied, so the caller can preempt a sequence and retry (same Conclusion).
//
// Prompts that start with the same tokens share the blocks of that prefix even when they
// arrive independently (prefix caching; "PagedAttention 与 vLLM 推理加速", §3.2 (3): requests
// with one system prompt keep a single copy of its K/V).  A full prompt block is found by
// its content: the content id of the block before it plus its own token ids, so a match
// means the whole token prefix matches.  Cached blocks nobody holds stay cached until their
// block is needed again, and are then evicted in the order they were released (a
// sequence's blocks tail first), after the plain free blocks are used up.
//
// Per decode step the work is O(number of sequences appended): a length check, at most one
// stack pop, and one slot computation each.  Plain single-threaded host code, no HIP.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <list>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pkv.h"

namespace {

struct Sequence {
  std::vector<int32_t> table;  // logical page -> physical block
  int32_t len = 0;             // tokens stored
};

}  // namespace

struct pkv_alloc {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_stack;  // back() is handed out next
  std::vector<int32_t> ref;         // references per physical block
  std::unordered_map<int64_t, Sequence> seqs;
  // Sequences preempted to the host: length and number of blocks to restore.
  std::unordered_map<int64_t, std::pair<int32_t, int32_t>> swapped;

  // Prefix cache.  A registered block is found by its content: the content id of the
  // block before it (-1 for a first block) and its own block_size token ids.  Entries are
  // indexed by a 64-bit hash of that content and confirmed by comparing it in full, so a
  // hash collision never makes a false match.  Content ids are never reused, so content
  // whose parent was evicted can no longer be looked up.
  std::unordered_multimap<uint64_t, int32_t> cache;
  std::vector<int32_t> blk_tokens;  // [num_blocks * block_size]: a registered block's tokens
  std::vector<int64_t> parent_of;   // per block: parent content id while registered
  std::vector<uint64_t> hash_of;    // per block: content hash while registered
  std::vector<int64_t> cid;         // per block: content id, -1 when not registered
  int64_t next_cid = 0;
  int32_t n_registered = 0;
  std::list<int32_t> evictable;  // registered blocks with no holder; front goes first
  std::vector<std::list<int32_t>::iterator> evict_pos;
  std::vector<char> in_evictable;

  bool taken(int64_t id) const { return seqs.count(id) || swapped.count(id); }

  // Blocks a call may take: free ones, then evictable cached ones.
  int64_t available() const { return int64_t(free_stack.size()) + int64_t(evictable.size()); }

  int32_t pop() {
    int32_t b;
    if (!free_stack.empty()) {
      b = free_stack.back();
      free_stack.pop_back();
    } else {
      b = evictable.front();
      evictable.pop_front();
      in_evictable[b] = 0;
      unregister(b);
    }
    ref[b] = 1;
    return b;
  }
  void unregister(int32_t b) {
    auto range = cache.equal_range(hash_of[b]);
    for (auto it = range.first; it != range.second; ++it)
      if (it->second == b) {
        cache.erase(it);
        break;
      }
    cid[b] = -1;
    --n_registered;
  }
  uint64_t content_hash(int64_t parent, const int32_t* toks) const {
    // 64-bit multiply-xorshift mixing of the parent id and each token.
    uint64_t h = uint64_t(parent) * 0x9E3779B97F4A7C15ull ^ 0xD6E8FEB86659FD93ull;
    for (int32_t i = 0; i < block_size; ++i) {
      h ^= uint32_t(toks[i]);
      h *= 0xBF58476D1CE4E5B9ull;
      h ^= h >> 31;
    }
#ifdef PKV_HASH_BITS
    // Test builds narrow the hash so that different contents collide all the time.
    h &= (uint64_t(1) << PKV_HASH_BITS) - 1;
#endif
    return h;
  }
  // The registered block holding this content, or -1.
  int32_t find(int64_t parent, const int32_t* toks) const {
    auto range = cache.equal_range(content_hash(parent, toks));
    for (auto it = range.first; it != range.second; ++it) {
      const int32_t b = it->second;
      if (parent_of[b] == parent &&
          std::memcmp(&blk_tokens[size_t(b) * block_size], toks,
                      size_t(block_size) * sizeof(int32_t)) == 0)
        return b;
    }
    return -1;
  }
  void register_block(int32_t b, int64_t parent, const int32_t* toks) {
    cid[b] = next_cid++;
    parent_of[b] = parent;
    hash_of[b] = content_hash(parent, toks);
    std::memcpy(&blk_tokens[size_t(b) * block_size], toks, size_t(block_size) * sizeof(int32_t));
    cache.emplace(hash_of[b], b);
    ++n_registered;
  }
  // One reference less on each block of a table (logical order).  Blocks left with none go
  // onto the free stack in logical order, or, if they hold a cached prefix, to the back of
  // the eviction order tail first.
  void release(const std::vector<int32_t>& table) {
    std::vector<int32_t> gone;
    for (int32_t b : table)
      if (--ref[b] == 0) gone.push_back(b);
    for (int32_t b : gone)
      if (cid[b] < 0) free_stack.push_back(b);
    for (auto it = gone.rbegin(); it != gone.rend(); ++it) {
      const int32_t b = *it;
      if (cid[b] < 0) continue;
      evictable.push_back(b);
      evict_pos[b] = std::prev(evictable.end());
      in_evictable[b] = 1;
    }
  }
  int64_t slot_of(const Sequence& s) const {
    // Token number s.len sits in logical page len / bs at offset len % bs.
    return int64_t(s.table[s.len / block_size]) * block_size + s.len % block_size;
  }
};

extern "C" {

pkv_status pkv_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                            pkv_alloc** out) {
  if (!out || num_blocks <= 0 || block_size <= 0) return PKV_ERR_INVALID_ARG;
  *out = nullptr;
  pkv_alloc* a = new (std::nothrow) pkv_alloc();
  if (!a) return PKV_ERR_INVALID_ARG;
  a->num_blocks = num_blocks;
  a->block_size = block_size;
  a->ref.assign(num_blocks, 0);
  a->blk_tokens.assign(size_t(num_blocks) * block_size, 0);
  a->parent_of.assign(num_blocks, -1);
  a->hash_of.assign(num_blocks, 0);
  a->cid.assign(num_blocks, -1);
  a->evict_pos.resize(num_blocks);
  a->in_evictable.assign(num_blocks, 0);
  a->free_stack.resize(num_blocks);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete a;
        return PKV_ERR_INVALID_ARG;
      }
      seen[b] = 1;
    }
  }
  // Stack top is the back, so the first pop returns free_order[0].
  for (int32_t i = 0; i < num_blocks; ++i)
    a->free_stack[num_blocks - 1 - i] = free_order ? free_order[i] : i;
  *out = a;
  return PKV_OK;
}

void pkv_alloc_destroy(pkv_alloc* a) { delete a; }

pkv_status pkv_seq_add(pkv_alloc* a, int64_t seq_id, int32_t num_tokens, int64_t* slots_out) {
  if (!a || num_tokens < 0 || (num_tokens > 0 && !slots_out)) return PKV_ERR_INVALID_ARG;
  if (a->taken(seq_id)) return PKV_ERR_DUPLICATE_SEQ;
  const int64_t need = (int64_t(num_tokens) + a->block_size - 1) / a->block_size;
  if (need > a->available()) return PKV_ERR_OUT_OF_BLOCKS;
  Sequence s;
  s.table.reserve(need);
  for (int64_t i = 0; i < need; ++i) s.table.push_back(a->pop());
  for (int32_t t = 0; t < num_tokens; ++t) {
    slots_out[t] = a->slot_of(s);
    ++s.len;
  }
  a->seqs.emplace(seq_id, std::move(s));
  return PKV_OK;
}

pkv_status pkv_seq_add_tokens(pkv_alloc* a, int64_t seq_id, const int32_t* tokens,
                              int32_t num_tokens, int64_t* slots_out, int32_t* n_cached_out) {
  if (!a || num_tokens < 0 || !n_cached_out) return PKV_ERR_INVALID_ARG;
  if (num_tokens > 0 && (!tokens || !slots_out)) return PKV_ERR_INVALID_ARG;
  if (a->taken(seq_id)) return PKV_ERR_DUPLICATE_SEQ;
  const int32_t bs = a->block_size;
  const int32_t full = num_tokens / bs;
  const int64_t nb = (int64_t(num_tokens) + bs - 1) / bs;
  // Longest run of leading full blocks whose prefixes are cached.
  std::vector<int32_t> hits;
  int64_t parent = -1;
  int64_t reused_idle = 0;
  for (int32_t j = 0; j < full; ++j) {
    const int32_t b = a->find(parent, tokens + int64_t(j) * bs);
    if (b < 0) break;
    hits.push_back(b);
    if (a->ref[b] == 0) ++reused_idle;
    parent = a->cid[b];
  }
  const int64_t need = nb - int64_t(hits.size());
  if (need > a->available() - reused_idle) return PKV_ERR_OUT_OF_BLOCKS;
  for (int32_t b : hits) {
    if (a->in_evictable[b]) {
      a->evictable.erase(a->evict_pos[b]);
      a->in_evictable[b] = 0;
    }
    ++a->ref[b];
  }
  Sequence s;
  s.table = hits;
  s.table.reserve(nb);
  for (int64_t j = int64_t(hits.size()); j < nb; ++j) {
    const int32_t b = a->pop();
    s.table.push_back(b);
    if ((j + 1) * bs <= num_tokens) {  // a full prompt block: register its content
      a->register_block(b, parent, tokens + j * bs);
      parent = a->cid[b];
    }
  }
  const int64_t shared = int64_t(hits.size()) * bs;
  for (int32_t t = 0; t < num_tokens; ++t)
    slots_out[t] = t < shared ? -1 : int64_t(s.table[t / bs]) * bs + t % bs;
  s.len = num_tokens;
  *n_cached_out = int32_t(shared);
  a->seqs.emplace(seq_id, std::move(s));
  return PKV_OK;
}

pkv_status pkv_seq_fork(pkv_alloc* a, int64_t parent_id, int64_t child_id) {
  if (!a) return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(parent_id);
  if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
  if (a->taken(child_id)) return PKV_ERR_DUPLICATE_SEQ;
  Sequence child = it->second;  // copy table and length
  for (int32_t b : child.table) ++a->ref[b];
  a->seqs.emplace(child_id, std::move(child));
  return PKV_OK;
}

pkv_status pkv_seq_append(pkv_alloc* a, const int64_t* seq_ids, int32_t n, int64_t* slots_out,
                          int32_t* cow_pairs_out, int32_t* n_cow_out) {
  if (!a || n < 0 || !n_cow_out) return PKV_ERR_INVALID_ARG;
  if (n > 0 && (!seq_ids || !slots_out || !cow_pairs_out)) return PKV_ERR_INVALID_ARG;
  // Validate everything and count the blocks this call needs before changing anything.
  std::vector<Sequence*> rows(n);
  {
    std::unordered_set<int64_t> distinct;
    distinct.reserve(size_t(n) * 2);
    for (int32_t i = 0; i < n; ++i) {
      auto it = a->seqs.find(seq_ids[i]);
      if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
      rows[i] = &it->second;
    }
    for (int32_t i = 0; i < n; ++i)
      if (!distinct.insert(seq_ids[i]).second) return PKV_ERR_INVALID_ARG;
  }
  int64_t need = 0;
  std::unordered_map<int32_t, int32_t> dropped;  // simulated reference losses from CoW
  for (int32_t i = 0; i < n; ++i) {
    const Sequence& s = *rows[i];
    if (s.len % a->block_size == 0) {
      ++need;
    } else {
      int32_t last = s.table.back();
      int32_t& d = dropped[last];
      if (a->ref[last] - d > 1) {
        ++need;
        ++d;
      }
    }
  }
  if (need > a->available()) return PKV_ERR_OUT_OF_BLOCKS;

  int32_t ncow = 0;
  for (int32_t i = 0; i < n; ++i) {
    Sequence& s = *rows[i];
    if (s.len % a->block_size == 0) {
      s.table.push_back(a->pop());
    } else if (a->ref[s.table.back()] > 1) {
      // Copy-on-write: the sharer moves to a private copy; the others keep the original.
      int32_t old = s.table.back();
      int32_t fresh = a->pop();
      --a->ref[old];
      s.table.back() = fresh;
      cow_pairs_out[2 * ncow] = old;
      cow_pairs_out[2 * ncow + 1] = fresh;
      ++ncow;
    }
    slots_out[i] = a->slot_of(s);
    ++s.len;
  }
  *n_cow_out = ncow;
  return PKV_OK;
}

pkv_status pkv_seq_extend(pkv_alloc* a, int64_t seq_id, int32_t n, int64_t* slots_out,
                          int32_t* cow_pairs_out, int32_t* n_cow_out) {
  if (!a || n < 0 || !n_cow_out) return PKV_ERR_INVALID_ARG;
  if (n > 0 && (!slots_out || !cow_pairs_out)) return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
  Sequence& s = it->second;
  // Only the first token can meet a shared, partly filled last block; every later one lands
  // in a private block.
  const bool cow = n > 0 && s.len % a->block_size != 0 && a->ref[s.table.back()] > 1;
  const int64_t blocks_after = (int64_t(s.len) + n + a->block_size - 1) / a->block_size;
  const int64_t need = blocks_after - int64_t(s.table.size()) + (cow ? 1 : 0);
  if (need > a->available()) return PKV_ERR_OUT_OF_BLOCKS;
  int32_t ncow = 0;
  if (cow) {
    const int32_t old = s.table.back();
    const int32_t fresh = a->pop();
    --a->ref[old];
    s.table.back() = fresh;
    cow_pairs_out[0] = old;
    cow_pairs_out[1] = fresh;
    ncow = 1;
  }
  for (int32_t i = 0; i < n; ++i) {
    if (s.len % a->block_size == 0) s.table.push_back(a->pop());
    slots_out[i] = a->slot_of(s);
    ++s.len;
  }
  *n_cow_out = ncow;
  return PKV_OK;
}

pkv_status pkv_seq_free(pkv_alloc* a, int64_t seq_id) {
  if (!a) return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
  a->release(it->second.table);
  a->seqs.erase(it);
  return PKV_OK;
}

pkv_status pkv_seq_swap_out(pkv_alloc* a, int64_t seq_id, int32_t max_blocks, int32_t* blocks_out,
                            int32_t* n_blocks_out) {
  if (!a || max_blocks < 0 || !n_blocks_out) return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
  const Sequence& s = it->second;
  const int32_t nb = int32_t(s.table.size());
  if (nb > max_blocks || (nb > 0 && !blocks_out)) return PKV_ERR_INVALID_ARG;
  for (int32_t i = 0; i < nb; ++i) blocks_out[i] = s.table[i];
  *n_blocks_out = nb;
  a->swapped[seq_id] = {s.len, nb};
  a->release(s.table);
  a->seqs.erase(it);
  return PKV_OK;
}

pkv_status pkv_seq_swap_in(pkv_alloc* a, int64_t seq_id, int32_t max_blocks, int32_t* blocks_out,
                           int32_t* n_blocks_out) {
  if (!a || max_blocks < 0 || !n_blocks_out) return PKV_ERR_INVALID_ARG;
  auto it = a->swapped.find(seq_id);
  if (it == a->swapped.end()) return PKV_ERR_UNKNOWN_SEQ;
  const int32_t len = it->second.first, nb = it->second.second;
  if (nb > max_blocks || (nb > 0 && !blocks_out)) return PKV_ERR_INVALID_ARG;
  if (nb > a->available()) return PKV_ERR_OUT_OF_BLOCKS;
  Sequence s;
  s.len = len;
  s.table.reserve(nb);
  for (int32_t i = 0; i < nb; ++i) {
    s.table.push_back(a->pop());
    blocks_out[i] = s.table.back();
  }
  *n_blocks_out = nb;
  a->swapped.erase(it);
  a->seqs.emplace(seq_id, std::move(s));
  return PKV_OK;
}

pkv_status pkv_get_block_tables(const pkv_alloc* a, const int64_t* seq_ids, int32_t n,
                                int32_t max_blocks, int32_t* tables_out, int32_t* lens_out) {
  if (!a || n < 0 || max_blocks < 0) return PKV_ERR_INVALID_ARG;
  if (n > 0 && (!seq_ids || (max_blocks > 0 && !tables_out))) return PKV_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
    if (int64_t(it->second.table.size()) > max_blocks) return PKV_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < n; ++i) {
    const Sequence& s = a->seqs.find(seq_ids[i])->second;
    int32_t* row = tables_out + int64_t(i) * max_blocks;
    const size_t k = s.table.size();
    if (k) std::memcpy(row, s.table.data(), k * sizeof(int32_t));
    std::fill(row + k, row + max_blocks, -1);
    if (lens_out) lens_out[i] = s.len;
  }
  return PKV_OK;
}

pkv_status pkv_shared_prefix_blocks(const pkv_alloc* a, const int64_t* seq_ids, int32_t n,
                                    int32_t* out) {
  if (!a || n < 0) return PKV_ERR_INVALID_ARG;
  if (n > 0 && (!seq_ids || !out)) return PKV_ERR_INVALID_ARG;
  for (int32_t i = 0; i < n; ++i)
    if (!a->seqs.count(seq_ids[i])) return PKV_ERR_UNKNOWN_SEQ;
  for (int32_t i = 0; i < n; ++i) {
    const Sequence& s = a->seqs.find(seq_ids[i])->second;
    int32_t k = 0;
    while (k < int32_t(s.table.size()) && a->ref[s.table[k]] > 1) ++k;
    out[i] = k;
  }
  return PKV_OK;
}

pkv_status pkv_prefix_groups(const pkv_alloc* a, const int64_t* seq_ids, int32_t n,
                             int32_t* group_start_out, int32_t* shared_blocks_out,
                             int32_t* n_groups_out) {
  if (!a || n < 0 || !group_start_out || !n_groups_out) return PKV_ERR_INVALID_ARG;
  if (n > 0 && (!seq_ids || !shared_blocks_out)) return PKV_ERR_INVALID_ARG;
  std::vector<const Sequence*> rows(n);
  for (int32_t i = 0; i < n; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
    rows[i] = &it->second;
  }
  int32_t g = 0;
  group_start_out[0] = 0;
  for (int32_t i = 0; i < n;) {
    // The run of rows whose tables start with row i's first block.
    int32_t j = i + 1;
    if (!rows[i]->table.empty())
      while (j < n && !rows[j]->table.empty() && rows[j]->table[0] == rows[i]->table[0]) ++j;
    // Leading entries all members agree on, cut to the full blocks every member's length covers.
    int64_t k = 0;
    if (j - i >= 2) {
      k = int64_t(rows[i]->table.size());
      for (int32_t r = i; r < j; ++r) {
        const auto& t = rows[r]->table;
        int64_t c = 0;
        while (c < k && c < int64_t(t.size()) && t[c] == rows[i]->table[c]) ++c;
        k = std::min<int64_t>({k, c, rows[r]->len / a->block_size});
      }
    }
    if (k > 0) {
      for (int32_t r = i; r < j; ++r) shared_blocks_out[r] = int32_t(k);
      group_start_out[++g] = j;
    } else {
      for (int32_t r = i; r < j; ++r) {
        shared_blocks_out[r] = 0;
        group_start_out[++g] = r + 1;
      }
    }
    i = j;
  }
  *n_groups_out = g;
  return PKV_OK;
}

pkv_status pkv_seq_length(const pkv_alloc* a, int64_t seq_id, int32_t* len_out) {
  if (!a || !len_out) return PKV_ERR_INVALID_ARG;
  auto it = a->seqs.find(seq_id);
  if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
  *len_out = it->second.len;
  return PKV_OK;
}

pkv_status pkv_seq_lengths(const pkv_alloc* a, const int64_t* seq_ids, int32_t n,
                           int32_t* lens_out) {
  if (!a || n < 0) return PKV_ERR_INVALID_ARG;
  if (n > 0 && (!seq_ids || !lens_out)) return PKV_ERR_INVALID_ARG;
  // Resolve every id first, so that an unknown one leaves lens_out untouched.
  std::vector<int32_t> lens(n);
  for (int32_t i = 0; i < n; ++i) {
    auto it = a->seqs.find(seq_ids[i]);
    if (it == a->seqs.end()) return PKV_ERR_UNKNOWN_SEQ;
    lens[i] = it->second.len;
  }
  std::copy(lens.begin(), lens.end(), lens_out);
  return PKV_OK;
}

int32_t pkv_num_free_blocks(const pkv_alloc* a) {
  return a ? int32_t(a->available()) : -1;
}

int32_t pkv_num_cached_blocks(const pkv_alloc* a) { return a ? a->n_registered : -1; }

int32_t pkv_block_refcount(const pkv_alloc* a, int32_t block) {
  if (!a || block < 0 || block >= a->num_blocks) return -1;
  return a->ref[block];
}

pkv_status pkv_usage(const pkv_alloc* a, int64_t* tokens_stored, int64_t* slots_allocated) {
  if (!a || !tokens_stored || !slots_allocated) return PKV_ERR_INVALID_ARG;
  int64_t tok = 0;
  for (const auto& kv : a->seqs) tok += kv.second.len;
  int64_t used = a->num_blocks - a->available();
  *tokens_stored = tok;
  *slots_allocated = used * a->block_size;
  return PKV_OK;
}

const char* pkv_status_str(pkv_status s) {
  switch (s) {
    case PKV_OK: return "PKV_OK";
    case PKV_ERR_INVALID_ARG: return "PKV_ERR_INVALID_ARG";
    case PKV_ERR_OUT_OF_BLOCKS: return "PKV_ERR_OUT_OF_BLOCKS";
    case PKV_ERR_UNKNOWN_SEQ: return "PKV_ERR_UNKNOWN_SEQ";
    case PKV_ERR_DUPLICATE_SEQ: return "PKV_ERR_DUPLICATE_SEQ";
    case PKV_ERR_UNSUPPORTED: return "PKV_ERR_UNSUPPORTED";
    case PKV_ERR_WORKSPACE: return "PKV_ERR_WORKSPACE";
    case PKV_ERR_HIP: return "PKV_ERR_HIP";
    default: return "PKV_ERR_UNKNOWN_STATUS";
  }
}

int32_t pkv_version(void) { return 100; }

}  // extern "C"
