// Randomised operation sequences against the host block allocator through its C ABI, for a
// build with AddressSanitizer and UndefinedBehaviorSanitizer (host code only).  After every
// call it checks the allocator's invariants from the outside: free + referenced blocks =
// pool size, reference counts equal the number of tables holding each block, and a failed
// call changes nothing.  It also keeps its own model of the pools' content: every slot holds
// an id standing for what was written there (for a prompt token, the whole token prefix
// ending at it; for other tokens a fresh id), block copies and swaps move these ids, and
// after every call each sequence must read back, through its block table, exactly the ids of
// its own tokens.  Exit status 0 = all checks passed.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <vector>

#include "pkv.h"

namespace {

uint64_t rng_state = 0x9E3779B97F4A7C15ull;
uint32_t next_u32() {  // xorshift64*
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return uint32_t((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
uint32_t below(uint32_t n) { return next_u32() % n; }

int fail(const char* what, int iter) {
  std::fprintf(stderr, "invariant violated at op %d: %s\n", iter, what);
  return 1;
}

struct Snapshot {
  int32_t free_blocks;
  int32_t cached_blocks;
  std::vector<int32_t> refs;
  std::map<int64_t, std::vector<int32_t>> tables;
  std::map<int64_t, int32_t> lens;
};

Snapshot snap(const pkv_alloc* a, int32_t nblocks, const std::vector<int64_t>& ids) {
  Snapshot s;
  s.free_blocks = pkv_num_free_blocks(a);
  s.cached_blocks = pkv_num_cached_blocks(a);
  for (int32_t b = 0; b < nblocks; ++b) s.refs.push_back(pkv_block_refcount(a, b));
  for (int64_t id : ids) {
    int32_t len = 0;
    if (pkv_seq_length(a, id, &len) != PKV_OK) continue;
    std::vector<int32_t> row(size_t(nblocks) + 1);
    if (pkv_get_block_tables(a, &id, 1, nblocks + 1, row.data(), nullptr) != PKV_OK) continue;
    while (!row.empty() && row.back() == -1) row.pop_back();
    s.tables[id] = row;
    s.lens[id] = len;
  }
  return s;
}

bool same(const Snapshot& x, const Snapshot& y) {
  return x.free_blocks == y.free_blocks && x.cached_blocks == y.cached_blocks && x.refs == y.refs && x.tables == y.tables && x.lens == y.lens;
}

}  // namespace

int main(int argc, char** argv) {
  const int iters = argc > 1 ? std::atoi(argv[1]) : 20000;
  const std::vector<int64_t> ids = {0, 1, 2, 3, 4, 5, 6, 7};
  for (int round = 0; round < 40; ++round) {
    const int32_t nblocks = 1 + int32_t(below(24));
    const int32_t bs = 1 << below(5);
    std::vector<int32_t> order(nblocks);
    for (int32_t i = 0; i < nblocks; ++i) order[i] = i;
    for (int32_t i = nblocks - 1; i > 0; --i) std::swap(order[i], order[below(uint32_t(i) + 1)]);
    pkv_alloc* a = nullptr;
    if (pkv_alloc_create(nblocks, bs, round % 2 ? order.data() : nullptr, &a) != PKV_OK) return fail("create", -1);
    // Content model: what each slot holds, each sequence's tokens, and swapped-out copies.
    std::vector<int64_t> pool(size_t(nblocks) * bs, -1);
    std::map<int64_t, std::vector<int64_t>> content;
    std::map<int64_t, std::pair<std::vector<int64_t>, std::vector<int64_t>>> parked;
    std::map<std::vector<int32_t>, int64_t> prefix_ids;
    int64_t next_id = 1;
    auto copy_block = [&](int32_t from, int32_t to) {
      for (int32_t i = 0; i < bs; ++i) pool[size_t(to) * bs + i] = pool[size_t(from) * bs + i];
    };
    // A few "system prompts" that prompts start with, so that cached prefixes repeat.
    std::vector<std::vector<int32_t>> systems(3);
    for (auto& sp : systems) {
      sp.resize(below(uint32_t(3 * bs + 1)));
      for (auto& t : sp) t = int32_t(below(3));
    }
    for (int it = 0; it < iters / 40; ++it) {
      const Snapshot before = snap(a, nblocks, ids);
      const uint32_t op = below(10);
      pkv_status st = PKV_OK;
      if (op == 0) {
        const int32_t n = int32_t(below(uint32_t(3 * bs + 2)));
        std::vector<int64_t> slots(size_t(n) + 1);
        const int64_t id = ids[below(8)];
        st = pkv_seq_add(a, id, n, slots.data());
        if (st == PKV_OK) {
          auto& c = content[id];
          for (int32_t t = 0; t < n; ++t) c.push_back(pool[slots[t]] = next_id++);
        }
      } else if (op == 1) {
        const int64_t p = ids[below(8)], c = ids[below(8)];
        st = pkv_seq_fork(a, p, c);
        if (st == PKV_OK) content[c] = content[p];
      } else if (op == 2) {
        const int64_t id = ids[below(8)];
        st = pkv_seq_free(a, id);
        if (st == PKV_OK) content.erase(id);
      } else if (op == 6 || op == 7) {
        std::vector<int32_t> blocks(size_t(nblocks) + 1);
        int32_t nb = -1;
        const int64_t id = ids[below(8)];
        st = op == 6 ? pkv_seq_swap_out(a, id, nblocks, blocks.data(), &nb)
                     : pkv_seq_swap_in(a, id, nblocks, blocks.data(), &nb);
        if (st == PKV_OK && (nb < 0 || nb > nblocks)) return fail("swap block count", it);
        if (st == PKV_OK && op == 6) {
          auto& park = parked[id];
          park.first.clear();
          for (int32_t i = 0; i < nb; ++i)
            for (int32_t j = 0; j < bs; ++j) park.first.push_back(pool[size_t(blocks[i]) * bs + j]);
          park.second = content[id];
          content.erase(id);
        } else if (st == PKV_OK) {
          auto& park = parked[id];
          for (int32_t i = 0; i < nb; ++i)
            for (int32_t j = 0; j < bs; ++j) pool[size_t(blocks[i]) * bs + j] = park.first[size_t(i) * bs + j];
          content[id] = park.second;
          parked.erase(id);
        }
      } else if (op == 8 || op == 9) {
        std::vector<int32_t> toks = systems[below(3)];
        for (uint32_t k = below(uint32_t(2 * bs + 2)); k > 0; --k) toks.push_back(int32_t(below(3)));
        std::vector<int64_t> slots(toks.size() + 1);
        int32_t ncached = -1;
        const int64_t id = ids[below(8)];
        st = pkv_seq_add_tokens(a, id, toks.empty() ? nullptr : toks.data(),
                                int32_t(toks.size()), slots.data(), &ncached);
        if (st == PKV_OK) {
          auto& c = content[id];
          std::vector<int32_t> prefix;
          for (size_t t = 0; t < toks.size(); ++t) {
            prefix.push_back(toks[t]);
            auto f = prefix_ids.emplace(prefix, next_id);
            if (f.second) ++next_id;
            c.push_back(f.first->second);
            if (slots[t] >= 0) pool[slots[t]] = f.first->second;
          }
        }
        if (st == PKV_OK && (ncached < 0 || ncached > int32_t(toks.size()) || ncached % bs))
          return fail("cached token count", it);
        for (int32_t t = 0; st == PKV_OK && t < int32_t(toks.size()); ++t)
          if ((t < ncached) != (slots[t] < 0)) return fail("cached slots", it);
      } else if (op == 5) {
        const int32_t n = int32_t(below(uint32_t(2 * bs + 3)));
        std::vector<int64_t> slots(size_t(n) + 1);
        int32_t pairs[2] = {-1, -1}, ncow = -1;
        const int64_t id = ids[below(8)];
        st = pkv_seq_extend(a, id, n, slots.data(), pairs, &ncow);
        if (st == PKV_OK && (ncow < 0 || ncow > 1)) return fail("extend cow count", it);
        if (st == PKV_OK) {
          if (ncow) copy_block(pairs[0], pairs[1]);
          for (int32_t t = 0; t < n; ++t) content[id].push_back(pool[slots[t]] = next_id++);
        }
      } else {
        const int32_t n = 1 + int32_t(below(4));
        std::vector<int64_t> seqs(n);
        for (auto& s : seqs) s = ids[below(8)];
        std::vector<int64_t> slots(n);
        std::vector<int32_t> pairs(2 * size_t(n));
        int32_t ncow = -1;
        st = pkv_seq_append(a, seqs.data(), n, slots.data(), pairs.data(), &ncow);
        if (st == PKV_OK && (ncow < 0 || ncow > n)) return fail("cow count", it);
        if (st == PKV_OK) {
          for (int32_t i = 0; i < ncow; ++i) copy_block(pairs[2 * i], pairs[2 * i + 1]);
          for (int32_t i = 0; i < n; ++i) content[seqs[i]].push_back(pool[slots[i]] = next_id++);
        }
      }
      const Snapshot after = snap(a, nblocks, ids);
      if (st != PKV_OK && !same(before, after)) return fail("failed call changed state", it);
      // Invariants of the state after the call.
      std::vector<int32_t> count(nblocks, 0);
      for (const auto& kv : after.tables) {
        const int64_t need = (after.lens.at(kv.first) + bs - 1) / bs;
        if (int64_t(kv.second.size()) != need) return fail("table length", it);
        for (int32_t b : kv.second) {
          if (b < 0 || b >= nblocks) return fail("block id range", it);
          ++count[b];
        }
      }
      int32_t referenced = 0;
      for (int32_t b = 0; b < nblocks; ++b) {
        if (count[b] != after.refs[b]) return fail("reference count", it);
        referenced += count[b] > 0;
      }
      if (referenced + after.free_blocks != nblocks) return fail("free + referenced", it);
      if (after.cached_blocks < 0 || after.cached_blocks > nblocks) return fail("cached count", it);
      // Every sequence reads back its own tokens' content through its table.
      if (after.tables.size() != content.size()) return fail("sequence set", it);
      for (const auto& kv : after.tables) {
        const auto& want = content[kv.first];
        if (int64_t(want.size()) != after.lens.at(kv.first)) return fail("content length", it);
        for (size_t t = 0; t < want.size(); ++t)
          if (pool[size_t(kv.second[t / bs]) * bs + t % bs] != want[t]) return fail("read-back content", it);
      }
      int32_t shared = -1;
      for (const auto& kv : after.tables) {
        int64_t id = kv.first;
        if (pkv_shared_prefix_blocks(a, &id, 1, &shared) != PKV_OK) return fail("shared query", it);
        int32_t k = 0;
        while (k < int32_t(kv.second.size()) && after.refs[kv.second[k]] > 1) ++k;
        if (shared != k) return fail("shared prefix count", it);
      }
    }
    pkv_alloc_destroy(a);
  }
  std::printf("ok\n");
  return 0;
}
