// Host-side KV block manager (libpabm.so).  The contract, and the passages it
// follows, are in include/pa_block_manager.h.
//
// Data structures (all O(1) per operation except where noted):
//  * free list: an intrusive doubly linked list over block ids (next/prev
//    arrays), first in first out, so a block taken back for prefix reuse can
//    be unlinked from the middle;
//  * per block: reference count and generation (bumped whenever the block is
//    handed out); with the prefix cache, whether it is registered, its key,
//    its parent block (the block before it in the sequence it was cached
//    from, -1 for a first block) with that block's generation at the time,
//    and its token ids;
//  * prefix cache: key -> block.  A lookup is a hit only when the block's
//    token ids equal the new sequence's and its parent is the block the new
//    sequence already took for the previous position; matching stops at the
//    first miss, so by induction every shared block was produced by exactly
//    the same token prefix (the parent's generation rules out a parent that
//    was evicted and handed out again);
//  * per sequence: block table, length and, while its token ids are known,
//    the key and block of its last full block plus the ids of the tokens in
//    its partly filled tail block.
#include "../../include/pa_block_manager.h"

#include <climits>
#include <cstring>
#include <memory>
#include <new>
#include <unordered_map>
#include <algorithm>
#include <vector>

namespace {

constexpr uint64_t kFnvOffset = 14695981039346656037ull;
constexpr uint64_t kFnvPrime = 1099511628211ull;

uint64_t fnv1a(uint64_t h, const unsigned char* p, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= kFnvPrime;
  }
  return h;
}

// Key of a full block: FNV-1a over the previous block's key (8 bytes, least
// significant first; 0 for a first block) followed by the block's token ids
// (4 bytes each, least significant first).
uint64_t block_key(uint64_t parent_key, const int32_t* tokens, int block_size) {
  unsigned char b[8];
  for (int i = 0; i < 8; ++i) b[i] = (unsigned char)(parent_key >> (8 * i));
  uint64_t h = fnv1a(kFnvOffset, b, 8);
  for (int t = 0; t < block_size; ++t) {
    const uint32_t v = (uint32_t)tokens[t];
    unsigned char w[4] = {(unsigned char)v, (unsigned char)(v >> 8), (unsigned char)(v >> 16),
                          (unsigned char)(v >> 24)};
    h = fnv1a(h, w, 4);
  }
  return h;
}

struct Sequence {
  std::vector<int64_t> table;
  int64_t length = 0;
  bool hashing = false;           // token ids known for the whole sequence
  uint64_t last_key = 0;          // key of the last full block (0 if none)
  int64_t last_full = -1;         // physical block of the last full block
  std::vector<int32_t> tail_tokens;
  uint64_t stamp = 0;             // last append step that touched it
};

}  // namespace

struct pa_bm {
  int64_t num_blocks = 0;
  int block_size = 0;
  bool prefix_cache = false;

  std::vector<int64_t> refcount;
  std::vector<uint64_t> gen;
  // free list
  std::vector<int64_t> next, prev;
  std::vector<unsigned char> in_free;
  int64_t head = -1, tail = -1, nfree = 0;
  // prefix cache
  std::vector<unsigned char> cached;
  std::vector<uint64_t> key;
  std::vector<int64_t> parent;
  std::vector<uint64_t> parent_gen;
  std::vector<int32_t> tokens;   // num_blocks * block_size when the cache is on
  std::unordered_map<uint64_t, int64_t> cache;

  std::unordered_map<int64_t, Sequence> seqs;
  int64_t prefix_hit_blocks = 0;
  int64_t copies = 0;
  uint64_t step = 0;              // append steps so far (duplicate detection)
  std::vector<Sequence*> batch;   // scratch of pa_bm_append_slots

  void push_back_free(int64_t b) {
    next[b] = -1;
    prev[b] = tail;
    if (tail >= 0) next[tail] = b; else head = b;
    tail = b;
    in_free[b] = 1;
    ++nfree;
  }
  void unlink_free(int64_t b) {
    if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
    if (next[b] >= 0) prev[next[b]] = prev[b]; else tail = prev[b];
    next[b] = prev[b] = -1;
    in_free[b] = 0;
    --nfree;
  }
  void uncache(int64_t b) {
    if (!cached[b]) return;
    auto it = cache.find(key[b]);
    if (it != cache.end() && it->second == b) cache.erase(it);
    cached[b] = 0;
  }
  // Takes the block at the head of the free list (evicting a cached prefix
  // block there); callers have checked nfree.
  int64_t allocate() {
    const int64_t b = head;
    unlink_free(b);
    uncache(b);
    refcount[b] = 1;
    ++gen[b];
    return b;
  }
  void release(int64_t b) {
    if (--refcount[b] == 0) push_back_free(b);
  }
  // Registers full block b (key k, parent block p, token ids tok) unless the
  // key is taken.
  void register_block(int64_t b, uint64_t k, int64_t p, const int32_t* tok) {
    if (!prefix_cache || cached[b] || cache.count(k)) return;
    cache.emplace(k, b);
    cached[b] = 1;
    key[b] = k;
    parent[b] = p;
    parent_gen[b] = p >= 0 ? gen[p] : 0;
    std::memcpy(&tokens[(size_t)b * block_size], tok, sizeof(int32_t) * block_size);
  }
  // The cached block for position i of a sequence whose previous position
  // holds block p and whose block has key k and token ids tok, or -1.
  int64_t lookup(uint64_t k, int64_t p, const int32_t* tok) const {
    auto it = cache.find(k);
    if (it == cache.end()) return -1;
    const int64_t b = it->second;
    if (parent[b] != p || (p >= 0 && parent_gen[b] != gen[p])) return -1;
    if (std::memcmp(&tokens[(size_t)b * block_size], tok, sizeof(int32_t) * block_size) != 0)
      return -1;
    return b;
  }
  int64_t blocks_for(int64_t length) const { return (length + block_size - 1) / block_size; }
};

extern "C" {

uint64_t pa_bm_fnv1a64(uint64_t seed, const void* data, int64_t bytes) {
  if (data == nullptr || bytes <= 0) return seed;
  return fnv1a(seed, static_cast<const unsigned char*>(data), bytes);
}

const char* pa_bm_status_string(int status) {
  switch (status) {
    case PA_BM_OK: return "ok";
    case PA_BM_INVALID: return "invalid argument";
    case PA_BM_EXHAUSTED: return "not enough free blocks";
    case PA_BM_UNKNOWN_SEQ: return "unknown sequence";
    case PA_BM_EXISTS: return "sequence already registered";
    case PA_BM_NOMEM: return "host allocation failed";
    case PA_BM_CORRUPT: return "block manager invariant broken";
    default: return "unknown status";
  }
}

int pa_bm_create(int64_t num_blocks, int block_size, const int64_t* free_order, int prefix_cache,
                 pa_bm** out) {
  if (out == nullptr) return PA_BM_INVALID;
  *out = nullptr;
  if (num_blocks <= 0 || block_size <= 0 || num_blocks > ((int64_t)1 << 40)) return PA_BM_INVALID;
  try {
    std::unique_ptr<pa_bm> m(new pa_bm());
    m->num_blocks = num_blocks;
    m->block_size = block_size;
    m->prefix_cache = prefix_cache != 0;
    m->refcount.assign(num_blocks, 0);
    m->gen.assign(num_blocks, 0);
    m->next.assign(num_blocks, -1);
    m->prev.assign(num_blocks, -1);
    m->in_free.assign(num_blocks, 0);
    m->cached.assign(num_blocks, 0);
    if (m->prefix_cache) {
      m->key.assign(num_blocks, 0);
      m->parent.assign(num_blocks, -1);
      m->parent_gen.assign(num_blocks, 0);
      m->tokens.assign((size_t)num_blocks * block_size, 0);
    }
    if (free_order == nullptr) {
      for (int64_t b = 0; b < num_blocks; ++b) m->push_back_free(b);
    } else {
      std::vector<unsigned char> seen(num_blocks, 0);
      for (int64_t i = 0; i < num_blocks; ++i) {
        const int64_t b = free_order[i];
        if (b < 0 || b >= num_blocks || seen[b]) return PA_BM_INVALID;   // not a permutation
        seen[b] = 1;
        m->push_back_free(b);
      }
    }
    *out = m.release();
    return PA_BM_OK;
  } catch (const std::bad_alloc&) {
    return PA_BM_NOMEM;
  }
}

void pa_bm_destroy(pa_bm* bm) { delete bm; }

int pa_bm_add_sequence(pa_bm* bm, int64_t seq, const int32_t* tokens, int64_t length,
                       int64_t* reused_tokens) {
  if (bm == nullptr || seq < 0 || length < 0) return PA_BM_INVALID;
  if (reused_tokens != nullptr) *reused_tokens = 0;
  if (bm->seqs.count(seq)) return PA_BM_EXISTS;
  try {
    const int bs = bm->block_size;
    const int64_t nblocks = bm->blocks_for(length);
    const int64_t nfull = length / bs;
    const bool hashing = bm->prefix_cache && tokens != nullptr;
    // Leading full blocks already cached (no state is changed yet).
    std::vector<int64_t> hits;
    std::vector<uint64_t> keys;
    if (hashing) {
      keys.resize(nfull);
      uint64_t k = 0;
      for (int64_t i = 0; i < nfull; ++i) {
        k = block_key(k, tokens + i * bs, bs);
        keys[i] = k;
      }
      int64_t p = -1;
      for (int64_t i = 0; i < nfull; ++i) {
        const int64_t b = bm->lookup(keys[i], p, tokens + i * bs);
        if (b < 0) break;
        hits.push_back(b);
        p = b;
      }
    }
    int64_t revived = 0;
    for (int64_t b : hits) revived += bm->in_free[b] ? 1 : 0;
    const int64_t fresh = nblocks - (int64_t)hits.size();
    if (bm->nfree - revived < fresh) return PA_BM_EXHAUSTED;

    Sequence s;
    s.table.reserve(nblocks);
    s.length = length;
    s.hashing = hashing;
    if (hashing) s.tail_tokens.reserve(bs);
    // Commit: shared blocks first (taken off the free list if unreferenced),
    // then fresh ones.
    for (int64_t b : hits) {
      if (bm->in_free[b]) bm->unlink_free(b);
      ++bm->refcount[b];
      s.table.push_back(b);
    }
    for (int64_t i = (int64_t)hits.size(); i < nblocks; ++i) s.table.push_back(bm->allocate());
    if (hashing) {
      for (int64_t i = (int64_t)hits.size(); i < nfull; ++i)
        bm->register_block(s.table[i], keys[i], i > 0 ? s.table[i - 1] : -1, tokens + i * bs);
      if (nfull > 0) {
        s.last_key = keys[nfull - 1];
        s.last_full = s.table[nfull - 1];
      }
      s.tail_tokens.assign(tokens + nfull * bs, tokens + length);
    }
    bm->prefix_hit_blocks += (int64_t)hits.size();
    if (reused_tokens != nullptr) *reused_tokens = (int64_t)hits.size() * bs;
    bm->seqs.emplace(seq, std::move(s));
    return PA_BM_OK;
  } catch (const std::bad_alloc&) {
    return PA_BM_NOMEM;
  }
}

int pa_bm_append_slots(pa_bm* bm, const int64_t* seqs, const int32_t* tokens, int64_t n,
                       int64_t* slots, int64_t* copies, int64_t* num_copies) {
  if (bm == nullptr || n < 0 || (n > 0 && (seqs == nullptr || slots == nullptr || copies == nullptr)) ||
      num_copies == nullptr)
    return PA_BM_INVALID;
  *num_copies = 0;
  try {
    const int bs = bm->block_size;
    // Validate and count the blocks this step takes, with the counts the
    // step itself changes (two sequences sharing one tail: only the first
    // writer copies).
    std::vector<Sequence*>& ss = bm->batch;
    ss.resize(n);
    const uint64_t step = ++bm->step;
    std::unordered_map<int64_t, int64_t> tail_refs;   // only for shared tails
    int64_t need = 0;
    for (int64_t i = 0; i < n; ++i) {
      auto it = bm->seqs.find(seqs[i]);
      if (it == bm->seqs.end()) return PA_BM_UNKNOWN_SEQ;
      Sequence& s = it->second;
      if (s.stamp == step) return PA_BM_INVALID;   // one token per sequence per step
      s.stamp = step;
      ss[i] = &s;
      if (s.length % bs == 0) {
        ++need;
      } else {
        const int64_t t = s.table.back();
        if (bm->refcount[t] > 1) {
          auto r = tail_refs.find(t);
          if (r == tail_refs.end()) r = tail_refs.emplace(t, bm->refcount[t]).first;
          if (r->second > 1) {
            ++need;
            --r->second;
          }
        }
      }
    }
    if (need > bm->nfree) return PA_BM_EXHAUSTED;
    // Room for one more block in every table (geometric growth), so the
    // commit below cannot fail halfway.
    for (int64_t i = 0; i < n; ++i) {
      std::vector<int64_t>& t = ss[i]->table;
      if (t.size() == t.capacity()) t.reserve(t.size() < 8 ? 8 : 2 * t.size());
    }

    int64_t nc = 0;
    for (int64_t i = 0; i < n; ++i) {
      Sequence& s = *ss[i];
      const int64_t len = s.length;
      if (len % bs == 0) {
        s.table.push_back(bm->allocate());
      } else {
        const int64_t t = s.table.back();
        if (bm->refcount[t] > 1) {
          const int64_t fresh = bm->allocate();
          copies[2 * nc] = t;
          copies[2 * nc + 1] = fresh;
          ++nc;
          --bm->refcount[t];
          s.table.back() = fresh;
        }
      }
      const int64_t block = s.table[len / bs];
      slots[i] = block * bs + len % bs;
      s.length = len + 1;
      if (s.hashing) {
        if (tokens == nullptr) {
          s.hashing = false;        // token ids of this sequence are no longer known
          s.tail_tokens.clear();
        } else {
          s.tail_tokens.push_back(tokens[i]);
          if (s.length % bs == 0) {   // the block just filled: cache it
            const uint64_t k = block_key(s.last_key, s.tail_tokens.data(), bs);
            bm->register_block(block, k, s.last_full, s.tail_tokens.data());
            s.last_key = k;
            s.last_full = block;
            s.tail_tokens.clear();
          }
        }
      }
    }
    bm->copies += nc;
    *num_copies = nc;
    return PA_BM_OK;
  } catch (const std::bad_alloc&) {
    return PA_BM_NOMEM;
  }
}

int pa_bm_fork(pa_bm* bm, int64_t parent, int64_t child) {
  if (bm == nullptr || child < 0) return PA_BM_INVALID;
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return PA_BM_UNKNOWN_SEQ;
  if (bm->seqs.count(child)) return PA_BM_EXISTS;
  try {
    Sequence c = it->second;   // copies table, length and token state
    for (int64_t b : c.table) ++bm->refcount[b];
    bm->seqs.emplace(child, std::move(c));
    return PA_BM_OK;
  } catch (const std::bad_alloc&) {
    return PA_BM_NOMEM;
  }
}

int pa_bm_free_sequence(pa_bm* bm, int64_t seq) {
  if (bm == nullptr) return PA_BM_INVALID;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_BM_UNKNOWN_SEQ;
  for (int64_t b : it->second.table) bm->release(b);
  bm->seqs.erase(it);
  return PA_BM_OK;
}

int pa_bm_fork_many(pa_bm* bm, const int64_t* parents, const int64_t* children, int64_t n) {
  if (bm == nullptr || n < 0 || (n > 0 && (parents == nullptr || children == nullptr)))
    return PA_BM_INVALID;
  try {
    // Check the whole batch first: pair i may fork a child made by an
    // earlier pair, never an unknown sequence; every child is new.
    std::unordered_map<int64_t, int64_t> made;   // child -> its parent in this batch
    made.reserve((size_t)n);
    for (int64_t i = 0; i < n; ++i) {
      if (children[i] < 0) return PA_BM_INVALID;
      if (!bm->seqs.count(parents[i]) && !made.count(parents[i])) return PA_BM_UNKNOWN_SEQ;
      if (bm->seqs.count(children[i]) || made.count(children[i])) return PA_BM_EXISTS;
      made.emplace(children[i], parents[i]);
    }
    int64_t done = 0;
    try {
      for (; done < n; ++done) {
        Sequence c = bm->seqs.at(parents[done]);
        for (int64_t b : c.table) ++bm->refcount[b];
        bm->seqs.emplace(children[done], std::move(c));
      }
    } catch (const std::bad_alloc&) {
      // Undo the pairs already applied, newest first.
      for (int64_t i = done - 1; i >= 0; --i) {
        auto it = bm->seqs.find(children[i]);
        for (int64_t b : it->second.table) --bm->refcount[b];
        bm->seqs.erase(it);
      }
      return PA_BM_NOMEM;
    }
    return PA_BM_OK;
  } catch (const std::bad_alloc&) {
    return PA_BM_NOMEM;
  }
}

int pa_bm_free_many(pa_bm* bm, const int64_t* seqs, int64_t n) {
  if (bm == nullptr || n < 0 || (n > 0 && seqs == nullptr)) return PA_BM_INVALID;
  try {
    std::unordered_map<int64_t, char> seen;
    seen.reserve((size_t)n);
    for (int64_t i = 0; i < n; ++i) {
      if (!bm->seqs.count(seqs[i])) return PA_BM_UNKNOWN_SEQ;
      if (!seen.emplace(seqs[i], 1).second) return PA_BM_INVALID;   // listed twice
    }
  } catch (const std::bad_alloc&) {
    return PA_BM_NOMEM;
  }
  for (int64_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    for (int64_t b : it->second.table) bm->release(b);
    bm->seqs.erase(it);
  }
  return PA_BM_OK;
}

int pa_bm_length(const pa_bm* bm, int64_t seq, int64_t* length) {
  if (bm == nullptr || length == nullptr) return PA_BM_INVALID;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return PA_BM_UNKNOWN_SEQ;
  *length = it->second.length;
  return PA_BM_OK;
}

int pa_bm_block_tables(const pa_bm* bm, const int64_t* seqs, int64_t n, int64_t max_blocks,
                       int32_t pad, int32_t* tables, int32_t* context_lens) {
  if (bm == nullptr || n < 0 || max_blocks < 0 || (n > 0 && (seqs == nullptr || tables == nullptr)))
    return PA_BM_INVALID;
  for (int64_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return PA_BM_UNKNOWN_SEQ;
    if ((int64_t)it->second.table.size() > max_blocks || it->second.length > INT32_MAX)
      return PA_BM_INVALID;
  }
  if (bm->num_blocks > INT32_MAX) return PA_BM_INVALID;   // block ids must fit the int32 tables
  for (int64_t i = 0; i < n; ++i) {
    const Sequence& s = bm->seqs.find(seqs[i])->second;
    int32_t* row = tables + i * max_blocks;
    const int64_t nb = (int64_t)s.table.size();
    for (int64_t j = 0; j < nb; ++j) row[j] = (int32_t)s.table[j];
    for (int64_t j = nb; j < max_blocks; ++j) row[j] = pad;
    if (context_lens != nullptr) context_lens[i] = (int32_t)s.length;
  }
  return PA_BM_OK;
}

int pa_bm_shared_prefix(const pa_bm* bm, const int64_t* seqs, int64_t n,
                        const int64_t* group_start, int64_t num_groups, int32_t* prefix_lens) {
  if (bm == nullptr || n < 0 || num_groups < 0 ||
      (n > 0 && (seqs == nullptr || prefix_lens == nullptr)) || group_start == nullptr)
    return PA_BM_INVALID;
  if (group_start[0] != 0 || group_start[num_groups] != n) return PA_BM_INVALID;
  for (int64_t g = 0; g < num_groups; ++g)
    if (group_start[g + 1] < group_start[g]) return PA_BM_INVALID;
  std::vector<const Sequence*> members((size_t)n);
  for (int64_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return PA_BM_UNKNOWN_SEQ;
    members[(size_t)i] = &it->second;
  }
  for (int64_t g = 0; g < num_groups; ++g) {
    const int64_t lo = group_start[g], hi = group_start[g + 1];
    int64_t shared = 0;
    if (hi - lo >= 2) {
      // Leading blocks every member holds (the same physical block), and at
      // most the shortest member's length in tokens.
      int64_t blocks = INT64_MAX, min_len = INT64_MAX;
      for (int64_t i = lo; i < hi; ++i) {
        blocks = std::min<int64_t>(blocks, (int64_t)members[(size_t)i]->table.size());
        min_len = std::min<int64_t>(min_len, members[(size_t)i]->length);
      }
      const std::vector<int64_t>& first = members[(size_t)lo]->table;
      int64_t same = 0;
      while (same < blocks) {
        bool all = true;
        for (int64_t i = lo + 1; i < hi && all; ++i)
          all = members[(size_t)i]->table[(size_t)same] == first[(size_t)same];
        if (!all) break;
        ++same;
      }
      shared = std::min<int64_t>(same * bm->block_size, min_len);
    }
    if (shared > INT32_MAX) return PA_BM_INVALID;
    for (int64_t i = lo; i < hi; ++i) prefix_lens[i] = (int32_t)shared;
  }
  return PA_BM_OK;
}

int pa_bm_refcount(const pa_bm* bm, int64_t block, int64_t* refcount) {
  if (bm == nullptr || refcount == nullptr || block < 0 || block >= bm->num_blocks)
    return PA_BM_INVALID;
  *refcount = bm->refcount[block];
  return PA_BM_OK;
}

int pa_bm_get_stats(const pa_bm* bm, pa_bm_stats* out) {
  if (bm == nullptr || out == nullptr) return PA_BM_INVALID;
  pa_bm_stats s;
  std::memset(&s, 0, sizeof(s));
  s.num_blocks = bm->num_blocks;
  s.block_size = bm->block_size;
  s.free_blocks = bm->nfree;
  for (int64_t b = 0; b < bm->num_blocks; ++b) {
    if (bm->refcount[b] > 0) ++s.used_blocks;
    if (bm->refcount[b] > 1) ++s.shared_blocks;
    if (bm->cached[b]) {
      ++s.cached_blocks;
      if (bm->in_free[b]) ++s.cached_free_blocks;
    }
  }
  s.sequences = (int64_t)bm->seqs.size();
  for (const auto& kv : bm->seqs) {
    const Sequence& q = kv.second;
    s.tokens += q.length;
    s.table_slots += (int64_t)q.table.size() * bm->block_size;
    s.tail_slack += (int64_t)q.table.size() * bm->block_size - q.length;
  }
  s.prefix_hit_blocks = bm->prefix_hit_blocks;
  s.copies = bm->copies;
  *out = s;
  return PA_BM_OK;
}

int pa_bm_check(const pa_bm* bm) {
  if (bm == nullptr) return PA_BM_INVALID;
  try {
    std::vector<int64_t> refs(bm->num_blocks, 0);
    for (const auto& kv : bm->seqs) {
      const Sequence& s = kv.second;
      if ((int64_t)s.table.size() != bm->blocks_for(s.length)) return PA_BM_CORRUPT;
      for (int64_t b : s.table) {
        if (b < 0 || b >= bm->num_blocks) return PA_BM_CORRUPT;
        ++refs[b];
      }
    }
    int64_t listed = 0;
    std::vector<unsigned char> seen(bm->num_blocks, 0);
    for (int64_t b = bm->head, p = -1; b >= 0; p = b, b = bm->next[b]) {
      if (b >= bm->num_blocks || seen[b] || bm->prev[b] != p || !bm->in_free[b]) return PA_BM_CORRUPT;
      seen[b] = 1;
      if (++listed > bm->num_blocks) return PA_BM_CORRUPT;
    }
    if (listed != bm->nfree) return PA_BM_CORRUPT;
    for (int64_t b = 0; b < bm->num_blocks; ++b) {
      if (refs[b] != bm->refcount[b]) return PA_BM_CORRUPT;
      if ((refs[b] == 0) != (seen[b] != 0)) return PA_BM_CORRUPT;   // free iff unreferenced
    }
    for (const auto& kv : bm->cache) {
      const int64_t b = kv.second;
      if (b < 0 || b >= bm->num_blocks || !bm->cached[b] || bm->key[b] != kv.first) return PA_BM_CORRUPT;
    }
    for (int64_t b = 0; b < bm->num_blocks; ++b) {
      if (!bm->cached[b]) continue;
      auto it = bm->cache.find(bm->key[b]);
      if (it == bm->cache.end() || it->second != b) return PA_BM_CORRUPT;
    }
    return PA_BM_OK;
  } catch (const std::bad_alloc&) {
    return PA_BM_NOMEM;
  }
}

}  // extern "C"
