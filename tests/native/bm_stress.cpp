// Random-operation stress of the host block manager, built with the host
// compiler's address and undefined-behaviour sanitizers by
// tests/test_bm_sanitize.py.  Every operation is followed by pa_bm_check;
// any failure exits non-zero.
#include "../../include/pa_block_manager.h"

#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

static int fail(const char* what, int st) {
  std::fprintf(stderr, "%s: %s\n", what, pa_bm_status_string(st));
  return 1;
}

static int run(unsigned seed, int prefix_cache) {
  std::mt19937_64 rng(seed);
  const int64_t nb = 64 + (int64_t)(rng() % 256);
  const int bs = 1 << (rng() % 5);
  pa_bm* bm = nullptr;
  int st = pa_bm_create(nb, bs, nullptr, prefix_cache, &bm);
  if (st) return fail("create", st);
  std::vector<int64_t> live;
  std::vector<std::vector<int32_t>> toks;   // per sequence id, its token ids
  int64_t next_id = 0;
  const int vocab = 3;                      // tiny vocabulary: many shared prefixes
  for (int op = 0; op < 20000; ++op) {
    const int kind = (int)(rng() % 5);
    if (kind == 0 || live.empty()) {
      const int64_t len = (int64_t)(rng() % (4 * bs + 1));
      std::vector<int32_t> t(len);
      for (auto& x : t) x = (int32_t)(rng() % vocab);
      int64_t reused = 0;
      st = pa_bm_add_sequence(bm, next_id, rng() % 2 ? t.data() : nullptr, len, &reused);
      if (st == PA_BM_OK) {
        live.push_back(next_id);
        toks.resize(next_id + 1);
        toks[next_id] = t;
        ++next_id;
      } else if (st != PA_BM_EXHAUSTED) {
        return fail("add", st);
      }
    } else if (kind == 1) {
      std::vector<int64_t> batch;
      for (int64_t s : live)
        if (rng() % 2) batch.push_back(s);
      std::vector<int32_t> nt(batch.size());
      for (auto& x : nt) x = (int32_t)(rng() % vocab);
      std::vector<int64_t> slots(batch.size()), copies(2 * batch.size() + 2);
      int64_t nc = 0;
      st = pa_bm_append_slots(bm, batch.data(), rng() % 4 ? nt.data() : nullptr,
                              (int64_t)batch.size(), slots.data(), copies.data(), &nc);
      if (st != PA_BM_OK && st != PA_BM_EXHAUSTED) return fail("append", st);
      for (int64_t i = 0; st == PA_BM_OK && i < (int64_t)batch.size(); ++i)
        if (slots[i] < 0 || slots[i] >= nb * bs) return fail("slot range", PA_BM_CORRUPT);
    } else if (kind == 2 && rng() % 2) {
      const int64_t p = live[rng() % live.size()];
      st = pa_bm_fork(bm, p, next_id);
      if (st) return fail("fork", st);
      live.push_back(next_id);
      toks.resize(next_id + 1);
      ++next_id;
    } else if (kind == 2) {
      // batched: up to three children, a later one may fork an earlier one
      const int k = 1 + (int)(rng() % 3);
      std::vector<int64_t> parents, children;
      for (int j = 0; j < k; ++j) {
        parents.push_back(j > 0 && rng() % 2 ? children.back() : live[rng() % live.size()]);
        children.push_back(next_id + j);
      }
      st = pa_bm_fork_many(bm, parents.data(), children.data(), k);
      if (st) return fail("fork_many", st);
      for (int64_t c : children) live.push_back(c);
      next_id += k;
      toks.resize(next_id);
    } else if (rng() % 2 || live.size() < 2) {
      const size_t i = rng() % live.size();
      st = pa_bm_free_sequence(bm, live[i]);
      if (st) return fail("free", st);
      live[i] = live.back();
      live.pop_back();
    } else {
      // batched: two distinct sequences, plus a rejected call listing one twice
      const size_t i = rng() % live.size();
      size_t j = rng() % (live.size() - 1);
      if (j >= i) ++j;
      const int64_t dup[2] = {live[i], live[i]};
      if (pa_bm_free_many(bm, dup, 2) != PA_BM_INVALID) return fail("free_many dup", PA_BM_CORRUPT);
      const int64_t two[2] = {live[i], live[j]};
      st = pa_bm_free_many(bm, two, 2);
      if (st) return fail("free_many", st);
      const int64_t a = live[i], b = live[j];
      std::vector<int64_t> rest;
      for (int64_t x : live)
        if (x != a && x != b) rest.push_back(x);
      live.swap(rest);
    }
    st = pa_bm_check(bm);
    if (st) return fail("check", st);
  }
  pa_bm_stats s;
  st = pa_bm_get_stats(bm, &s);
  if (st) return fail("stats", st);
  if (s.free_blocks + s.used_blocks != s.num_blocks) return fail("stats sum", PA_BM_CORRUPT);
  pa_bm_destroy(bm);
  return 0;
}

int main() {
  for (unsigned seed = 1; seed <= 12; ++seed)
    for (int pc = 0; pc < 2; ++pc)
      if (run(seed, pc)) {
        std::fprintf(stderr, "seed %u prefix_cache %d failed\n", seed, pc);
        return 1;
      }
  std::printf("ok\n");
  return 0;
}
