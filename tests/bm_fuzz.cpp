// Randomized allocate / append / free (preempt) sequences against the block
// manager of the C ABI, with the invariants that "Nano-vLLM part 1" sections
// 3.2 and 4 fix checked after every operation.  Built by
// tests/test_block_manager_sanitized.py with AddressSanitizer and
// UndefinedBehaviorSanitizer (host code only); stops at the first failure.
//
//   bm_fuzz <seed> <operations>
//
// Invariants:
//  - a sequence of n tokens holds ceil(n / block_size) blocks, none twice;
//  - a block's reference count is the number of live tables listing it, and
//    the free count is the pool minus the distinct listed blocks (4.2, 4.3);
//  - a block listed by several tables is a full block of each, at the same
//    index, after identical token prefixes (4.2: shared blocks hold the same
//    whole prefix; nobody appends into them);
//  - slots are table[p / bs] * bs + p % bs (4.1);
//  - a "no space" answer changes nothing (3.2: the caller preempts);
//  - allocate reports a block-aligned cached prefix and leaves one block to
//    compute.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <set>
#include <vector>

#include "pagedkv.h"

namespace {

struct Model {
  std::map<int64_t, std::vector<int32_t>> tokens;  // live sequences
};

[[noreturn]] void fail(const char* what, long a = 0, long b = 0) {
  std::fprintf(stderr, "bm_fuzz: %s (%ld, %ld)\n", what, a, b);
  std::exit(1);
}

std::vector<int32_t> table_of(pkv_block_manager* m, int64_t id) {
  const int32_t n = pkv_bm_block_table(m, id, nullptr, 0);
  if (n < 0) fail("block_table of a live sequence", static_cast<long>(id), n);
  std::vector<int32_t> t(static_cast<size_t>(n) + 2);
  if (pkv_bm_block_table(m, id, t.data(), n + 2) != n) fail("block_table count");
  if (t[n] != -1 || t[n + 1] != -1) fail("block_table padding");
  t.resize(static_cast<size_t>(n));
  return t;
}

void check(pkv_block_manager* m, const Model& md, int32_t num_blocks, int32_t bs) {
  std::map<int32_t, int32_t> refs;
  std::map<int32_t, std::vector<std::pair<int64_t, int32_t>>> where;  // block -> (seq, index)
  for (const auto& [id, toks] : md.tokens) {
    const int32_t n = static_cast<int32_t>(toks.size());
    if (pkv_bm_seq_len(m, id) != n) fail("seq_len", static_cast<long>(id), n);
    const std::vector<int32_t> t = table_of(m, id);
    if (static_cast<int32_t>(t.size()) != (n + bs - 1) / bs) fail("blocks per sequence", n, t.size());
    std::set<int32_t> seen;
    for (size_t i = 0; i < t.size(); ++i) {
      if (t[i] < 0 || t[i] >= num_blocks) fail("block id out of range", t[i]);
      if (!seen.insert(t[i]).second) fail("block listed twice in one table", t[i]);
      ++refs[t[i]];
      where[t[i]].push_back({id, static_cast<int32_t>(i)});
    }
    std::vector<int32_t> slots(static_cast<size_t>(n));
    if (n > 0 && pkv_bm_slots(m, id, 0, n, slots.data()) != n) fail("slots count");
    for (int32_t p = 0; p < n; ++p)
      if (slots[p] != t[p / bs] * bs + p % bs) fail("slot formula", p, slots[p]);
  }
  for (int32_t b = 0; b < num_blocks; ++b) {
    const auto it = refs.find(b);
    const int32_t want = it == refs.end() ? 0 : it->second;
    if (pkv_bm_ref_count(m, b) != want) fail("reference count", b, pkv_bm_ref_count(m, b));
  }
  if (pkv_bm_num_free(m) != num_blocks - static_cast<int32_t>(refs.size()))
    fail("free count", pkv_bm_num_free(m), num_blocks - static_cast<long>(refs.size()));
  for (const auto& [b, users] : where) {
    if (users.size() < 2) continue;
    const auto& [id0, i0] = users[0];
    const std::vector<int32_t>& t0 = md.tokens.at(id0);
    for (const auto& [id, i] : users) {
      const std::vector<int32_t>& tk = md.tokens.at(id);
      if (i != i0) fail("shared block at different indices", b);
      const size_t end = static_cast<size_t>(i + 1) * bs;
      if (tk.size() < end || t0.size() < end) fail("shared block not full", b);
      for (size_t p = 0; p < end; ++p)
        if (tk[p] != t0[p]) fail("shared block after different prefixes", b, static_cast<long>(p));
    }
  }
}

}  // namespace

int main(int argc, char** argv) {
  const uint64_t seed = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 1;
  const int ops = argc > 2 ? std::atoi(argv[2]) : 2000;
  std::mt19937_64 rng(seed);
  auto uni = [&](int lo, int hi) { return std::uniform_int_distribution<int>(lo, hi)(rng); };
  const int32_t bs = 1 << uni(2, 5);           // 4 .. 32 tokens per block
  const int32_t num_blocks = uni(8, 64);
  pkv_block_manager* m = pkv_bm_create(num_blocks, bs);
  if (!m) fail("create");
  if (pkv_bm_create(0, bs) || pkv_bm_create(num_blocks, 0)) fail("create accepted bad sizes");
  // a few shared "system prompts", so that prefixes repeat and blocks get shared
  std::vector<std::vector<int32_t>> prompts(4);
  for (auto& p : prompts) {
    p.resize(static_cast<size_t>(uni(0, 3 * bs)));
    for (auto& t : p) t = uni(0, 9);
  }
  Model md;
  int64_t next_id = 100;
  for (int op = 0; op < ops; ++op) {
    const int kind = uni(0, 9);
    if (kind <= 3) {  // admit a sequence
      std::vector<int32_t> toks = prompts[static_cast<size_t>(uni(0, 3))];
      const int extra = uni(toks.empty() ? 1 : 0, 2 * bs);
      for (int i = 0; i < extra; ++i) toks.push_back(uni(0, 9));
      const int32_t free_before = pkv_bm_num_free(m);
      const int32_t r = pkv_bm_allocate(m, next_id, toks.data(), static_cast<int32_t>(toks.size()));
      if (r == PKV_BM_NO_SPACE) {
        if (pkv_bm_num_free(m) != free_before || pkv_bm_seq_len(m, next_id) != PKV_BM_ERR_ARG)
          fail("no-space allocate changed the manager");
      } else {
        const int32_t n = static_cast<int32_t>(toks.size());
        if (r < 0 || r % bs != 0 || r > ((n + bs - 1) / bs - 1) * bs) fail("cached prefix", r, n);
        md.tokens[next_id] = toks;
      }
      ++next_id;
    } else if (kind <= 7 && !md.tokens.empty()) {  // decode: one token for a live sequence
      auto it = md.tokens.begin();
      std::advance(it, uni(0, static_cast<int>(md.tokens.size()) - 1));
      const int32_t tok = uni(0, 9);
      const int32_t free_before = pkv_bm_num_free(m);
      const std::vector<int32_t> t_before = table_of(m, it->first);
      const int32_t r = pkv_bm_append(m, it->first, tok);
      if (r == PKV_BM_NO_SPACE) {
        if (pkv_bm_num_free(m) != free_before || table_of(m, it->first) != t_before)
          fail("no-space append changed the manager");
        // preempt the longest other sequence, as the scheduler would
        int64_t victim = -1;
        size_t longest = 0;
        for (const auto& [id, tk] : md.tokens)
          if (id != it->first && tk.size() >= longest) { victim = id; longest = tk.size(); }
        if (victim >= 0) {
          if (pkv_bm_free(m, victim) != 0) fail("free of a live sequence");
          md.tokens.erase(victim);
        }
      } else if (r == 0) {
        it->second.push_back(tok);
      } else {
        fail("append status", r);
      }
    } else if (!md.tokens.empty()) {  // a sequence finishes
      auto it = md.tokens.begin();
      std::advance(it, uni(0, static_cast<int>(md.tokens.size()) - 1));
      if (pkv_bm_free(m, it->first) != 0) fail("free of a live sequence");
      md.tokens.erase(it);
    }
    // invalid requests are refused and change nothing
    int32_t one = 1, out[4];
    if (pkv_bm_free(m, -5) != PKV_BM_ERR_ARG || pkv_bm_append(m, -5, 1) != PKV_BM_ERR_ARG ||
        pkv_bm_allocate(m, 7, &one, 0) != PKV_BM_ERR_ARG || pkv_bm_ref_count(m, num_blocks) != PKV_BM_ERR_ARG ||
        pkv_bm_ref_count(m, -1) != PKV_BM_ERR_ARG)
      fail("invalid request accepted");
    if (!md.tokens.empty()) {
      const auto& [id, tk] = *md.tokens.begin();
      const int32_t n = static_cast<int32_t>(tk.size());
      if (pkv_bm_slots(m, id, n, n + 1, out) != PKV_BM_ERR_ARG || pkv_bm_slots(m, id, 1, 0, out) != PKV_BM_ERR_ARG ||
          pkv_bm_allocate(m, id, &one, 1) != PKV_BM_ERR_ARG)
        fail("invalid request accepted");
    }
    check(m, md, num_blocks, bs);
  }
  for (const auto& [id, tk] : md.tokens) pkv_bm_free(m, id);
  if (pkv_bm_num_free(m) != num_blocks) fail("blocks lost after freeing everything");
  pkv_bm_destroy(m);
  std::printf("bm_fuzz seed %llu: %d operations, block size %d, %d blocks: ok\n",
              static_cast<unsigned long long>(seed), ops, bs, num_blocks);
  return 0;
}
