// Control-plane block manager: the CPU side that hands block tables and slot
// mappings to the GPU data plane.
//
// "Nano-vLLM part 1", section 4: a sequence is cut into fixed-size blocks
// (4.1); every full block's content is hashed and a hash -> block id map lets
// a new sequence reuse blocks holding the same prefix by raising their
// reference counts (4.2); the manager runs on the CPU and tracks only
// metadata, and a freed block is marked free at once but its GPU memory is not
// cleared, only overwritten when the block is handed out again (4.3).
// Section 3.2: when no block is left for a sequence's next token the
// scheduler preempts a sequence; here allocation and append report that
// condition and change nothing, and the caller frees (preempts) a sequence.
//
// Readings where the page is silent:
//  - A block's hash covers its tokens and the hash of the block before it, so
//    equal hashes mean equal whole prefixes (K/V at a position depend on every
//    earlier token).  Only full blocks are hashed and shared; a hit is also
//    checked against the stored tokens and the previous hash.
//  - Prefix hits are taken from the first block on and stop at the first
//    miss.  When every block of a prompt would hit, the last one is treated
//    as a miss so that at least one query row is left to compute and no
//    shared block is written.
//  - Free blocks form a FIFO: freed blocks go to the back, new blocks come
//    from the front, so a freed block keeps its cached content (and its hash
//    entry) as long as possible; a block taken from the free list for new
//    content drops its old hash entry.  A sequence's blocks are released last
//    block first, so the blocks of its prefix, the likeliest to be shared,
//    are the last of them to be overwritten.
#include <cstdint>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"

namespace {

constexpr uint64_t kFnvOffset = 1469598103934665603ull;
constexpr uint64_t kFnvPrime = 1099511628211ull;

// 64-bit FNV-1a over the previous block's hash and this block's token ids
// (little-endian bytes).
uint64_t block_hash(uint64_t prev, const int32_t* tokens, int32_t n) {
  uint64_t h = kFnvOffset;
  auto mix = [&](uint64_t v, int bytes) {
    for (int i = 0; i < bytes; ++i) {
      h ^= (v >> (8 * i)) & 0xFFu;
      h *= kFnvPrime;
    }
  };
  mix(prev, 8);
  for (int32_t i = 0; i < n; ++i) mix(static_cast<uint32_t>(tokens[i]), 4);
  return h;
}

struct Block {
  int32_t ref = 0;
  bool hashed = false;
  bool free = true;
  uint64_t hash = 0;
  uint64_t prev_hash = 0;
  std::vector<int32_t> tokens;  // content of a hashed (full) block
};

struct Seq {
  std::vector<int32_t> table;
  std::vector<int32_t> tokens;
  uint64_t tail_hash = 0;  // hash of the last full block (0 before the first)
};

}  // namespace

struct pkv_block_manager {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<Block> blocks;
  std::deque<int32_t> free_list;
  int32_t n_free = 0;  // blocks in free_list that are still free
  std::unordered_map<uint64_t, int32_t> by_hash;
  std::unordered_map<int64_t, Seq> seqs;

  // Take the next free block for new content (the caller checked n_free).
  int32_t take_free() {
    for (;;) {
      const int32_t b = free_list.front();
      free_list.pop_front();
      Block& blk = blocks[b];
      if (!blk.free) continue;  // left the list through a cache hit
      blk.free = false;
      --n_free;
      if (blk.hashed) {
        auto it = by_hash.find(blk.hash);
        if (it != by_hash.end() && it->second == b) by_hash.erase(it);
        blk.hashed = false;
        blk.tokens.clear();
      }
      blk.ref = 1;
      return b;
    }
  }

  // Cached block holding `tokens` after a prefix hashing to `prev`, or -1.
  int32_t lookup(uint64_t h, uint64_t prev, const int32_t* tokens) const {
    auto it = by_hash.find(h);
    if (it == by_hash.end()) return -1;
    const Block& blk = blocks[it->second];
    if (!blk.hashed || blk.prev_hash != prev ||
        static_cast<int32_t>(blk.tokens.size()) != block_size)
      return -1;
    for (int32_t i = 0; i < block_size; ++i)
      if (blk.tokens[i] != tokens[i]) return -1;
    return it->second;
  }

  void register_full(int32_t b, uint64_t h, uint64_t prev, const int32_t* tokens) {
    Block& blk = blocks[b];
    blk.hashed = true;
    blk.hash = h;
    blk.prev_hash = prev;
    blk.tokens.assign(tokens, tokens + block_size);
    by_hash[h] = b;
  }

  void release(int32_t b) {
    Block& blk = blocks[b];
    if (--blk.ref == 0) {
      blk.free = true;
      free_list.push_back(b);
      ++n_free;
    }
  }
};

extern "C" {

pkv_block_manager* pkv_bm_create(int32_t num_blocks, int32_t block_size) {
  if (num_blocks <= 0 || block_size <= 0) return nullptr;
  pkv_block_manager* m = new (std::nothrow) pkv_block_manager();
  if (!m) return nullptr;
  m->num_blocks = num_blocks;
  m->block_size = block_size;
  m->blocks.resize(static_cast<size_t>(num_blocks));
  for (int32_t b = 0; b < num_blocks; ++b) m->free_list.push_back(b);
  m->n_free = num_blocks;
  return m;
}

void pkv_bm_destroy(pkv_block_manager* m) { delete m; }

int32_t pkv_bm_num_free(const pkv_block_manager* m) { return m ? m->n_free : -1; }

int32_t pkv_bm_allocate(pkv_block_manager* m, int64_t seq_id, const int32_t* tokens, int32_t n) {
  if (!m || n <= 0 || !tokens) return PKV_BM_ERR_ARG;
  if (m->seqs.count(seq_id)) return PKV_BM_ERR_ARG;
  const int32_t bs = m->block_size;
  const int32_t nblocks = (n + bs - 1) / bs;
  const int32_t nfull = n / bs;
  // prefix hits: full blocks from the first on, up to the first miss
  std::vector<int32_t> hit;
  std::vector<uint64_t> hashes;
  uint64_t prev = 0;
  for (int32_t i = 0; i < nfull; ++i) {
    const uint64_t h = block_hash(prev, tokens + static_cast<size_t>(i) * bs, bs);
    hashes.push_back(h);
    if (static_cast<int32_t>(hit.size()) == i) {
      const int32_t b = m->lookup(h, prev, tokens + static_cast<size_t>(i) * bs);
      if (b >= 0) hit.push_back(b);
    }
    prev = h;
  }
  if (static_cast<int32_t>(hit.size()) == nblocks) hit.pop_back();  // keep one block to compute
  int32_t free_hits = 0;
  for (int32_t b : hit) free_hits += m->blocks[b].free ? 1 : 0;
  const int32_t misses = nblocks - static_cast<int32_t>(hit.size());
  if (misses + free_hits > m->n_free) return PKV_BM_NO_SPACE;

  Seq s;
  s.tokens.assign(tokens, tokens + n);
  for (int32_t b : hit) {
    Block& blk = m->blocks[b];
    if (blk.free) {  // cached content of a freed block, reused before it was overwritten
      blk.free = false;
      --m->n_free;
    }
    ++blk.ref;
    s.table.push_back(b);
  }
  uint64_t p = static_cast<int32_t>(hit.size()) > 0 ? hashes[hit.size() - 1] : 0;
  for (int32_t i = static_cast<int32_t>(hit.size()); i < nblocks; ++i) {
    const int32_t b = m->take_free();
    s.table.push_back(b);
    if (i < nfull) {
      m->register_full(b, hashes[i], p, tokens + static_cast<size_t>(i) * bs);
      p = hashes[i];
    }
  }
  s.tail_hash = nfull > 0 ? hashes[nfull - 1] : 0;
  const int32_t cached = static_cast<int32_t>(hit.size()) * bs;
  m->seqs.emplace(seq_id, std::move(s));
  return cached;
}

int32_t pkv_bm_append(pkv_block_manager* m, int64_t seq_id, int32_t token) {
  if (!m) return PKV_BM_ERR_ARG;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PKV_BM_ERR_ARG;
  Seq& s = it->second;
  const int32_t bs = m->block_size;
  const int32_t n = static_cast<int32_t>(s.tokens.size());
  if (n % bs == 0) {  // the last block is full: the token needs a new one
    if (m->n_free == 0) return PKV_BM_NO_SPACE;
    s.table.push_back(m->take_free());
  }
  s.tokens.push_back(token);
  if ((n + 1) % bs == 0) {  // the last block just filled up: make it findable
    const int32_t* blk_tokens = s.tokens.data() + (n + 1 - bs);
    const uint64_t h = block_hash(s.tail_hash, blk_tokens, bs);
    m->register_full(s.table.back(), h, s.tail_hash, blk_tokens);
    s.tail_hash = h;
  }
  return 0;
}

int32_t pkv_bm_free(pkv_block_manager* m, int64_t seq_id) {
  if (!m) return PKV_BM_ERR_ARG;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PKV_BM_ERR_ARG;
  const std::vector<int32_t>& t = it->second.table;
  for (auto b = t.rbegin(); b != t.rend(); ++b) m->release(*b);
  m->seqs.erase(it);
  return 0;
}

int32_t pkv_bm_seq_len(const pkv_block_manager* m, int64_t seq_id) {
  if (!m) return PKV_BM_ERR_ARG;
  auto it = m->seqs.find(seq_id);
  return it == m->seqs.end() ? PKV_BM_ERR_ARG : static_cast<int32_t>(it->second.tokens.size());
}

int32_t pkv_bm_block_table(const pkv_block_manager* m, int64_t seq_id, int32_t* out,
                           int32_t max_blocks) {
  if (!m) return PKV_BM_ERR_ARG;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PKV_BM_ERR_ARG;
  const std::vector<int32_t>& t = it->second.table;
  const int32_t n = static_cast<int32_t>(t.size());
  if (out) {
    for (int32_t i = 0; i < max_blocks; ++i) out[i] = i < n ? t[i] : -1;
  }
  return n;
}

int32_t pkv_bm_slots(const pkv_block_manager* m, int64_t seq_id, int32_t from, int32_t to,
                     int32_t* out) {
  if (!m || !out) return PKV_BM_ERR_ARG;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PKV_BM_ERR_ARG;
  const Seq& s = it->second;
  if (from < 0 || to < from || to > static_cast<int32_t>(s.tokens.size())) return PKV_BM_ERR_ARG;
  const int32_t bs = m->block_size;
  for (int32_t p = from; p < to; ++p) out[p - from] = s.table[p / bs] * bs + p % bs;
  return to - from;
}

int32_t pkv_bm_ref_count(const pkv_block_manager* m, int32_t block_id) {
  if (!m || block_id < 0 || block_id >= m->num_blocks) return PKV_BM_ERR_ARG;
  return m->blocks[block_id].ref;
}

}  // extern "C"
