// Host block pool for the paged KV cache, with hash-chained prefix reuse and
// least-recently-released eviction: the block manager of a paged cache
// ("rvLLM: High-performance LLM inference in Rust", architecture diagram,
// "Block Manager (paged KV)") with prefix caching as "Litellama" describes it
// (section "Features", Prefix Caching: block hashes chained so shared
// prompts are stored once and reused, released blocks evicted in LRU order
// under capacity pressure).
//
// Rules (the statement of them that include/padecode.h gives):
//  * a full 16-token block is identified by FNV-1a-64 over the 8
//    little-endian bytes of its parent's hash (the pool seed for block 0)
//    followed by its 16 token ids as 4-byte little-endian integers; a match
//    also compares parent and tokens, so a hash collision never shares data;
//  * add_sequence reuses the longest run of leading cached blocks, takes the
//    rest (and a partial last block) from the free queue, registers its new
//    full blocks, and changes nothing when the queue cannot supply them;
//  * the free queue holds the blocks no sequence uses, least recently
//    released first; taking one evicts its cache entry; a sequence releases
//    its blocks last first.
// The free queue is an intrusive doubly linked list over block ids, so a
// cached block found in it leaves it in O(1).

#include <stdint.h>
#include <string.h>

#include <new>
#include <unordered_map>
#include <vector>

#include "padecode.h"

namespace {

constexpr int kBlock = 16;
constexpr uint64_t kFnvOffset = 0xCBF29CE484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001B3ull;

uint64_t fnv1a_bytes(uint64_t h, const uint8_t* p, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= kFnvPrime;
  }
  return h;
}

uint64_t chain_hash(uint64_t parent, const int32_t* tokens) {
  uint8_t buf[8 + 4 * kBlock];
  for (int i = 0; i < 8; ++i) buf[i] = (uint8_t)(parent >> (8 * i));
  for (int t = 0; t < kBlock; ++t) {
    const uint32_t v = (uint32_t)tokens[t];
    for (int i = 0; i < 4; ++i) buf[8 + 4 * t + i] = (uint8_t)(v >> (8 * i));
  }
  return fnv1a_bytes(kFnvOffset, buf, sizeof(buf));
}

struct Block {
  int32_t ref = 0;
  bool keyed = false;   // a registered full block: hash, parent, tokens valid
  uint64_t hash = 0, parent = 0;
  int32_t tokens[kBlock];
  int32_t prev = -1, next = -1;   // free-queue links
  bool in_free = false;
};

struct Seq {
  std::vector<int32_t> tokens;
  std::vector<int32_t> blocks;
  uint64_t parent = 0;
};

}  // namespace

struct pa_block_pool {
  uint64_t seed;
  std::vector<Block> blocks;
  int32_t head = -1, tail = -1, nfree = 0;
  std::unordered_map<uint64_t, int32_t> cached;
  std::unordered_map<int64_t, Seq> seqs;

  void push_back(int32_t b) {
    Block& x = blocks[b];
    x.prev = tail;
    x.next = -1;
    if (tail >= 0) blocks[tail].next = b; else head = b;
    tail = b;
    x.in_free = true;
    ++nfree;
  }
  void unlink(int32_t b) {
    Block& x = blocks[b];
    if (x.prev >= 0) blocks[x.prev].next = x.next; else head = x.next;
    if (x.next >= 0) blocks[x.next].prev = x.prev; else tail = x.prev;
    x.prev = x.next = -1;
    x.in_free = false;
    --nfree;
  }
  int32_t take_free() {   // least recently released; evicts its cache entry
    const int32_t b = head;
    unlink(b);
    Block& x = blocks[b];
    if (x.keyed) {
      auto it = cached.find(x.hash);
      if (it != cached.end() && it->second == b) cached.erase(it);
      x.keyed = false;
    }
    return b;
  }
  int32_t lookup(uint64_t h, uint64_t parent, const int32_t* tokens) const {
    auto it = cached.find(h);
    if (it == cached.end()) return -1;
    const Block& x = blocks[it->second];
    if (!x.keyed || x.hash != h || x.parent != parent ||
        memcmp(x.tokens, tokens, sizeof(x.tokens)) != 0)
      return -1;
    return it->second;
  }
  void enroll(int32_t b, uint64_t h, uint64_t parent, const int32_t* tokens) {
    Block& x = blocks[b];
    x.keyed = true;
    x.hash = h;
    x.parent = parent;
    memcpy(x.tokens, tokens, sizeof(x.tokens));
    cached.emplace(h, b);   // keeps an existing entry for the same hash
  }
};

extern "C" {

pa_status pa_pool_create(int32_t num_blocks, uint64_t seed, pa_block_pool** pool) {
  if (!pool) return PA_ERR_NULL;
  *pool = nullptr;
  if (num_blocks < 1) return PA_ERR_SHAPE;
  try {
    pa_block_pool* p = new pa_block_pool();
    p->seed = seed;
    p->blocks.resize(num_blocks);
    for (int32_t b = 0; b < num_blocks; ++b) p->push_back(b);
    *pool = p;
  } catch (const std::bad_alloc&) {
    return PA_ERR_CAPACITY;
  }
  return PA_OK;
}

void pa_pool_destroy(pa_block_pool* pool) { delete pool; }

pa_status pa_pool_add_sequence(pa_block_pool* p, int64_t seq_id, const int32_t* tokens,
                               int32_t num_tokens, int32_t* cached_tokens) {
  if (!p || (!tokens && num_tokens > 0)) return PA_ERR_NULL;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (p->seqs.count(seq_id)) return PA_ERR_STATE;
  try {
    const int32_t nfull = num_tokens / kBlock;
    const bool partial = num_tokens % kBlock != 0;
    std::vector<uint64_t> hashes(nfull), parents(nfull);
    std::vector<int32_t> hits;
    uint64_t parent = p->seed;
    for (int32_t i = 0; i < nfull; ++i) {
      const int32_t* bt = tokens + (size_t)kBlock * i;
      const uint64_t h = chain_hash(parent, bt);
      hashes[i] = h;
      parents[i] = parent;
      if ((int32_t)hits.size() == i) {
        const int32_t b = p->lookup(h, parent, bt);
        if (b >= 0) hits.push_back(b);
      }
      parent = h;
    }
    int32_t need = (nfull - (int32_t)hits.size()) + (partial ? 1 : 0);
    for (int32_t b : hits)
      if (p->blocks[b].ref == 0) ++need;
    if (need > p->nfree) return PA_ERR_CAPACITY;

    Seq s;
    s.tokens.assign(tokens, tokens + num_tokens);
    s.blocks.reserve(nfull + (partial ? 1 : 0));
    for (int32_t b : hits) {
      if (p->blocks[b].ref == 0) p->unlink(b);
      ++p->blocks[b].ref;
      s.blocks.push_back(b);
    }
    for (int32_t i = (int32_t)hits.size(); i < nfull; ++i) {
      const int32_t b = p->take_free();
      p->blocks[b].ref = 1;
      p->enroll(b, hashes[i], parents[i], tokens + (size_t)kBlock * i);
      s.blocks.push_back(b);
    }
    if (partial) {
      const int32_t b = p->take_free();
      p->blocks[b].ref = 1;
      s.blocks.push_back(b);
    }
    s.parent = nfull ? hashes[nfull - 1] : p->seed;
    p->seqs.emplace(seq_id, std::move(s));
    if (cached_tokens) *cached_tokens = kBlock * (int32_t)hits.size();
  } catch (const std::bad_alloc&) {
    return PA_ERR_CAPACITY;
  }
  return PA_OK;
}

pa_status pa_pool_append_token(pa_block_pool* p, int64_t seq_id, int32_t token) {
  if (!p) return PA_ERR_NULL;
  auto it = p->seqs.find(seq_id);
  if (it == p->seqs.end()) return PA_ERR_STATE;
  Seq& s = it->second;
  try {
    if (s.tokens.size() % kBlock == 0) {
      if (p->nfree == 0) return PA_ERR_CAPACITY;
      s.blocks.reserve(s.blocks.size() + 1);
      s.tokens.reserve(s.tokens.size() + 1);
      const int32_t b = p->take_free();
      p->blocks[b].ref = 1;
      s.blocks.push_back(b);
    }
    s.tokens.push_back(token);
  } catch (const std::bad_alloc&) {
    return PA_ERR_CAPACITY;
  }
  if (s.tokens.size() % kBlock == 0) {
    const int32_t* bt = s.tokens.data() + s.tokens.size() - kBlock;
    const uint64_t h = chain_hash(s.parent, bt);
    p->enroll(s.blocks.back(), h, s.parent, bt);
    s.parent = h;
  }
  return PA_OK;
}

pa_status pa_pool_free_sequence(pa_block_pool* p, int64_t seq_id) {
  if (!p) return PA_ERR_NULL;
  auto it = p->seqs.find(seq_id);
  if (it == p->seqs.end()) return PA_ERR_STATE;
  const std::vector<int32_t>& bl = it->second.blocks;
  for (auto r = bl.rbegin(); r != bl.rend(); ++r)
    if (--p->blocks[*r].ref == 0) p->push_back(*r);
  p->seqs.erase(it);
  return PA_OK;
}

int32_t pa_pool_num_free(const pa_block_pool* p) { return p ? p->nfree : -1; }

pa_status pa_pool_block_table(const pa_block_pool* p, const int64_t* seq_ids, int32_t num_seqs,
                              int32_t max_blocks_per_seq, int32_t pad_block,
                              int32_t* block_table, int32_t* context_lens) {
  if (!p || (num_seqs > 0 && (!seq_ids || !block_table))) return PA_ERR_NULL;
  if (num_seqs < 0 || max_blocks_per_seq < 1) return PA_ERR_SHAPE;
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = p->seqs.find(seq_ids[i]);
    if (it == p->seqs.end()) return PA_ERR_STATE;
    if ((int64_t)it->second.blocks.size() > max_blocks_per_seq) return PA_ERR_SHAPE;
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Seq& s = p->seqs.find(seq_ids[i])->second;
    int32_t* row = block_table + (size_t)i * max_blocks_per_seq;
    const int32_t n = (int32_t)s.blocks.size();
    for (int32_t j = 0; j < max_blocks_per_seq; ++j) row[j] = j < n ? s.blocks[j] : pad_block;
    if (context_lens) context_lens[i] = (int32_t)s.tokens.size();
  }
  return PA_OK;
}

pa_status pa_pool_shared_prefix(const pa_block_pool* p, const int64_t* seq_ids, int32_t num_seqs,
                                int32_t* prefix_blocks) {
  if (!p || !prefix_blocks || (num_seqs > 0 && !seq_ids)) return PA_ERR_NULL;
  if (num_seqs < 0) return PA_ERR_SHAPE;
  const Seq* ref = nullptr;   // the longest sequence, the first among equals
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = p->seqs.find(seq_ids[i]);
    if (it == p->seqs.end()) return PA_ERR_STATE;
    if (!ref || it->second.tokens.size() > ref->tokens.size()) ref = &it->second;
  }
  if (!ref) {
    *prefix_blocks = 0;
    return PA_OK;
  }
  // every sequence must agree with the longest on each of its own full
  // blocks below the answer: one that differs at block j < its full blocks
  // bounds the answer by j
  size_t shared = ref->tokens.size() / kBlock;
  for (int32_t i = 0; i < num_seqs; ++i) {
    const Seq& s = p->seqs.find(seq_ids[i])->second;
    const size_t full = s.tokens.size() / kBlock;
    for (size_t j = 0; j < full && j < shared; ++j)
      if (s.blocks[j] != ref->blocks[j]) {
        shared = j;
        break;
      }
  }
  *prefix_blocks = (int32_t)shared;
  return PA_OK;
}

}  // extern "C"
