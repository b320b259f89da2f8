// Host-side KV block manager: which physical 16-token blocks each sequence
// owns, the block tables and slot mappings the kernels read, prefix sharing
// of full blocks, and release / eviction / rollback.
//
// What it does, from the pages: the KV-cache manager owns logical blocks,
// block tables, the prefix cache, and allocation and release (micro-vLLM wiki,
// layer description "KVCacheManager"; feature list "Paged KV Cache、prefix
// cache 和请求抢占"). Blocks are allocated and released on demand and shared
// through prefix caching; when blocks are scarce, admission control keeps
// the engine correct ("从零手写 vLLM 核心：mini-vllm 项目深度解析", section
// "2. 分页KV缓存（PagedAttention）"). Speculative decoding needs KV rollback
// (same write-up, "工程启示").
//
// Design:
//  * A full block is identified by a chained content hash: the hash of its
//    parent block and its 16 token ids. A prompt's leading full blocks whose
//    chain is already registered are shared (reference counted) instead of
//    allocated and rewritten.
//  * Released blocks go to the tail of the free queue; a block that still
//    carries a hash stays findable in the index until the queue hands it out
//    again (least recently released first), when its hash is dropped.
//  * Slots are flat rows of the pool: slot = block * 16 + offset.
//  * Rollback drops a sequence's newest tokens (rejected drafts); it never
//    modifies a block another sequence shares.
#include <limits.h>
#include <stdint.h>

#include <list>
#include <new>
#include <unordered_map>
#include <vector>

#include "mvk.h"

namespace {

constexpr int32_t kBlock = 16;
// Sizes stay far from int32 overflow: slots are block * 16 + offset, and
// token counts are rounded up to whole blocks.
constexpr int32_t kMaxBlocks = INT32_MAX / kBlock;
constexpr int32_t kMaxTokens = INT32_MAX / 2;

struct Block {
  int32_t ref = 0;
  uint64_t hash = 0;   // chained content hash, when registered
  bool hashed = false;
  bool in_free = true;
  std::list<int32_t>::iterator free_pos;
};

struct Sequence {
  std::vector<int32_t> blocks;
  std::vector<int32_t> tokens;  // token ids of every cached position
  int32_t hashed_blocks = 0;    // leading full blocks whose hash is known
  std::vector<uint64_t> hashes; // chained hash of each full block
};

// 64-bit mix of the parent hash and a block's token ids (splitmix64 finaliser
// over an FNV-style fold): collisions are not excluded, so a hit is also
// checked against the block's token ids.
uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

uint64_t block_hash(uint64_t parent, const int32_t* tokens) {
  uint64_t h = mix64(parent + 0x9E3779B97F4A7C15ull);
  for (int i = 0; i < kBlock; ++i) h = mix64(h ^ (uint64_t)(uint32_t)tokens[i]);
  return h;
}

}  // namespace

struct mvk_block_manager {
  int32_t num_blocks;
  bool prefix_cache;
  std::vector<Block> blocks;
  std::vector<std::vector<int32_t>> block_tokens;   // token ids of registered blocks
  std::list<int32_t> free_queue;                    // front = next to hand out
  std::unordered_map<uint64_t, int32_t> index;      // hash -> block
  std::unordered_map<int64_t, Sequence> seqs;

  mvk_block_manager(int32_t n, bool prefix)
      : num_blocks(n), prefix_cache(prefix), blocks(n), block_tokens(n) {
    for (int32_t b = 0; b < n; ++b) {
      free_queue.push_back(b);
      blocks[b].free_pos = std::prev(free_queue.end());
    }
  }

  // A registered full block with this hash and these tokens, or -1.
  int32_t lookup(uint64_t h, const int32_t* tokens) const {
    if (!prefix_cache) return -1;
    auto it = index.find(h);
    if (it == index.end()) return -1;
    const std::vector<int32_t>& t = block_tokens[it->second];
    for (int i = 0; i < kBlock; ++i)
      if (t[i] != tokens[i]) return -1;
    return it->second;
  }

  void unregister(int32_t b) {
    if (!blocks[b].hashed) return;
    auto it = index.find(blocks[b].hash);
    if (it != index.end() && it->second == b) index.erase(it);
    blocks[b].hashed = false;
  }

  void take(int32_t b) {  // a block leaves the free queue (reuse or fresh)
    Block& blk = blocks[b];
    if (blk.in_free) {
      free_queue.erase(blk.free_pos);
      blk.in_free = false;
    }
    ++blk.ref;
  }

  int32_t pop_free() {  // the least recently released block, its hash dropped
    const int32_t b = free_queue.front();
    unregister(b);
    take(b);
    return b;
  }

  void release(int32_t b) {
    Block& blk = blocks[b];
    if (--blk.ref == 0) {
      free_queue.push_back(b);
      blk.free_pos = std::prev(free_queue.end());
      blk.in_free = true;
    }
  }

  void register_block(int32_t b, uint64_t h, const int32_t* tokens) {
    if (!prefix_cache) return;
    auto it = index.find(h);
    if (it != index.end() && it->second != b) return;  // an equal block is already findable
    blocks[b].hash = h;
    blocks[b].hashed = true;
    block_tokens[b].assign(tokens, tokens + kBlock);
    index[h] = b;
  }

  // Hash and register every newly full block of s.
  void register_full(Sequence& s) {
    const int32_t full = (int32_t)s.tokens.size() / kBlock;
    while (s.hashed_blocks < full) {
      const int32_t i = s.hashed_blocks;
      const uint64_t parent = i ? s.hashes[i - 1] : 0;
      const uint64_t h = block_hash(parent, s.tokens.data() + (size_t)i * kBlock);
      s.hashes.push_back(h);
      register_block(s.blocks[i], h, s.tokens.data() + (size_t)i * kBlock);
      ++s.hashed_blocks;
    }
  }

  // Leading full blocks of a prompt already cached, and blocks still needed.
  void plan(const int32_t* tokens, int32_t n, int32_t* hits, int32_t* need) const {
    int32_t h_count = 0;
    uint64_t parent = 0;
    // the last token of a prompt is always recomputed: its block is not reused
    const int32_t full = (n - 1) / kBlock;
    for (int32_t i = 0; i < full; ++i) {
      const uint64_t h = block_hash(parent, tokens + (size_t)i * kBlock);
      if (lookup(h, tokens + (size_t)i * kBlock) < 0) break;
      parent = h;
      ++h_count;
    }
    const int32_t total = (n + kBlock - 1) / kBlock;
    int32_t need_new = total - h_count;
    // cached blocks that sit in the free queue are taken out of it when reused
    int32_t in_free = 0;
    parent = 0;
    for (int32_t i = 0; i < h_count; ++i) {
      const uint64_t h = block_hash(parent, tokens + (size_t)i * kBlock);
      const int32_t b = lookup(h, tokens + (size_t)i * kBlock);
      if (blocks[b].in_free) ++in_free;
      parent = h;
    }
    *hits = h_count;
    *need = need_new + in_free;  // free-queue entries the admission consumes
  }
};

extern "C" {

mvk_block_manager* mvk_bm_create(int32_t num_blocks, int32_t block_size, int32_t prefix_cache) {
  if (num_blocks <= 0 || num_blocks > kMaxBlocks || block_size != kBlock) return nullptr;
  return new (std::nothrow) mvk_block_manager(num_blocks, prefix_cache != 0);
}

void mvk_bm_destroy(mvk_block_manager* m) { delete m; }

int32_t mvk_bm_num_free(const mvk_block_manager* m) {
  return m ? (int32_t)m->free_queue.size() : -1;
}

int32_t mvk_bm_can_admit(const mvk_block_manager* m, const int32_t* token_ids,
                         int32_t num_tokens, int32_t* cached_tokens) {
  if (!m || num_tokens <= 0 || num_tokens > kMaxTokens || !token_ids)
    return MVK_ERR_INVALID_ARGUMENT;
  int32_t hits, need;
  m->plan(token_ids, num_tokens, &hits, &need);
  if (cached_tokens) *cached_tokens = hits * kBlock;
  return need <= (int32_t)m->free_queue.size() ? MVK_OK : MVK_ERR_OUT_OF_BLOCKS;
}

int32_t mvk_bm_admit(mvk_block_manager* m, int64_t seq_id, const int32_t* token_ids,
                     int32_t num_tokens, int32_t* cached_tokens) {
  if (!m || num_tokens <= 0 || num_tokens > kMaxTokens || !token_ids)
    return MVK_ERR_INVALID_ARGUMENT;
  if (m->seqs.count(seq_id)) return MVK_ERR_INVALID_ARGUMENT;
  int32_t hits, need;
  m->plan(token_ids, num_tokens, &hits, &need);
  if (need > (int32_t)m->free_queue.size()) return MVK_ERR_OUT_OF_BLOCKS;
  Sequence s;
  s.tokens.assign(token_ids, token_ids + num_tokens);
  uint64_t parent = 0;
  for (int32_t i = 0; i < hits; ++i) {  // shared leading blocks
    const uint64_t h = block_hash(parent, token_ids + (size_t)i * kBlock);
    const int32_t b = m->lookup(h, token_ids + (size_t)i * kBlock);
    m->take(b);
    s.blocks.push_back(b);
    s.hashes.push_back(h);
    parent = h;
  }
  s.hashed_blocks = hits;
  const int32_t total = (num_tokens + kBlock - 1) / kBlock;
  for (int32_t i = hits; i < total; ++i) s.blocks.push_back(m->pop_free());
  m->register_full(s);
  if (cached_tokens) *cached_tokens = hits * kBlock;
  m->seqs.emplace(seq_id, std::move(s));
  return MVK_OK;
}

int32_t mvk_bm_append(mvk_block_manager* m, int64_t seq_id, int32_t token_id, int32_t* slot) {
  if (!m || !slot) return MVK_ERR_INVALID_ARGUMENT;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return MVK_ERR_INVALID_ARGUMENT;
  Sequence& s = it->second;
  const int32_t pos = (int32_t)s.tokens.size();
  if (pos >= kMaxTokens) return MVK_ERR_INVALID_ARGUMENT;
  if (pos % kBlock == 0) {  // the last block is full: one more
    if (m->free_queue.empty()) return MVK_ERR_OUT_OF_BLOCKS;
    s.blocks.push_back(m->pop_free());
  }
  s.tokens.push_back(token_id);
  *slot = s.blocks[pos / kBlock] * kBlock + pos % kBlock;
  m->register_full(s);
  return MVK_OK;
}

int32_t mvk_bm_rollback(mvk_block_manager* m, int64_t seq_id, int32_t num_tokens) {
  if (!m || num_tokens < 0) return MVK_ERR_INVALID_ARGUMENT;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return MVK_ERR_INVALID_ARGUMENT;
  Sequence& s = it->second;
  const int32_t len = (int32_t)s.tokens.size();
  if (num_tokens > len) return MVK_ERR_INVALID_ARGUMENT;
  const int32_t new_len = len - num_tokens;
  const int32_t keep_blocks = (new_len + kBlock - 1) / kBlock;
  // a kept block that loses tokens must not be shared: it will be rewritten
  const int32_t first_touched = new_len / kBlock;
  if (first_touched < keep_blocks && m->blocks[s.blocks[first_touched]].ref > 1)
    return MVK_ERR_INVALID_ARGUMENT;
  while ((int32_t)s.blocks.size() > keep_blocks) {
    m->release(s.blocks.back());
    s.blocks.pop_back();
  }
  const int32_t full = new_len / kBlock;
  if (s.hashed_blocks > full) {
    for (int32_t i = full; i < s.hashed_blocks && i < keep_blocks; ++i)
      m->unregister(s.blocks[i]);
    s.hashed_blocks = full;
    s.hashes.resize(full);
  }
  s.tokens.resize(new_len);
  return MVK_OK;
}

int32_t mvk_bm_release(mvk_block_manager* m, int64_t seq_id) {
  if (!m) return MVK_ERR_INVALID_ARGUMENT;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return MVK_ERR_INVALID_ARGUMENT;
  // newest blocks first, so a sequence's prefix stays cached longest
  for (auto b = it->second.blocks.rbegin(); b != it->second.blocks.rend(); ++b) m->release(*b);
  m->seqs.erase(it);
  return MVK_OK;
}

int32_t mvk_bm_seq_info(const mvk_block_manager* m, int64_t seq_id, int32_t* num_tokens,
                        int32_t* num_blocks) {
  if (!m) return MVK_ERR_INVALID_ARGUMENT;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return MVK_ERR_INVALID_ARGUMENT;
  if (num_tokens) *num_tokens = (int32_t)it->second.tokens.size();
  if (num_blocks) *num_blocks = (int32_t)it->second.blocks.size();
  return MVK_OK;
}

int32_t mvk_bm_block_table(const mvk_block_manager* m, int64_t seq_id, int32_t* table,
                           int32_t max_blocks) {
  if (!m || !table || max_blocks < 0) return MVK_ERR_INVALID_ARGUMENT;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return MVK_ERR_INVALID_ARGUMENT;
  const std::vector<int32_t>& b = it->second.blocks;
  if ((int32_t)b.size() > max_blocks) return MVK_ERR_INVALID_ARGUMENT;
  for (int32_t i = 0; i < max_blocks; ++i) table[i] = i < (int32_t)b.size() ? b[i] : -1;
  return MVK_OK;
}

int32_t mvk_bm_slots(const mvk_block_manager* m, int64_t seq_id, int32_t first_token,
                     int32_t count, int32_t* slots) {
  if (!m || !slots || first_token < 0 || count < 0) return MVK_ERR_INVALID_ARGUMENT;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return MVK_ERR_INVALID_ARGUMENT;
  const Sequence& s = it->second;
  if ((int64_t)first_token + count > (int64_t)s.tokens.size()) return MVK_ERR_INVALID_ARGUMENT;
  for (int32_t i = 0; i < count; ++i) {
    const int32_t t = first_token + i;
    slots[i] = s.blocks[t / kBlock] * kBlock + t % kBlock;
  }
  return MVK_OK;
}

int32_t mvk_bm_block_ref(const mvk_block_manager* m, int32_t block) {
  if (!m || block < 0 || block >= m->num_blocks) return -1;
  return m->blocks[block].ref;
}

}  // extern "C"
