// Host-side prefix cache: finds the physical blocks that already hold the
// K/V of a prompt's leading full blocks, so a new sequence can share them
// through the block table instead of recomputing them ("KV Cache
// 优化与内存管理深度解析：PagedAttention 原理与实践", `HashBasedCaching`:
// block hashing, cache keys, the prefix lookup walk-through; "5.KV Cache 管理
// & PagedAttention", question 20, match the prefix, take references, allocate
// the rest, release at zero; "paged-attention-and-vllm-inference",
// `PrefixCacheManager`).
//
// The key of block i of a prompt is the whole token prefix up to the end of
// that block (the pages' prefix-hash strategy), not the block's own tokens:
// a block's K/V depend on every earlier token, so equal block contents
// after different histories must not match.  The cache is a trie with one
// node per cached block: node = (parent node, the block's bs tokens) ->
// physical block.  Lookups go through a hash table on (parent node id,
// tokens), and every hit is verified by comparing the parent id and the
// tokens, so a hash collision can never yield a wrong block.
//
// Reference counting goes through the allocator: the cache holds one
// reference on every cached block; a match takes one more on each returned
// block for the caller.  Every block a match or insert walks past gets the
// next value of a per-cache counter (in prefix order), so "least recently
// used" is a strict order.  Eviction removes least-recently-used leaves (a
// node with cached children stays, so every cached block remains
// reachable) that nobody but the cache references, and releases them.
// Plain CPU code, one mutex; no device calls.
#include <stdint.h>

#include <mutex>
#include <unordered_map>
#include <vector>

#include "../../include/pa.h"

namespace pa {
int set_error(int code, const char* msg);
int32_t bm_block_size(const pa_block_manager* m);
void alloc_add_user(pa_allocator* a);
void alloc_drop_user(pa_allocator* a);
}

namespace {

struct Node {
  int64_t parent;               // node id, -1 for the root
  std::vector<int32_t> tokens;  // the block's tokens
  int32_t block;                // physical block id
  int32_t children = 0;         // cached child nodes
  uint64_t last_use = 0;        // LRU stamp
  bool live = false;
};

uint64_t mix64(uint64_t x) {
  x ^= x >> 30;
  x *= 0xbf58476d1ce4e5b9ull;
  x ^= x >> 27;
  x *= 0x94d049bb133111ebull;
  x ^= x >> 31;
  return x;
}

uint64_t key_hash(int64_t parent, const int32_t* tokens, int32_t bs) {
  uint64_t h = mix64((uint64_t)parent + 0x9e3779b97f4a7c15ull);
  for (int32_t i = 0; i < bs; ++i) h = mix64(h ^ (uint64_t)(uint32_t)tokens[i]);
  return h;
}

}  // namespace

struct pa_prefix_cache {
  std::mutex mu;
  pa_allocator* a = nullptr;
  int32_t bs = 0;
  std::vector<Node> nodes;
  std::vector<int64_t> free_nodes;
  std::unordered_multimap<uint64_t, int64_t> index;  // key hash -> node id
  uint64_t clock = 0;
  int32_t live = 0;

  // node id for (parent, tokens), or -1
  int64_t find(int64_t parent, const int32_t* tokens) const {
    const uint64_t h = key_hash(parent, tokens, bs);
    auto range = index.equal_range(h);
    for (auto it = range.first; it != range.second; ++it) {
      const Node& n = nodes[it->second];
      if (n.parent != parent) continue;
      bool same = true;
      for (int32_t i = 0; i < bs && same; ++i) same = n.tokens[i] == tokens[i];
      if (same) return it->second;
    }
    return -1;
  }

  void unindex(int64_t id) {
    const Node& n = nodes[id];
    const uint64_t h = key_hash(n.parent, n.tokens.data(), bs);
    auto range = index.equal_range(h);
    for (auto it = range.first; it != range.second; ++it)
      if (it->second == id) {
        index.erase(it);
        return;
      }
  }
};

extern "C" {

pa_prefix_cache* pa_pc_create(pa_allocator* a, int32_t block_size) {
  if (!a || block_size <= 0) {
    pa::set_error(PA_ERR_INVALID_ARG, "need an allocator and a positive block size");
    return nullptr;
  }
  pa_prefix_cache* c = new pa_prefix_cache;
  c->a = a;
  c->bs = block_size;
  pa::alloc_add_user(a);
  return c;
}

void pa_pc_destroy(pa_prefix_cache* c) {
  if (!c) return;
  for (const Node& n : c->nodes)
    if (n.live) pa_alloc_decref(c->a, n.block);
  pa_allocator* a = c->a;
  delete c;
  pa::alloc_drop_user(a);
}

int32_t pa_pc_match(pa_prefix_cache* c, const int32_t* tokens, int64_t n_tokens,
                    int32_t* blocks_out, int32_t max_blocks) {
  if (!c || n_tokens < 0 || max_blocks < 0 || (n_tokens > 0 && !tokens) ||
      (max_blocks > 0 && !blocks_out))
    return pa::set_error(PA_ERR_INVALID_ARG, "invalid arguments");
  std::lock_guard<std::mutex> g(c->mu);
  const int64_t full = n_tokens / c->bs;
  const int32_t limit = (int32_t)(full < max_blocks ? full : max_blocks);
  int64_t parent = -1;
  int32_t k = 0;
  for (; k < limit; ++k) {
    const int64_t id = c->find(parent, tokens + (int64_t)k * c->bs);
    if (id < 0) break;
    c->nodes[id].last_use = ++c->clock;
    blocks_out[k] = c->nodes[id].block;
    parent = id;
  }
  // a reference on each returned block for the caller
  for (int32_t i = 0; i < k; ++i) {
    const int rc = pa_alloc_incref(c->a, blocks_out[i]);
    if (rc) {
      for (int32_t j = 0; j < i; ++j) pa_alloc_decref(c->a, blocks_out[j]);
      return rc;
    }
  }
  return k;
}

int32_t pa_pc_insert(pa_prefix_cache* c, const int32_t* tokens, int64_t n_tokens,
                     const int32_t* blocks, int32_t n_blocks) {
  if (!c || n_tokens < 0 || n_blocks < 0 || (n_tokens > 0 && !tokens) || (n_blocks > 0 && !blocks))
    return pa::set_error(PA_ERR_INVALID_ARG, "invalid arguments");
  std::lock_guard<std::mutex> g(c->mu);
  const int64_t full = n_tokens / c->bs;
  const int32_t count = (int32_t)(full < n_blocks ? full : n_blocks);
  // the blocks must be allocated (the cache is about to share them)
  for (int32_t i = 0; i < count; ++i)
    if (pa_alloc_refcount(c->a, blocks[i]) <= 0)
      return pa::set_error(PA_ERR_BAD_BLOCK, "a block to cache is not allocated");
  int64_t parent = -1;
  int32_t added = 0;
  for (int32_t i = 0; i < count; ++i) {
    const int32_t* t = tokens + (int64_t)i * c->bs;
    int64_t id = c->find(parent, t);
    if (id < 0) {
      // new node: the cache takes a reference on the caller's block
      const int rc = pa_alloc_incref(c->a, blocks[i]);
      if (rc) return rc;
      if (!c->free_nodes.empty()) {
        id = c->free_nodes.back();
        c->free_nodes.pop_back();
      } else {
        id = (int64_t)c->nodes.size();
        c->nodes.emplace_back();
      }
      Node& n = c->nodes[id];
      n.parent = parent;
      n.tokens.assign(t, t + c->bs);
      n.block = blocks[i];
      n.children = 0;
      n.live = true;
      if (parent >= 0) ++c->nodes[parent].children;
      c->index.emplace(key_hash(parent, t, c->bs), id);
      ++c->live;
      ++added;
    }
    c->nodes[id].last_use = ++c->clock;
    parent = id;
  }
  return added;
}

int32_t pa_pc_evict(pa_prefix_cache* c, int32_t max_blocks) {
  if (!c || max_blocks < 0) return pa::set_error(PA_ERR_INVALID_ARG, "invalid arguments");
  std::lock_guard<std::mutex> g(c->mu);
  int32_t freed = 0;
  while (freed < max_blocks) {
    // least recently used leaf that only the cache references
    int64_t victim = -1;
    for (int64_t id = 0; id < (int64_t)c->nodes.size(); ++id) {
      const Node& n = c->nodes[id];
      if (!n.live || n.children > 0 || pa_alloc_refcount(c->a, n.block) != 1) continue;
      if (victim < 0 || n.last_use < c->nodes[victim].last_use) victim = id;
    }
    if (victim < 0) break;
    Node& n = c->nodes[victim];
    c->unindex(victim);
    if (n.parent >= 0) --c->nodes[n.parent].children;
    pa_alloc_decref(c->a, n.block);
    n.live = false;
    n.tokens.clear();
    c->free_nodes.push_back(victim);
    --c->live;
    ++freed;
  }
  return freed;
}

int32_t pa_pc_size(const pa_prefix_cache* c) {
  if (!c) return pa::set_error(PA_ERR_INVALID_ARG, "null prefix cache");
  std::lock_guard<std::mutex> g(const_cast<pa_prefix_cache*>(c)->mu);
  return c->live;
}

}  // extern "C"

// Admission of a new sequence through the prefix cache ("5.KV Cache 管理 &
// PagedAttention", question 20, allocate_with_prefix: the table starts with
// the matched blocks, each with one more reference; blocks are allocated
// for the remaining tokens; the sequence's prefix is then cached).  Built on
// the public calls above and the block manager's, so the locking stays
// theirs: match, attach the matched blocks to the new sequence, release the
// match's own references, reserve a slot per remaining token, offer the
// sequence's full blocks to the cache.
extern "C" int64_t pa_bm_add_sequence_cached(pa_block_manager* m, pa_prefix_cache* c,
                                             int64_t seq_id, const int32_t* tokens,
                                             int64_t n_tokens, int64_t* slots_out) {
  if (!m || !c || n_tokens < 0 || (n_tokens > 0 && (!tokens || !slots_out)))
    return pa::set_error(PA_ERR_INVALID_ARG, "invalid arguments");
  if (n_tokens > 0x7FFFFFFFLL) return pa::set_error(PA_ERR_INVALID_ARG, "sequence too long");
  const int32_t bs = c->bs;
  if (pa::bm_block_size(m) != bs)
    return pa::set_error(PA_ERR_INVALID_ARG, "block manager and prefix cache block sizes differ");
  const int32_t full = (int32_t)(n_tokens / bs);
  std::vector<int32_t> matched((size_t)full + 1);
  const int32_t k = pa_pc_match(c, tokens, n_tokens, matched.data(), full);
  if (k < 0) return k;
  int rc = pa_bm_add_sequence(m, seq_id, matched.data(), k, (int64_t)k * bs);
  // the sequence took its own references (or failed): drop the match's
  for (int32_t i = 0; i < k; ++i) pa_alloc_decref(c->a, matched[i]);
  if (rc) return rc;
  const int64_t first = (int64_t)k * bs;
  for (int64_t t = first; t < n_tokens; ++t) {
    int32_t src, dst;
    rc = pa_bm_append_slot(m, seq_id, &slots_out[t - first], &src, &dst);
    if (rc) {
      pa_bm_free_sequence(m, seq_id);  // back to the state before the call
      return rc;
    }
  }
  const int32_t nb = pa_bm_num_blocks_of(m, seq_id);
  std::vector<int32_t> table((size_t)(nb > 0 ? nb : 1));
  int32_t len32 = 0;
  rc = pa_bm_export(m, &seq_id, 1, nb, table.data(), &len32);
  if (rc == PA_OK) rc = pa_pc_insert(c, tokens, n_tokens, table.data(), nb);
  if (rc < 0) {
    pa_bm_free_sequence(m, seq_id);
    return rc;
  }
  return first;
}
