// Host-side block allocator and sequence block manager (plain C++, no device
// calls).
//
// Allocator: "5.KV Cache 管理 & PagedAttention", question 9 -- a stack of
// free block ids (allocation pops the top; an empty stack is an
// out-of-blocks error), made thread-safe with a lock (9.2), with per-block
// reference counts for sharing (9.4).  Where the page has no guard, this
// implementation refuses: ids outside [0, N), incref/decref of a block that
// is not allocated (which also rules out double free and underflow).
//
// Sequence manager: the same page, question 10 (allocate blocks as the
// sequence grows), question 12 (a token at position L goes to logical block
// L / bs, offset L % bs; a new block when L fills the table), question 18
// (fork shares every block; writing into a shared block first moves the
// writer to a fresh copy), question 20 (a shared prefix is attached by
// taking a reference on existing blocks).
#include <mutex>
#include <unordered_map>
#include <vector>

#include "../../include/pa.h"

namespace pa {
int set_error(int code, const char* msg);
void alloc_add_user(pa_allocator* a);
void alloc_drop_user(pa_allocator* a);
}

struct pa_allocator {
  std::mutex mu;
  int32_t n = 0;
  std::vector<int32_t> free_stack;  // top = back()
  std::vector<int32_t> ref;
  // Managers and prefix caches built on this allocator release references
  // through it when they are destroyed, so its memory outlives them: a
  // destroy request while any of them lives only marks it, and the last one
  // to go frees it (callers such as garbage collectors may destroy the
  // three in any order).
  int32_t users = 0;
  bool doomed = false;
};

struct pa_block_manager {
  struct Seq {
    std::vector<int32_t> table;
    int64_t len = 0;
  };
  std::mutex mu;
  pa_allocator* a = nullptr;
  int32_t bs = 0;
  std::unordered_map<int64_t, Seq> seqs;
};

namespace {

int alloc_locked(pa_allocator* a, int32_t* out) {
  if (a->free_stack.empty()) return pa::set_error(PA_ERR_OUT_OF_BLOCKS, "all blocks are in use");
  const int32_t b = a->free_stack.back();
  a->free_stack.pop_back();
  a->ref[b] = 1;
  *out = b;
  return PA_OK;
}

int check_allocated_locked(const pa_allocator* a, int32_t b) {
  if (b < 0 || b >= a->n) return pa::set_error(PA_ERR_BAD_BLOCK, "block id out of range");
  if (a->ref[b] == 0) return pa::set_error(PA_ERR_BAD_BLOCK, "block is not allocated");
  return PA_OK;
}

int decref_locked(pa_allocator* a, int32_t b) {
  int rc = check_allocated_locked(a, b);
  if (rc) return rc;
  if (--a->ref[b] == 0) a->free_stack.push_back(b);
  return PA_OK;
}

}  // namespace

extern "C" {

pa_allocator* pa_alloc_create(int32_t num_blocks, const int32_t* free_order) {
  if (num_blocks < 0) {
    pa::set_error(PA_ERR_INVALID_ARG, "num_blocks must be >= 0");
    return nullptr;
  }
  pa_allocator* a = new pa_allocator;
  a->n = num_blocks;
  a->ref.assign(num_blocks, 0);
  a->free_stack.resize(num_blocks);
  if (free_order) {
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < num_blocks; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete a;
        pa::set_error(PA_ERR_INVALID_ARG, "free_order must be a permutation of 0..N-1");
        return nullptr;
      }
      seen[b] = 1;
      a->free_stack[i] = b;
    }
  } else {
    for (int32_t i = 0; i < num_blocks; ++i) a->free_stack[i] = i;
  }
  return a;
}

void pa_alloc_destroy(pa_allocator* a) {
  if (!a) return;
  {
    std::lock_guard<std::mutex> g(a->mu);
    if (a->users > 0) {
      a->doomed = true;
      return;
    }
  }
  delete a;
}

int pa_alloc_allocate(pa_allocator* a, int32_t* block_out) {
  if (!a || !block_out) return pa::set_error(PA_ERR_INVALID_ARG, "null argument");
  std::lock_guard<std::mutex> g(a->mu);
  return alloc_locked(a, block_out);
}

int pa_alloc_incref(pa_allocator* a, int32_t block) {
  if (!a) return pa::set_error(PA_ERR_INVALID_ARG, "null allocator");
  std::lock_guard<std::mutex> g(a->mu);
  int rc = check_allocated_locked(a, block);
  if (rc) return rc;
  ++a->ref[block];
  return PA_OK;
}

int pa_alloc_decref(pa_allocator* a, int32_t block) {
  if (!a) return pa::set_error(PA_ERR_INVALID_ARG, "null allocator");
  std::lock_guard<std::mutex> g(a->mu);
  return decref_locked(a, block);
}

int32_t pa_alloc_num_free(const pa_allocator* a) {
  if (!a) return pa::set_error(PA_ERR_INVALID_ARG, "null allocator");
  std::lock_guard<std::mutex> g(const_cast<pa_allocator*>(a)->mu);
  return (int32_t)a->free_stack.size();
}

int32_t pa_alloc_num_blocks(const pa_allocator* a) {
  if (!a) return pa::set_error(PA_ERR_INVALID_ARG, "null allocator");
  return a->n;
}

int32_t pa_alloc_refcount(const pa_allocator* a, int32_t block) {
  if (!a) return pa::set_error(PA_ERR_INVALID_ARG, "null allocator");
  std::lock_guard<std::mutex> g(const_cast<pa_allocator*>(a)->mu);
  if (block < 0 || block >= a->n) return pa::set_error(PA_ERR_BAD_BLOCK, "block id out of range");
  return a->ref[block];
}

pa_block_manager* pa_bm_create(pa_allocator* a, int32_t block_size) {
  if (!a || block_size <= 0) {
    pa::set_error(PA_ERR_INVALID_ARG, "need an allocator and a positive block size");
    return nullptr;
  }
  pa_block_manager* m = new pa_block_manager;
  m->a = a;
  m->bs = block_size;
  pa::alloc_add_user(a);
  return m;
}

void pa_bm_destroy(pa_block_manager* m) {
  if (!m) return;
  pa_allocator* a = m->a;
  delete m;
  pa::alloc_drop_user(a);
}

int pa_bm_add_sequence(pa_block_manager* m, int64_t seq_id, const int32_t* shared_blocks,
                       int32_t n_shared, int64_t shared_tokens) {
  if (!m || n_shared < 0 || (n_shared > 0 && !shared_blocks) || shared_tokens < 0)
    return pa::set_error(PA_ERR_INVALID_ARG, "invalid arguments");
  if (shared_tokens > (int64_t)n_shared * m->bs)
    return pa::set_error(PA_ERR_INVALID_ARG, "shared tokens exceed the shared blocks");
  std::lock_guard<std::mutex> g(m->mu);
  if (m->seqs.count(seq_id)) return pa::set_error(PA_ERR_INVALID_ARG, "sequence id already exists");
  std::lock_guard<std::mutex> ga(m->a->mu);
  for (int32_t i = 0; i < n_shared; ++i) {
    int rc = check_allocated_locked(m->a, shared_blocks[i]);
    if (rc) return rc;
  }
  pa_block_manager::Seq s;
  s.table.assign(shared_blocks, shared_blocks + n_shared);
  s.len = shared_tokens;
  for (int32_t b : s.table) ++m->a->ref[b];
  m->seqs.emplace(seq_id, std::move(s));
  return PA_OK;
}

int pa_bm_append_slot(pa_block_manager* m, int64_t seq_id, int64_t* slot_out, int32_t* cow_src,
                      int32_t* cow_dst) {
  if (!m || !slot_out) return pa::set_error(PA_ERR_INVALID_ARG, "invalid arguments");
  std::lock_guard<std::mutex> g(m->mu);
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return pa::set_error(PA_ERR_NOT_FOUND, "unknown sequence id");
  pa_block_manager::Seq& s = it->second;
  std::lock_guard<std::mutex> ga(m->a->mu);
  int32_t src = -1, dst = -1;
  const int64_t idx = s.len / m->bs;
  if (s.len % m->bs == 0 && idx == (int64_t)s.table.size()) {
    int32_t nb;
    int rc = alloc_locked(m->a, &nb);
    if (rc) return rc;
    s.table.push_back(nb);
  } else {
    const int32_t blk = s.table[idx];
    if (m->a->ref[blk] > 1) {
      int32_t nb;
      int rc = alloc_locked(m->a, &nb);
      if (rc) return rc;
      decref_locked(m->a, blk);
      s.table[idx] = nb;
      src = blk;
      dst = nb;
    }
  }
  *slot_out = (int64_t)s.table[idx] * m->bs + s.len % m->bs;
  s.len += 1;
  if (cow_src) *cow_src = src;
  if (cow_dst) *cow_dst = dst;
  return PA_OK;
}

int pa_bm_fork(pa_block_manager* m, int64_t parent_id, int64_t child_id) {
  if (!m) return pa::set_error(PA_ERR_INVALID_ARG, "null manager");
  std::lock_guard<std::mutex> g(m->mu);
  auto it = m->seqs.find(parent_id);
  if (it == m->seqs.end()) return pa::set_error(PA_ERR_NOT_FOUND, "unknown parent sequence");
  if (m->seqs.count(child_id)) return pa::set_error(PA_ERR_INVALID_ARG, "child id already exists");
  pa_block_manager::Seq c = it->second;
  std::lock_guard<std::mutex> ga(m->a->mu);
  for (int32_t b : c.table) ++m->a->ref[b];
  m->seqs.emplace(child_id, std::move(c));
  return PA_OK;
}

int pa_bm_free_sequence(pa_block_manager* m, int64_t seq_id) {
  if (!m) return pa::set_error(PA_ERR_INVALID_ARG, "null manager");
  std::lock_guard<std::mutex> g(m->mu);
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return pa::set_error(PA_ERR_NOT_FOUND, "unknown sequence id");
  std::lock_guard<std::mutex> ga(m->a->mu);
  for (int32_t b : it->second.table) decref_locked(m->a, b);
  m->seqs.erase(it);
  return PA_OK;
}

int64_t pa_bm_seq_len(const pa_block_manager* m, int64_t seq_id) {
  if (!m) return pa::set_error(PA_ERR_INVALID_ARG, "null manager");
  std::lock_guard<std::mutex> g(const_cast<pa_block_manager*>(m)->mu);
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return pa::set_error(PA_ERR_NOT_FOUND, "unknown sequence id");
  return it->second.len;
}

int32_t pa_bm_num_blocks_of(const pa_block_manager* m, int64_t seq_id) {
  if (!m) return pa::set_error(PA_ERR_INVALID_ARG, "null manager");
  std::lock_guard<std::mutex> g(const_cast<pa_block_manager*>(m)->mu);
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return pa::set_error(PA_ERR_NOT_FOUND, "unknown sequence id");
  return (int32_t)it->second.table.size();
}

int pa_bm_export(const pa_block_manager* m, const int64_t* seq_ids, int32_t n, int32_t max_blocks,
                 int32_t* block_tables, int32_t* seq_lens) {
  if (!m || n < 0 || max_blocks < 0 || (n > 0 && (!seq_ids || !block_tables || !seq_lens)))
    return pa::set_error(PA_ERR_INVALID_ARG, "invalid arguments");
  std::lock_guard<std::mutex> g(const_cast<pa_block_manager*>(m)->mu);
  for (int32_t i = 0; i < n; ++i) {
    auto it = m->seqs.find(seq_ids[i]);
    if (it == m->seqs.end()) return pa::set_error(PA_ERR_NOT_FOUND, "unknown sequence id");
    if ((int64_t)it->second.table.size() > max_blocks)
      return pa::set_error(PA_ERR_INVALID_ARG, "a block table does not fit in max_blocks");
    if (it->second.len > 0x7FFFFFFF) return pa::set_error(PA_ERR_INVALID_ARG, "sequence too long");
  }
  for (int32_t i = 0; i < n; ++i) {
    const auto& s = m->seqs.find(seq_ids[i])->second;
    int32_t* row = block_tables + (int64_t)i * max_blocks;
    for (int32_t j = 0; j < max_blocks; ++j) row[j] = j < (int32_t)s.table.size() ? s.table[j] : -1;
    seq_lens[i] = (int32_t)s.len;
  }
  return PA_OK;
}

}  // extern "C"

namespace pa {
// block size of a manager (for the prefix-cache admission, which must use
// the same one)
int32_t bm_block_size(const pa_block_manager* m) { return m ? m->bs : 0; }

void alloc_add_user(pa_allocator* a) {
  std::lock_guard<std::mutex> g(a->mu);
  ++a->users;
}

// the allocator is freed here when it was destroyed while this user lived
void alloc_drop_user(pa_allocator* a) {
  bool free_it;
  {
    std::lock_guard<std::mutex> g(a->mu);
    free_it = --a->users == 0 && a->doomed;
  }
  if (free_it) delete a;
}
}  // namespace pa
