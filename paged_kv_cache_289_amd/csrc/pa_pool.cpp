// Host-side pool of physical KV blocks: the allocator behind the block tables.
//
// The cache is a pool of fixed-size blocks handed out as sequences grow, so a
// sequence of L tokens holds ceil(L / B) blocks and wastes fewer than B slots
// ("Scaling inference with vLLM", paging paragraph; "vLLM: LLM Inference That
// Doesn't Waste Your GPU", section "PagedAttention: virtual memory for KV").
// Sequences with a common start physically share its blocks instead of copying
// them ("Scaling inference with vLLM", prefix-sharing paragraph): a fork takes
// the parent's table and raises every block's reference count.  A block goes
// back to the free list when no table holds it.  Before a sequence writes into
// a partially filled block that other tables also hold, it gets a private copy
// (copy-on-write): the append returns the (source, destination) pair for the
// caller to copy on the device (paged_kv_copy_blocks) before the new tokens are
// written (paged_kv_append).  Full shared blocks are never written again.
//
// Free blocks sit on a LIFO stack (O(1) take and give back); released
// sequence ids are reused.  Every entry point takes the pool's mutex.
#include <mutex>
#include <new>
#include <vector>

#include "paged_attn.h"

struct paged_block_pool {
  struct Seq {
    bool live = false;
    int64_t len = 0;
    std::vector<int32_t> blocks;
  };
  int block_size = 0;
  int num_blocks = 0;
  std::vector<int32_t> free_stack;
  std::vector<int32_t> ref;
  std::vector<Seq> seqs;
  std::vector<int> free_ids;
  mutable std::mutex mu;

  bool valid_seq(int s) const { return s >= 0 && s < (int)seqs.size() && seqs[s].live; }

  int32_t take() {
    const int32_t b = free_stack.back();
    free_stack.pop_back();
    ref[b] = 1;
    return b;
  }
  void drop(int32_t b) {
    if (--ref[b] == 0) free_stack.push_back(b);
  }
  int new_seq() {
    int s;
    if (!free_ids.empty()) {
      s = free_ids.back();
      free_ids.pop_back();
    } else {
      s = (int)seqs.size();
      seqs.emplace_back();
    }
    seqs[s].live = true;
    seqs[s].len = 0;
    seqs[s].blocks.clear();
    return s;
  }
};

namespace {
int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }
}  // namespace

extern "C" {

paged_block_pool* paged_pool_create(int num_blocks, int block_size) {
  if (num_blocks < 1 || block_size < 1) return nullptr;
  paged_block_pool* p = new (std::nothrow) paged_block_pool;
  if (!p) return nullptr;
  p->block_size = block_size;
  p->num_blocks = num_blocks;
  p->ref.assign(num_blocks, 0);
  p->free_stack.reserve(num_blocks);
  for (int b = num_blocks - 1; b >= 0; --b) p->free_stack.push_back(b);   // block 0 first
  return p;
}

void paged_pool_destroy(paged_block_pool* pool) { delete pool; }

int paged_pool_num_free(const paged_block_pool* pool) {
  if (!pool) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(pool->mu);
  return (int)pool->free_stack.size();
}

int paged_pool_refcount(const paged_block_pool* pool, int block) {
  if (!pool) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(pool->mu);
  if (block < 0 || block >= pool->num_blocks) return PA_ERR_INVALID;
  return pool->ref[block];
}

int paged_seq_create(paged_block_pool* pool) {
  if (!pool) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(pool->mu);
  return pool->new_seq();
}

int paged_seq_fork(paged_block_pool* pool, int parent) {
  if (!pool) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(pool->mu);
  if (!pool->valid_seq(parent)) return PA_ERR_INVALID;
  const int s = pool->new_seq();              // (may reallocate seqs: index afterwards)
  pool->seqs[s].blocks = pool->seqs[parent].blocks;
  pool->seqs[s].len = pool->seqs[parent].len;
  for (int32_t b : pool->seqs[s].blocks) ++pool->ref[b];
  return s;
}

int paged_seq_release(paged_block_pool* pool, int seq) {
  if (!pool) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(pool->mu);
  if (!pool->valid_seq(seq)) return PA_ERR_INVALID;
  paged_block_pool::Seq& q = pool->seqs[seq];
  for (int32_t b : q.blocks) pool->drop(b);
  q.blocks.clear();
  q.len = 0;
  q.live = false;
  pool->free_ids.push_back(seq);
  return PA_OK;
}

int paged_seq_append(paged_block_pool* pool, int seq, int num_tokens, int32_t* copy_pairs,
                     int max_pairs, int* num_pairs) {
  if (!pool || !num_pairs) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(pool->mu);
  if (!pool->valid_seq(seq)) return PA_ERR_INVALID;
  if (num_tokens < 0 || max_pairs < 0) return PA_ERR_SHAPE;
  *num_pairs = 0;
  if (num_tokens == 0) return PA_OK;
  paged_block_pool::Seq& q = pool->seqs[seq];
  const int64_t B = pool->block_size, L = q.len;
  const bool cow = L % B != 0 && pool->ref[q.blocks.back()] > 1;
  const int64_t grow = ceil_div64(L + num_tokens, B) - ceil_div64(L, B);
  if (grow + (cow ? 1 : 0) > (int64_t)pool->free_stack.size()) return PA_ERR_NO_BLOCKS;
  if (cow && (max_pairs < 1 || !copy_pairs)) return PA_ERR_SHAPE;
  if (cow) {
    const int32_t old = q.blocks.back();
    const int32_t fresh = pool->take();
    copy_pairs[0] = old;
    copy_pairs[1] = fresh;
    *num_pairs = 1;
    q.blocks.back() = fresh;
    pool->drop(old);
  }
  for (int64_t i = 0; i < grow; ++i) q.blocks.push_back(pool->take());
  q.len = L + num_tokens;
  return PA_OK;
}

int paged_seq_length(const paged_block_pool* pool, int seq) {
  if (!pool) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(pool->mu);
  if (!pool->valid_seq(seq)) return PA_ERR_INVALID;
  const int64_t L = pool->seqs[seq].len;
  return L > 0x7fffffff ? PA_ERR_SHAPE : (int)L;
}

int paged_seq_blocks(const paged_block_pool* pool, int seq, int32_t* out, int max_blocks) {
  if (!pool) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(pool->mu);
  if (!pool->valid_seq(seq)) return PA_ERR_INVALID;
  const std::vector<int32_t>& b = pool->seqs[seq].blocks;
  if (max_blocks < (int)b.size()) return PA_ERR_SHAPE;
  if (!b.empty() && !out) return PA_ERR_NULL;
  for (size_t i = 0; i < b.size(); ++i) out[i] = b[i];
  return (int)b.size();
}

}  // extern "C"
