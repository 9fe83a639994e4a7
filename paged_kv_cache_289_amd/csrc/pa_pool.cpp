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
// Prefix caching.  The pages' server hashes each page's token content, so
// that requests with the same first N tokens share N / B physical pages
// without recomputing them ("Local_LLM_03_vLLM_Architecture", prefix-caching
// slide; "vLLM: LLM Inference That Doesn't Waste Your GPU", section "Prefix
// caching").  Here a full block whose K/V are written is registered
// (paged_seq_commit) under a chained 64-bit key of its tokens and its parent's
// key; an empty sequence then takes every leading full block registered under
// the same token prefix (paged_seq_match_prefix).  A hit is verified, not
// trusted: the entry keeps the block's tokens and its parent block, and both
// must equal the candidate's (the parent of a live cached block is live, since
// every table holds a whole prefix of blocks, so by induction a match means
// exactly the same token prefix).  A block leaves the cache when it is freed.
//
// Free blocks sit on a LIFO stack (O(1) take and give back); released
// sequence ids are reused.  Every entry point takes the pool's mutex.
#include <algorithm>
#include <mutex>
#include <new>
#include <unordered_map>
#include <vector>

#include "paged_attn.h"

struct paged_block_pool {
  struct Seq {
    bool live = false;
    int64_t len = 0;
    std::vector<int32_t> blocks;
    std::vector<uint64_t> keys;   // cache keys of the leading full blocks known so far
  };
  struct CacheEntry {
    int32_t block;
    int32_t parent_block;         // -1 for a sequence's first block
    std::vector<int32_t> tokens;
  };
  int block_size = 0;
  int num_blocks = 0;
  std::vector<int32_t> free_stack;
  std::vector<int32_t> ref;
  std::vector<Seq> seqs;
  std::vector<int> free_ids;
  std::unordered_map<uint64_t, CacheEntry> cache;
  std::vector<uint64_t> cached_key;   // per block: its key while it is cached
  std::vector<uint8_t> is_cached;
  mutable std::mutex mu;

  bool valid_seq(int s) const { return s >= 0 && s < (int)seqs.size() && seqs[s].live; }

  int32_t take() {
    const int32_t b = free_stack.back();
    free_stack.pop_back();
    ref[b] = 1;
    return b;
  }
  void drop(int32_t b) {
    if (--ref[b] != 0) return;
    if (is_cached[b]) {
      auto it = cache.find(cached_key[b]);
      if (it != cache.end() && it->second.block == b) cache.erase(it);
      is_cached[b] = 0;
    }
    free_stack.push_back(b);
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
    seqs[s].keys.clear();
    return s;
  }
};

namespace {
int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// splitmix64 finalizer (Steele, Lea and Flood's SplitMix generator, as
// published by Vigna): a bijective 64-bit mix.
uint64_t mix64(uint64_t x) {
  x += 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

constexpr uint64_t kRootKey = 0x243F6A8885A308D3ull;   // parent key of a first block

// Key of a full block: its parent's key, then each token id, mixed in turn.
uint64_t block_key(uint64_t parent, const int32_t* tokens, int n) {
  uint64_t h = mix64(parent);
  for (int i = 0; i < n; ++i) h = mix64(h ^ (uint32_t)tokens[i]);
  return h;
}
}  // namespace

extern "C" {

paged_block_pool* paged_pool_create(int num_blocks, int block_size) {
  if (num_blocks < 1 || block_size < 1) return nullptr;
  paged_block_pool* p = new (std::nothrow) paged_block_pool;
  if (!p) return nullptr;
  p->block_size = block_size;
  p->num_blocks = num_blocks;
  p->ref.assign(num_blocks, 0);
  p->cached_key.assign(num_blocks, 0);
  p->is_cached.assign(num_blocks, 0);
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
  pool->seqs[s].keys = pool->seqs[parent].keys;
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
  q.keys.clear();
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

int paged_seq_match_prefix(paged_block_pool* pool, int seq, const int32_t* tokens,
                           int num_tokens) {
  if (!pool) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(pool->mu);
  if (!pool->valid_seq(seq) || pool->seqs[seq].len != 0) return PA_ERR_INVALID;
  if (num_tokens < 0) return PA_ERR_SHAPE;
  if (num_tokens > 0 && !tokens) return PA_ERR_NULL;
  paged_block_pool::Seq& q = pool->seqs[seq];
  const int B = pool->block_size;
  uint64_t parent = kRootKey;
  int32_t parent_block = -1;
  int64_t j = 0;
  for (; (j + 1) * B <= num_tokens; ++j) {
    const int32_t* t = tokens + j * B;
    const uint64_t k = block_key(parent, t, B);
    auto it = pool->cache.find(k);
    if (it == pool->cache.end()) break;
    const paged_block_pool::CacheEntry& e = it->second;
    if (e.parent_block != parent_block || !std::equal(e.tokens.begin(), e.tokens.end(), t)) break;
    q.blocks.push_back(e.block);
    q.keys.push_back(k);
    ++pool->ref[e.block];
    parent = k;
    parent_block = e.block;
  }
  q.len = j * B;
  return (int)q.len;
}

int paged_seq_commit(paged_block_pool* pool, int seq, const int32_t* tokens, int num_tokens) {
  if (!pool) return PA_ERR_NULL;
  std::lock_guard<std::mutex> g(pool->mu);
  if (!pool->valid_seq(seq)) return PA_ERR_INVALID;
  paged_block_pool::Seq& q = pool->seqs[seq];
  if (num_tokens < 0 || num_tokens > q.len) return PA_ERR_SHAPE;
  if (num_tokens > 0 && !tokens) return PA_ERR_NULL;
  const int B = pool->block_size;
  int added = 0;
  uint64_t parent = q.keys.empty() ? kRootKey : q.keys.back();
  for (int64_t j = (int64_t)q.keys.size(); (j + 1) * B <= num_tokens; ++j) {
    const int32_t* t = tokens + j * B;
    const uint64_t k = block_key(parent, t, B);
    const int32_t b = q.blocks[j];
    if (!pool->cache.count(k) && !pool->is_cached[b]) {
      pool->cache.emplace(k, paged_block_pool::CacheEntry{b, j ? q.blocks[j - 1] : -1,
                                                          std::vector<int32_t>(t, t + B)});
      pool->is_cached[b] = 1;
      pool->cached_key[b] = k;
      ++added;
    }
    q.keys.push_back(k);
    parent = k;
  }
  return added;
}

}  // extern "C"
