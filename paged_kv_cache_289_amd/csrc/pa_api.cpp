// C-ABI host layer of libpagedattn.so: argument validation (pure host code,
// before any HIP call), the partition planner, workspace sizing and dispatch to
// the kernel launchers.  Declarations and conventions: include/paged_attn.h.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <cmath>

#include "pa_internal.h"

namespace {

bool dtype_ok(int dt) { return dt == PA_F32 || dt == PA_F16 || dt == PA_BF16; }
int elem_bytes(int dt) { return dt == PA_F32 ? 4 : dt == PA_FP8_E4M3 ? 1 : 2; }
// the entry points that only move cache bytes also take 8-bit caches
bool kv_dtype_ok(int dt) { return dtype_ok(dt) || dt == PA_FP8_E4M3; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// events of paged_attn_set_kernel_events, per host thread
thread_local pa::KernelEvents t_events;

// Shared shape checks of the attention entry points.  Returns PA_OK or an error.
int check_attn_shapes(int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
                      int num_blocks, int max_blocks_per_seq, int max_context_len, int dtype,
                      int out_dtype, int partition_tokens, float scale) {
  if (num_seqs < 0 || num_heads < 1 || num_kv_heads < 1 || head_dim < 1 || block_size < 1 ||
      num_blocks < 1 || max_blocks_per_seq < 1 || max_context_len < 0 || partition_tokens < 0)
    return PA_ERR_SHAPE;
  if (num_heads % num_kv_heads != 0) return PA_ERR_SHAPE;
  if (!dtype_ok(dtype) || !(out_dtype == PA_F32 || out_dtype == dtype)) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (block_size != 8 && block_size != 16 && block_size != 32) return PA_ERR_UNSUPPORTED;
  if (num_heads / num_kv_heads > 16) return PA_ERR_UNSUPPORTED;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size) return PA_ERR_SHAPE;
  if (partition_tokens > 0 && partition_tokens % block_size != 0) return PA_ERR_SHAPE;
  if (!isfinite(scale)) return PA_ERR_SHAPE;
  return PA_OK;
}

int resolve_partition(int partition_tokens, int num_seqs, int num_heads, int num_kv_heads,
                      int block_size, int max_context_len, int max_q_len) {
  return partition_tokens > 0
             ? partition_tokens
             : paged_attn_default_partition(num_seqs, num_heads, num_kv_heads, block_size,
                                            max_context_len, max_q_len);
}

// Partition-mode workspace: fp32 (max, sum) pairs [rows][H][P], padded to a
// multiple of 4 floats so that the partial outputs after them start on a
// 16-byte boundary (the kernels move them as 16-byte vectors), then fp32
// partial outputs [rows][H][P][D].
size_t partial_ml_floats(int rows, int num_heads, int max_parts) {
  return ((size_t)rows * num_heads * max_parts * 2 + 3) / 4 * 4;
}

size_t workspace_bytes_for(int rows, int num_heads, int head_dim, int max_parts) {
  if (max_parts <= 1) return 0;
  return (partial_ml_floats(rows, num_heads, max_parts) +
          (size_t)rows * num_heads * max_parts * head_dim) * sizeof(float);
}

void split_workspace(void* ws, int rows, int num_heads, int max_parts, pa::AttnArgs* a) {
  float* base = static_cast<float*>(ws);
  a->ws_ml = base;
  a->ws_o = base + partial_ml_floats(rows, num_heads, max_parts);
}

// Balanced-split decode plan.  Work items are (sequence, KV head, block);
// `bound` is the most there can be.  With partition_tokens > 0 every wave takes
// partition_tokens / B blocks; otherwise the launch is the resident wave count
// and the device splits the items evenly.
struct SplitPlan {
  bool use = false;
  int chunk = 0;          // 0: decided on the device
  int waves = 0;          // waves launched (multiple of kWaves)
  int workgroups = 0;
};

// items of the balanced split at most: every (sequence, KV head) costs its
// blocks plus kSegItems
int64_t split_bound(int num_seqs, int num_kv_heads, int block_size, int max_context_len) {
  return (int64_t)num_seqs * num_kv_heads * (ceil_div(max_context_len, block_size) + pa::kSegItems);
}

SplitPlan plan_split(int num_seqs, int num_kv_heads, int block_size, int max_context_len,
                     int partition_tokens, int resident_waves) {
  SplitPlan p;
  if (num_seqs > pa::kMaxSplitSeqs) return p;
  p.use = true;
  const int64_t bound = split_bound(num_seqs, num_kv_heads, block_size, max_context_len);
  int64_t waves;
  if (partition_tokens > 0) {
    p.chunk = partition_tokens / block_size;
    waves = (bound + p.chunk - 1) / p.chunk;
  } else {
    waves = std::min<int64_t>(bound, std::min(resident_waves, pa::kMaxSplitWaves));
  }
  waves = std::max<int64_t>(1, waves);
  p.workgroups = (int)((waves + pa::kWaves - 1) / pa::kWaves);
  p.waves = p.workgroups * pa::kWaves;
  return p;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Split-mode workspace, each region on a 256-byte boundary (whole cache
// lines): the int32 plan [2 + S + 1] that the merge reads, then fp32 (max, sum)
// pairs and fp32 partial outputs for (S Hk + waves) slots x G heads.
struct SplitLayout {
  size_t plan = 0, ml = 0, o = 0, total = 0;
};

SplitLayout split_layout(int num_seqs, int num_heads, int num_kv_heads, int head_dim, int waves) {
  SplitLayout l;
  const size_t slots = (size_t)num_seqs * num_kv_heads + waves;
  const size_t group = (size_t)(num_heads / num_kv_heads);
  l.plan = 0;
  l.ml = align256((size_t)(3 + num_seqs) * sizeof(int32_t));
  l.o = l.ml + align256(slots * group * 2 * sizeof(float));
  l.total = l.o + slots * group * (size_t)head_dim * sizeof(float);
  return l;
}

size_t split_workspace_bytes(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                             int waves) {
  return split_layout(num_seqs, num_heads, num_kv_heads, head_dim, waves).total;
}

void split_workspace_ptrs(void* ws, int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                          int waves, pa::AttnArgs* a) {
  const SplitLayout l = split_layout(num_seqs, num_heads, num_kv_heads, head_dim, waves);
  char* base = static_cast<char*>(ws);
  a->plan = reinterpret_cast<int*>(base + l.plan);
  a->ws_ml = reinterpret_cast<float*>(base + l.ml);
  a->ws_o = reinterpret_cast<float*>(base + l.o);
}

// Balanced-split multi-query calls: several query tokens per sequence, rows
// that fit fewer than four 32-row tiles per KV head (the token layout),
// head_dim 128, the library's own work split (partition_tokens 0) and a
// bounded number of (sequence, KV head, row tile) units.  Applies to bf16 and
// f16; the workspace size covers it whatever the dtype.
int64_t mq_split_units(int num_seqs, int max_q_len, int num_heads, int num_kv_heads) {
  const int group = num_heads / num_kv_heads;
  return (int64_t)num_seqs * num_kv_heads * ceil_div(max_q_len * group, 32);
}

bool mq_split_shape(int num_seqs, int max_q_len, int num_heads, int num_kv_heads, int head_dim,
                    int partition_tokens) {
  if (partition_tokens != 0 || head_dim != 128 || max_q_len < 2 || num_seqs < 1 ||
      num_seqs > pa::kMaxSplitSeqs || num_kv_heads < 1 || num_heads % num_kv_heads)
    return false;
  if (pa::multiq_rows_mode(max_q_len, num_heads / num_kv_heads)) return false;
  return mq_split_units(num_seqs, max_q_len, num_heads, num_kv_heads) <= pa::kMqMaxSplitUnits;
}

// Waves of a split launch: one per item at most, kMqMaxSplitWaves at most
// (fewer where fewer are resident), in whole workgroups.  The workspace is
// sized for the device-independent bound.
int mq_split_waves(int64_t units, int max_context_len, int resident) {
  const int64_t items = units * (ceil_div(max_context_len, 32) + pa::kMqSegItemsMax);
  const int64_t w =
      std::max<int64_t>(1, std::min<int64_t>(items, std::min(resident, pa::kMqMaxSplitWaves)));
  return (int)((w + pa::kWaves - 1) / pa::kWaves * pa::kWaves);
}

// Its workspace, each region on a 256-byte boundary: the int32 plan
// [2 + S + 1] that the merge reads, then fp32 (max, sum) pairs and fp32 partial
// outputs for (units + waves) slots x 32 rows.
SplitLayout mq_split_layout(int num_seqs, int max_q_len, int num_heads, int num_kv_heads,
                            int head_dim, int waves) {
  SplitLayout l;
  const size_t rows =
      ((size_t)mq_split_units(num_seqs, max_q_len, num_heads, num_kv_heads) + waves) * 32;
  l.plan = 0;
  l.ml = align256((size_t)(3 + num_seqs) * sizeof(int32_t));
  l.o = l.ml + align256(rows * 2 * sizeof(float));
  l.total = l.o + rows * (size_t)head_dim * sizeof(float);
  return l;
}

// Waves the workspace must allow for when the launch size is not known yet
// (it depends on the device's CU count and the kernel's occupancy).
int split_waves_bound(int num_seqs, int num_kv_heads, int block_size, int max_context_len,
                      int partition_tokens) {
  return plan_split(num_seqs, num_kv_heads, block_size, max_context_len, partition_tokens,
                    pa::kMaxSplitWaves).waves;
}

// CUs of the current device (cached per device; threads that race on the first
// query store the same value, atomically).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (!n) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n < 1)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace

extern "C" {

int paged_attn_set_kernel_events(void* start, void* stop) {
  if ((start == nullptr) != (stop == nullptr)) return PA_ERR_NULL;
  t_events.start = static_cast<hipEvent_t>(start);
  t_events.stop = static_cast<hipEvent_t>(stop);
  return PA_OK;
}

const char* paged_attn_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "a required pointer is NULL";
    case PA_ERR_SHAPE: return "inconsistent or negative sizes";
    case PA_ERR_UNSUPPORTED: return "unsupported dtype, head_dim, block_size, group or alignment";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP launch or runtime error";
    case PA_ERR_NO_BLOCKS: return "block pool has too few free blocks";
    case PA_ERR_INVALID: return "unknown or released sequence id, or block id outside the pool";
    case PA_ERR_SCRATCH:
      return "the call needs more device scratch than the allocation-free entry point holds "
             "(32 MiB per GPU)";
    default: return "unknown status";
  }
}

int paged_attn_default_partition(int num_seqs, int num_heads, int num_kv_heads, int block_size,
                                 int max_context_len, int max_q_len) {
  int part;
  if (max_q_len > 1) {
    // multi-token queries: one workgroup per (row unit, KV head, sequence,
    // partition), a row unit being one 32-row tile, or four of them when a
    // sequence has that many rows.  Partitions are sized so that the longest
    // context is covered by about 2048 workgroups (one-tile units) or 512
    // (four-tile units: two resident per CU, each doing four times the work),
    // in 32-token tiles, between 256 and 4096 tokens.
    const int group = num_kv_heads > 0 ? std::max(1, num_heads / num_kv_heads) : 1;
    const int tiles = ceil_div(max_q_len * group, 32);
    const bool rows = pa::multiq_rows_mode(max_q_len, group);
    const int64_t units = (int64_t)std::max(1, num_seqs) * std::max(1, num_kv_heads) *
                          (rows ? ceil_div(tiles, pa::kWaves) : tiles);
    int64_t want = (int64_t)max_context_len * units / (rows ? 512 : 2048);
    want = std::min<int64_t>(4096, std::max<int64_t>(256, want));
    part = (int)((want + 31) / 32 * 32);
  } else {
    part = 2048;
  }
  if (part % block_size) part = ceil_div(part, block_size) * block_size;
  return part;
}

int paged_attn_multiq_uses_split(int num_seqs, int max_q_len, int num_heads, int num_kv_heads,
                                 int head_dim, int dtype, int partition_tokens) {
  return (dtype == PA_BF16 || dtype == PA_F16) &&
                 mq_split_shape(num_seqs, max_q_len, num_heads, num_kv_heads, head_dim,
                                partition_tokens)
             ? 1
             : 0;
}

size_t paged_attn_workspace_size(int num_seqs, int total_q, int max_q_len, int num_heads,
                                 int num_kv_heads, int head_dim, int block_size,
                                 int max_context_len, int partition_tokens) {
  if (num_seqs < 0 || total_q < 0 || max_q_len < 0 || num_heads < 1 || num_kv_heads < 1 ||
      head_dim < 1 || block_size < 1 || max_context_len < 0 || partition_tokens < 0)
    return 0;
  if (partition_tokens > 0 && partition_tokens % block_size) return 0;
  if (num_heads % num_kv_heads) return 0;
  if (max_q_len <= 1 && num_seqs <= pa::kMaxSplitSeqs) {   // balanced-split decode
    if (num_seqs == 0) return 0;
    const int waves = split_waves_bound(num_seqs, num_kv_heads, block_size, max_context_len,
                                        partition_tokens);
    return split_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim, waves);
  }
  const int part = resolve_partition(partition_tokens, num_seqs, num_heads, num_kv_heads,
                                     block_size, max_context_len, max_q_len);
  const int max_parts = ceil_div(max_context_len, part);
  const size_t parts_bytes = workspace_bytes_for(total_q, num_heads, head_dim, max_parts);
  if (mq_split_shape(num_seqs, max_q_len, num_heads, num_kv_heads, head_dim, partition_tokens))
    return std::max(parts_bytes,
                    mq_split_layout(num_seqs, max_q_len, num_heads, num_kv_heads, head_dim,
                                    mq_split_waves(mq_split_units(num_seqs, max_q_len, num_heads,
                                                                  num_kv_heads),
                                                   max_context_len, pa::kMqMaxSplitWaves))
                        .total);
  return parts_bytes;
}

}  // extern "C"

namespace {

// paged_attn_decode with an optional per-(row, head) log-sum-exp output (log2
// units) and the profiling events to use.
int decode_core(void* out, const void* q, const void* k_cache, const void* v_cache,
                const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                int num_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                int max_blocks_per_seq, int max_context_len, float scale, int dtype, int out_dtype,
                int partition_tokens, void* workspace, size_t workspace_bytes, pa_stream_t stream,
                float* lse, const pa::KernelEvents& ev, float out_scale = 1.f,
                bool device_sized = false, int len_offset = 0, bool split_no_merge = false,
                pa::AttnArgs* used = nullptr) {
  // device_sized: the workspace is the allocation-free entry point's scratch,
  // checked against what this device's launch needs (PA_ERR_SCRATCH if it is
  // too small) rather than against the device-independent size.
  // len_offset: subtracted from every context length (the tails of a
  // shared-prefix decode).  split_no_merge: with the balanced split, leave the
  // pieces in the workspace (the caller merges them); `used` receives the
  // launch's arguments (plan and workspace regions).
  // (8-bit caches come with bf16 queries: the query type is what the checks see)
  int rc = check_attn_shapes(num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                             max_blocks_per_seq, max_context_len,
                             dtype == PA_FP8_E4M3 ? PA_BF16 : dtype, out_dtype, partition_tokens,
                             scale);
  if (rc != PA_OK) return rc;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_UNSUPPORTED;

  pa::AttnArgs a{};
  a.out_scale = out_scale;
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.q_offsets = nullptr;
  a.num_seqs = num_seqs;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_heads / num_kv_heads;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.pool_blocks = num_blocks;
  a.max_context_len = max_context_len;
  a.max_q_len = 1;
  a.causal = 0;
  a.out_dtype = out_dtype;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.lse = lse;
  a.len_offset = len_offset;

  if (num_seqs <= pa::kMaxSplitSeqs) {
    // the workspace is checked against the device-independent bound (what
    // paged_attn_workspace_size returns) before any HIP call
    if (!device_sized) {
      const int bound_waves = split_waves_bound(num_seqs, num_kv_heads, block_size,
                                                max_context_len, partition_tokens);
      const size_t need = split_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim,
                                                bound_waves);
      if (!workspace || workspace_bytes < need || !aligned16(workspace)) return PA_ERR_WORKSPACE;
    }
    // balanced split over the resident waves of this device
    const int wgs = pa::split_workgroups_per_cu(dtype, head_dim, block_size, a.group);
    const int resident = std::min(pa::kMaxSplitWaves,
                                  device_cus() * wgs * pa::kWaves);
    const SplitPlan sp = plan_split(num_seqs, num_kv_heads, block_size, max_context_len,
                                    partition_tokens, resident);
    if (device_sized &&
        workspace_bytes < split_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim,
                                                sp.waves))
      return PA_ERR_SCRATCH;
    split_workspace_ptrs(workspace, num_seqs, num_heads, num_kv_heads, head_dim, sp.waves, &a);
    a.chunk_blocks = sp.chunk;
    a.split_workgroups = sp.workgroups;
    a.part = 0;
    a.max_parts = 0;
    a.no_merge = split_no_merge ? 1 : 0;
  } else {
    const int part = resolve_partition(partition_tokens, num_seqs, num_heads, num_kv_heads,
                                       block_size, max_context_len, 1);
    const int max_parts = std::max(1, ceil_div(max_context_len, part));
    const size_t need = workspace_bytes_for(num_seqs, num_heads, head_dim, max_parts);
    if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
      return device_sized ? PA_ERR_SCRATCH : PA_ERR_WORKSPACE;
    if (need > 0) split_workspace(workspace, num_seqs, num_heads, max_parts, &a);
    a.part = part;
    a.max_parts = max_parts;
    a.plan = nullptr;
  }
  if ((dtype == PA_BF16 || dtype == PA_F16 || dtype == PA_FP8_E4M3) && head_dim == 128 &&
      a.plan && len_offset == 0 && !split_no_merge && !used && partition_tokens == 0 &&
      (int64_t)num_seqs * num_kv_heads <= pa::kMqMaxSplitUnits) {
    // Head_dim 128: the same balanced split, over (sequence, KV head, 32-token
    // tile) items, with the products on the matrix cores (the multi-query
    // split kernel without query offsets; an 8-bit cache is widened to f16).
    // Its pieces use the decode's slots, (S Hk + waves) x G, for at most
    // kMqMaxSplitWaves waves: within the workspace checked above, and checked
    // again against the allocation-free entry point's scratch.
    const int wgs = pa::multiq_split_workgroups_per_cu(dtype, block_size);
    const int waves = mq_split_waves((int64_t)num_seqs * num_kv_heads, max_context_len,
                                     device_cus() * wgs * pa::kWaves);
    if (device_sized &&
        workspace_bytes < split_workspace_bytes(num_seqs, num_heads, num_kv_heads, head_dim, waves))
      return PA_ERR_SCRATCH;
    split_workspace_ptrs(workspace, num_seqs, num_heads, num_kv_heads, head_dim, waves, &a);
    a.split_workgroups = waves / pa::kWaves;
    a.chunk_blocks = 0;
    hipError_t e = pa::launch_split_decode(dtype, block_size, num_seqs, a,
                                           static_cast<hipStream_t>(stream), ev);
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
  }
  if (used) *used = a;
  hipError_t e = pa::launch_decode(dtype, head_dim, block_size, a.group, num_seqs, a,
                                   static_cast<hipStream_t>(stream), ev);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

extern "C" {

int paged_attn_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                      int num_heads, int num_kv_heads, int head_dim, int block_size,
                      int num_blocks, int max_blocks_per_seq, int max_context_len, float scale,
                      int dtype, int out_dtype, int partition_tokens, void* workspace,
                      size_t workspace_bytes, pa_stream_t stream) {
  // 8-bit caches come with bf16 queries and per-tensor scales: only
  // paged_attn_decode_fp8kv takes them (it also rejects the shapes they cannot serve)
  if (!dtype_ok(dtype)) return PA_ERR_UNSUPPORTED;
  return decode_core(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                     max_context_len, scale, dtype, out_dtype, partition_tokens, workspace,
                     workspace_bytes, stream, nullptr, t_events);
}

int paged_attn_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                              int block_size, int num_blocks, int max_blocks_per_seq,
                              int max_context_len, float scale, int dtype, int out_dtype,
                              int partition_tokens, pa_stream_t stream) {
  // every scalar and pointer check before the first HIP call
  if (!dtype_ok(dtype)) return PA_ERR_UNSUPPORTED;
  const int rc = check_attn_shapes(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                   num_blocks, max_blocks_per_seq, max_context_len, dtype,
                                   out_dtype, partition_tokens, scale);
  if (rc != PA_OK) return rc;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_UNSUPPORTED;
  void* scratch = nullptr;
  if (pa::scratch_buffer(&scratch) != hipSuccess) return PA_ERR_HIP;
  return decode_core(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                     max_context_len, scale, dtype, out_dtype, partition_tokens, scratch,
                     pa::kScratchBytes, stream, nullptr, t_events, 1.f, /*device_sized=*/true);
}

}  // extern "C"

namespace {

// paged_attn_multiq with an optional log-sum-exp output and the events to use.
int multiq_core(void* out, const void* q, const void* k_cache, const void* v_cache,
                const int32_t* block_tables, const int32_t* context_lens,
                const int32_t* q_offsets, int num_seqs, int total_q, int max_q_len,
                int num_heads, int num_kv_heads, int head_dim, int block_size, int num_blocks,
                int max_blocks_per_seq, int max_context_len, float scale, int causal, int dtype,
                int out_dtype, int partition_tokens, void* workspace, size_t workspace_bytes,
                pa_stream_t stream, float* lse, const pa::KernelEvents& ev, int no_merge = 0,
                int fixed_rows = 0) {
  // fixed_rows > 0: one sequence of fixed_rows query rows whose length is
  // max_context_len (context_lens and q_offsets unused); only with no_merge
  if (fixed_rows > 0 && (!no_merge || num_seqs != 1 || total_q != fixed_rows)) return PA_ERR_SHAPE;
  int rc = check_attn_shapes(num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                             max_blocks_per_seq, max_context_len, dtype, out_dtype,
                             partition_tokens, scale);
  if (rc != PA_OK) return rc;
  if (total_q < 0 || max_q_len < 0 || (total_q > 0 && max_q_len < 1)) return PA_ERR_SHAPE;
  if ((int64_t)max_q_len * num_seqs < total_q) return PA_ERR_SHAPE;
  if (num_seqs == 0 || total_q == 0) return PA_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables ||
      (fixed_rows == 0 && (!context_lens || !q_offsets)))
    return PA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_UNSUPPORTED;

  if (!no_merge && fixed_rows == 0 &&
      paged_attn_multiq_uses_split(num_seqs, max_q_len, num_heads, num_kv_heads, head_dim, dtype,
                                   partition_tokens)) {
    // balanced split over the resident waves of this device; the workspace is
    // checked against the device-independent bound before any HIP call
    const int64_t units = mq_split_units(num_seqs, max_q_len, num_heads, num_kv_heads);
    if (!workspace || !aligned16(workspace) ||
        workspace_bytes <
            mq_split_layout(num_seqs, max_q_len, num_heads, num_kv_heads, head_dim,
                            mq_split_waves(units, max_context_len, pa::kMqMaxSplitWaves))
                .total)
      return PA_ERR_WORKSPACE;
    const int resident = device_cus() * pa::multiq_split_workgroups_per_cu(dtype, block_size) *
                         pa::kWaves;
    const int waves = mq_split_waves(units, max_context_len, resident);
    const int workgroups = waves / pa::kWaves;
    const SplitLayout l = mq_split_layout(num_seqs, max_q_len, num_heads, num_kv_heads, head_dim,
                                          waves);
    pa::AttnArgs a{};
    char* wsb = static_cast<char*>(workspace);
    a.plan = reinterpret_cast<int*>(wsb + l.plan);
    a.ws_ml = reinterpret_cast<float*>(wsb + l.ml);
    a.ws_o = reinterpret_cast<float*>(wsb + l.o);
    a.split_workgroups = workgroups;
    a.out = out;
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.q_offsets = q_offsets;
    a.num_seqs = num_seqs;
    a.num_heads = num_heads;
    a.num_kv_heads = num_kv_heads;
    a.group = num_heads / num_kv_heads;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.pool_blocks = num_blocks;
    a.max_context_len = max_context_len;
    a.max_q_len = max_q_len;
    a.causal = causal ? 1 : 0;
    a.out_dtype = out_dtype;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.out_scale = 1.f;
    a.lse = lse;
    hipError_t e = pa::launch_multiq(dtype, head_dim, block_size, a.group, num_seqs, a,
                                     static_cast<hipStream_t>(stream), ev);
    if (e == hipErrorNotSupported) return PA_ERR_UNSUPPORTED;
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
  }

  const int part = resolve_partition(partition_tokens, num_seqs, num_heads, num_kv_heads,
                                     block_size, max_context_len, max_q_len);
  const int max_parts = std::max(1, ceil_div(max_context_len, part));
  const int rows = total_q;
  const size_t need = workspace_bytes_for(rows, num_heads, head_dim, max_parts);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return PA_ERR_WORKSPACE;

  pa::AttnArgs a{};
  a.out = out;
  if (need > 0) split_workspace(workspace, rows, num_heads, max_parts, &a);
  a.num_seqs = num_seqs;
  a.plan = nullptr;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.q_offsets = q_offsets;
  a.num_heads = num_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_heads / num_kv_heads;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.pool_blocks = num_blocks;
  a.max_context_len = max_context_len;
  a.part = part;
  a.max_parts = max_parts;
  a.max_q_len = max_q_len;
  a.causal = causal ? 1 : 0;
  a.out_dtype = out_dtype;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.out_scale = 1.f;
  a.lse = lse;
  a.no_merge = no_merge;
  a.fixed_rows = fixed_rows;
  hipError_t e = pa::launch_multiq(dtype, head_dim, block_size, a.group, num_seqs, a,
                                   static_cast<hipStream_t>(stream), ev);
  if (e == hipErrorNotSupported) return PA_ERR_UNSUPPORTED;
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

extern "C" {

int paged_attn_multiq(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens,
                      const int32_t* q_offsets, int num_seqs, int total_q, int max_q_len,
                      int num_heads, int num_kv_heads, int head_dim, int block_size,
                      int num_blocks, int max_blocks_per_seq, int max_context_len, float scale,
                      int causal, int dtype, int out_dtype, int partition_tokens,
                      void* workspace, size_t workspace_bytes, pa_stream_t stream) {
  return multiq_core(out, q, k_cache, v_cache, block_tables, context_lens, q_offsets, num_seqs,
                     total_q, max_q_len, num_heads, num_kv_heads, head_dim, block_size,
                     num_blocks, max_blocks_per_seq, max_context_len, scale, causal, dtype,
                     out_dtype, partition_tokens, workspace, workspace_bytes, stream, nullptr,
                     t_events);
}

int paged_kv_gather(void* k_out, void* v_out, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens,
                    const int32_t* token_offsets, int num_seqs, int num_kv_heads, int head_dim,
                    int block_size, int num_blocks, int max_blocks_per_seq, int dtype,
                    pa_stream_t stream) {
  if (num_seqs < 0 || num_kv_heads < 1 || head_dim < 1 || block_size < 1 || num_blocks < 1 ||
      max_blocks_per_seq < 1)
    return PA_ERR_SHAPE;
  if (!kv_dtype_ok(dtype)) return PA_ERR_UNSUPPORTED;
  if ((head_dim * elem_bytes(dtype)) % 16 != 0) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (!k_out || !v_out || !k_cache || !v_cache || !block_tables || !context_lens ||
      !token_offsets)
    return PA_ERR_NULL;
  if (!aligned16(k_out) || !aligned16(v_out) || !aligned16(k_cache) || !aligned16(v_cache))
    return PA_ERR_UNSUPPORTED;
  hipError_t e = pa::launch_gather(k_out, v_out, k_cache, v_cache, block_tables, context_lens,
                                    token_offsets, num_seqs, num_kv_heads, head_dim, block_size,
                                    num_blocks, max_blocks_per_seq, elem_bytes(dtype),
                                    static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"

namespace {

// Workspace of the shared-prefix decode: int32 {q_offsets[2], prefix_len[1],
// tail_lens[S]}, fp32 outputs and log-sum-exps of both parts, then the
// workspaces of the prefix multi-query call and of the tail decode, each
// starting on a 256-byte boundary.
struct CascadeLayout {
  size_t out1 = 0, out2 = 0, lse1 = 0, lse2 = 0, mq = 0, dec = 0, total = 0;
  size_t mq_bytes = 0, dec_bytes = 0;
};

CascadeLayout cascade_layout(int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                             int block_size, int max_context_len, int prefix_blocks) {
  CascadeLayout c;
  const size_t S = (size_t)num_seqs, rows = S * num_heads;
  const int prefix_tokens = prefix_blocks * block_size;
  size_t off = 0;
  c.out1 = off;  off = align256(off + rows * head_dim * sizeof(float));
  c.out2 = off;  off = align256(off + rows * head_dim * sizeof(float));
  c.lse1 = off;  off = align256(off + rows * sizeof(float));
  c.lse2 = off;  off = align256(off + rows * sizeof(float));
  c.mq_bytes = paged_attn_workspace_size(1, num_seqs, num_seqs, num_heads, num_kv_heads,
                                         head_dim, block_size, prefix_tokens, 0);
  c.mq = off;    off = align256(off + c.mq_bytes);
  c.dec_bytes = paged_attn_workspace_size(num_seqs, num_seqs, 1, num_heads, num_kv_heads,
                                          head_dim, block_size, max_context_len - prefix_tokens, 0);
  c.dec = off;   off = align256(off + c.dec_bytes);
  c.total = off;
  return c;
}

}  // namespace

extern "C" {

size_t paged_attn_shared_prefix_workspace_size(int num_seqs, int num_heads, int num_kv_heads,
                                               int head_dim, int block_size, int max_context_len,
                                               int prefix_blocks) {
  if (num_seqs < 0 || num_heads < 1 || num_kv_heads < 1 || head_dim < 1 || block_size < 1 ||
      max_context_len < 0 || prefix_blocks < 0 || num_heads % num_kv_heads)
    return 0;
  if ((int64_t)prefix_blocks * block_size > max_context_len) return 0;
  if (num_seqs == 0) return 0;
  if (prefix_blocks == 0)
    return paged_attn_workspace_size(num_seqs, num_seqs, 1, num_heads, num_kv_heads, head_dim,
                                     block_size, max_context_len, 0);
  return cascade_layout(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                        max_context_len, prefix_blocks).total;
}

int paged_attn_decode_shared_prefix(void* out, const void* q, const void* k_cache,
                                    const void* v_cache, const int32_t* block_tables,
                                    const int32_t* context_lens, int num_seqs, int num_heads,
                                    int num_kv_heads, int head_dim, int block_size,
                                    int num_blocks, int max_blocks_per_seq, int max_context_len,
                                    int prefix_blocks, float scale, int dtype, int out_dtype,
                                    void* workspace, size_t workspace_bytes,
                                    pa_stream_t stream) {
  int rc = check_attn_shapes(num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                             max_blocks_per_seq, max_context_len, dtype, out_dtype, 0, scale);
  if (rc != PA_OK) return rc;
  if (prefix_blocks < 0 || prefix_blocks > max_blocks_per_seq ||
      (int64_t)prefix_blocks * block_size > max_context_len)
    return PA_ERR_SHAPE;
  if (num_seqs == 0) return PA_OK;
  const pa::KernelEvents none{};
  if (prefix_blocks == 0)
    return decode_core(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_heads,
                       num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                       max_context_len, scale, dtype, out_dtype, 0, workspace, workspace_bytes,
                       stream, nullptr, none);
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens) return PA_ERR_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_UNSUPPORTED;
  const CascadeLayout c = cascade_layout(num_seqs, num_heads, num_kv_heads, head_dim, block_size,
                                         max_context_len, prefix_blocks);
  if (!workspace || workspace_bytes < c.total || !aligned16(workspace)) return PA_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  float* o1 = reinterpret_cast<float*>(ws + c.out1);
  float* o2 = reinterpret_cast<float*>(ws + c.out2);
  float* l1 = reinterpret_cast<float*>(ws + c.lse1);
  float* l2 = reinterpret_cast<float*>(ws + c.lse2);
  const int prefix_tokens = prefix_blocks * block_size;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // the shared prefix: every sequence's query as one row of a single sequence
  // over row 0's first blocks, the partition partials left in the workspace
  const int part = resolve_partition(0, 1, num_heads, num_kv_heads, block_size, prefix_tokens,
                                     num_seqs);
  const int n_parts = std::max(1, ceil_div(prefix_tokens, part));
  rc = multiq_core(o1, q, k_cache, v_cache, block_tables, nullptr, nullptr, 1, num_seqs,
                   num_seqs, num_heads, num_kv_heads, head_dim, block_size, num_blocks,
                   max_blocks_per_seq, prefix_tokens, scale, 0, dtype, PA_F32, 0,
                   c.mq_bytes ? ws + c.mq : nullptr, c.mq_bytes, stream, l1, none,
                   /*no_merge=*/1, /*fixed_rows=*/num_seqs);
  if (rc != PA_OK) return rc;
  // each sequence's own tail: its table from entry prefix_blocks on (same row
  // stride), its length less the prefix; with the balanced split the pieces
  // stay in the workspace for the fold
  pa::AttnArgs ta{};
  rc = decode_core(o2, q, k_cache, v_cache, block_tables + prefix_blocks, context_lens, num_seqs,
                   num_heads, num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                   max_context_len - prefix_tokens, scale, dtype, PA_F32, 0,
                   c.dec_bytes ? ws + c.dec : nullptr, c.dec_bytes, stream, l2, none, 1.f, false,
                   prefix_tokens, /*split_no_merge=*/true, &ta);
  if (rc != PA_OK) return rc;
  pa::CascadeFold f{};
  f.out = out;
  f.out_dtype = out_dtype;
  f.num_seqs = num_seqs;
  f.num_heads = num_heads;
  f.num_kv_heads = num_kv_heads;
  f.group = num_heads / num_kv_heads;
  f.context_lens = context_lens;
  f.prefix_tokens = prefix_tokens;
  f.tail_max_len = max_context_len - prefix_tokens;
  f.p_ml = reinterpret_cast<const float*>(ws + c.mq);
  f.p_o = f.p_ml + partial_ml_floats(num_seqs, num_heads, n_parts);
  f.n_parts = n_parts;
  f.o1 = o1;
  f.lse1 = l1;
  f.plan = ta.plan;
  f.t_ml = ta.ws_ml;
  f.t_o = ta.ws_o;
  f.o2 = o2;
  f.lse2 = l2;
  hipError_t e = pa::launch_cascade_fold(f, head_dim, st);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int paged_attn_decode_fp8kv(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens,
                            int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                            int block_size, int num_blocks, int max_blocks_per_seq,
                            int max_context_len, float scale, float k_scale, float v_scale,
                            int out_dtype, int partition_tokens, void* workspace,
                            size_t workspace_bytes, pa_stream_t stream) {
  if (!(std::isfinite(k_scale) && std::isfinite(v_scale)) || !(k_scale > 0.f) ||
      !(v_scale > 0.f))
    return PA_ERR_SHAPE;
  if (out_dtype != PA_F32 && out_dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (num_kv_heads > 0 && num_heads % num_kv_heads == 0 && num_heads / num_kv_heads > 8)
    return PA_ERR_UNSUPPORTED;
  // the tensor scales go into the score scale and the output factor
  const float qk = scale * k_scale;
  if (!std::isfinite(qk)) return PA_ERR_SHAPE;
  return decode_core(out, q, k_cache, v_cache, block_tables, context_lens, num_seqs, num_heads,
                     num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                     max_context_len, qk, PA_FP8_E4M3, out_dtype, partition_tokens, workspace,
                     workspace_bytes, stream, nullptr, t_events, v_scale);
}

int paged_kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                    const int32_t* block_tables, const int32_t* context_lens,
                    const int32_t* q_offsets, int num_seqs, int total_new, int num_kv_heads,
                    int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                    int max_context_len, int dtype, pa_stream_t stream) {
  if (num_seqs < 0 || total_new < 0 || num_kv_heads < 1 || head_dim < 1 || block_size < 1 ||
      num_blocks < 1 || max_blocks_per_seq < 1 || max_context_len < 0)
    return PA_ERR_SHAPE;
  if ((int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size) return PA_ERR_SHAPE;
  if (total_new > 0 && num_seqs == 0) return PA_ERR_SHAPE;
  if (!kv_dtype_ok(dtype)) return PA_ERR_UNSUPPORTED;
  if ((head_dim * elem_bytes(dtype)) % 16 != 0) return PA_ERR_UNSUPPORTED;
  // one thread per 16-byte chunk: the grid must fit a 32-bit workgroup count
  const int64_t chunks = (int64_t)total_new * num_kv_heads * (head_dim * elem_bytes(dtype) / 16);
  if (chunks / 256 >= 0x7fffffff) return PA_ERR_SHAPE;
  if (total_new == 0) return PA_OK;
  if (!k_cache || !v_cache || !k_new || !v_new || !block_tables || !context_lens || !q_offsets)
    return PA_ERR_NULL;
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
    return PA_ERR_UNSUPPORTED;
  hipError_t e = pa::launch_append(k_cache, v_cache, k_new, v_new, block_tables, context_lens,
                                   q_offsets, num_seqs, total_new, num_kv_heads, head_dim,
                                   block_size, num_blocks, max_blocks_per_seq, max_context_len,
                                   elem_bytes(dtype), static_cast<hipStream_t>(stream),
                                   t_events);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int paged_kv_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int num_pairs,
                         int num_kv_heads, int head_dim, int block_size, int num_blocks,
                         int dtype, pa_stream_t stream) {
  if (num_pairs < 0 || num_kv_heads < 1 || head_dim < 1 || block_size < 1 || num_blocks < 1)
    return PA_ERR_SHAPE;
  if (!kv_dtype_ok(dtype)) return PA_ERR_UNSUPPORTED;
  if (((int64_t)num_kv_heads * block_size * head_dim * elem_bytes(dtype)) % 16 != 0)
    return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!k_cache || !v_cache || !pairs) return PA_ERR_NULL;
  if (!aligned16(k_cache) || !aligned16(v_cache)) return PA_ERR_UNSUPPORTED;
  hipError_t e = pa::launch_copy_blocks(k_cache, v_cache, pairs, num_pairs, num_kv_heads,
                                        head_dim, block_size, num_blocks, elem_bytes(dtype),
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int paged_attn_check_inputs(const int32_t* block_tables, const int32_t* context_lens,
                            int num_seqs, int block_size, int num_blocks, int max_blocks_per_seq,
                            int max_context_len, int32_t* bad_count, pa_stream_t stream) {
  if (num_seqs < 0 || block_size < 1 || num_blocks < 1 || max_blocks_per_seq < 1 ||
      max_context_len < 0)
    return PA_ERR_SHAPE;
  if (!bad_count || (num_seqs > 0 && (!block_tables || !context_lens))) return PA_ERR_NULL;
  hipError_t e = pa::launch_check(block_tables, context_lens, num_seqs, block_size, num_blocks,
                                  max_blocks_per_seq, max_context_len, bad_count,
                                  static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int paged_hbm_read(const void* buf, size_t bytes, uint32_t* sink, int workgroups,
                   int nontemporal, pa_stream_t stream) {
  if (bytes == 0) return PA_OK;
  if (!buf || !sink) return PA_ERR_NULL;
  if (bytes % 16 != 0 || !aligned16(buf)) return PA_ERR_UNSUPPORTED;
  if (workgroups < 0 || nontemporal < 0 || nontemporal > 2) return PA_ERR_SHAPE;
  // (the direct-to-LDS mode holds 64 KiB of LDS per workgroup: two per CU)
  if (workgroups == 0) workgroups = device_cus() * (nontemporal == 2 ? 2 : 8);
  hipError_t e = pa::launch_stream_read(buf, bytes, sink, workgroups, nontemporal,
                                        static_cast<hipStream_t>(stream));
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"
