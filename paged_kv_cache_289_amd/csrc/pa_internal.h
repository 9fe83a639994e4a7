// Internal interface between the C-ABI host layer (pa_api.cpp) and the kernel
// translation units.  Every launcher enqueues on the given stream and returns
// the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "paged_attn.h"

namespace pa {

// Threads per workgroup of the attention kernels (four wave64s).
#ifndef PA_WAVES
#define PA_WAVES 4
#endif
constexpr int kWaves = PA_WAVES;
constexpr int kThreads = 64 * kWaves;

// Multi-token queries: a workgroup takes four 32-row tiles of one (sequence,
// KV head) over the same K/V tiles when a sequence can have that many rows
// (n * G > 96); otherwise it takes one row tile and splits the tokens.
inline bool multiq_rows_mode(int max_q_len, int group) {
  return (max_q_len * group + 31) / 32 >= kWaves;
}

// Balanced-split decode: most sequences per call it handles (their prefix sums
// live in LDS), and most waves it launches (the workspace is sized for this).
constexpr int kMaxSplitSeqs = 8192;
constexpr int kMaxSplitWaves = 8192;
// The split prices every (sequence, KV head) segment at its blocks plus this
// many items: a wave that starts a segment loads its query and waits for its
// first block with nothing else in flight, and stores its result at the end.
#ifndef PA_SEG_ITEMS
#define PA_SEG_ITEMS 4
#endif
constexpr int kSegItems = PA_SEG_ITEMS;
// Balanced-split multi-query calls (few query rows per KV head, head_dim
// 128): the fixed cost per (sequence, KV head, row tile) in 32-token tiles, the
// most waves launched and the most units (sequence x KV head x row tile) they
// take (the workspace holds a 32-row piece per unit and per wave).
// It is larger for an 8-bit cache, whose key tiles take half the bytes (and so
// less time) of a 16-bit one against the same fixed cost; kMqSegItemsMax bounds
// it for the host's sizing.
constexpr int mq_seg_items(int kv_dtype) { return kv_dtype == PA_FP8_E4M3 ? 4 : 2; }
constexpr int kMqSegItemsMax = 4;
constexpr int kMqMaxSplitWaves = 4096;
constexpr int kMqMaxSplitUnits = 16384;

// Arguments of the decode / multi-query partial kernels and of the merge.
struct AttnArgs {
  void* out;                 // [rows][H][D], out_dtype
  float* ws_ml;              // [rows][H][P_max][2] (running max in log2 units, sum)
  float* ws_o;               // [rows][H][P_max][D] unnormalized partial outputs
  const void* q;             // [rows][H][D]
  const void* k_cache;       // [NB][Hk][B][D]
  const void* v_cache;
  const int32_t* block_tables;  // [S][mbs]
  const int32_t* context_lens;  // [S]
  const int32_t* q_offsets;     // [S+1] (multi-query only)
  int num_seqs;              // S
  int num_heads;             // H
  int num_kv_heads;          // Hk
  int group;                 // G = H / Hk
  int max_blocks_per_seq;    // mbs
  int pool_blocks;           // physical blocks in the K/V pools
  int max_context_len;
  int part;                  // partition length in tokens (multiple of B)
  int max_parts;             // P_max = ceil(max_context_len / part)
  int max_q_len;
  int causal;
  int out_dtype;
  float scale_log2;          // scale * log2(e): scores are kept in log2 units
  float out_scale;           // factor on every final output (1, or the V scale of 8-bit caches)
  // balanced split, decode or multi-query (plan != nullptr)
  int* plan;                 // [2 + S + 1]: chunk, total items, item prefix sums
  // optional: per (row, query head) log-sum-exp of the scores in log2 units,
  // m + log2(l) (-inf for a row with no visible key), written with the output
  float* lse;
  int chunk_blocks;          // items per wave (0: split evenly over the launch)
  int split_workgroups;      // workgroups launched
  // leave the partials in the workspace for the caller's own merge instead of
  // launching merge_kernel (multi-token calls) or split_merge_kernel (decode)
  int no_merge;
  // subtracted from every context length before it is clamped to
  // [0, max_context_len] (the tails of a shared-prefix decode)
  int len_offset;
  // > 0: one sequence whose query rows are 0 .. fixed_rows - 1 and whose
  // length is max_context_len; q_offsets and context_lens are not read (the
  // prefix pass of a shared-prefix decode)
  int fixed_rows;
};

// Optional events recorded right around a call's main kernel (profiling aid).
struct KernelEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

hipError_t launch_decode(int dtype, int head_dim, int block_size, int group, int num_seqs,
                         const AttnArgs& a, hipStream_t stream, const KernelEvents& ev);

// Resident workgroups per CU of the split decode kernel for this configuration.
int split_workgroups_per_cu(int dtype, int head_dim, int block_size, int group);
int multiq_split_workgroups_per_cu(int dtype, int block_size);
// decode at head_dim 128 (bf16, f16 or 8-bit K/V) through the multi-query
// balanced-split kernel on the matrix cores, and its merge
hipError_t launch_split_decode(int dtype, int block_size, int num_seqs, const AttnArgs& a,
                               hipStream_t st, const KernelEvents& ev);

hipError_t launch_multiq(int dtype, int head_dim, int block_size, int group, int num_seqs,
                         const AttnArgs& a, hipStream_t stream, const KernelEvents& ev);

hipError_t launch_gather(void* k_out, void* v_out, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens,
                         const int32_t* token_offsets, int num_seqs, int num_kv_heads,
                         int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                         int elem_bytes, hipStream_t stream);

hipError_t launch_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                         const int32_t* block_tables, const int32_t* context_lens,
                         const int32_t* q_offsets, int num_seqs, int total_new, int num_kv_heads,
                         int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                         int max_context_len, int elem_bytes, hipStream_t stream,
                         const KernelEvents& ev);

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int num_pairs,
                              int num_kv_heads, int head_dim, int block_size, int num_blocks,
                              int elem_bytes, hipStream_t stream);

// Final rows of the shared-prefix decode: the prefix pass's n_parts partition
// partials (or, with one partition, its normalized output o1 and lse1) and the
// tail pass's output -- with the balanced split (plan != nullptr), the pieces
// it left in its workspace, or o2 and lse2 for a (sequence, KV head) that one
// wave covered; otherwise o2 and lse2 -- combined by log-sum-exp.
struct CascadeFold {
  void* out;
  int out_dtype, num_seqs, num_heads, num_kv_heads, group;
  const int32_t* context_lens;
  int prefix_tokens, tail_max_len;
  const float *p_ml, *p_o;   // prefix partials [rows][H][n_parts][2], [..][D]
  int n_parts;
  const float *o1, *lse1;
  const int* plan;           // tail split plan, or nullptr
  const float *t_ml, *t_o;   // tail pieces
  const float *o2, *lse2;
};
hipError_t launch_cascade_fold(const CascadeFold& f, int head_dim, hipStream_t stream);

// mode 0: grid-stride, cached loads; 1: grid-stride, non-temporal; 2: each
// wave its own contiguous share through direct-to-LDS loads (non-temporal)
hipError_t launch_stream_read(const void* buf, size_t bytes, unsigned* sink, int workgroups,
                              int mode, hipStream_t stream);

// Device scratch of the allocation-free decode entry point: kScratchBytes in
// a file-scope device array, one copy per GPU (pa_noalloc.hip).  Returns the
// current device's copy, looked up once per device.
constexpr size_t kScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;
hipError_t scratch_buffer(void** ptr);

hipError_t launch_check(const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                        int block_size, int num_blocks, int max_blocks_per_seq,
                        int max_context_len, int32_t* bad_count, hipStream_t stream);

}  // namespace pa
