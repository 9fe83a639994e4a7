/*
 * paged_attn.h -- C ABI of libpagedattn.so, paged attention for MI355X (gfx950).
 *
 * What the library computes.  The KV cache of every sequence is cut into
 * fixed-size blocks (16 tokens by default) that sit anywhere in one shared
 * physical pool; a per-sequence block table maps logical positions to physical
 * blocks, and the attention kernel gathers K/V from the scattered blocks
 * through it ("Local_LLM_03_vLLM_Architecture", PagedAttention slide; "vLLM:
 * LLM Inference That Doesn't Waste Your GPU", section "PagedAttention: virtual
 * memory for KV").  Each query token attends over every prior cached token
 * ("Local_LLM_03_vLLM_Architecture", KV-cache slide).  Several sequences may
 * point at the same physical blocks for a shared prompt prefix ("Scaling
 * inference with vLLM", prefix-sharing paragraph); K/V are only read, so that
 * aliasing is always allowed.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All array pointers are DEVICE pointers owned by the caller.  The library
 *    allocates nothing, keeps no pointer after return, and never synchronizes:
 *    work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *    The device work of a call is kernel launches only (no memory sets or
 *    copies; any plan is computed on the device), so a call may be captured
 *    into a HIP graph, its output and workspace given, and replayed: every
 *    replay gives the same bytes as the call made directly.  The first call
 *    on a device (made outside a capture) fills the library's per-device
 *    caches (compute units, occupancies, the allocation-free scratch address).
 *  - Element counts are in elements, byte counts in bytes.
 *  - Pool layout: k_cache and v_cache are separate, contiguous
 *        [num_blocks][num_kv_heads][block_size][head_dim]
 *    arrays.  Token t of sequence s lives in physical block
 *    block_tables[s * max_blocks_per_seq + t / block_size], slot t % block_size.
 *    block_tables is int32 [num_seqs][max_blocks_per_seq], row-major; only the
 *    first ceil(context_lens[s] / block_size) entries of row s are read.
 *  - context_lens[s] (int32, device) counts every key the queries of s may
 *    see, including the query tokens' own K/V, which the caller has already
 *    written into the pool.  Values <= 0 give zero output rows.
 *  - Grouped-query attention: query head h reads KV head h / (num_heads /
 *    num_kv_heads) (contiguous groups).
 *  - Scores are scale * <q, k>; softmax accumulates in fp32.
 *  - Scalar arguments are validated on the host before any HIP call; a bad
 *    argument returns a negative pa_status and enqueues nothing.  Device
 *    contents are trusted: context_lens[s] must not exceed max_context_len and
 *    every table entry that is read must be in [0, num_blocks).
 *    paged_attn_check_inputs() verifies both on the device when in doubt.
 *  - Supported: dtype in {PA_F32, PA_F16, PA_BF16} (q, k_cache, v_cache share
 *    it); out_dtype PA_F32 or equal to dtype; head_dim in {64, 128};
 *    block_size in {8, 16, 32}; num_heads % num_kv_heads == 0 with
 *    num_heads / num_kv_heads <= 16.  Anything else: PA_ERR_UNSUPPORTED.
 *  - Thread safety: every entry point may be called from several host threads
 *    at once.  Global state: per-device caches of device properties (filled
 *    once, atomically), and the profiling events of
 *    paged_attn_set_kernel_events, which are per host thread.
 */
#ifndef PAGED_ATTN_H
#define PAGED_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL                       */
  PA_ERR_SHAPE = -2,       /* inconsistent or negative sizes                   */
  PA_ERR_UNSUPPORTED = -3, /* dtype / head_dim / block_size / group not built  */
  PA_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required       */
  PA_ERR_HIP = -5,         /* a HIP launch or runtime call failed              */
  PA_ERR_NO_BLOCKS = -6,   /* the block pool has too few free blocks           */
  PA_ERR_INVALID = -7,     /* unknown or released sequence id, bad block id    */
  PA_ERR_SCRATCH = -8      /* more scratch than paged_attn_decode_noalloc has  */
} pa_status;

/* PA_FP8_E4M3: 8-bit floating-point codes (sign, 4 exponent bits with bias 7,
   3 mantissa bits, no infinities; the all-ones magnitude is NaN): the K/V pools
   of paged_attn_decode_fp8kv, and a valid dtype for the entry points that only
   move cache bytes (paged_kv_gather, paged_kv_append, paged_kv_copy_blocks). */
typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2, PA_FP8_E4M3 = 3 } pa_dtype;

/* Opaque to this header; it is a hipStream_t. */
typedef void* pa_stream_t;

/*
 * Bytes of device workspace that paged_attn_decode (total_q == num_seqs,
 * max_q_len == 1) or paged_attn_multiq needs for these shapes when called
 * with the same partition_tokens (0 = the library's choice).  The workspace
 * holds the work plan and the fp32 (max, sum, unnormalized output) partials of
 * the context pieces that the log-sum-exp merge combines; its contents need no
 * initialization and are overwritten by every call (so calls that may run
 * concurrently need separate workspaces).  0 is a legal answer (no merge
 * needed; only for multi-token calls whose contexts fit one partition).
 * Returns 0 as well for arguments the entry points would reject.
 */
size_t paged_attn_workspace_size(int num_seqs, int total_q, int max_q_len, int num_heads,
                                 int num_kv_heads, int head_dim, int block_size,
                                 int max_context_len, int partition_tokens);

/*
 * Decode step: one query token per sequence.
 *   out  [num_seqs][num_heads][head_dim]  (out_dtype)
 *   q    [num_seqs][num_heads][head_dim]  (dtype)
 * For each (s, h): out = sum_t softmax_t(scale * <q, k_t>) v_t over the
 * context_lens[s] keys of KV head h / G of sequence s, gathered through the
 * block table (the decode step's attention over every prior token,
 * "Local_LLM_03_vLLM_Architecture", KV-cache and PagedAttention slides).
 * The (sequence, KV head, block) items are cut into equal pieces, one per
 * resident wave; pieces of one context are merged by log-sum-exp in a second
 * kernel.  partition_tokens = 0 lets the library size the pieces; a positive
 * multiple of block_size fixes each piece at that many tokens.  Batches of
 * more than 8192 sequences use fixed context partitions instead.  With
 * partition_tokens 0 at head_dim 128 (bf16, f16, and the 8-bit cache of
 * paged_attn_decode_fp8kv; up to 16384 (sequence, KV head) pairs) the items are
 * 32-token tiles and the products run on the matrix cores (fp32 accumulation;
 * P is carried to about 2^-16 in bf16 and rounded to f16 in f16); otherwise
 * the products run on the vector ALUs in fp32.  The two agree to within that
 * rounding, not bit for bit; a given call always takes the same one.
 */
int paged_attn_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens,
                      int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                      int block_size, int num_blocks, int max_blocks_per_seq,
                      int max_context_len, float scale, int dtype, int out_dtype,
                      int partition_tokens, void* workspace, size_t workspace_bytes,
                      pa_stream_t stream);

/*
 * paged_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, result and kernels as
 * paged_attn_decode; the work plan and partials go to a scratch array of
 * 32 MiB that the library holds in device memory, one per GPU, until the
 * process ends.  The call allocates nothing.  A call that would need more
 * scratch than that (the need depends on the batch, the heads and the device's
 * resident waves; the Llama-3-8B/70B decode layers use under 14 MiB) returns
 * PA_ERR_SCRATCH and enqueues nothing.  Every call on a GPU uses that GPU's one
 * array and nothing in it needs to start at any value, but calls whose work may
 * overlap on one GPU (several streams, several host threads) race on it and
 * must be serialized by the caller.
 */
int paged_attn_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                              int block_size, int num_blocks, int max_blocks_per_seq,
                              int max_context_len, float scale, int dtype, int out_dtype,
                              int partition_tokens, pa_stream_t stream);

/*
 * Several query tokens per sequence: the k guessed tokens that speculative
 * decoding verifies in one pass ("Scaling inference with vLLM", speculative
 * decoding paragraph) or a chunk of a prompt processed as one prefill batch
 * ("Local_LLM_03_vLLM_Architecture", chunked-prefill slide).
 *   out  [total_q][num_heads][head_dim]  (out_dtype)
 *   q    [total_q][num_heads][head_dim]  (dtype)
 *   q_offsets  int32 [num_seqs + 1], device: rows of sequence s are
 *              q_offsets[s] .. q_offsets[s+1]-1, q_offsets[0] == 0,
 *              q_offsets[num_seqs] == total_q, n_s = q_offsets[s+1]-q_offsets[s]
 *              <= max_q_len.
 * The n_s rows are the last n_s positions of the context.  With causal != 0,
 * row i of s sees keys t <= context_lens[s] - n_s + i (requires
 * context_lens[s] >= n_s); with causal == 0 every row sees all keys.
 * The contraction runs on bf16/fp16 MFMA with fp32 accumulation (dtype PA_F32
 * runs a vector-ALU path).  Other conventions as paged_attn_decode.
 * Work split: with partition_tokens 0, bf16/f16 calls at head_dim 128 whose
 * rows fit in at most three 32-row tiles per KV head (max_q_len * num_heads /
 * num_kv_heads <= 96, max_q_len >= 2) cut the (sequence, KV head, row tile,
 * 32-key tile) list into equal chunks, one per resident wave, and merge the
 * pieces of a (sequence, KV head, row tile) that several waves share
 * (paged_attn_multiq_uses_split says which calls do); other calls use fixed
 * context partitions of partition_tokens (0: paged_attn_default_partition).
 */
int paged_attn_multiq(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens,
                      const int32_t* q_offsets, int num_seqs, int total_q, int max_q_len,
                      int num_heads, int num_kv_heads, int head_dim, int block_size,
                      int num_blocks, int max_blocks_per_seq, int max_context_len, float scale,
                      int causal, int dtype, int out_dtype, int partition_tokens,
                      void* workspace, size_t workspace_bytes, pa_stream_t stream);

/*
 * Block-table walk alone: copy each sequence's K and V, in logical order, out
 * of the paged pool into contiguous arrays (the gather that the attention
 * kernels fuse; "Local_LLM_03_vLLM_Architecture", PagedAttention slide).
 *   k_out, v_out   [token_offsets[num_seqs]][num_kv_heads][head_dim] (dtype)
 *   token_offsets  int32 [num_seqs + 1], device; token t of sequence s goes
 *                  to row token_offsets[s] + t; token_offsets[s+1] -
 *                  token_offsets[s] must equal context_lens[s].
 * Bytes are copied unchanged (bit-exact).  A table entry that is read and lies
 * outside [0, num_blocks) is never dereferenced: the rows of its tokens are
 * written as zeros.
 */
int paged_kv_gather(void* k_out, void* v_out, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* context_lens,
                    const int32_t* token_offsets, int num_seqs, int num_kv_heads, int head_dim,
                    int block_size, int num_blocks, int max_blocks_per_seq, int dtype,
                    pa_stream_t stream);

/*
 * Device-side check of the contents the attention entry points trust:
 * counts sequences whose context_lens[s] is negative or above
 * max_context_len, and table entries among the first
 * ceil(context_lens[s] / block_size) of each row that fall outside
 * [0, num_blocks).  Writes the count (int32) to *bad_count (device); it is
 * zero when the inputs are safe to pass to the attention entry points.
 */
int paged_attn_check_inputs(const int32_t* block_tables, const int32_t* context_lens,
                            int num_seqs, int block_size, int num_blocks, int max_blocks_per_seq,
                            int max_context_len, int32_t* bad_count, pa_stream_t stream);

/*
 * Profiling aid.  With both arguments non-NULL (hipEvent_t handles), every
 * later paged_attn_decode / paged_attn_multiq / paged_kv_append call made from
 * this host thread
 * launches its main kernel with hipExtLaunchKernel, which stamps `start` and
 * `stop` with that dispatch's own start and end on the call's stream (a
 * partition merge, if any, runs after `stop`), so the elapsed time between
 * them is that kernel's duration.  NULL, NULL turns it off.  The
 * events are caller-owned and must outlive the calls that record them.
 * Returns PA_ERR_NULL if exactly one argument is NULL.
 */
int paged_attn_set_kernel_events(void* start, void* stop);

/* Partition length (tokens) that the library picks when partition_tokens is 0
   for multi-token queries that do not take the balanced split, or for decode
   batches above 8192 sequences (other decode calls use the balanced split and
   no fixed partition). */
int paged_attn_default_partition(int num_seqs, int num_heads, int num_kv_heads, int block_size,
                                 int max_context_len, int max_q_len);

/* 1 if paged_attn_multiq with these sizes, dtype and partition_tokens splits
   its work evenly over the resident waves (the balanced split described at
   paged_attn_multiq), 0 if it uses fixed context partitions.  Host-only. */
int paged_attn_multiq_uses_split(int num_seqs, int max_q_len, int num_heads, int num_kv_heads,
                                 int head_dim, int dtype, int partition_tokens);

/*
 * Decode over a shared prefix.  Same result as paged_attn_decode (same
 * arguments and conventions), for calls whose block tables all start with the
 * same prefix_blocks physical blocks -- requests with a common start that
 * share its pages ("Scaling inference with vLLM", prefix-sharing paragraph;
 * "Local_LLM_03_vLLM_Architecture", prefix-caching slide) -- and whose
 * context_lens are all at least prefix_blocks * block_size.  Those are
 * preconditions, not checked on the device; outside them the result is
 * undefined.
 *
 * The prefix is attended once for all sequences: one multi-query pass treats
 * the num_seqs decode queries as num_seqs rows over the shared keys (matrix
 * cores, each prefix K/V tile read once per group of rows), a decode pass
 * covers each sequence's own tail (its table from entry prefix_blocks on),
 * and a last kernel combines the two normalized parts by their log-sum-exps.
 * prefix_blocks == 0 is a plain decode.
 *
 * workspace: device, at least paged_attn_shared_prefix_workspace_size(...)
 * bytes, 16-byte aligned, no initialization needed.  Errors as for
 * paged_attn_decode, plus PA_ERR_SHAPE for prefix_blocks < 0, beyond
 * max_blocks_per_seq, or covering more than max_context_len tokens.
 */
size_t paged_attn_shared_prefix_workspace_size(int num_seqs, int num_heads, int num_kv_heads,
                                               int head_dim, int block_size, int max_context_len,
                                               int prefix_blocks);
int paged_attn_decode_shared_prefix(void* out, const void* q, const void* k_cache,
                                    const void* v_cache, const int32_t* block_tables,
                                    const int32_t* context_lens, int num_seqs, int num_heads,
                                    int num_kv_heads, int head_dim, int block_size,
                                    int num_blocks, int max_blocks_per_seq, int max_context_len,
                                    int prefix_blocks, float scale, int dtype, int out_dtype,
                                    void* workspace, size_t workspace_bytes, pa_stream_t stream);

/*
 * Decode over an 8-bit KV cache.  The same call as paged_attn_decode, with
 * k_cache and v_cache holding PA_FP8_E4M3 codes (1 byte per element, the same
 * [num_blocks][num_kv_heads][block_size][head_dim] layout) and one scale per
 * tensor: the keys are k_scale * (decoded code) and the values v_scale *
 * (decoded code).  Half the K/V bytes of a 16-bit cache.  The pages apply
 * "fewer bits, faster memory access" to weights ("Scaling inference with
 * vLLM", quantization paragraph); here it is applied to the cache the decode
 * streams.
 *
 * q is bf16 [num_seqs][num_heads][head_dim] (converted to f16 in the kernel:
 * exact for |q| in f16's normal range); out_dtype is PA_F32 or PA_BF16.
 * Accumulation is fp32.  Codes are widened exactly; the NaN codes are not
 * supported.  Supported: head_dim 64 and 128 with block_size 8/16/32,
 * groups num_heads / num_kv_heads of at most 8.
 * partition_tokens, the workspace (paged_attn_workspace_size(...) for the same
 * shapes and partition_tokens) and the errors are as for paged_attn_decode,
 * plus PA_ERR_SHAPE for k_scale or v_scale not finite and positive.
 */
int paged_attn_decode_fp8kv(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* context_lens,
                            int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                            int block_size, int num_blocks, int max_blocks_per_seq,
                            int max_context_len, float scale, float k_scale, float v_scale,
                            int out_dtype, int partition_tokens, void* workspace,
                            size_t workspace_bytes, pa_stream_t stream);

/* Static description of a status code. */
const char* paged_attn_status_string(int status);

/* ------------------------------------------------------------------------
 * Filling and sharing the cache
 * ------------------------------------------------------------------------ */

/*
 * Writes the K and V of new tokens into their slots of the pool.  Each decode
 * step adds the new tokens' K/V to the cache that later steps read ("vLLM:
 * LLM Inference That Doesn't Waste Your GPU", section "KV cache, in one
 * picture"), at the slot its position maps to through the block table
 * ("Local_LLM_03_vLLM_Architecture", PagedAttention slide).
 *
 * k_new, v_new: DEVICE [total_new][num_kv_heads][head_dim], dtype.  The new
 * tokens of sequence s are rows q_offsets[s] .. q_offsets[s+1]-1 (int32
 * [num_seqs+1], device, non-decreasing, q_offsets[num_seqs] == total_new).
 * With the attention calls' convention, context_lens[s] already counts them,
 * so new token i of s goes to position t = context_lens[s] - n_s + i, i.e.
 * block block_tables[s][t / block_size], slot t % block_size, every KV head.
 * Bytes are copied unchanged.  Call it before the attention call that reads
 * the new tokens, on the same stream.  Tokens whose position falls outside
 * [0, max_context_len) or whose table entry is outside [0, num_blocks) are
 * skipped (nothing is written out of bounds).  Slots written by two new
 * tokens at once (tables that alias a block being written) are a caller
 * error: the pool below never lets a sequence write into a shared block.
 * Errors: PA_ERR_NULL, PA_ERR_SHAPE (negative sizes, max_context_len beyond
 * max_blocks_per_seq * block_size, total_new > 0 with num_seqs == 0),
 * PA_ERR_UNSUPPORTED (dtype, or a row not a multiple of 16 bytes, or
 * pointers not 16-byte aligned), PA_ERR_HIP.
 */
int paged_kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                    const int32_t* block_tables, const int32_t* context_lens,
                    const int32_t* q_offsets, int num_seqs, int total_new, int num_kv_heads,
                    int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                    int max_context_len, int dtype, pa_stream_t stream);

/*
 * Copies whole blocks of both pools: for p < num_pairs, block pairs[2p+1]
 * receives what block pairs[2p] holds (every KV head and slot of K and of V).
 * pairs is DEVICE int32 [num_pairs][2]; destinations must be distinct and
 * never a source.  This is the device half of copy-on-write: run the pairs
 * that paged_seq_append returns before paged_kv_append writes the new tokens.
 * Pairs with an id outside [0, num_blocks) are skipped.  Errors as for
 * paged_kv_append.
 */
int paged_kv_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int num_pairs,
                         int num_kv_heads, int head_dim, int block_size, int num_blocks,
                         int dtype, pa_stream_t stream);

/*
 * Host-side block pool: the allocator that hands out the physical blocks the
 * tables point at.  A sequence of L tokens holds ceil(L / block_size) blocks,
 * so it wastes fewer than block_size slots ("Scaling inference with vLLM",
 * paging paragraph; "vLLM: LLM Inference That Doesn't Waste Your GPU",
 * section "PagedAttention: virtual memory for KV").  A fork shares all of
 * the parent's blocks instead of copying them ("Scaling inference with vLLM",
 * prefix-sharing paragraph); every block counts the tables that hold it and
 * returns to the free list when none does.
 *
 * Everything here is HOST memory and host work (no HIP call).  Sequence ids
 * are small non-negative ints; a released id may be handed out again.  Each
 * call takes the pool's mutex, so a pool may be shared between threads.
 *
 * paged_pool_create returns NULL for num_blocks < 1, block_size < 1 or when
 * out of host memory.  The int-returning calls return a negative pa_status
 * on error: PA_ERR_NULL for a NULL pool (or output pointer), PA_ERR_INVALID
 * for an unknown or released sequence id or a block id outside the pool.
 *
 * paged_seq_append grows a sequence by num_tokens (>= 0) and allocates the
 * blocks they need.  If the sequence's last block is partially filled and
 * also held by another table, the sequence first gets a fresh copy of it
 * (copy-on-write): the (source, destination) pair is written to copy_pairs
 * (host int32, room for max_pairs pairs; at most one pair per call) and
 * *num_pairs says how many; the caller copies them on the device with
 * paged_kv_copy_blocks before writing the new tokens.  All or nothing:
 * PA_ERR_NO_BLOCKS (too few free blocks) and PA_ERR_SHAPE (num_tokens < 0,
 * or a copy is needed and max_pairs < 1) leave the pool unchanged.
 *
 * paged_seq_blocks writes the sequence's block ids, in logical order, to
 * out (host, room for max_blocks entries) and returns how many; PA_ERR_SHAPE
 * if max_blocks is too small.  Those ids are the sequence's block-table row.
 */
typedef struct paged_block_pool paged_block_pool;
paged_block_pool* paged_pool_create(int num_blocks, int block_size);
void paged_pool_destroy(paged_block_pool* pool);
int paged_pool_num_free(const paged_block_pool* pool);
int paged_pool_refcount(const paged_block_pool* pool, int block);
int paged_seq_create(paged_block_pool* pool);
int paged_seq_fork(paged_block_pool* pool, int parent);
int paged_seq_release(paged_block_pool* pool, int seq);
int paged_seq_append(paged_block_pool* pool, int seq, int num_tokens, int32_t* copy_pairs,
                     int max_pairs, int* num_pairs);
int paged_seq_length(const paged_block_pool* pool, int seq);
int paged_seq_blocks(const paged_block_pool* pool, int seq, int32_t* out, int max_blocks);

/*
 * Prefix caching on the pool.  The pages' server hashes each page's token
 * content, so that requests with the same first N tokens share N / block_size
 * physical pages and skip recomputing them ("Local_LLM_03_vLLM_Architecture",
 * prefix-caching slide; "vLLM: LLM Inference That Doesn't Waste Your GPU",
 * section "Prefix caching").
 *
 * paged_seq_commit registers the full blocks among the sequence's first
 * num_tokens tokens (host int32 token ids, the sequence's own tokens from its
 * start; num_tokens <= its length; call it once their K/V are written).  A
 * token prefix that is already registered keeps its block.  Returns how many
 * blocks were newly registered.
 *
 * paged_seq_match_prefix gives an EMPTY sequence (length 0, else
 * PA_ERR_INVALID) every leading full block registered under exactly the same
 * token prefix as tokens[0 .. num_tokens): the blocks join its table (their
 * reference counts go up) and its length becomes the returned number of
 * tokens, a multiple of block_size.  Their K/V are already in the pool; the
 * caller appends and computes only the rest.  Hits are verified against the
 * stored tokens and parent block, so a hash collision never shares a block.
 * A block leaves the cache when it returns to the free list.
 */
int paged_seq_commit(paged_block_pool* pool, int seq, const int32_t* tokens, int num_tokens);
int paged_seq_match_prefix(paged_block_pool* pool, int seq, const int32_t* tokens,
                           int num_tokens);

/*
 * Measurement aid, not part of the attention path: one plain streaming read of
 * `bytes` bytes (a multiple of 16) at `buf` (16-byte aligned) by `workgroups`
 * workgroups of 256 threads.  `nontemporal` selects the pattern: 0, 16-byte
 * vectors in a grid-stride loop (0 workgroups = eight per compute unit); 1, the
 * same with the non-temporal hint; 2, each wave its own contiguous share in
 * 8 KiB steps by direct-to-LDS loads with the non-temporal hint, two stages per
 * wave (0 workgroups = two per compute unit; the bytes past the waves' shares in
 * a grid-stride loop).  Other values give PA_ERR_SHAPE.  It gives the HBM read
 * rate this device sustains, the practical ceiling to set the paged kernels'
 * bandwidth figures against.  `sink` (one uint32, device) is written only by a
 * data-dependent branch that keeps the loads live; its value means nothing.
 * Errors as for the other entry points.
 */
int paged_hbm_read(const void* buf, size_t bytes, uint32_t* sink, int workgroups,
                   int nontemporal, pa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_ATTN_H */
