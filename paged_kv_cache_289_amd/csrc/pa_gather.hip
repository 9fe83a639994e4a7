// Block-table walk alone: copy every sequence's K and V out of the paged pool
// into contiguous [tokens][Hk][D] arrays, in logical order (the gather that the
// PagedAttention kernel performs through the per-sequence table of physical
// block ids, "Local_LLM_03_vLLM_Architecture", PagedAttention slide).  Bytes
// are moved unchanged, so the result can be compared bit for bit.
//
// Also the device-side input check: context lengths in [0, max_context_len]
// and table entries in [0, num_blocks) for every block a sequence uses.
#include "pa_common.h"

namespace pa {

// One workgroup per (logical block j, KV head g, sequence s); 16-byte copies.
// Source (block phys, head g) is one contiguous B*D*elem chunk; destination
// rows are token-major with stride Hk*D elements.  A table entry outside
// [0, NB) is never dereferenced: its tokens' rows are written as zeros.
__global__ __launch_bounds__(256) void gather_kernel(
    uint4* __restrict__ k_out, uint4* __restrict__ v_out, const uint4* __restrict__ kc,
    const uint4* __restrict__ vc, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ lens, const int32_t* __restrict__ tok_off, int Hk, int vec_per_row,
    int B, int NB, int mbs) {
  const int j = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int L = min(max(lens[s], 0), mbs * B);
  const int t0 = j * B;
  if (t0 >= L) return;
  const int ntok = min(B, L - t0);
  const int id = tables[(size_t)s * mbs + j];
  const bool valid = id >= 0 && id < NB;
  const size_t src0 = (((size_t)(valid ? id : 0) * Hk + g) * B) * vec_per_row;
  const size_t dst_row0 = (size_t)tok_off[s] + t0;
  for (int i = threadIdx.x; i < ntok * vec_per_row; i += blockDim.x) {
    const int r = i / vec_per_row, c = i % vec_per_row;
    const size_t dst = ((dst_row0 + r) * Hk + g) * vec_per_row + c;
    k_out[dst] = valid ? kc[src0 + i] : make_uint4(0, 0, 0, 0);
    v_out[dst] = valid ? vc[src0 + i] : make_uint4(0, 0, 0, 0);
  }
}

hipError_t launch_gather(void* k_out, void* v_out, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, const int32_t* context_lens,
                         const int32_t* token_offsets, int num_seqs, int num_kv_heads,
                         int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                         int elem_bytes, hipStream_t st) {
  const int vec_per_row = head_dim * elem_bytes / 16;
  dim3 grid(max_blocks_per_seq, num_kv_heads, num_seqs);
  hipLaunchKernelGGL(gather_kernel, grid, dim3(256), 0, st, reinterpret_cast<uint4*>(k_out),
                     reinterpret_cast<uint4*>(v_out), reinterpret_cast<const uint4*>(k_cache),
                     reinterpret_cast<const uint4*>(v_cache), block_tables, context_lens,
                     token_offsets, num_kv_heads, vec_per_row, block_size, num_blocks,
                     max_blocks_per_seq);
  return hipGetLastError();
}

// Single workgroup: every thread counts its share of bad entries, a tree sum
// in LDS totals them, thread 0 writes the count (no atomics, no memset).
__global__ __launch_bounds__(256) void check_kernel(const int32_t* __restrict__ tables,
                                                    const int32_t* __restrict__ lens, int S, int B,
                                                    int NB, int mbs, int max_ctx,
                                                    int32_t* __restrict__ bad) {
  __shared__ int part[256];
  int cnt = 0;
  for (int s = 0; s < S; ++s) {
    const int L = lens[s];
    if (threadIdx.x == 0 && (L < 0 || L > max_ctx)) ++cnt;
    const int used = min(max(L, 0), max_ctx);
    const int nb = min((used + B - 1) / B, mbs);
    for (int j = threadIdx.x; j < nb; j += blockDim.x) {
      const int id = tables[(size_t)s * mbs + j];
      cnt += (id < 0 || id >= NB) ? 1 : 0;
    }
  }
  part[threadIdx.x] = cnt;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *bad = part[0];
}

hipError_t launch_check(const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                        int block_size, int num_blocks, int max_blocks_per_seq,
                        int max_context_len, int32_t* bad_count, hipStream_t st) {
  hipLaunchKernelGGL(check_kernel, dim3(1), dim3(256), 0, st, block_tables, context_lens,
                     num_seqs, block_size, num_blocks, max_blocks_per_seq, max_context_len,
                     bad_count);
  return hipGetLastError();
}

}  // namespace pa
