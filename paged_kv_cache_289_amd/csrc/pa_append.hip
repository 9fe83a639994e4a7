// Filling the paged cache: the K/V of new tokens go into the slots their
// positions map to through the block table (token t of a sequence sits in
// block table[t / B], slot t % B, "Local_LLM_03_vLLM_Architecture",
// PagedAttention slide; each decode step adds the new token's K/V to the cache
// that later steps reuse, "vLLM: LLM Inference That Doesn't Waste Your GPU",
// section "KV cache, in one picture").  And whole-block copies, which give a
// sequence its own copy of a block that other tables share before it writes
// into it.  Bytes are moved unchanged.
#include <algorithm>

#include "pa_common.h"

namespace pa {

// One wave per new token: its Hk rows of cpr 16-byte chunks are contiguous in
// the new K/V ([token][Hk][cpr]), so lane l takes chunks l, l + 64, ... of
// the token.  The first P chunks of K and of V per lane (P full passes of
// the wave, chosen by the launcher so that they are all in range) are loaded
// before anything else, without conditions, since their addresses depend on
// the token only; the token's sequence and slot are found meanwhile, once per
// wave (a binary search over q_offsets, in scalar loads), and the stores
// follow.  New token i of sequence s (rows q_offsets[s] .. q_offsets[s+1]-1)
// takes position L_s - n_s + i, L_s = context_lens[s] counting the new
// tokens.  Positions outside [0, max_context_len), table entries past
// max_blocks_per_seq and block ids outside [0, num_blocks) are skipped, never
// written; all of these are per token.
template <int P>
__global__ __launch_bounds__(256, 8) void append_kernel(
    uint4* __restrict__ kc, uint4* __restrict__ vc, const uint4* __restrict__ kn,
    const uint4* __restrict__ vn, const int32_t* __restrict__ tables,
    const int32_t* __restrict__ lens, const int32_t* __restrict__ qoff, int S, int total_new,
    int Hk, int cpr, int B, int NB, int mbs, int max_ctx) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  const int tok = __builtin_amdgcn_readfirstlane((int)blockIdx.x * (256 / 64) + (int)(threadIdx.x >> 6));
  if (tok >= total_new) return;
  const int nch = Hk * cpr;   // >= 64 P
  // the token's rows: wave-uniform bases, 32-bit per-lane offsets
  const u32x4* ksrc = reinterpret_cast<const u32x4*>(kn) + (size_t)tok * nch;
  const u32x4* vsrc = reinterpret_cast<const u32x4*>(vn) + (size_t)tok * nch;
  u32x4 kb[P > 0 ? P : 1], vb[P > 0 ? P : 1];
#pragma unroll
  for (int u = 0; u < P; ++u) {
    kb[u] = ksrc[lane + 64 * u];
    vb[u] = vsrc[lane + 64 * u];
  }
  // the sequence of the token: the last s with q_offsets[s] <= tok
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (qoff[mid] <= tok) lo = mid;
    else hi = mid - 1;
  }
  const int q0 = qoff[lo], n = qoff[lo + 1] - q0;
  if (tok < q0 || tok >= q0 + n) return;          // offsets that do not cover the token
  const int64_t t = (int64_t)lens[lo] - n + (tok - q0);
  if (t < 0 || t >= max_ctx) return;
  const int j = (int)(t / B);
  if (j >= mbs) return;
  const int phys = tables[(size_t)lo * mbs + j];
  if (phys < 0 || phys >= NB) return;
  // chunk c = g cpr + cc of the token goes to row (phys, g, t mod B), chunk cc
  const size_t dst0 = ((size_t)phys * Hk * B + (size_t)(t % B)) * cpr;
  u32x4* kdst = reinterpret_cast<u32x4*>(kc) + dst0;
  u32x4* vdst = reinterpret_cast<u32x4*>(vc) + dst0;
  const unsigned head_stride = (unsigned)(B * cpr);
  auto off_of = [&](int c) { return (unsigned)(c / cpr) * head_stride + (unsigned)(c % cpr); };
#pragma unroll
  for (int u = 0; u < P; ++u) {
    const unsigned o = off_of(lane + 64 * u);
    kdst[o] = kb[u];
    vdst[o] = vb[u];
  }
  for (int c = lane + 64 * P; c < nch; c += 64) {   // the rest of the token's chunks
    const unsigned o = off_of(c);
    kdst[o] = ksrc[c];
    vdst[o] = vsrc[c];
  }
}

hipError_t launch_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                         const int32_t* block_tables, const int32_t* context_lens,
                         const int32_t* q_offsets, int num_seqs, int total_new, int num_kv_heads,
                         int head_dim, int block_size, int num_blocks, int max_blocks_per_seq,
                         int max_context_len, int elem_bytes, hipStream_t st,
                         const KernelEvents& ev) {
  int cpr = head_dim * elem_bytes / 16;
  const dim3 grid((unsigned)(((int64_t)total_new + 3) / 4));   // four tokens per workgroup
  uint4* kc = reinterpret_cast<uint4*>(k_cache);
  uint4* vc = reinterpret_cast<uint4*>(v_cache);
  const uint4* kn = reinterpret_cast<const uint4*>(k_new);
  const uint4* vn = reinterpret_cast<const uint4*>(v_new);
  // full passes of a wave over a token's chunks issued up front
  const int full = num_kv_heads * cpr / 64;
  const void* fn = full >= 4   ? reinterpret_cast<const void*>(append_kernel<4>)
                   : full >= 2 ? reinterpret_cast<const void*>(append_kernel<2>)
                   : full >= 1 ? reinterpret_cast<const void*>(append_kernel<1>)
                               : reinterpret_cast<const void*>(append_kernel<0>);
  void* args[] = {&kc, &vc, &kn, &vn, &block_tables, &context_lens, &q_offsets, &num_seqs,
                  &total_new, &num_kv_heads, &cpr, &block_size, &num_blocks,
                  &max_blocks_per_seq, &max_context_len};
  if (ev.start || ev.stop)   // profiling: events stamped by the dispatch itself
    return hipExtLaunchKernel(fn, grid, dim3(256), args, 0, st, ev.start, ev.stop, 0);
  const hipError_t e = hipLaunchKernel(fn, grid, dim3(256), args, 0, st);
  return e != hipSuccess ? e : hipGetLastError();
}

// Workgroups (x, p): pair p = blockIdx.y + k gridDim.y copies block src into
// block dst, every KV head and slot of K and of V; x strides over the block's
// 16-byte vectors.  Pairs with an id outside [0, num_blocks) are skipped.
// Destinations are distinct and never a source (the caller's contract), so
// the copies do not depend on each other.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint4* __restrict__ kc,
                                                          uint4* __restrict__ vc,
                                                          const int32_t* __restrict__ pairs,
                                                          int n, int64_t vec_per_block, int NB) {
  for (int p = blockIdx.y; p < n; p += gridDim.y) {
    const int src = pairs[2 * p], dst = pairs[2 * p + 1];
    if (src < 0 || src >= NB || dst < 0 || dst >= NB) continue;
    const size_t s0 = (size_t)src * vec_per_block, d0 = (size_t)dst * vec_per_block;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < vec_per_block;
         i += (int64_t)gridDim.x * blockDim.x) {
      kc[d0 + i] = kc[s0 + i];
      vc[d0 + i] = vc[s0 + i];
    }
  }
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int num_pairs,
                              int num_kv_heads, int head_dim, int block_size, int num_blocks,
                              int elem_bytes, hipStream_t st) {
  const int64_t vpb = (int64_t)num_kv_heads * block_size * head_dim * elem_bytes / 16;
  const int64_t per_pair = std::min<int64_t>((vpb + 255) / 256, 64);
  dim3 grid((unsigned)per_pair, (unsigned)std::min(num_pairs, 65535));
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(256), 0, st,
                     reinterpret_cast<uint4*>(k_cache), reinterpret_cast<uint4*>(v_cache), pairs,
                     num_pairs, vpb, num_blocks);
  return hipGetLastError();
}

}  // namespace pa
