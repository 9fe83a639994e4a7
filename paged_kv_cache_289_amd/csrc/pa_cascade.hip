// Decode over a shared prefix in two passes.  When every block table starts
// with the same physical blocks (requests with a common start share those
// pages, "Scaling inference with vLLM", prefix-sharing paragraph;
// "Local_LLM_03_vLLM_Architecture", prefix-caching slide), attention over a
// sequence's keys splits into the shared prefix and its own tail.  Softmax over
// the union is the log-sum-exp combination of the two parts:
//   out = (2^lse1 o1 + 2^lse2 o2) / (2^lse1 + 2^lse2)
// with o1, o2 the normalized outputs over each part and lse1, lse2 (log2
// units) their log-sum-exps.  The prefix part is one multi-query call in which
// the S decode queries are S rows over the same keys, so each prefix K/V tile
// is read once per group of rows instead of once per sequence.
#include "pa_common.h"

namespace pa {

// q_offsets {0, S} and length {P B} of the prefix call; tail length of every
// sequence.  One thread per sequence.
__global__ __launch_bounds__(256) void cascade_prep_kernel(const int32_t* __restrict__ lens, int S,
                                                           int prefix_tokens, int max_ctx,
                                                           int32_t* __restrict__ qoff,
                                                           int32_t* __restrict__ plen,
                                                           int32_t* __restrict__ tail) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) {
    qoff[0] = 0;
    qoff[1] = S;
    plen[0] = prefix_tokens;
  }
  if (i < S) {
    const int L = min(max(lens[i], 0), max_ctx);
    tail[i] = max(L - prefix_tokens, 0);
  }
}

// One thread per output element: the log-sum-exp combination of the two parts.
__global__ __launch_bounds__(256) void cascade_combine_kernel(
    void* __restrict__ out, const float* __restrict__ o1, const float* __restrict__ lse1,
    const float* __restrict__ o2, const float* __restrict__ lse2, int64_t n, int D,
    int out_dtype) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int64_t r = i / D;
  const float a = lse1[r], b = lse2[r];
  const float M = fmaxf(a, b);
  if (M == kNegInf) {
    store_out(out, i, 0.f, out_dtype);
    return;
  }
  const float w1 = fast_exp2(a - M), w2 = fast_exp2(b - M);
  store_out(out, i, (w1 * o1[i] + w2 * o2[i]) / (w1 + w2), out_dtype);
}

hipError_t launch_cascade_prep(const int32_t* context_lens, int num_seqs, int prefix_tokens,
                               int max_context_len, int32_t* q_offsets, int32_t* prefix_len,
                               int32_t* tail_lens, hipStream_t st) {
  const int wgs = (num_seqs + 255) / 256;
  hipLaunchKernelGGL(cascade_prep_kernel, dim3(wgs > 0 ? wgs : 1), dim3(256), 0, st, context_lens,
                     num_seqs, prefix_tokens, max_context_len, q_offsets, prefix_len, tail_lens);
  return hipGetLastError();
}

hipError_t launch_cascade_combine(void* out, const float* o1, const float* lse1, const float* o2,
                                  const float* lse2, int64_t rows, int head_dim, int out_dtype,
                                  hipStream_t st) {
  const int64_t n = rows * head_dim;
  hipLaunchKernelGGL(cascade_combine_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     out, o1, lse1, o2, lse2, n, head_dim, out_dtype);
  return hipGetLastError();
}

}  // namespace pa
