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

// One workgroup per (sequence, query head), thread d owns dim d.  The prefix
// pass left n_parts partition partials (max m_p, sum l_p, unnormalized o_p, in
// log2 units) when it had several, else its normalized output o1 and lse1 (one
// "partial" with m = lse1, l = 1); the tail pass left its normalized output o2
// and lse2 (a partial with m = lse2, l = 1).  All are folded in one
// log-sum-exp: out = sum 2^(m - M) o / sum 2^(m - M) l.
template <int D>
__global__ __launch_bounds__(D) void cascade_combine_kernel(
    void* __restrict__ out, const float* __restrict__ ws_ml, const float* __restrict__ ws_o,
    int max_parts, int n_parts, const float* __restrict__ o1, const float* __restrict__ lse1,
    const float* __restrict__ o2, const float* __restrict__ lse2, int out_dtype) {
  const int64_t r = (int64_t)blockIdx.x * gridDim.y + blockIdx.y;   // (sequence, head) row
  const int d = threadIdx.x;
  constexpr int kMax = 16;   // partials loaded per round
  float M = lse2[r], num = 0.f, den = 0.f;
  const float t_o = o2[r * D + d];
  if (n_parts <= 1) {
    const float m1 = lse1[r];
    const float mx = fmaxf(M, m1);
    if (mx == kNegInf) {
      store_out(out, r * D + d, 0.f, out_dtype);
      return;
    }
    const float w1 = fast_exp2(m1 - mx), w2 = fast_exp2(M - mx);
    store_out(out, r * D + d, (w1 * o1[r * D + d] + w2 * t_o) / (w1 + w2), out_dtype);
    return;
  }
  // start from the tail's part, then fold the prefix partials in rounds
  const bool tail = M != kNegInf;
  num = tail ? t_o : 0.f;
  den = tail ? 1.f : 0.f;
  const float* ml = ws_ml + 2 * r * max_parts;
  const float* po = ws_o + r * max_parts * D + d;
  for (int p0 = 0; p0 < n_parts; p0 += kMax) {
    float pm[kMax], pl[kMax], pv[kMax];
#pragma unroll
    for (int k = 0; k < kMax; ++k) {
      const int pk = min(p0 + k, n_parts - 1);
      pm[k] = ml[2 * pk];
      pl[k] = ml[2 * pk + 1];
      pv[k] = po[(size_t)pk * D];
    }
    float mx = M;
#pragma unroll
    for (int k = 0; k < kMax; ++k)
      if (p0 + k < n_parts) mx = fmaxf(mx, pm[k]);
    const float ms = (mx == kNegInf) ? 0.f : mx;
    const float rs = fast_exp2(M - ms);
    num *= rs;
    den *= rs;
#pragma unroll
    for (int k = 0; k < kMax; ++k) {
      const float wt = (p0 + k < n_parts) ? fast_exp2(pm[k] - ms) : 0.f;
      num = __builtin_fmaf(wt, pv[k], num);
      den = __builtin_fmaf(wt, pl[k], den);
    }
    M = mx;
  }
  store_out(out, r * D + d, den > 0.f ? num / den : 0.f, out_dtype);
}

hipError_t launch_cascade_prep(const int32_t* context_lens, int num_seqs, int prefix_tokens,
                               int max_context_len, int32_t* q_offsets, int32_t* prefix_len,
                               int32_t* tail_lens, hipStream_t st) {
  const int wgs = (num_seqs + 255) / 256;
  hipLaunchKernelGGL(cascade_prep_kernel, dim3(wgs > 0 ? wgs : 1), dim3(256), 0, st, context_lens,
                     num_seqs, prefix_tokens, max_context_len, q_offsets, prefix_len, tail_lens);
  return hipGetLastError();
}

hipError_t launch_cascade_combine(void* out, const float* ws_ml, const float* ws_o, int max_parts,
                                  int n_parts, const float* o1, const float* lse1, const float* o2,
                                  const float* lse2, int num_seqs, int num_heads, int head_dim,
                                  int out_dtype, hipStream_t st) {
  const dim3 grid(num_seqs, num_heads);
  if (head_dim == 64)
    hipLaunchKernelGGL(cascade_combine_kernel<64>, grid, dim3(64), 0, st, out, ws_ml, ws_o,
                       max_parts, n_parts, o1, lse1, o2, lse2, out_dtype);
  else
    hipLaunchKernelGGL(cascade_combine_kernel<128>, grid, dim3(128), 0, st, out, ws_ml, ws_o,
                       max_parts, n_parts, o1, lse1, o2, lse2, out_dtype);
  return hipGetLastError();
}

}  // namespace pa
