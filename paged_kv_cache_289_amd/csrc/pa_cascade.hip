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
// is read once per group of rows instead of once per sequence.  Both parts
// leave unnormalized partials (max, sum, o) where they split the work, and one
// fold below takes all of them at once.
#include "pa_common.h"

namespace pa {

// Thread c owns 4 consecutive dims of one (sequence, query head) row, so a
// 256-thread workgroup covers 1,024 of a sequence's H * D outputs.  Every
// part is a triple (m, l, o): a partial's max (log2 units), sum and
// unnormalized output, or a normalized output o with m = its log-sum-exp and
// l = 1.  out = sum 2^(m - M) o / sum 2^(m - M) l over the prefix partials and
// the tail's pieces.  The prefix partials are loaded first (they need nothing
// else); the tail's plan and length alongside them; then its pieces.
template <int D>
__global__ __launch_bounds__(256) void cascade_fold_kernel(const CascadeFold f) {
  constexpr int kChunks = D / 4;
  constexpr int kBatch = 8;
  const int H = f.num_heads, Hk = f.num_kv_heads, G = f.group;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= H * kChunks) return;
  const int hq = c / kChunks, d0 = (c % kChunks) * 4;
  const int s = blockIdx.y;
  const int g = hq / G, h = hq - g * G;
  const size_t r = (size_t)s * H + hq;

  float M = kNegInf, den = 0.f;
  float num[4] = {0.f, 0.f, 0.f, 0.f};
  // fold up to kBatch parts (entries k < n count)
  auto fold = [&](int n, const float (&pm)[kBatch], const float (&pl)[kBatch],
                  const float4 (&pv)[kBatch]) {
    float mx = M;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      if (k >= n) break;
      mx = fmaxf(mx, pm[k]);
    }
    const float ms = (mx == kNegInf) ? 0.f : mx;
    const float rs = fast_exp2(M - ms);
    den *= rs;
#pragma unroll
    for (int e = 0; e < 4; ++e) num[e] *= rs;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      if (k >= n) break;   // (entries past n may be unset)
      const float wt = fast_exp2(pm[k] - ms);
      num[0] = __builtin_fmaf(wt, pv[k].x, num[0]);
      num[1] = __builtin_fmaf(wt, pv[k].y, num[1]);
      num[2] = __builtin_fmaf(wt, pv[k].z, num[2]);
      num[3] = __builtin_fmaf(wt, pv[k].w, num[3]);
      den = __builtin_fmaf(wt, pl[k], den);
    }
    M = mx;
  };

  // the tail's length and plan (independent of the prefix loads below)
  const int Lraw = as_const(f.context_lens)[s];
  const int Lt = min(max(Lraw - f.prefix_tokens, 0), f.tail_max_len);
  int chunk = 1, p0 = 0, p1 = 0;
  if (f.plan) {
    const ConstI32Ptr plan = as_const(f.plan);
    chunk = plan[0];
    p0 = plan[2 + s];
    p1 = plan[3 + s];
  }

  // the prefix part
  if (f.n_parts <= 1) {
    float pm[kBatch], pl[kBatch];
    float4 pv[kBatch];
    pm[0] = f.lse1[r];
    pl[0] = 1.f;
    pv[0] = *reinterpret_cast<const float4*>(f.o1 + r * D + d0);
    fold(1, pm, pl, pv);
  } else {
    const float* ml = f.p_ml + 2 * r * f.n_parts;
    const float* po = f.p_o + r * f.n_parts * D + d0;
    for (int q0 = 0; q0 < f.n_parts; q0 += kBatch) {
      float pm[kBatch], pl[kBatch];
      float4 pv[kBatch];
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const int pk = min(q0 + k, f.n_parts - 1);
        pm[k] = ml[2 * pk];
        pl[k] = ml[2 * pk + 1];
        pv[k] = *reinterpret_cast<const float4*>(po + (size_t)pk * D);
      }
      fold(f.n_parts - q0, pm, pl, pv);
    }
  }

  // the tail part
  if (Lt > 0) {
    const int c = p1 - p0;   // (s, g)'s items: its own cost, then its blocks
    const int a0 = Hk * p0 + g * c;
    const int w0 = f.plan ? (a0 + kSegItems) / chunk : 0, w1 = f.plan ? (a0 + c - 1) / chunk : 0;
    if (w0 == w1) {   // written as a normalized output with its log-sum-exp
      float pm[kBatch], pl[kBatch];
      float4 pv[kBatch];
      pm[0] = f.lse2[r];
      pl[0] = 1.f;
      pv[0] = *reinterpret_cast<const float4*>(f.o2 + r * D + d0);
      fold(1, pm, pl, pv);
    } else {          // wave w left its piece in slot (s Hk + g + w) G + h
      const size_t base = (size_t)s * Hk + g;
      for (int w = w0; w <= w1; w += kBatch) {
        float pm[kBatch], pl[kBatch];
        float4 pv[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          const size_t sl = (base + min(w + k, w1)) * G + h;
          pm[k] = f.t_ml[2 * sl];
          pl[k] = f.t_ml[2 * sl + 1];
          pv[k] = *reinterpret_cast<const float4*>(f.t_o + sl * D + d0);
        }
        fold(w1 + 1 - w, pm, pl, pv);
      }
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const size_t oidx = r * D + d0;
#pragma unroll
  for (int e = 0; e < 4; ++e) store_out(f.out, oidx + e, num[e] * inv, f.out_dtype);
}

hipError_t launch_cascade_fold(const CascadeFold& f, int head_dim, hipStream_t st) {
  const int chunks = f.num_heads * head_dim / 4;
  const dim3 grid((chunks + 255) / 256, f.num_seqs);
  if (head_dim == 64)
    hipLaunchKernelGGL(cascade_fold_kernel<64>, grid, dim3(256), 0, st, f);
  else
    hipLaunchKernelGGL(cascade_fold_kernel<128>, grid, dim3(256), 0, st, f);
  return hipGetLastError();
}

}  // namespace pa
