// Paged decode attention for gfx950: one query token per sequence.
//
// The cache is read through each sequence's block table of physical block ids
// (the PagedAttention kernel that gathers K/V from scattered blocks,
// "Local_LLM_03_vLLM_Architecture", PagedAttention slide).  One workgroup owns
// one (partition of the context, KV head, sequence); all G query heads of the
// KV head's group are served from the same K/V bytes (GQA-8 in the slide's
// KV sizing), so every K/V byte is read from HBM once.
//
// Lane layout (wave64).  A token's head_dim row of one KV head is D*elem
// bytes; LPT = D*elem/16 lanes hold it as one 16-byte vector each, and a wave
// covers TPL = 64/LPT tokens per load instruction.  A B-token block of one KV
// head is contiguous (B*D*elem bytes), so each load instruction reads
// TPL*D*elem contiguous bytes: full 128-byte lines, no over-fetch.
//
// Per block: QK partial dots (bf16/f16 dot2, fp32 FMA for f32) on the lane's
// 16 bytes, a DPP all-reduce over the LPT lanes of the token, online softmax in
// base 2 (scores pre-multiplied by scale*log2 e), and PV accumulated in fp32 on
// the same lanes, which already hold that token's V dims.  The next block's
// K/V loads are issued before the current block is computed.
//
// Epilogue: the TPL token rows of a wave, then the four waves, are merged by
// log-sum-exp; a sequence whose context fits one partition writes the final
// output, otherwise the partition's (max, sum, unnormalized output) goes to
// the workspace and merge_kernel combines the partitions.
#include <type_traits>

#include "pa_common.h"

namespace pa {

#ifndef PA_NBUF
#define PA_NBUF 2
#endif
constexpr int NBUF = PA_NBUF;   // register ring depth: blocks in flight per wave + 1

template <int D>
__device__ inline void merge_rows(const AttnArgs& a, size_t row, int g, int n_parts);

template <int DT, int D, int B, int GP>
__global__ __launch_bounds__(kThreads) void decode_partial_kernel(const AttnArgs a) {
  using E = Elem<DT>;
  constexpr int EPL = E::kPerVec;   // elements per lane per token
  constexpr int LPT = D / EPL;      // lanes per token row
  constexpr int TPL = 64 / LPT;     // token rows per wave
  constexpr int LPB = B / TPL;      // vector loads per block per tensor per lane
  static_assert(LPT * EPL == D && TPL * LPT == 64 && LPB * TPL == B, "layout");

  const int p = blockIdx.x, g = blockIdx.y;
  const int H = a.num_heads, G = a.group;
  // Decode: blockIdx.z is the sequence and its one query row.  Per-row mode
  // (multi-token queries without MFMA): blockIdx.z = s * max_q_len + i is row i
  // of sequence s, which sees the first L_s - n_s + i + 1 keys when causal.
  int s = blockIdx.z, qrow = blockIdx.z;
  int L = min(max(a.context_lens[s], 0), a.max_context_len);
  if (a.q_offsets) {
    s = blockIdx.z / a.max_q_len;
    const int i = blockIdx.z % a.max_q_len;
    const int q0 = a.q_offsets[s], n = a.q_offsets[s + 1] - q0;
    if (i >= n) return;
    qrow = q0 + i;
    L = min(max(a.context_lens[s], 0), a.max_context_len);
    if (a.causal) L = max(0, min(L, L - n + i + 1));
  }
  const int n_parts = (L + a.part - 1) / a.part;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
  const int row = lane / LPT, col = lane % LPT;
  const size_t head0 = (size_t)qrow * H + (size_t)g * G;   // first query head of the group

  if (n_parts == 0) {  // empty context: zero output rows, written by partition 0
    if (p == 0)
      for (int i = tid; i < G * D; i += kThreads) store_out(a.out, head0 * D + i, 0.f, a.out_dtype);
    return;
  }
  if (p >= n_parts) return;

  // query vectors of the group (zero for padded heads h >= G)
  uint4 qv[GP];
  const uint4* qsrc = reinterpret_cast<const uint4*>(a.q);
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    if (h < G) qv[h] = qsrc[((head0 + h) * D) / EPL + col];
    else qv[h] = make_uint4(0, 0, 0, 0);
  }

  float m[GP], l[GP], o[GP][EPL];
#pragma unroll
  for (int h = 0; h < GP; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[h][e] = 0.f;
  }

  const int tok0 = p * a.part;
  const int tok_end = min(tok0 + a.part, L);
  const int blk_end = (tok_end + B - 1) / B;
  const int32_t* tbl = a.block_tables + (size_t)s * a.max_blocks_per_seq;
  const uint4* kc = reinterpret_cast<const uint4*>(a.k_cache);
  const uint4* vc = reinterpret_cast<const uint4*>(a.v_cache);
  // vector index of (block phys, head g, row 0, col) and the stride between
  // the TPL-token groups of a block
  constexpr int kVecPerBlockHead = B * D / EPL;
  const size_t lane_off = (size_t)row * (D / EPL) + col;
  const size_t head_off = (size_t)g * kVecPerBlockHead;
  const size_t blk_stride = (size_t)a.num_kv_heads * kVecPerBlockHead;

  // A ring of NBUF register buffers per wave: while block j is computed, the
  // loads of blocks j + kWaves .. j + (NBUF-1) kWaves are in flight, and the
  // block id needed by the next issue is fetched one step ahead.  The ring is
  // rotated by a fully unrolled loop, so every buffer index is a compile-time
  // constant (registers, never scratch).
  //
  // Loads are raw buffer loads: the (block, KV head) slice base is built in
  // SGPRs from the block id, each lane adds a fixed offset, and no load sits
  // under a branch, so the compiler can wait for exactly the buffer it needs.
  // A block past the wave's range gets a zero-size descriptor: its loads
  // return zeros without touching memory.
  //
  // In the last block of a sequence the slots at or beyond L may hold anything
  // (stale or poisoned data).  There every lane's slot is clamped to the last
  // valid one, so only real tokens are ever loaded, and the scores of the
  // clamped duplicates are set to -inf: they get weight exactly 0.
  constexpr int kRowBytes = D * E::kBytes;
  constexpr int kSliceBytes = B * kRowBytes;   // one (block, KV head) slice
  const size_t blk_bytes = (size_t)a.num_kv_heads * kSliceBytes;
  const char* kbase = static_cast<const char*>(a.k_cache) + (size_t)g * kSliceBytes;
  const char* vbase = static_cast<const char*>(a.v_cache) + (size_t)g * kSliceBytes;
  uint4 kbuf[NBUF][LPB], vbuf[NBUF][LPB];
  auto load_block = [&](int jj, int phys, bool in_range, uint4 (&kr)[LPB], uint4 (&vr)[LPB]) {
    const int last = min(B - 1, L - 1 - jj * B);   // last valid slot (wave-uniform)
    const int nrec = in_range ? kSliceBytes : 0;
    const size_t boff = (size_t)phys * blk_bytes;
    const BufRsrc rk = make_rsrc(kbase + boff, nrec);
    const BufRsrc rv = make_rsrc(vbase + boff, nrec);
    int voff[LPB];
#pragma unroll
    for (int i = 0; i < LPB; ++i) voff[i] = min(i * TPL + row, last) * kRowBytes + col * 16;
    // keep the issue order K then V, and keep both ahead of the compute that
    // follows, so each wait covers exactly the buffer being consumed
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < LPB; ++i) kr[i] = buffer_load16(rk, voff[i]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < LPB; ++i) vr[i] = buffer_load16(rv, voff[i]);
    __builtin_amdgcn_sched_barrier(0);
  };

  auto compute_block = [&](int jj, const uint4 (&kr)[LPB], const uint4 (&vr)[LPB]) {
    // QK: partial dot on the lane's 16 bytes, all-reduce over the token's lanes
    float sc[LPB][GP];
#pragma unroll
    for (int i = 0; i < LPB; ++i)
#pragma unroll
      for (int h = 0; h < GP; ++h)
        sc[i][h] = group_sum<LPT>(E::dot(qv[h], kr[i], 0.f)) * a.scale_log2;
    if ((jj + 1) * B > L) {   // wave-uniform: only the last block of the sequence
#pragma unroll
      for (int i = 0; i < LPB; ++i) {
        const bool valid = jj * B + i * TPL + row < L;
#pragma unroll
        for (int h = 0; h < GP; ++h) sc[i][h] = valid ? sc[i][h] : kNegInf;
      }
    }
    // online softmax in base 2
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      float mx = m[h];
#pragma unroll
      for (int i = 0; i < LPB; ++i) mx = fmaxf(mx, sc[i][h]);
      const float ms = (mx == kNegInf) ? 0.f : mx;
      const float alpha = fast_exp2(m[h] - ms);
      m[h] = mx;
      sc[0][h] = fast_exp2(sc[0][h] - ms);
      float psum = sc[0][h];
#pragma unroll
      for (int i = 1; i < LPB; ++i) {
        sc[i][h] = fast_exp2(sc[i][h] - ms);
        psum += sc[i][h];
      }
      l[h] = __builtin_fmaf(l[h], alpha, psum);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] *= alpha;
    }
    // PV: each V element is widened once and used for all GP heads
#pragma unroll
    for (int i = 0; i < LPB; ++i) {
      float vf[EPL];
      E::to_float(vr[i], vf);
#pragma unroll
      for (int e = 0; e < EPL; ++e)
#pragma unroll
        for (int h = 0; h < GP; ++h) o[h][e] = __builtin_fmaf(sc[i][h], vf[e], o[h][e]);
    }
  };

  // blocks of this wave: j, j + kWaves, j + 2 kWaves, ... < blk_end
  int j = tok0 / B + wave;
  const int jmax = blk_end - 1;   // table reads are clamped here (always in bounds)
#pragma unroll
  for (int b = 0; b + 1 < NBUF; ++b) {
    const int jb = j + b * kWaves;
    load_block(jb, tbl[min(jb, jmax)], jb < blk_end, kbuf[b], vbuf[b]);
  }
  constexpr int kAhead = (NBUF - 1) * kWaves;   // distance of the block issued next
  int id_next = tbl[min(j + kAhead, jmax)];
  bool done = j >= blk_end;
  while (!done) {
#pragma unroll
    for (int u = 0; u < NBUF; ++u) {
      const int jn = j + kAhead;
      const int id_after = tbl[min(jn + kWaves, jmax)];
      load_block(jn, id_next, jn < blk_end, kbuf[(u + NBUF - 1) % NBUF],
                 vbuf[(u + NBUF - 1) % NBUF]);
      compute_block(j, kbuf[u], vbuf[u]);
      id_next = id_after;
      j += kWaves;
      if (j >= blk_end) {
        done = true;
        break;
      }
    }
  }

  // merge the TPL token rows of the wave (lanes col, col+LPT, ...)
#pragma unroll
  for (int off = LPT; off < 64; off <<= 1) {
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      const float m2 = __shfl_xor(m[h], off, 64);
      const float l2 = __shfl_xor(l[h], off, 64);
      const float mx = fmaxf(m[h], m2);
      const float ms = (mx == kNegInf) ? 0.f : mx;
      const float a1 = fast_exp2(m[h] - ms), a2 = fast_exp2(m2 - ms);
      l[h] = l[h] * a1 + l2 * a2;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] = o[h][e] * a1 + __shfl_xor(o[h][e], off, 64) * a2;
      m[h] = mx;
    }
  }

  // merge the waves through LDS
  __shared__ float sm_o[kWaves][GP][D];
  __shared__ float sm_m[kWaves][GP], sm_l[kWaves][GP];
  if (row == 0) {
#pragma unroll
    for (int h = 0; h < GP; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_o[wave][h][col * EPL + e] = o[h][e];
      if (col == 0) {
        sm_m[wave][h] = m[h];
        sm_l[wave][h] = l[h];
      }
    }
  }
  __syncthreads();

  const bool final_out = (n_parts == 1);
  for (int i = tid; i < G * D; i += kThreads) {
    const int h = i / D, d = i % D;
    float mx = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, sm_m[w][h]);
    const float ms = (mx == kNegInf) ? 0.f : mx;
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = fast_exp2(sm_m[w][h] - ms);
      num = __builtin_fmaf(wt, sm_o[w][h][d], num);
      den = __builtin_fmaf(wt, sm_l[w][h], den);
    }
    const size_t hh = head0 + h;
    if (final_out) {
      store_out(a.out, hh * D + d, den > 0.f ? num / den : 0.f, a.out_dtype);
    } else {
      const size_t slot = hh * a.max_parts + p;
      a.ws_o[slot * D + d] = num;
      if (d == 0) {
        a.ws_ml[2 * slot] = mx;
        a.ws_ml[2 * slot + 1] = den;
      }
    }
  }
}

// Log-sum-exp merge of the partitions of one (row, KV-head group):
// M = max_p m_p, out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
// The loads of different partitions are independent, so the loops are unrolled
// to keep several in flight.
template <int D>
__device__ inline void merge_rows(const AttnArgs& a, size_t row, int g, int n_parts) {
  const int H = a.num_heads, G = a.group;
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
    const int h = i / D, d = i % D;
    const size_t hh = row * H + (size_t)g * G + h;
    const float* ml = a.ws_ml + 2 * hh * a.max_parts;
    const float* po = a.ws_o + hh * a.max_parts * D + d;
    float mx = kNegInf;
#pragma unroll 8
    for (int p = 0; p < n_parts; ++p) mx = fmaxf(mx, ml[2 * p]);
    const float ms = (mx == kNegInf) ? 0.f : mx;
    float num = 0.f, den = 0.f;
#pragma unroll 8
    for (int p = 0; p < n_parts; ++p) {
      const float wt = fast_exp2(ml[2 * p] - ms);
      num = __builtin_fmaf(wt, po[(size_t)p * D], num);
      den = __builtin_fmaf(wt, ml[2 * p + 1], den);
    }
    store_out(a.out, hh * D + d, den > 0.f ? num / den : 0.f, a.out_dtype);
  }
}

// Separate merge launch.  Rows with a single partition were finished by the
// partial kernel.
template <int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(const AttnArgs a) {
  const int g = blockIdx.y, s = blockIdx.z;
  size_t row = s;
  int L = min(max(a.context_lens[s], 0), a.max_context_len);
  if (a.q_offsets) {  // multi-token queries: blockIdx.x = row within the sequence
    const int q0 = a.q_offsets[s], n = a.q_offsets[s + 1] - q0;
    const int i = blockIdx.x;
    if (i >= n) return;
    row = (size_t)q0 + i;
    if (a.causal) L = max(0, min(L, L - n + i + 1));
  }
  const int n_parts = (L + a.part - 1) / a.part;
  if (n_parts <= 1) return;
  merge_rows<D>(a, row, g, n_parts);
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
// Merge launch shared with the multi-query kernel (rows = query tokens).
hipError_t launch_merge(int head_dim, int num_seqs, const AttnArgs& a, hipStream_t st) {
  dim3 mgrid(a.q_offsets ? a.max_q_len : 1, a.num_kv_heads, num_seqs);
  if (head_dim == 64)
    hipLaunchKernelGGL((merge_kernel<64>), mgrid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((merge_kernel<128>), mgrid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <int DT, int D, int B, int GP>
static hipError_t launch_decode_t(int num_seqs, const AttnArgs& a, hipStream_t st,
                                  const KernelEvents& ev) {
  // per-row mode launches one grid row per (sequence, query row) slot
  const int rows = a.q_offsets ? num_seqs * a.max_q_len : num_seqs;
  dim3 grid(a.max_parts, a.num_kv_heads, rows);
  if (ev.start) hipEventRecord(ev.start, st);
  hipLaunchKernelGGL((decode_partial_kernel<DT, D, B, GP>), grid, dim3(kThreads), 0, st, a);
  hipError_t e = hipGetLastError();
  if (ev.stop) hipEventRecord(ev.stop, st);
  if (e != hipSuccess || a.max_parts <= 1) return e;
  return launch_merge(D, num_seqs, a, st);
}

template <int DT, int D, int B>
static hipError_t dispatch_g(int group, int num_seqs, const AttnArgs& a, hipStream_t st,
                             const KernelEvents& ev) {
  if (group <= 1) return launch_decode_t<DT, D, B, 1>(num_seqs, a, st, ev);
  if (group <= 2) return launch_decode_t<DT, D, B, 2>(num_seqs, a, st, ev);
  if (group <= 4) return launch_decode_t<DT, D, B, 4>(num_seqs, a, st, ev);
  if (group <= 8) return launch_decode_t<DT, D, B, 8>(num_seqs, a, st, ev);
  return launch_decode_t<DT, D, B, 16>(num_seqs, a, st, ev);
}

template <int DT, int D>
static hipError_t dispatch_b(int block_size, int group, int num_seqs, const AttnArgs& a,
                             hipStream_t st, const KernelEvents& ev) {
  switch (block_size) {
    case 8: return dispatch_g<DT, D, 8>(group, num_seqs, a, st, ev);
    case 16: return dispatch_g<DT, D, 16>(group, num_seqs, a, st, ev);
    default: return dispatch_g<DT, D, 32>(group, num_seqs, a, st, ev);
  }
}

template <int DT>
static hipError_t dispatch_d(int head_dim, int block_size, int group, int num_seqs,
                             const AttnArgs& a, hipStream_t st, const KernelEvents& ev) {
  if (head_dim == 64) return dispatch_b<DT, 64>(block_size, group, num_seqs, a, st, ev);
  return dispatch_b<DT, 128>(block_size, group, num_seqs, a, st, ev);
}

hipError_t launch_decode(int dtype, int head_dim, int block_size, int group, int num_seqs,
                         const AttnArgs& a, hipStream_t st, const KernelEvents& ev) {
  switch (dtype) {
    case PA_F32: return dispatch_d<PA_F32>(head_dim, block_size, group, num_seqs, a, st, ev);
    case PA_F16: return dispatch_d<PA_F16>(head_dim, block_size, group, num_seqs, a, st, ev);
    default: return dispatch_d<PA_BF16>(head_dim, block_size, group, num_seqs, a, st, ev);
  }
}

}  // namespace pa
