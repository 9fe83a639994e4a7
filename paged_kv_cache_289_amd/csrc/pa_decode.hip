// Paged decode attention for gfx950: one query token per sequence.
//
// The cache is read through each sequence's block table of physical block ids
// (the PagedAttention kernel that gathers K/V from scattered blocks,
// "Local_LLM_03_vLLM_Architecture", PagedAttention slide).  All G query heads of
// a KV head's group are served from the same K/V bytes (GQA-8 in the slide's
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
// base 2 (the scale times log2 e is applied inside the exponent's FMA), and PV
// accumulated in fp32 on the same lanes, which already hold that token's V dims.
//
// Lazy rescaling.  The running max m only moves when a score exceeds it by
// more than kRescaleLog2 (log2 units); otherwise the block's weights are taken
// against the stale m, so they are at most 2^kRescaleLog2 and the o / l
// rescale is skipped.  After the first block of a run that is nearly every
// block.  o and l always refer to the stored m, so partials and merges are
// unchanged.  m starts at a finite sentinel, which keeps rows without any
// valid token free of inf - inf.
//
// Two ways to cut the work into waves:
//  * split (decode default): every (sequence, KV head, block) item, with a
//    fixed cost item per (sequence, KV head), is numbered in one list and each
//    resident wave takes an equal contiguous chunk, so all waves finish
//    together whatever the mix of context lengths.  A chunk that
//    covers a whole (sequence, KV head) writes the output; pieces of a longer
//    one write (max, sum, unnormalized output) partials that split_merge_kernel
//    combines by log-sum-exp.
//  * partitions (multi-token fp32 rows, very large batches): one workgroup per
//    (context partition, KV head, row); its four waves interleave the
//    partition's blocks and merge through LDS; merge_kernel combines
//    partitions.
#include <atomic>
#include <type_traits>

#include "pa_common.h"

namespace pa {

#ifndef PA_NBUF
#define PA_NBUF 2
#endif
constexpr int NBUF = PA_NBUF;   // register ring depth: blocks in flight per wave + 1

// Positive exponent scale for scale_log2 (the sign goes into q, 0 into a tiny
// value that leaves every weight at exactly 1).
__device__ inline float exp_scale(float scale_log2) {
  return fmaxf(fabsf(scale_log2), 1e-30f);
}

// ---------------------------------------------------------------------------
// one wave's walk over some blocks of one (row, KV head)
// ---------------------------------------------------------------------------
template <int DT, int D, int B, int GP>
struct DecodeWave {
  using E = Elem<DT>;
  using Vec = typename E::Vec;             // a lane's vector of one token row
  static constexpr int EPL = E::kPerVec;   // elements per lane per token
  static constexpr int LPT = D / EPL;      // lanes per token row
  static constexpr int TPL = 64 / LPT;     // token rows per wave
  static constexpr int LPB = B / TPL;      // vector loads per block per tensor per lane
  static constexpr int kRowBytes = D * E::kBytes;
  static constexpr int kSliceBytes = B * kRowBytes;   // one (block, KV head) slice
  static_assert(LPT * EPL == D && TPL * LPT == 64 && LPB * TPL == B, "layout");

  // Weights computed once per row.  When a token row is one 16-lane DPP row,
  // all 16 lanes of the row hold the same LPB x GP scores after the
  // all-reduce.  Lane c then evaluates only scores c, c + 16, ... (whose head
  // is c % GP, as GP divides 16) and the row's weights are broadcast back for
  // PV.  Each lane keeps the running sum of its own weights (l_lane) against
  // the max of its head (m_lane); the per-head sums are gathered at the end.
  static constexpr bool kOwnExp = (LPT == 16);
  static constexpr int kScores = LPB * GP;
  static constexpr int kScoresPerLane = (kScores + 15) / 16;
  // With a multiple of 16 scores, the 16 lanes of a row reduce-scatter them
  // instead: each exchange step halves the values a lane carries, and lane c
  // ends with exactly the sums it evaluates (scores c, c + 16, ...), with no
  // selection afterwards.
  static constexpr bool kScatter = kOwnExp && kScores % 16 == 0;

  int row, col;                 // token row within a load, 16-byte column
  typename E::QVec qv[GP];
  float m[GP], l[GP], o[GP][EPL];
  float m_lane, l_lane;         // kOwnExp: this lane's head (col % GP)

  __device__ explicit DecodeWave(int lane) : row(lane / LPT), col(lane % LPT) {}

  // query vectors of heads head0 .. head0 + G - 1 (zero for padded heads),
  // sign-flipped when the scale is negative (exact in every storage type)
  __device__ void load_q(const void* q, size_t head0, int G, float scale_log2) {
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      qv[h] = (h < G) ? E::load_q(q, (head0 + h) * D + (size_t)col * EPL) : E::zero_q();
      if (scale_log2 < 0.f) E::flip_q(qv[h]);
    }
  }

  __device__ void reset() {
#pragma unroll
    for (int h = 0; h < GP; ++h) {
      m[h] = kMaxInit;
      l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[h][e] = 0.f;
    }
    m_lane = kMaxInit;
    l_lane = 0.f;
  }


  // the score with index 16 K + c in lane c of each row: four select levels
  // on c's bits.  The selects are written as v_cndmask instructions: left to
  // itself the compiler turns the tree into a lane-indexed scratch lookup.
  // (k is a compile-time constant after unrolling)
  __device__ float own_score(const float (&sc)[LPB][GP], int k, const uint64_t (&bit)[4]) const {
    float t0[8], t1[4], t2[2];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      t0[j] = lane_select(score_at_rt(sc, 16 * k + 2 * j), score_at_rt(sc, 16 * k + 2 * j + 1), bit[0]);
#pragma unroll
    for (int j = 0; j < 4; ++j) t1[j] = lane_select(t0[2 * j], t0[2 * j + 1], bit[1]);
#pragma unroll
    for (int j = 0; j < 2; ++j) t2[j] = lane_select(t1[2 * j], t1[2 * j + 1], bit[2]);
    return lane_select(t2[0], t2[1], bit[3]);
  }
  // score n of the block (token load n / GP, head n % GP), -inf past the end;
  // n is a compile-time constant after unrolling
  __device__ static float score_at_rt(const float (&sc)[LPB][GP], int n) {
    return n < kScores ? sc[n / GP][n % GP] : kNegInf;
  }

  // One reduce-scatter step over the lane pairs of DPP pattern CTRL, whose two
  // lanes differ in the bit that `mask` selects: of each pair of values (the
  // first and second halves of x), a lane keeps the half its bit names and adds
  // its partner's copy of that half, which the partner sends.
  // (Plain selects, not inline asm: the compiler must see which instruction
  // writes each value a DPP exchange reads, to keep the wait states that DPP
  // needs after a vector write of its operand.  All selects come first, then
  // the exchanges, so most reads sit far from their writes anyway.)
  template <int CTRL, int N>
  __device__ static void scatter_step(float (&x)[kScores], bool upper) {
    float send[N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i) send[i] = upper ? x[i] : x[i + N / 2];
#pragma unroll
    for (int i = 0; i < N / 2; ++i) x[i] = upper ? x[i + N / 2] : x[i];
#pragma unroll
    for (int i = 0; i < N / 2; ++i) x[i] += dpp<CTRL>(send[i]);
  }
  // Partial dots of the block's scores -> in lane c (of each 16-lane row) the
  // full scores c + 16 k, k < kScoresPerLane, in own[k].  Partners are lanes
  // c ^ 15 (row mirror), c ^ 7 (half-row mirror), c ^ 2 and c ^ 1 (quad
  // permutes): each keeps its partner's bits above the one it flips, so the
  // two always hold the same set of values, and halving by bits 3, 2, 1, 0 in
  // turn leaves lane c with entries kM c .. kM c + kM - 1 of the initial order,
  // which therefore holds score c + 16 k at entry kM c + k.
  __device__ void scores_scatter(const Vec (&kr)[LPB], float (&own)[kScoresPerLane]) const {
    constexpr int kM = kScoresPerLane;
    float x[kScores];
#pragma unroll
    for (int j = 0; j < kScores; ++j) {
      const int n = j / kM + 16 * (j % kM);   // score n: token load n / GP, head n % GP
      x[j] = E::dot0(qv[n % GP], kr[n / GP]);
    }
    scatter_step<kDppRowMirror, kScores>(x, (col >> 3) & 1);
    scatter_step<kDppRowHalfMirror, kScores / 2>(x, (col >> 2) & 1);
    scatter_step<kDppQuadXor2, kScores / 4>(x, (col >> 1) & 1);
    scatter_step<kDppQuadXor1, kScores / 8>(x, col & 1);
#pragma unroll
    for (int k = 0; k < kM; ++k) own[k] = x[k];
  }

  // One block with reduce-scattered scores: QK, the online softmax on the
  // lane's own scores (head col % GP) and PV with the row's weights broadcast
  // back from the lanes that evaluated them.
  __device__ void compute_block_scatter(int jj, const Vec (&kr)[LPB], const Vec (&vr)[LPB],
                                        int L, float c) {
    constexpr int kM = kScoresPerLane;
    float own[kM];
    scores_scatter(kr, own);
    if ((jj + 1) * B > L) {   // wave-uniform: only the last block of the sequence
      asm volatile("");
#pragma unroll
      for (int k = 0; k < kM; ++k) {
        const int i = (col + 16 * k) / GP;   // this score's token load
        own[k] = (jj * B + i * TPL + row < L) ? own[k] : kNegInf;
      }
    }
    // Lazy rescaling (see the header): compare the lane's scores with the
    // running max of their head.
    float mx = own[0];
#pragma unroll
    for (int k = 1; k < kM; ++k) mx = fmaxf(mx, own[k]);
    mx *= c;
    if (__builtin_amdgcn_ballot_w64(mx > m_lane + kRescaleLog2) != 0) {   // wave-uniform, rare
      // the max over the row's lanes of the same head (lanes c, c + GP, ...)
#pragma unroll
      for (int sh = GP; sh < 16; sh *= 2) mx = fmaxf(mx, row_ror(mx, sh));
      const float mn = fmaxf(m_lane, mx);
      const float alpha = fast_exp2(m_lane - mn);
      m_lane = mn;
      l_lane *= alpha;
#pragma unroll
      for (int h = 0; h < GP; ++h) {   // lane h evaluates head h
        const float ah = row_bcast(alpha, h);
        m[h] = row_bcast(m_lane, h);
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[h][e] *= ah;
      }
    }
    float pk[kM];
#pragma unroll
    for (int k = 0; k < kM; ++k) {
      pk[k] = fast_exp2(__builtin_fmaf(own[k], c, -m_lane));
      l_lane += pk[k];
    }
    // PV: each V element is widened once and used for all GP heads
#pragma unroll
    for (int i = 0; i < LPB; ++i) {
      float pf[GP];
#pragma unroll
      for (int h = 0; h < GP; ++h) pf[h] = row_bcast(pk[(i * GP + h) / 16], (i * GP + h) % 16);
      float vf[EPL];
      E::to_float(vr[i], vf);
#pragma unroll
      for (int e = 0; e < EPL; ++e)
#pragma unroll
        for (int h = 0; h < GP; ++h) o[h][e] = __builtin_fmaf(pf[h], vf[e], o[h][e]);
    }
  }

  // Blocks j = j_begin, j_begin + step, ... < j_end of the sequence whose table
  // is tbl and whose visible length is L (j_end <= ceil(L / B)).
  //
  // A ring of NBUF register buffers: while block j is computed, the loads of
  // the next NBUF-1 blocks are in flight, and the block id needed by the next
  // issue is fetched one step ahead.  The ring is rotated by a fully unrolled
  // loop, so every buffer index is a compile-time constant.  Loads are raw
  // buffer loads with the (block, KV head) slice base built in SGPRs and no
  // load under a branch, so each wait covers exactly the buffer consumed.  A
  // block past the range gets a zero-size descriptor (zeros, no memory access).
  //
  // In the last block of a sequence the slots at or beyond L may hold anything
  // (stale or poisoned data): that block's descriptor ends after slot L - 1,
  // so lanes on later slots read zeros without touching memory, and their
  // scores are set to -inf, which gives them weight exactly 0.  Every lane's
  // offset inside a block is therefore the same for all blocks and is
  // computed once.  (Offsets recomputed per block would be written at the top
  // of the ring, and the compiler may give them registers of a buffer that is
  // still loading on some path, which makes it drain the ring there.)
  //
  // Streaming (NT) loads carry the non-temporal hint: K/V bytes that no other
  // wave reads again should not push reused lines (block tables, queries,
  // partials, and shared blocks) out of the caches.
  template <bool NT>
  __device__ void run(const int32_t* tbl_ptr, int L, int j_begin, int j_end, int step,
                      const char* kbase, const char* vbase, size_t blk_bytes, float scale_log2) {
    const ConstI32Ptr tbl = as_const(tbl_ptr);
    const float c = exp_scale(scale_log2);
    uint64_t colbit[4];   // lanes whose column has bit b set (for own_score)
#pragma unroll
    for (int b = 0; b < 4; ++b) colbit[b] = __builtin_amdgcn_ballot_w64((col >> b) & 1);
    Vec kbuf[NBUF][LPB], vbuf[NBUF][LPB];
    // The lane's byte offset inside a (block, KV head) slice for its first
    // load; load i adds a constant, which goes in the load's scalar/immediate
    // offset, so all loads share one offset register that nothing in the ring
    // ever writes.  (A register written at the top of the ring would have to
    // wait for every load still pending into it on any path, which the
    // compiler covers by draining the whole ring there.)
    const int voff0 = row * kRowBytes + col * (int)sizeof(Vec);
    auto load_block = [&](int jj, int phys, bool in_range, Vec (&kr)[LPB], Vec (&vr)[LPB]) {
      // the slots below L (wave-uniform; at least one for a block in range)
      const int nrec = in_range ? min(L - jj * B, B) * kRowBytes : 0;
      const size_t boff = (size_t)phys * blk_bytes;
      const BufRsrc rk = make_rsrc(kbase + boff, nrec);
      const BufRsrc rv = make_rsrc(vbase + boff, nrec);
      // keep the issue order K then V, and both ahead of the compute that
      // follows, so each wait covers exactly the buffer being consumed
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < LPB; ++i) kr[i] = buffer_load_vec<Vec, NT>(rk, voff0, i * TPL * kRowBytes);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < LPB; ++i) vr[i] = buffer_load_vec<Vec, NT>(rv, voff0, i * TPL * kRowBytes);
      __builtin_amdgcn_sched_barrier(0);
    };

    auto compute_block = [&](int jj, const Vec (&kr)[LPB], const Vec (&vr)[LPB]) {
      if constexpr (kScatter) {
        compute_block_scatter(jj, kr, vr, L, c);
        return;
      }
      // QK: partial dot on the lane's 16 bytes, all-reduce over the token's lanes
      float part[LPB * GP];
#pragma unroll
      for (int i = 0; i < LPB; ++i)
#pragma unroll
        for (int h = 0; h < GP; ++h) part[i * GP + h] = E::dot0(qv[h], kr[i]);
      group_sum_all<LPT>(part);
      float sc[LPB][GP];
#pragma unroll
      for (int i = 0; i < LPB; ++i)
#pragma unroll
        for (int h = 0; h < GP; ++h) sc[i][h] = part[i * GP + h];
      if ((jj + 1) * B > L) {   // wave-uniform: only the last block of the sequence
        asm volatile("");       // keep this a branch (not selects on every block)
#pragma unroll
        for (int i = 0; i < LPB; ++i) {
          const bool valid = jj * B + i * TPL + row < L;
#pragma unroll
          for (int h = 0; h < GP; ++h) sc[i][h] = valid ? sc[i][h] : kNegInf;
        }
      }
      // online softmax in base 2 with lazy rescaling
      float mb[GP];
      bool up = false;
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        float t = sc[0][h];
#pragma unroll
        for (int i = 1; i < LPB; ++i) t = fmaxf(t, sc[i][h]);
        mb[h] = t * c;
        up |= mb[h] > m[h] + kRescaleLog2;
      }
      if (__builtin_amdgcn_ballot_w64(up) != 0) {   // wave-uniform, rare
        float alpha_lane = 1.f;
#pragma unroll
        for (int h = 0; h < GP; ++h) {
          const float mn = fmaxf(m[h], mb[h]);
          const float alpha = fast_exp2(m[h] - mn);
          m[h] = mn;
          l[h] *= alpha;
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[h][e] *= alpha;
          if (kOwnExp && col % GP == h) {
            alpha_lane = alpha;
            m_lane = mn;
          }
        }
        l_lane *= alpha_lane;
      }
      float pf[LPB][GP];   // the weights of the lane's row
      if constexpr (kOwnExp) {
        float pk[kScoresPerLane];
#pragma unroll
        for (int k = 0; k < kScoresPerLane; ++k) {
          const float sk = own_score(sc, k, colbit);
          pk[k] = fast_exp2(__builtin_fmaf(sk, c, -m_lane));
          l_lane += pk[k];
        }
#pragma unroll
        for (int i = 0; i < LPB; ++i)
#pragma unroll
          for (int h = 0; h < GP; ++h) pf[i][h] = row_bcast(pk[(i * GP + h) / 16], (i * GP + h) % 16);
      } else {
#pragma unroll
        for (int h = 0; h < GP; ++h) {
          float psum = 0.f;
#pragma unroll
          for (int i = 0; i < LPB; ++i) {
            pf[i][h] = fast_exp2(__builtin_fmaf(sc[i][h], c, -m[h]));
            psum += pf[i][h];
          }
          l[h] += psum;
        }
      }
      // PV: each V element is widened once and used for all GP heads
#pragma unroll
      for (int i = 0; i < LPB; ++i) {
        float vf[EPL];
        E::to_float(vr[i], vf);
#pragma unroll
        for (int e = 0; e < EPL; ++e)
#pragma unroll
          for (int h = 0; h < GP; ++h) o[h][e] = __builtin_fmaf(pf[i][h], vf[e], o[h][e]);
      }
    };

    if (j_begin >= j_end) return;
    int j = j_begin;
    const int jmax = j_end - 1;   // table reads are clamped here (always in bounds)
#pragma unroll
    for (int b = 0; b + 1 < NBUF; ++b) {
      const int jb = j + b * step;
      load_block(jb, tbl[min(jb, jmax)], jb < j_end, kbuf[b], vbuf[b]);
    }
    const int ahead = (NBUF - 1) * step;   // distance of the block issued next
    int id_next = tbl[min(j + ahead, jmax)];
    bool done = false;
    while (!done) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        const int jn = j + ahead;
        const int id_after = tbl[min(jn + step, jmax)];
        load_block(jn, id_next, jn < j_end, kbuf[(u + NBUF - 1) % NBUF],
                   vbuf[(u + NBUF - 1) % NBUF]);
        compute_block(j, kbuf[u], vbuf[u]);
        id_next = id_after;
        j += step;
        if (j >= j_end) {
          done = true;
          break;
        }
      }
    }
  }

  // Merge the TPL token rows of the wave (lanes col, col + LPT, ...) by
  // log-sum-exp; afterwards every row holds the wave's state.
  __device__ void merge_rows_in_wave() {
    if constexpr (kOwnExp) {   // per-head sums from the lanes' own sums
#pragma unroll
      for (int h = 0; h < GP; ++h) {
        float t = 0.f;
#pragma unroll
        for (int j = h; j < 16; j += GP) t += row_bcast(l_lane, j);
        l[h] = t;
      }
    }
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
  }
};

// ---------------------------------------------------------------------------
// split kernel: equal chunks of the flattened (sequence, KV head, block) list
// ---------------------------------------------------------------------------
// Each (sequence, KV head) with nb[s] > 0 blocks is c[s] = kSegItems + nb[s]
// items: its fixed cost (starting a segment: the query, the first block's
// latency, the final stores), then its blocks.  Items are numbered
// f = Hk pre[s] + g c[s] + k (pre: exclusive prefix sum of c); wave w takes f
// in [w chunk, (w+1) chunk), and item k >= kSegItems is block k - kSegItems.
// A length mix with many short segments would otherwise leave the waves that
// draw them far behind the others.  Workgroup 0 stores the plan for the
// merge: plan[0] = chunk, plan[1] = total items, plan[2 ..] = pre[0 .. S].
template <int DT, int D, int B, int GP>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(const AttnArgs a) {
  using W = DecodeWave<DT, D, B, GP>;
  extern __shared__ int sm_pre[];   // [S + 1] prefix sums of items per sequence
  __shared__ int sm_wsum[kWaves], sm_wne[kWaves];
  const int S = a.num_seqs, H = a.num_heads, Hk = a.num_kv_heads, G = a.group;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int X = kSegItems;

  // Items per sequence (per KV head: its blocks plus X if it has any) and
  // their prefix sums, 256 sequences per round: an inclusive scan inside each
  // wave (shuffles), then the wave totals through LDS (two barriers per
  // round).  The non-empty sequences are counted alongside.
  int carry = 0, nonempty = 0;
  if (tid == 0) sm_pre[0] = 0;
  for (int base = 0; base < S; base += kThreads) {
    const int s = base + tid;
    const int L = s < S ? min(max(a.context_lens[s] - a.len_offset, 0), a.max_context_len) : 0;
    const int nbs = (L + B - 1) / B;
    int v = nbs > 0 ? nbs + X : 0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(v, off, 64);
      v += lane >= off ? t : 0;
    }
    const uint64_t ne = __builtin_amdgcn_ballot_w64(nbs > 0);   // (all lanes take part)
    if (lane == 63) {
      sm_wsum[wave] = v;
      sm_wne[wave] = __builtin_popcountll(ne);
    }
    __syncthreads();
    int before = carry;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int t = sm_wsum[w];
      before += w < wave ? t : 0;
      carry += t;
      nonempty += sm_wne[w];
    }
    if (s < S) sm_pre[s + 1] = before + v;
    __syncthreads();
  }
  const int total = Hk * __builtin_amdgcn_readfirstlane(sm_pre[S]);
  // More table entries than pool blocks means some block serves several
  // sequences (a shared prefix): then K/V lines are worth keeping in the
  // caches.  Otherwise every block is (almost surely) read once: stream it.
  const int entries = __builtin_amdgcn_readfirstlane(sm_pre[S] - X * nonempty);
  const bool stream = entries <= a.pool_blocks;
  const int nwaves = gridDim.x * kWaves;
  const int chunk = a.chunk_blocks > 0 ? a.chunk_blocks : max(1, (total + nwaves - 1) / nwaves);
  if (blockIdx.x == 0) {
    if (tid == 0) {
      a.plan[0] = chunk;
      a.plan[1] = total;
    }
    for (int s = tid; s <= S; s += kThreads) a.plan[2 + s] = sm_pre[s];
  }

  const int wid = blockIdx.x * kWaves + wave;
  int f = wid * chunk;
  const int f_end = min(f + chunk, total);
  if (f >= total) return;

  // Locate the first item: the sequence s with Hk pre[s] <= f < Hk pre[s+1].
  // Values read from LDS are per-lane to the compiler; readfirstlane keeps the
  // walk in scalar registers, so block ids come from scalar loads and the
  // vector-memory waits in the block loop stay exact.
  auto pre_at = [&](int i) { return __builtin_amdgcn_readfirstlane(sm_pre[i]); };
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (Hk * pre_at(mid) <= f) lo = mid;
    else hi = mid - 1;
  }
  int s = lo;
  int c = pre_at(s + 1) - pre_at(s);   // items of each KV head of s (> 0)
  const int r0 = f - Hk * pre_at(s);
  int g = r0 / c, k = r0 % c;          // k: item within (s, g); its first X are no block

  W w(lane);
  const size_t blk_bytes = (size_t)Hk * W::kSliceBytes;
  const ConstI32Ptr lens = as_const(a.context_lens);
  while (f < f_end) {
    if (k < X) {                      // the segment's own cost: no block
      f += X - k;
      k = X;
      if (f >= f_end) break;
    }
    const int nb = c - X, j = k - X;
    const int L = min(max(lens[s] - a.len_offset, 0), a.max_context_len);
    const int n_here = min(nb - j, f_end - f);
    const size_t head0 = (size_t)s * H + (size_t)g * G;
    w.load_q(a.q, head0, G, a.scale_log2);
    w.reset();
    const int32_t* tbl = a.block_tables + (size_t)s * a.max_blocks_per_seq;
    const char* kb = static_cast<const char*>(a.k_cache) + (size_t)g * W::kSliceBytes;
    const char* vb = static_cast<const char*>(a.v_cache) + (size_t)g * W::kSliceBytes;
    if (stream)
      w.template run<true>(tbl, L, j, j + n_here, 1, kb, vb, blk_bytes, a.scale_log2);
    else
      w.template run<false>(tbl, L, j, j + n_here, 1, kb, vb, blk_bytes, a.scale_log2);
    w.merge_rows_in_wave();
    if (w.row == 0) {
      // (compile-time head loops keep the state in registers)
      if (j == 0 && n_here == nb) {   // the whole (sequence, KV head): final output
#pragma unroll
        for (int h = 0; h < GP; ++h) {
          if (h >= G) break;
          const float inv = w.l[h] > 0.f ? a.out_scale / w.l[h] : 0.f;
#pragma unroll
          for (int e = 0; e < W::EPL; ++e)
            store_out(a.out, (head0 + h) * D + w.col * W::EPL + e, w.o[h][e] * inv, a.out_dtype);
          if (a.lse && w.col == 0) a.lse[head0 + h] = lse2_of(w.m[h], w.l[h]);
        }
      } else {                        // a piece: partial for the merge
        const size_t slot = ((size_t)s * Hk + g + wid) * G;
#pragma unroll
        for (int h = 0; h < GP; ++h) {
          if (h >= G) break;
          float* po = a.ws_o + (slot + h) * D + w.col * W::EPL;
#pragma unroll
          for (int e = 0; e < W::EPL; ++e) po[e] = w.o[h][e];
          if (w.col == 0) {
            a.ws_ml[2 * (slot + h)] = w.m[h];
            a.ws_ml[2 * (slot + h) + 1] = w.l[h];
          }
        }
      }
    }
    f += n_here;
    k += n_here;
    if (k == c && f < f_end) {        // next KV head, or the next non-empty sequence
      k = 0;
      if (++g == Hk) {
        g = 0;
        do {
          ++s;
        } while (pre_at(s + 1) == pre_at(s));
        c = pre_at(s + 1) - pre_at(s);
      }
    }
  }
}

// Merge of the split kernel's pieces for one sequence; thread c owns 4
// consecutive dims of one query head (16-byte loads of the pieces' partial
// outputs), so a 256-thread workgroup covers 1,024 of the sequence's H*D
// outputs.  The items of (s, g) are [a0, a0 + c) with a0 = Hk pre[s] + g c,
// its blocks the last c - kSegItems of them, so the waves that covered its
// blocks are (a0 + kSegItems) / chunk .. (a0 + c - 1) / chunk, and wave w
// left its piece in slot (s Hk + g + w) G + h.  Empty contexts get zero
// rows.  The plan, the length and the prefix sums are read together, then the
// pieces' (max, sum, o) in batches of independent loads.
template <int D>
__global__ __launch_bounds__(256) void split_merge_kernel(const AttnArgs a) {
  constexpr int kChunks = D / 4;   // 4-dim chunks per head
  const int H = a.num_heads, Hk = a.num_kv_heads, G = a.group;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= H * kChunks) return;
  const int hq = c / kChunks, d0 = (c % kChunks) * 4;
  const int s = blockIdx.y;
  const int g = hq / G, h = hq - g * G;
  const ConstI32Ptr plan = as_const(a.plan);
  const int Lraw = as_const(a.context_lens)[s] - a.len_offset;
  const int chunk = plan[0];
  const int p0 = plan[2 + s], p1 = plan[3 + s];
  const size_t oidx = ((size_t)s * H + hq) * D + d0;
  if (min(max(Lraw, 0), a.max_context_len) == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) store_out(a.out, oidx + e, 0.f, a.out_dtype);
    if (a.lse && d0 == 0) a.lse[(size_t)s * H + hq] = kNegInf;
    return;
  }
  // (s, g) holds items [a0, a0 + items): its own cost first, then its
  // blocks, which waves (a0 + kSegItems) / chunk .. (a0 + items - 1) / chunk
  // covered
  const int items = p1 - p0;
  const int a0 = Hk * p0 + g * items;
  const int w0 = (a0 + kSegItems) / chunk, w1 = (a0 + items - 1) / chunk;
  if (w0 == w1) return;               // written by its one wave
  const size_t base = (size_t)s * Hk + g;
  constexpr int kBatch = 8;
  float M = kNegInf, den = 0.f;
  float num[4] = {0.f, 0.f, 0.f, 0.f};
  for (int w = w0; w <= w1; w += kBatch) {
    float pm[kBatch], pl[kBatch];
    float4 pv[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const size_t sl = (base + min(w + k, w1)) * G + h;   // past the last piece: weight 0
      pm[k] = a.ws_ml[2 * sl];
      pl[k] = a.ws_ml[2 * sl + 1];
      pv[k] = *reinterpret_cast<const float4*>(a.ws_o + sl * D + d0);
    }
    float mx = M;
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      if (w + k <= w1) mx = fmaxf(mx, pm[k]);
    const float ms = (mx == kNegInf) ? 0.f : mx;
    const float r = fast_exp2(M - ms);
    den *= r;
#pragma unroll
    for (int e = 0; e < 4; ++e) num[e] *= r;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float wt = (w + k <= w1) ? fast_exp2(pm[k] - ms) : 0.f;
      num[0] = __builtin_fmaf(wt, pv[k].x, num[0]);
      num[1] = __builtin_fmaf(wt, pv[k].y, num[1]);
      num[2] = __builtin_fmaf(wt, pv[k].z, num[2]);
      num[3] = __builtin_fmaf(wt, pv[k].w, num[3]);
      den = __builtin_fmaf(wt, pl[k], den);
    }
    M = mx;
  }
  const float inv = den > 0.f ? a.out_scale / den : 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) store_out(a.out, oidx + e, num[e] * inv, a.out_dtype);
  if (a.lse && d0 == 0) a.lse[(size_t)s * H + hq] = lse2_of(M, den);
}

// ---------------------------------------------------------------------------
// partition kernel: one workgroup per (partition, KV head, row)
// ---------------------------------------------------------------------------
template <int DT, int D, int B, int GP>
__global__ __launch_bounds__(kThreads) void decode_partition_kernel(const AttnArgs a) {
  using W = DecodeWave<DT, D, B, GP>;
  constexpr int EPL = W::EPL;
  const int p = blockIdx.x, g = blockIdx.y;
  const int H = a.num_heads, G = a.group;
  // Decode: blockIdx.z is the sequence and its one query row.  Per-row mode
  // (multi-token queries without MFMA): blockIdx.z = s * max_q_len + i is row i
  // of sequence s, which sees the first L_s - n_s + i + 1 keys when causal.
  // (fixed_rows: one sequence of fixed_rows rows and length max_context_len)
  const bool rows_mode = a.q_offsets || a.fixed_rows > 0;
  int s = blockIdx.z, qrow = blockIdx.z, i = 0, n = 1;
  if (rows_mode) {
    s = blockIdx.z / a.max_q_len;
    i = blockIdx.z % a.max_q_len;
    const int q0 = a.fixed_rows > 0 ? 0 : a.q_offsets[s];
    n = a.fixed_rows > 0 ? a.fixed_rows : a.q_offsets[s + 1] - q0;
    if (i >= n) return;
    qrow = q0 + i;
  }
  // context_lens is read only once s is known (blockIdx.z may exceed S)
  int L = a.fixed_rows > 0 ? a.max_context_len
                           : min(max(a.context_lens[s] - a.len_offset, 0), a.max_context_len);
  if (rows_mode && a.causal) L = max(0, min(L, L - n + i + 1));
  const int n_parts = (L + a.part - 1) / a.part;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
  const size_t head0 = (size_t)qrow * H + (size_t)g * G;       // first query head of the group

  if (n_parts == 0) {  // empty context: zero output rows, written by partition 0
    if (p == 0)
      for (int i = tid; i < G * D; i += kThreads) store_out(a.out, head0 * D + i, 0.f, a.out_dtype);
    if (p == 0 && a.lse && tid < G) a.lse[head0 + tid] = kNegInf;
    return;
  }
  if (p >= n_parts) return;

  W w(lane);
  w.load_q(a.q, head0, G, a.scale_log2);
  w.reset();
  const int tok0 = p * a.part;
  const int blk_end = (min(tok0 + a.part, L) + B - 1) / B;
  // (rows of one sequence, and partitions, re-read blocks: cached loads)
  w.template run<false>(a.block_tables + (size_t)s * a.max_blocks_per_seq, L, tok0 / B + wave,
                        blk_end, kWaves,
        static_cast<const char*>(a.k_cache) + (size_t)g * W::kSliceBytes,
        static_cast<const char*>(a.v_cache) + (size_t)g * W::kSliceBytes,
        (size_t)a.num_kv_heads * W::kSliceBytes, a.scale_log2);
  w.merge_rows_in_wave();

  // merge the waves through LDS
  __shared__ float sm_o[kWaves][GP][D];
  __shared__ float sm_m[kWaves][GP], sm_l[kWaves][GP];
  if (w.row == 0) {
#pragma unroll
    for (int h = 0; h < GP; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) sm_o[wave][h][w.col * EPL + e] = w.o[h][e];
      if (w.col == 0) {
        sm_m[wave][h] = w.m[h];
        sm_l[wave][h] = w.l[h];
      }
    }
  }
  __syncthreads();

  const bool final_out = (n_parts == 1);
  for (int i = tid; i < G * D; i += kThreads) {
    const int h = i / D, d = i % D;
    float mx = kNegInf;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) mx = fmaxf(mx, sm_m[v][h]);
    const float ms = (mx == kNegInf) ? 0.f : mx;
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      const float wt = fast_exp2(sm_m[v][h] - ms);
      num = __builtin_fmaf(wt, sm_o[v][h][d], num);
      den = __builtin_fmaf(wt, sm_l[v][h], den);
    }
    const size_t hh = head0 + h;
    if (final_out) {
      store_out(a.out, hh * D + d, den > 0.f ? a.out_scale * num / den : 0.f, a.out_dtype);
      if (a.lse && d == 0) a.lse[hh] = lse2_of(mx, den);
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

// Log-sum-exp merge of the partitions of one row: M = max_p m_p,
// out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.  Thread c of the row
// owns 4 consecutive dims of one query head (16-byte loads of the partials;
// the partial outputs start on a 16-byte boundary), so a 256-thread workgroup
// covers 1,024 of the row's H*D outputs.  Rows with a single partition were
// finished by the partial kernel.  The length (and the row's place in its
// sequence) is read first, then every partition's (max, sum, o) in batches of
// independent loads.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const AttnArgs a) {
  constexpr int kChunks = D / 4;   // 4-dim chunks per head
  const int H = a.num_heads;
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= H * kChunks) return;
  const int hq = c / kChunks, d0 = (c % kChunks) * 4;
  const int s = blockIdx.z;
  size_t row = s;
  int L = min(max(a.context_lens[s] - a.len_offset, 0), a.max_context_len);
  if (a.q_offsets) {  // multi-token queries: blockIdx.y = row within the sequence
    const int q0 = a.q_offsets[s], n = a.q_offsets[s + 1] - q0;
    const int i = blockIdx.y;
    if (i >= n) return;
    row = (size_t)q0 + i;
    if (a.causal) L = max(0, min(L, L - n + i + 1));
  }
  const int n_parts = (L + a.part - 1) / a.part;
  if (n_parts <= 1) return;
  const size_t hh = row * H + hq;
  const float* ml = a.ws_ml + 2 * hh * a.max_parts;
  const float* po = a.ws_o + hh * a.max_parts * D + d0;
  constexpr int kBatch = 8;
  float M = kNegInf, den = 0.f;
  float num[4] = {0.f, 0.f, 0.f, 0.f};
  for (int p0 = 0; p0 < n_parts; p0 += kBatch) {
    float pm[kBatch], pl[kBatch];
    float4 pv[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int pk = min(p0 + k, n_parts - 1);   // repeats past the end get weight 0
      pm[k] = ml[2 * pk];
      pl[k] = ml[2 * pk + 1];
      pv[k] = *reinterpret_cast<const float4*>(po + (size_t)pk * D);
    }
    float mx = M;
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      if (p0 + k < n_parts) mx = fmaxf(mx, pm[k]);
    const float ms = (mx == kNegInf) ? 0.f : mx;
    const float r = fast_exp2(M - ms);
    den *= r;
#pragma unroll
    for (int e = 0; e < 4; ++e) num[e] *= r;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float wt = (p0 + k < n_parts) ? fast_exp2(pm[k] - ms) : 0.f;
      num[0] = __builtin_fmaf(wt, pv[k].x, num[0]);
      num[1] = __builtin_fmaf(wt, pv[k].y, num[1]);
      num[2] = __builtin_fmaf(wt, pv[k].z, num[2]);
      num[3] = __builtin_fmaf(wt, pv[k].w, num[3]);
      den = __builtin_fmaf(wt, pl[k], den);
    }
    M = mx;
  }
  const float inv = den > 0.f ? a.out_scale / den : 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) store_out(a.out, hh * D + d0 + e, num[e] * inv, a.out_dtype);
  if (a.lse && d0 == 0) a.lse[hh] = lse2_of(M, den);
}

// ---------------------------------------------------------------------------
// launch
// ---------------------------------------------------------------------------
hipError_t launch_merge(int head_dim, int num_seqs, const AttnArgs& a, hipStream_t st) {
  const int chunks = a.num_heads * head_dim / 4;   // 4-dim chunks of a row
  dim3 mgrid((chunks + 255) / 256, a.q_offsets ? a.max_q_len : 1, num_seqs);
  if (head_dim == 64)
    hipLaunchKernelGGL((merge_kernel<64>), mgrid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((merge_kernel<128>), mgrid, dim3(256), 0, st, a);
  return hipGetLastError();
}

// Resident workgroups per CU of the split kernel (occupancy query, cached;
// threads that race on the first query store the same value, atomically).
template <int DT, int D, int B, int GP>
static int split_wgs_per_cu() {
  static std::atomic<int> cached{0};
  int n = cached.load(std::memory_order_relaxed);
  if (!n) {
    const size_t smem = ((size_t)kMaxSplitSeqs + 1) * sizeof(int);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void*>(decode_split_kernel<DT, D, B, GP>), kThreads,
            smem) != hipSuccess || n < 1)
      n = 1;
    cached.store(n, std::memory_order_relaxed);
  }
  return n;
}

template <int DT, int D, int B, int GP>
static hipError_t launch_decode_t(int num_seqs, const AttnArgs& a, hipStream_t st,
                                  const KernelEvents& ev) {
  if (a.plan) {   // balanced split
    const size_t smem = ((size_t)num_seqs + 1) * sizeof(int);
    hipError_t e = launch_main(decode_split_kernel<DT, D, B, GP>, dim3(a.split_workgroups),
                               dim3(kThreads), smem, st, ev, a);
    if (e != hipSuccess || a.no_merge) return e;
    const int chunks = a.num_heads * D / 4;   // 4-dim chunks of a sequence's outputs
    hipLaunchKernelGGL((split_merge_kernel<D>), dim3((chunks + 255) / 256, num_seqs), dim3(256), 0,
                       st, a);
    return hipGetLastError();
  }
  // per-row mode launches one grid row per (sequence, query row) slot
  const int rows = (a.q_offsets || a.fixed_rows > 0) ? num_seqs * a.max_q_len : num_seqs;
  dim3 grid(a.max_parts, a.num_kv_heads, rows);
  hipError_t e = launch_main(decode_partition_kernel<DT, D, B, GP>, grid, dim3(kThreads), 0, st,
                             ev, a);
  if (e != hipSuccess || a.max_parts <= 1 || a.no_merge) return e;
  return launch_merge(D, num_seqs, a, st);
}

// Compile-time dispatch over (dtype, head_dim, block_size, padded group).
template <typename F>
static auto with_config(int dtype, int head_dim, int block_size, int group, F&& f) {
  auto by_g = [&](auto dt, auto d, auto b) {
    using I1 = std::integral_constant<int, 1>;
    if (group <= 1) return f(dt, d, b, I1{});
    if (group <= 2) return f(dt, d, b, std::integral_constant<int, 2>{});
    if (group <= 4) return f(dt, d, b, std::integral_constant<int, 4>{});
    if (group <= 8) return f(dt, d, b, std::integral_constant<int, 8>{});
    // (8-bit caches stop at groups of 8; the host rejects larger groups)
    constexpr bool kNo16 = decltype(dt)::value == PA_FP8_E4M3;
    return f(dt, d, b, std::integral_constant<int, kNo16 ? 8 : 16>{});
  };
  auto by_b = [&](auto dt, auto d) {
    if (block_size == 8) return by_g(dt, d, std::integral_constant<int, 8>{});
    if (block_size == 16) return by_g(dt, d, std::integral_constant<int, 16>{});
    return by_g(dt, d, std::integral_constant<int, 32>{});
  };
  auto by_d = [&](auto dt) {
    if (head_dim == 64) return by_b(dt, std::integral_constant<int, 64>{});
    return by_b(dt, std::integral_constant<int, 128>{});
  };
  if (dtype == PA_F32) return by_d(std::integral_constant<int, PA_F32>{});
  if (dtype == PA_F16) return by_d(std::integral_constant<int, PA_F16>{});
  if (dtype == PA_FP8_E4M3) return by_d(std::integral_constant<int, PA_FP8_E4M3>{});
  return by_d(std::integral_constant<int, PA_BF16>{});
}

hipError_t launch_decode(int dtype, int head_dim, int block_size, int group, int num_seqs,
                         const AttnArgs& a, hipStream_t st, const KernelEvents& ev) {
  return with_config(dtype, head_dim, block_size, group, [&](auto dt, auto d, auto b, auto gp) {
    return launch_decode_t<decltype(dt)::value, decltype(d)::value, decltype(b)::value,
                           decltype(gp)::value>(num_seqs, a, st, ev);
  });
}

int split_workgroups_per_cu(int dtype, int head_dim, int block_size, int group) {
  return with_config(dtype, head_dim, block_size, group, [&](auto dt, auto d, auto b, auto gp) {
    return split_wgs_per_cu<decltype(dt)::value, decltype(d)::value, decltype(b)::value,
                            decltype(gp)::value>();
  });
}

}  // namespace pa
