// Multi-token queries: speculative verification (the k guessed tokens a target
// model checks in one pass, "Scaling inference with vLLM", speculative decoding
// paragraph) and prefill chunks ("Local_LLM_03_vLLM_Architecture",
// chunked-prefill slide).  The n query rows of a sequence are its last n
// positions; with the causal mask row i sees keys t <= L - n + i.
//
// bf16/f16: matrix-core kernel.  For one KV head g of sequence s, the query
// rows are the n*G pairs (i, h) of the group (row r = i*G + h), tiled by 32.
// Each wave owns one 32-row tile and walks 32-token K/V tiles of a context
// partition with v_mfma_f32_32x32x16 (fp32 accumulation):
//
//   S^T = K Q^T      A = K tile (token x dims), B = Q^T; in the result lane l
//                    holds 16 of the 32 tokens of row m = l % 32, so the row's
//                    softmax max/sum is 16 in-lane steps plus one exchange
//                    with lane l ^ 32 (v_permlane32_swap, no LDS).
//   O^T += V^T P^T   B = P^T comes straight out of the score registers
//                    (rounded to the input dtype).  A = V^T holds, in lane l,
//                    V at dim 32b + l % 32 for exactly the tokens whose
//                    probabilities the lane holds, in the same order (the
//                    contraction order over a tile's tokens is free, as long
//                    as both operands share it).  With K/V staged in LDS
//                    (rows layout below) two LDS transpose reads
//                    (ds_read_b64_tr_b16) give it per 16-token step; with
//                    K/V loaded straight into registers (token layout) an
//                    MFMA of V with an identity puts V into that layout.
//
// The four waves of a workgroup split the partition's tiles, each keeping its
// next tile's loads in flight while it computes one; their (max, sum, O)
// states are merged through LDS, then written as the final output or as a
// partition partial for merge_kernel.  fp32: every query row runs the decode
// kernel over its own visible length.
#include "pa_common.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2v_t __attribute__((ext_vector_type(2)));
typedef float f32x2v_t __attribute__((ext_vector_type(2)));

template <int DT> struct Mma;

template <> struct Mma<PA_BF16> {
  static constexpr uint32_t kOne = 0x3F80u;   // 1.0
  __device__ static inline f32x16_t mma(const uint4& a, const uint4& b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  // two floats -> two bf16 rounded to nearest even (v_cvt_pk_bf16_f32), lo in the low half
  __device__ static inline uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v_t{lo, hi}, bf16x2v_t));
  }
  // two floats that are bf16 values already: their upper halves (exact)
  __device__ static inline uint32_t pack2_exact(float lo, float hi) {
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
  }
};

template <> struct Mma<PA_F16> {
  static constexpr uint32_t kOne = 0x3C00u;   // 1.0
  __device__ static inline f32x16_t mma(const uint4& a, const uint4& b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2v_t{lo, hi}, f16x2v_t));
  }
  // two floats that are f16 values already (rounding toward zero changes nothing)
  __device__ static inline uint32_t pack2_exact(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
  }
};

template <int DT>
__device__ inline uint4 pack8(const f32x16_t& x, int base) {
  using M = Mma<DT>;
  return make_uint4(M::pack2(x[base + 0], x[base + 1]), M::pack2(x[base + 2], x[base + 3]),
                    M::pack2(x[base + 4], x[base + 5]), M::pack2(x[base + 6], x[base + 7]));
}

template <int DT>
__device__ inline uint4 pack8_exact(const f32x16_t& x, int base) {
  using M = Mma<DT>;
  return make_uint4(M::pack2_exact(x[base + 0], x[base + 1]), M::pack2_exact(x[base + 2], x[base + 3]),
                    M::pack2_exact(x[base + 4], x[base + 5]), M::pack2_exact(x[base + 6], x[base + 7]));
}

// token offset (within a 32-token tile) of C-layout register v in lane half hh
__device__ constexpr int tile_token(int v, int hh) { return 8 * (v / 4) + 4 * hh + (v % 4); }

// ROWS = false: one 32-row tile per workgroup; its four waves take
//   interleaved 32-token tiles of the partition (each staging its own tiles
//   through its own LDS area) and merge through LDS at the end.
// ROWS = true:  four row tiles per workgroup, one per wave, over the same
//   tokens; the 256 threads stage each K/V tile once into a double-buffered LDS
//   area that all four waves read.  Used when a sequence has many query rows
//   (prefill chunks), where it cuts the K/V traffic per row by four.
//
// Staging: a K or V tile is 32 token rows of D elements.  Thread c of the
// stagers loads 16-byte chunks c, c + NP, ... in memory order (a wave reads
// four whole rows, 1 KiB, per instruction) and writes them to LDS rows padded
// by 16 bytes, from which each lane reads its MFMA operands (row = token
// mcol, 16 bytes per k-step) without bank conflicts.
template <int DT, int D, int B, bool ROWS>
__device__ __forceinline__ void multiq_mfma_body(const AttnArgs& a) {
  using M = Mma<DT>;
  constexpr int KS = D / 16;   // k-steps of QK over head_dim
  constexpr int DB = D / 32;   // 32-dim blocks of the output
  constexpr int kElem = 2;
  constexpr int kRowBytes = D * kElem;
  // LDS row strides.  K rows are read 16 bytes per lane, 16 rows per pass:
  // 16 bytes of padding (4 dwords) spread those rows over all banks.  V rows
  // are read by transpose reads, 4 rows x 64 bytes per half-wave: 64 bytes of
  // padding (16 dwords, so 16 or 48 dwords modulo the 64 banks) keeps those
  // four rows in disjoint banks.
  constexpr int RS = kRowBytes + 16;       // K
  constexpr int RSV = kRowBytes + 64;      // V
  constexpr int kTileBytes = 32 * RS;      // one K tile in LDS
  constexpr int kStageBytes = kTileBytes + 32 * RSV;   // a K tile and a V tile
  constexpr int CPR = kRowBytes / 16;      // 16-byte chunks per token row
  constexpr int NP = ROWS ? kThreads : 64; // threads staging one tile
  constexpr int kPer = 32 * CPR / NP;      // chunks per staging thread per tensor
  static_assert(kPer * NP == 32 * CPR && NP % CPR == 0, "staging layout");

  const int G = a.group, H = a.num_heads, Hk = a.num_kv_heads;
  const int rt_count = (a.max_q_len * G + 31) / 32;
  const int units = ROWS ? (rt_count + kWaves - 1) / kWaves : rt_count;
  // One workgroup per (row unit, partition, KV head, sequence), numbered so
  // that the row units of one (partition, KV head, sequence), which read the
  // same K/V tiles, run on one XCD.
  int wg = xcd_major(blockIdx.x, gridDim.x);
  const int ux = wg % units;
  wg /= units;
  const int p = wg % a.max_parts;
  wg /= a.max_parts;
  const int g = wg % Hk, s = wg / Hk;
  const int q0 = a.fixed_rows > 0 ? 0 : a.q_offsets[s];
  const int n = a.fixed_rows > 0 ? a.fixed_rows : a.q_offsets[s + 1] - q0;
  const int n_rows = n * G;
  const int wg_row0 = (ROWS ? ux * kWaves : ux) * 32;
  if (wg_row0 >= n_rows) return;       // workgroup-uniform
  const int L = a.fixed_rows > 0 ? a.max_context_len
                                 : min(max(a.context_lens[s], 0), a.max_context_len);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5;            // lane half: which 16 of a tile's 32 tokens
  const int mcol = lane & 31;          // this lane's query row within the tile
  const int rt = ROWS ? ux * kWaves + wave : ux;
  const bool wave_rows = rt * 32 < n_rows;   // (ROWS: a wave past the rows only stages)
  const int r = rt * 32 + mcol;
  const bool row_ok = wave_rows && r < n_rows;
  const int qi = row_ok ? r / G : 0;   // query token of the row
  const int qh = row_ok ? r % G : 0;   // head within the group
  auto visible = [&](int i) { return a.causal ? max(0, min(L, L - n + i + 1)) : L; };
  // visible keys of this row, of the wave's first and last rows, and of the
  // workgroup's last (most-seeing) row
  const int lrow = row_ok ? visible(qi) : 0;
  const int l_tile_max = wave_rows ? visible(min(rt * 32 + 31, n_rows - 1) / G) : 0;
  const int l_tile_min = wave_rows ? visible((rt * 32) / G) : 0;
  const int wg_rows = ROWS ? 32 * kWaves : 32;
  const int l_wg_max = visible(min(wg_row0 + wg_rows - 1, n_rows - 1) / G);
  const int parts_row = (lrow + a.part - 1) / a.part;
  const size_t out_row = ((size_t)(q0 + qi) * H + (size_t)g * G + qh);   // (token, head) index

  const int tok0 = p * a.part;
  if (L == 0) {  // nothing visible: zero rows, written once
    if (p == 0 && (ROWS || wave == 0) && row_ok)
      for (int d = hh * (D / 2); d < (hh + 1) * (D / 2); ++d) store_out(a.out, out_row * D + d, 0.f, a.out_dtype);
    if (p == 0 && (ROWS || wave == 0) && row_ok && a.lse && hh == 0) a.lse[out_row] = kNegInf;
    return;
  }
  if (tok0 >= l_wg_max) return;        // no row of this workgroup sees this partition
  const int wg_end = min(tok0 + a.part, l_wg_max);
  const int tok_end = min(tok0 + a.part, l_tile_max);   // this wave's keys end here
  const int lim = min(lrow, tok_end);  // this lane-row's keys end here (within the partition)

  // Q^T operand: row m = lane % 32, dims 16 ks + 8 hh .. +7
  uint4 qv[KS];
  {
    const uint4* qp = reinterpret_cast<const uint4*>(a.q) + (out_row * D + hh * 8) / 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qv[ks] = row_ok ? qp[2 * ks] : make_uint4(0, 0, 0, 0);
    // a negative scale goes into q's sign bits (exact), so the scores are
    // scaled by a positive c inside the exponent's FMA
    if (a.scale_log2 < 0.f) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qv[ks].x ^= 0x80008000u; qv[ks].y ^= 0x80008000u;
        qv[ks].z ^= 0x80008000u; qv[ks].w ^= 0x80008000u;
      }
    }
  }
  const float c = fmaxf(fabsf(a.scale_log2), 1e-30f);
  // identity operands selecting dims 0..15 and 16..31 of a 32-dim block
  uint4 eye[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    uint32_t w[4];
#pragma unroll
    for (int j2 = 0; j2 < 4; ++j2) {
      const int k0 = hh * 8 + 2 * j2 + 16 * kk;
      w[j2] = (k0 == mcol ? M::kOne : 0u) | ((k0 + 1 == mcol ? M::kOne : 0u) << 16);
    }
    eye[kk] = make_uint4(w[0], w[1], w[2], w[3]);
  }

  f32x16_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x16_t{};
  // running max (log2 units) starts at a finite sentinel below any score, so
  // rows that see no key stay free of inf - inf
  float m_run = kMaxInit, l_run = 0.f;

  const char* kbase = static_cast<const char*>(a.k_cache);
  const char* vbase = static_cast<const char*>(a.v_cache);

  // A 32-token tile spans 32 / B whole blocks; their ids are read with scalar
  // loads and each staging lane picks the one of its token.  Tokens at or past
  // L are clamped to the last valid one (their slots may hold anything) and
  // masked in the scores.
  static_assert(32 % B == 0, "tiles hold whole blocks");
  constexpr int kTileBlocks = 32 / B;
  const ConstI32Ptr tblc = as_const(a.block_tables + (size_t)s * a.max_blocks_per_seq);
  const int jlast = (L - 1) / B;
  // Staged chunks are held as a native vector type: copies of the uint4 struct
  // between global memory and LDS would pass through private memory.
  const int spid = ROWS ? tid : lane;  // this thread's staging index
  const int scol = spid % CPR;         // its 16-byte column
  // Chunk i of this thread: token tok_i of the tile, i.e. block tok_i / B of
  // the tile at slot tok_i % B; its byte offset inside a block of the pool
  // (head g, that slot, this column) is the same for every full tile.
  const size_t blk_stride = (size_t)Hk * B * kRowBytes;   // one physical block, all heads
  int chunk_off[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int tok = spid / CPR + i * (NP / CPR);
    chunk_off[i] = (g * B + tok % B) * kRowBytes + scol * 16;
  }
  auto stage_load = [&](int t0, u32x4_t (&sk)[kPer], u32x4_t (&sv)[kPer]) {
    int ids[kTileBlocks];
#pragma unroll
    for (int k = 0; k < kTileBlocks; ++k) ids[k] = tblc[min(t0 / B + k, jlast)];
    if (t0 + 32 <= L) {   // workgroup-uniform: a full tile (block ids from scalar loads)
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int jt = (spid / CPR + i * (NP / CPR)) / B;
        int phys = ids[0];
#pragma unroll
        for (int k = 1; k < kTileBlocks; ++k) phys = (jt == k) ? ids[k] : phys;
        const size_t boff = (size_t)phys * blk_stride;
        sk[i] = *reinterpret_cast<const u32x4_t*>(kbase + boff + chunk_off[i]);
        sv[i] = *reinterpret_cast<const u32x4_t*>(vbase + boff + chunk_off[i]);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int tok = spid / CPR + i * (NP / CPR);
      const int t = min(t0 + tok, L - 1);   // >= t0, since t0 < L
      const int jt = t / B - t0 / B;
      int phys = ids[0];
#pragma unroll
      for (int k = 1; k < kTileBlocks; ++k) phys = (jt == k) ? ids[k] : phys;
      const size_t off = (((size_t)phys * Hk + g) * B + (t % B)) * kRowBytes + scol * 16;
      sk[i] = *reinterpret_cast<const u32x4_t*>(kbase + off);
      sv[i] = *reinterpret_cast<const u32x4_t*>(vbase + off);
    }
  };
  // rows layout: 32-token tiles per loop step, and two LDS stages of a step each
  constexpr int kTps = 1;
  constexpr int kLdsBytes = ROWS ? 2 * kTps * kStageBytes : 16;   // (only the rows layout stages)
  __shared__ __attribute__((aligned(16))) char sm_kv[kLdsBytes];
  // base: K tile, base + kTileBytes: V tile
  auto stage_store = [&](char* base, const u32x4_t (&sk)[kPer], const u32x4_t (&sv)[kPer]) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int tok = spid / CPR + i * (NP / CPR);
      *reinterpret_cast<u32x4_t*>(base + tok * RS + scol * 16) = sk[i];
      *reinterpret_cast<u32x4_t*>(base + kTileBytes + tok * RSV + scol * 16) = sv[i];
    }
  };
  // this lane's K operands: token mcol, dims 16 ks + 8 hh .. +7
  auto lds_read_k = [&](const char* base, uint4 (&kr)[KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kr[ks] = *reinterpret_cast<const uint4*>(base + mcol * RS + 32 * ks + 16 * hh);
  };
  // this lane's V^T operands for dim block db and 16-token step ks: dim
  // 32 db + mcol, tokens 16 ks + 4 hh + (0..3) then 16 ks + 8 + 4 hh + (0..3),
  // the order of its probabilities.  In a transpose read, lane i of each
  // 16-lane group addresses row r0 + i / 4 at dims c0 + 4 (i % 4) .. + 3, and
  // lane j receives dim c0 + j of rows r0 .. r0 + 3.
  auto lds_read_vt = [&](const char* base, uint4 (&va)[DB][2]) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 LdsV4;
    const int trow = 4 * hh + (lane & 15) / 4;
    const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const char* p0 = base + kTileBytes + (16 * ks + trow) * RSV + (32 * db + tcol) * 2;
        const auto lo = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                      (LdsV4*)(__attribute__((address_space(3))) char*)p0));
        const auto hi = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                      (LdsV4*)(__attribute__((address_space(3))) char*)(p0 + 8 * RSV)));
        va[db][ks] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
  };

  // S^T = K Q^T of one tile: lane holds tokens t0 + tile_token(v, hh) of its row
  auto qk_tile = [&](const uint4 (&kr)[KS]) {
    f32x16_t sc = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) sc = M::mma(kr[ks], qv[ks], sc);
    return sc;
  };
  // masking and the online softmax of one tile's scores; returns the P^T
  // operands (pb: p rounded or cut to the input dtype, pl: bf16 residual)
  auto softmax_scores = [&](int t0, f32x16_t sc, uint4& pb0, uint4& pb1, uint4& pl0,
                            uint4& pl1) {
    float mx = kNegInf;
    if (t0 + 32 <= min(l_tile_min, tok_end)) {   // wave-uniform: no key of the tile is masked
#pragma unroll
      for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sc[v]);
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        sc[v] = (t0 + tile_token(v, hh) < lim) ? sc[v] : kNegInf;
        mx = fmaxf(mx, sc[v]);
      }
    }
    mx = max_halves(mx) * c;   // the row's tile max in log2 units (c > 0)
    // Lazy rescaling: the running max moves only when a score beats it by
    // more than kRescaleLog2; otherwise the weights are taken against the
    // stale max (so they are at most 2^kRescaleLog2) and o, l keep their scale.
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleLog2) != 0) {   // wave-uniform
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
    }
    float psum = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      sc[v] = fast_exp2(__builtin_fmaf(sc[v], c, -m_run));
      psum += sc[v];
    }
    l_run += sum_halves(psum);

    // P^T operands.  bf16 keeps 8 significant bits, too few for the
    // probabilities at short contexts, so P is split into a head (p with its
    // low 16 bits cleared, exact) and the residual p - head (exact in fp32,
    // then rounded to bf16), and both are multiplied: p is carried to about
    // 2^-16.  f16's 11 bits are used as they are (rounded to nearest).
    if constexpr (DT == PA_BF16) {
      f32x16_t res;
#pragma unroll
      for (int v = 0; v < 16; ++v)
        res[v] = sc[v] - __uint_as_float(__float_as_uint(sc[v]) & 0xffff0000u);
      pb0 = pack8_exact<DT>(sc, 0);
      pb1 = pack8_exact<DT>(sc, 8);
      pl0 = pack8<DT>(res, 0);
      pl1 = pack8<DT>(res, 8);
    } else {
      pb0 = pack8<DT>(sc, 0);
      pb1 = pack8<DT>(sc, 8);
    }
  };
  // O^T += V^T P^T for dim block db from its two 16-token V^T operands
  auto pv_block = [&](int db, const uint4& va0, const uint4& va1, const uint4& pb0,
                      const uint4& pb1, const uint4& pl0, const uint4& pl1) {
    o[db] = M::mma(va0, pb0, o[db]);
    o[db] = M::mma(va1, pb1, o[db]);
    if constexpr (DT == PA_BF16) {
      o[db] = M::mma(va0, pl0, o[db]);
      o[db] = M::mma(va1, pl1, o[db]);
    }
  };
  // token layout: V rows in registers (token mcol) -> V^T through the identity
  auto compute_tile = [&](int t0, const uint4 (&kr)[KS], const uint4 (&vr)[KS]) {
    uint4 pb0, pb1, pl0, pl1;
    softmax_scores(t0, qk_tile(kr), pb0, pb1, pl0, pl1);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      // V I reproduces the V values exactly, so repacking them is exact
      f32x16_t vt = M::mma(vr[2 * db], eye[0], f32x16_t{});
      vt = M::mma(vr[2 * db + 1], eye[1], vt);
      pv_block(db, pack8_exact<DT>(vt, 0), pack8_exact<DT>(vt, 8), pb0, pb1, pl0, pl1);
    }
  };

  if constexpr (ROWS) {
    // All four waves walk the workgroup's tokens [tok0, wg_end) in step, kTps
    // 32-token tiles per step: the step's tiles are read from one LDS stage
    // while the next step's are loaded into registers and then stored to the
    // other stage; one barrier per step.  The loop bounds are
    // workgroup-uniform, so every wave reaches every barrier, and the last
    // step is peeled off so that every load in the loop is unconditional.
    // (A wave whose rows see no key of a tile skips its compute; a tile of a
    // step that starts past the last key loads the step's first tile again
    // and is skipped.)
    auto compute_from = [&](int t0, const char* base) {
      if (t0 < tok_end) {   // wave-uniform: the wave's rows see keys in this tile
        uint4 kr[KS], va[DB][2];
        lds_read_k(base, kr);
        lds_read_vt(base, va);
        uint4 pb0, pb1, pl0, pl1;
        softmax_scores(t0, qk_tile(kr), pb0, pb1, pl0, pl1);
#pragma unroll
        for (int db = 0; db < DB; ++db) pv_block(db, va[db][0], va[db][1], pb0, pb1, pl0, pl1);
      }
    };
    auto load_step = [&](int t0, u32x4_t (&sk)[kTps][kPer], u32x4_t (&sv)[kTps][kPer]) {
#pragma unroll
      for (int u = 0; u < kTps; ++u) stage_load(t0 + 32 * u < L ? t0 + 32 * u : t0, sk[u], sv[u]);
    };
    auto store_step = [&](char* base, const u32x4_t (&sk)[kTps][kPer],
                          const u32x4_t (&sv)[kTps][kPer]) {
#pragma unroll
      for (int u = 0; u < kTps; ++u) stage_store(base + u * kStageBytes, sk[u], sv[u]);
    };
    auto compute_step = [&](int t0, const char* base) {
#pragma unroll
      for (int u = 0; u < kTps; ++u) compute_from(t0 + 32 * u, base + u * kStageBytes);
    };
    constexpr int kStep = 32 * kTps;
    int t0 = tok0;
    int buf = 0;
    u32x4_t sk[kTps][kPer], sv[kTps][kPer];
    load_step(t0, sk, sv);
    store_step(sm_kv, sk, sv);
    __syncthreads();
    while (t0 + kStep < wg_end) {
      load_step(t0 + kStep, sk, sv);
      __builtin_amdgcn_sched_barrier(0);
      compute_step(t0, sm_kv + buf * kTps * kStageBytes);
      buf ^= 1;
      store_step(sm_kv + buf * kTps * kStageBytes, sk, sv);
      __syncthreads();
      t0 += kStep;
    }
    compute_step(t0, sm_kv + buf * kTps * kStageBytes);
  } else {
    // Each wave takes tiles tok0 + 32 wave, + 32 kWaves, ... and loads them
    // straight into registers in the operand layout (lane (mcol, hh) reads
    // token t0 + mcol, 16 bytes per k-step).  Two register buffers: the next
    // tile's loads are issued (K, then V, before any of the compute) and stay
    // in flight while a tile is computed; the last tile issues nothing, so
    // each wait covers exactly the tile being consumed.
    auto load_tile = [&](int t0, uint4 (&kr)[KS], uint4 (&vr)[KS]) {
      const int t = min(t0 + mcol, L - 1);   // >= t0, since t0 < L
      const int jt = t / B - t0 / B;
      int phys = tblc[min(t0 / B, jlast)];
#pragma unroll
      for (int k = 1; k < kTileBlocks; ++k) {
        const int id = tblc[min(t0 / B + k, jlast)];
        phys = (jt == k) ? id : phys;
      }
      const size_t roff = (((size_t)phys * Hk + g) * B + (t % B)) * kRowBytes + hh * 16;
      const uint4* kp = reinterpret_cast<const uint4*>(kbase + roff);
      const uint4* vp = reinterpret_cast<const uint4*>(vbase + roff);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kr[ks] = kp[2 * ks];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) vr[ks] = vp[2 * ks];
    };
    constexpr int kStride = 32 * kWaves;
    int t0 = tok0 + 32 * wave;
    if (t0 < tok_end) {
      uint4 k0[KS], v0[KS], k1[KS], v1[KS];
      load_tile(t0, k0, v0);
      for (;;) {
        if (t0 + kStride >= tok_end) {
          compute_tile(t0, k0, v0);
          break;
        }
        load_tile(t0 + kStride, k1, v1);
        __builtin_amdgcn_sched_barrier(0);
        compute_tile(t0, k0, v0);
        t0 += kStride;
        if (t0 + kStride >= tok_end) {
          compute_tile(t0, k1, v1);
          break;
        }
        load_tile(t0 + kStride, k0, v0);
        __builtin_amdgcn_sched_barrier(0);
        compute_tile(t0, k1, v1);
        t0 += kStride;
      }
    }
  }

  if constexpr (!ROWS) {
    // merge the waves' states through LDS, one wave at a time, into wave 0
    __shared__ float sm_o[32][D + 4];
    __shared__ float sm_m[32], sm_l[32];
    for (int w = 1; w < kWaves; ++w) {
      if (wave == w) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v) sm_o[mcol][32 * db + tile_token(v, hh)] = o[db][v];
        if (hh == 0) {
          sm_m[mcol] = m_run;
          sm_l[mcol] = l_run;
        }
      }
      __syncthreads();
      if (wave == 0) {
        const float m2 = sm_m[mcol], l2 = sm_l[mcol];
        const float mxw = fmaxf(m_run, m2);
        const float ms = (mxw == kNegInf) ? 0.f : mxw;
        const float a1 = fast_exp2(m_run - ms), a2 = fast_exp2(m2 - ms);
        l_run = l_run * a1 + l2 * a2;
        m_run = mxw;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            o[db][v] = o[db][v] * a1 + sm_o[mcol][32 * db + tile_token(v, hh)] * a2;
      }
      __syncthreads();
    }
    if (wave != 0) return;
  }
  if (!row_ok) return;

  // lane (mcol, hh) holds dims 32 db + 8 c + 4 hh + (0..3) of its row
  if (parts_row <= 1) {
    if (p != 0) return;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        store_out(a.out, out_row * D + 32 * db + tile_token(v, hh), o[db][v] * inv, a.out_dtype);
    if (a.lse && hh == 0) a.lse[out_row] = lse2_of(m_run, l_run);
  } else if (p < parts_row) {
    const size_t slot = out_row * a.max_parts + p;
    float* po = a.ws_o + slot * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<float4*>(po + 32 * db + 8 * c + 4 * hh) =
            make_float4(o[db][4 * c], o[db][4 * c + 1], o[db][4 * c + 2], o[db][4 * c + 3]);
    if (hh == 0) {
      a.ws_ml[2 * slot] = m_run;
      a.ws_ml[2 * slot + 1] = l_run;
    }
  }
}

// The two layouts as kernels.  The rows layout fits two waves per SIMD
// (it holds one staged chunk per thread instead of two register tiles per
// wave), which lets one wave's softmax overlap the other's matrix products.
template <int DT, int D, int B>
__global__ __launch_bounds__(kThreads) void multiq_mfma_kernel(const AttnArgs a) {
  multiq_mfma_body<DT, D, B, false>(a);
}

template <int DT, int D, int B>
__global__ __launch_bounds__(kThreads, 2) void multiq_mfma_rows_kernel(const AttnArgs a) {
  multiq_mfma_body<DT, D, B, true>(a);
}

hipError_t launch_merge(int head_dim, int num_seqs, const AttnArgs& a, hipStream_t st);

template <int DT, int D, int B>
static hipError_t launch_mfma_t(int num_seqs, const AttnArgs& a, hipStream_t st,
                                const KernelEvents& ev) {
  const int rt_count = (a.max_q_len * a.group + 31) / 32;
  const bool rows = multiq_rows_mode(a.max_q_len, a.group);
  const int units = rows ? (rt_count + kWaves - 1) / kWaves : rt_count;
  dim3 grid(units * a.max_parts * a.num_kv_heads * num_seqs);
  const hipError_t e =
      rows ? launch_main(multiq_mfma_rows_kernel<DT, D, B>, grid, dim3(kThreads), 0, st, ev, a)
           : launch_main(multiq_mfma_kernel<DT, D, B>, grid, dim3(kThreads), 0, st, ev, a);
  if (e != hipSuccess || a.max_parts <= 1 || a.no_merge) return e;
  return launch_merge(D, num_seqs, a, st);
}

template <int DT, int D>
static hipError_t dispatch_mfma_b(int block_size, int num_seqs, const AttnArgs& a,
                                  hipStream_t st, const KernelEvents& ev) {
  switch (block_size) {
    case 8: return launch_mfma_t<DT, D, 8>(num_seqs, a, st, ev);
    case 16: return launch_mfma_t<DT, D, 16>(num_seqs, a, st, ev);
    default: return launch_mfma_t<DT, D, 32>(num_seqs, a, st, ev);
  }
}

template <int DT>
static hipError_t dispatch_mfma(int head_dim, int block_size, int num_seqs, const AttnArgs& a,
                                hipStream_t st, const KernelEvents& ev) {
  if (head_dim == 64) return dispatch_mfma_b<DT, 64>(block_size, num_seqs, a, st, ev);
  return dispatch_mfma_b<DT, 128>(block_size, num_seqs, a, st, ev);
}

hipError_t launch_multiq(int dtype, int head_dim, int block_size, int group, int num_seqs,
                         const AttnArgs& a, hipStream_t st, const KernelEvents& ev) {
  if (dtype == PA_BF16) return dispatch_mfma<PA_BF16>(head_dim, block_size, num_seqs, a, st, ev);
  if (dtype == PA_F16) return dispatch_mfma<PA_F16>(head_dim, block_size, num_seqs, a, st, ev);
  // fp32: vector-ALU path, each query row as a decode row over its visible length
  return launch_decode(dtype, head_dim, block_size, group, num_seqs, a, st, ev);
}

}  // namespace pa
