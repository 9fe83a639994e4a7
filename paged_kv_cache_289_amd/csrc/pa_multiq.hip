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
//                    as both operands share it).  With V staged in LDS
//                    (rows layout, and the token layout at head_dim 128) two
//                    LDS transpose reads (ds_read_b64_tr_b16) give it per
//                    16-token step; with V loaded straight into registers
//                    (token layout at head_dim 64) an MFMA of V with an
//                    identity puts V into that layout.
//
// Work split, few rows per KV head (token layout): by default (head_dim 128)
// a balanced split hands every resident wave an equal share of the flattened
// (sequence, KV head, row tile, key tile) list, and a merge kernel combines
// the pieces of units that several waves share; with fixed partitions the
// four waves of a workgroup split one partition's tiles and merge through
// LDS, then write the final output or a partial for merge_kernel.  Many rows
// (rows layout): four row tiles per workgroup share each staged K/V tile.
// fp32: every query row runs the decode kernel over its own visible length.
#include <atomic>
#include <type_traits>

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

// S^T = K Q^T of one 32-token tile: lane (m, hh) gets the scores of row m for
// tokens t0 + tile_token(v, hh)
template <int DT, int KS>
__device__ __forceinline__ f32x16_t tile_qk(const uint4 (&kr)[KS], const uint4 (&qv)[KS]) {
  f32x16_t sc = f32x16_t{};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) sc = Mma<DT>::mma(kr[ks], qv[ks], sc);
  return sc;
}

// Masking and the online softmax of one tile's scores: keys at or past lim
// (this lane's row) are masked unless the whole tile is visible to every row
// of the wave (`unmasked`, wave-uniform).  Updates the running (m, l, o) and
// returns the P^T operands (pb: p rounded or cut to the input dtype, pl: bf16
// residual).
template <int DT, int DB>
__device__ __forceinline__ void tile_softmax(f32x16_t sc, int t0, int hh, bool unmasked, int lim,
                                             float c, float& m_run, float& l_run,
                                             f32x16_t (&o)[DB], uint4& pb0, uint4& pb1,
                                             uint4& pl0, uint4& pl1) {
  float mx = kNegInf;
  if (unmasked) {
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
}

// O^T += V^T P^T for one 32-dim block from its two 16-token V^T operands
template <int DT>
__device__ __forceinline__ void tile_pv(f32x16_t& o, const uint4& va0, const uint4& va1,
                                        const uint4& pb0, const uint4& pb1, const uint4& pl0,
                                        const uint4& pl1) {
  o = Mma<DT>::mma(va0, pb0, o);
  o = Mma<DT>::mma(va1, pb1, o);
  if constexpr (DT == PA_BF16) {
    o = Mma<DT>::mma(va0, pl0, o);
    o = Mma<DT>::mma(va1, pl1, o);
  }
}

// Q^T operand of lane (m, hh): its row's query (token, head) out_row, dims
// 16 ks + 8 hh .. +7 (zeros for a lane without a row).  A negative scale goes
// into q's sign bits (exact), so the scores are scaled by a positive c inside
// the exponent's FMA.
template <int D>
__device__ __forceinline__ void load_q_operand(const void* q, size_t out_row, int hh, bool row_ok,
                                               float scale_log2, uint4 (&qv)[D / 16]) {
  constexpr int KS = D / 16;
  const uint4* qp = reinterpret_cast<const uint4*>(q) + (out_row * D + hh * 8) / 8;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qv[ks] = row_ok ? qp[2 * ks] : make_uint4(0, 0, 0, 0);
  if (scale_log2 < 0.f) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qv[ks].x ^= 0x80008000u; qv[ks].y ^= 0x80008000u;
      qv[ks].z ^= 0x80008000u; qv[ks].w ^= 0x80008000u;
    }
  }
}

// Token layout at head_dim 128: one wave walks 32-token tiles of one
// (sequence, KV head) through its own two 8 KiB LDS stages, one for the K tile
// and one for the V tile.  Both arrive by direct-to-LDS loads: a wave
// instruction moves four whole token rows (1 KiB, every lane 16 bytes), which
// keeps each load instruction on eight full 128-byte lines (loading K straight
// into the operand layout would touch 32 rows per instruction, 32 bytes of
// each).  Each stage row's 16-byte chunks are permuted (an XOR on the chunk
// index, see below) so that the operand reads out of LDS hit distinct banks.
// Tokens at or past L are clamped to the last valid one (their slots may hold
// anything) and masked in the scores.
template <int B>
struct TokenTileWalker {
  static constexpr int kRowBytes = 256;            // 128 16-bit elements
  static constexpr int kStageBytes = 32 * kRowBytes;
  static constexpr int kTileBlocks = 32 / B;
  static constexpr int KS = 8, DB = 4;
  const char* kbase;
  const char* vbase;
  ConstI32Ptr tblc;   // the sequence's block table
  int jlast;          // its last block, (L - 1) / B
  int L, Hk, g, lane;

  // physical block of token t of the tile at t0 (block ids from scalar loads)
  __device__ __forceinline__ int phys_of(int t0, int t) const {
    const int jt = t / B - t0 / B;
    int phys = tblc[min(t0 / B, jlast)];
#pragma unroll
    for (int k = 1; k < kTileBlocks; ++k) {
      const int id = tblc[min(t0 / B + k, jlast)];
      phys = (jt == k) ? id : phys;
    }
    return phys;
  }
  __device__ __forceinline__ size_t row_off(int phys, int t) const {
    return (((size_t)phys * Hk + g) * B + (t % B)) * kRowBytes;
  }
  // V stage: 16-byte chunk c of row r sits at position c ^ 4 (r mod 4), which
  // keeps the transpose reads (four rows by two chunks per 16 lanes) on
  // distinct banks.
  // V^T operands for dim block db and 16-token step ks: dim 32 db + m, tokens
  // 16 ks + 4 hh + (0..3) then 16 ks + 8 + 4 hh + (0..3), the order of the
  // lane's probabilities.  In a transpose read, lane i of each 16-lane group
  // addresses row r0 + i / 4 at dims c0 + 4 (i % 4) .. + 3, and lane j
  // receives dim c0 + j of rows r0 .. r0 + 3.
  __device__ __forceinline__ void read_vt(const char* stage, uint4 (&va)[DB][2]) const {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) v4i16 LdsV4;
    const int hh = lane >> 5;
    const int rsub = (lane & 15) / 4;
    const int cl = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
    const int off = (lane & 1) * 8;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int r0 = 16 * ks + 4 * hh + rsub, r1 = r0 + 8;
        const int c = 4 * db + cl;
        const char* p0 = stage + r0 * kRowBytes + ((c ^ (4 * (r0 & 3))) * 16) + off;
        const char* p1 = stage + r1 * kRowBytes + ((c ^ (4 * (r1 & 3))) * 16) + off;
        const auto lo = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                      (LdsV4*)(__attribute__((address_space(3))) char*)p0));
        const auto hi = __builtin_bit_cast(uint2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                      (LdsV4*)(__attribute__((address_space(3))) char*)p1));
        va[db][ks] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
  }

  // K stage: instruction i: lane l writes stage bytes 1024 i + 16 l, i.e. row
  // r = 4 i + l / 16 at position l % 16, which holds chunk (l % 16) ^ (r mod 16);
  // lane (m, hh) then reads chunk 2 ks + hh of row m, its operand for k-step ks
  // (16 rows of one lane half hit 16 distinct positions: no bank conflict).
  // NT: the non-temporal hint.
  template <bool NT>
  __device__ __forceinline__ void load_k(int t0, char* stage) const {
    load_k_part<NT, 8>(t0, stage, 0);
  }
  // instructions i0 .. i0 + N - 1 of load_k (tile rows 4 i0 .. 4 (i0 + N) - 1)
  template <bool NT, int N>
  __device__ __forceinline__ void load_k_part(int t0, char* stage, int i0) const {
    const int krow = lane >> 4;
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int i = i0 + j;
      const int r = 4 * i + krow;
      const int t = min(t0 + r, L - 1);
      const char* src = kbase + row_off(phys_of(t0, t), t) + (((lane & 15) ^ (r & 15)) * 16);
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(stage + 1024 * i),
                                       16, 0, NT ? kCpolNt : 0);
    }
  }
  __device__ __forceinline__ void read_k(const char* stage, uint4 (&kr)[KS]) const {
    typedef unsigned int u4v __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) const u4v LdsU4;
    const int m = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cpos = (2 * ks + hh) ^ (m & 15);
      const u4v x = *(LdsU4*)(__attribute__((address_space(3))) const char*)(stage + m * kRowBytes +
                                                                              cpos * 16);
      kr[ks] = make_uint4(x.x, x.y, x.z, x.w);
    }
  }
  // V stage: instruction i: lane l writes row 4 i + l / 16 at position l % 16,
  // which holds chunk (l % 16) ^ 4 (l / 16)
  template <bool NT>
  __device__ __forceinline__ void load_v(int t0, char* stage) const {
    load_v_part<NT, 8>(t0, stage, 0);
  }
  template <bool NT, int N>
  __device__ __forceinline__ void load_v_part(int t0, char* stage, int i0) const {
    const int vrow = lane >> 4, vchunk = (lane & 15) ^ (4 * (lane >> 4));
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int i = i0 + j;
      const int t = min(t0 + 4 * i + vrow, L - 1);
      const char* src = vbase + row_off(phys_of(t0, t), t) + vchunk * 16;
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(stage + 1024 * i),
                                       16, 0, NT ? kCpolNt : 0);
    }
  }

  // This lane's byte offsets, inside a stage, of its K operand chunks
  // (k-steps 0..7, as read_k) and of its V^T rows (dim blocks 0..3, as
  // read_vt; the second 16-token step and the second half of each add 4096
  // and 2048), plus `base`.
  __device__ __forceinline__ void lane_offsets(unsigned base, unsigned (&koff)[KS],
                                               unsigned (&voff)[DB]) const {
    const int m = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      koff[ks] = base + m * kRowBytes + (((2 * ks + hh) ^ (m & 15)) * 16);
    const int rsub = (lane & 15) / 4;
    const int cl = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int db = 0; db < DB; ++db)
      voff[db] = base + (4 * hh + rsub) * kRowBytes + (((4 * db + cl) ^ (4 * rsub)) * 16) +
                 (lane & 1) * 8;
  }
  // read_k and read_vt of one stage (K at byte KO past the offsets' base, V at
  // KO + 8192) in one asm block that ends by waiting for its own reads.  For
  // a stage read while loads into other stages are in flight: the compiler,
  // which cannot tell the stages apart, would wait for every load in flight
  // before a read it issues itself.
  template <int KO>
  __device__ __forceinline__ void read_stage_asm(const unsigned (&koff)[KS],
                                                 const unsigned (&voff)[DB], uint4 (&kr)[KS],
                                                 uint4 (&va)[DB][2]) const {
    typedef unsigned int u4v __attribute__((ext_vector_type(4)));
    typedef unsigned int u2v __attribute__((ext_vector_type(2)));
    u4v k[8];
    u2v v[4][4];
    asm volatile(
        "ds_read_b128 %0, %24 offset:%36\n\t"
        "ds_read_b128 %1, %25 offset:%36\n\t"
        "ds_read_b128 %2, %26 offset:%36\n\t"
        "ds_read_b128 %3, %27 offset:%36\n\t"
        "ds_read_b128 %4, %28 offset:%36\n\t"
        "ds_read_b128 %5, %29 offset:%36\n\t"
        "ds_read_b128 %6, %30 offset:%36\n\t"
        "ds_read_b128 %7, %31 offset:%36\n\t"
        "ds_read_b64_tr_b16 %8, %32 offset:%37\n\t"
        "ds_read_b64_tr_b16 %9, %32 offset:%38\n\t"
        "ds_read_b64_tr_b16 %10, %32 offset:%39\n\t"
        "ds_read_b64_tr_b16 %11, %32 offset:%40\n\t"
        "ds_read_b64_tr_b16 %12, %33 offset:%37\n\t"
        "ds_read_b64_tr_b16 %13, %33 offset:%38\n\t"
        "ds_read_b64_tr_b16 %14, %33 offset:%39\n\t"
        "ds_read_b64_tr_b16 %15, %33 offset:%40\n\t"
        "ds_read_b64_tr_b16 %16, %34 offset:%37\n\t"
        "ds_read_b64_tr_b16 %17, %34 offset:%38\n\t"
        "ds_read_b64_tr_b16 %18, %34 offset:%39\n\t"
        "ds_read_b64_tr_b16 %19, %34 offset:%40\n\t"
        "ds_read_b64_tr_b16 %20, %35 offset:%37\n\t"
        "ds_read_b64_tr_b16 %21, %35 offset:%38\n\t"
        "ds_read_b64_tr_b16 %22, %35 offset:%39\n\t"
        "ds_read_b64_tr_b16 %23, %35 offset:%40\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=v"(k[0]), "=v"(k[1]), "=v"(k[2]), "=v"(k[3]), "=v"(k[4]), "=v"(k[5]), "=v"(k[6]),
          "=v"(k[7]), "=v"(v[0][0]), "=v"(v[0][1]), "=v"(v[0][2]), "=v"(v[0][3]),
          "=v"(v[1][0]), "=v"(v[1][1]), "=v"(v[1][2]), "=v"(v[1][3]), "=v"(v[2][0]),
          "=v"(v[2][1]), "=v"(v[2][2]), "=v"(v[2][3]), "=v"(v[3][0]), "=v"(v[3][1]),
          "=v"(v[3][2]), "=v"(v[3][3])
        : "v"(koff[0]), "v"(koff[1]), "v"(koff[2]), "v"(koff[3]), "v"(koff[4]), "v"(koff[5]),
          "v"(koff[6]), "v"(koff[7]), "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]),
          "i"(KO), "i"(KO + 8192), "i"(KO + 8192 + 2048), "i"(KO + 8192 + 4096),
          "i"(KO + 8192 + 6144)
        : "memory");
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kr[ks] = make_uint4(k[ks].x, k[ks].y, k[ks].z, k[ks].w);
    // per dim block: 16-token step 0 (rows, rows + 8), then step 1
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        va[db][ks] = make_uint4(v[db][2 * ks].x, v[db][2 * ks].y, v[db][2 * ks + 1].x,
                                v[db][2 * ks + 1].y);
  }

  // The tiles t0, t0 + stride, ... below t_end (t0 < t_end, wave-uniform)
  // into the running (m, l, o); keys at or past lim are masked, and a tile
  // ending at or before unmask_end (wave-uniform) needs no mask.  Each step
  // waits for its tile, reads all of its operands out of the stages, and only
  // then (once those reads are back) loads the next tile into the same stages,
  // so the loads are in flight for the whole of the tile's compute.
  template <int DT, bool NT>
  __device__ __forceinline__ void walk(int t0, int t_end, int stride, const uint4 (&qv)[KS],
                                       float c, int lim, int unmask_end, char* kst, char* vst,
                                       f32x16_t (&o)[DB], float& m_run, float& l_run) const {
    const int hh = lane >> 5;
    t_end = __builtin_amdgcn_readfirstlane(t_end);
    load_k<NT>(t0, kst);
    load_v<NT>(t0, vst);
    for (;;) {
      uint4 kr[KS];
      read_k(kst, kr);
      uint4 va[DB][2];
      read_vt(vst, va);
      const bool more = t0 + stride < t_end;   // wave-uniform
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): the stages are read
      __builtin_amdgcn_sched_barrier(0);
      if (more) {
        load_k<NT>(t0 + stride, kst);
        load_v<NT>(t0 + stride, vst);
      }
      const f32x16_t sc = tile_qk<DT>(kr, qv);
      uint4 pb0, pb1, pl0, pl1;
      tile_softmax<DT>(sc, t0, hh, t0 + 32 <= unmask_end, lim, c, m_run, l_run, o, pb0, pb1, pl0,
                       pl1);
#pragma unroll
      for (int db = 0; db < DB; ++db) tile_pv<DT>(o[db], va[db][0], va[db][1], pb0, pb1, pl0, pl1);
      if (!more) break;
      t0 += stride;
    }
  }
};

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
  load_q_operand<D>(a.q, out_row, hh, row_ok, a.scale_log2, qv);
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
  // token layout at head_dim 128: a K stage and a V stage of 32 rows per wave
  constexpr bool kStaged = !ROWS && D == 128;
  constexpr int kVTile = 32 * kRowBytes;
  __shared__ __attribute__((aligned(16))) char sm_kst[kStaged ? kWaves * kVTile : 16];
  __shared__ __attribute__((aligned(16))) char sm_vst[kStaged ? kWaves * kVTile : 16];
  // rows layout at head_dim 128: four stages, each a K tile and then its V
  // tile (16 KiB), filled by direct-to-LDS loads
  constexpr bool kPipe = ROWS && D == 128;
  constexpr int kPipeStage = 2 * 32 * kRowBytes;
  __shared__ __attribute__((aligned(16))) char sm_pipe[kPipe ? 4 * kPipeStage : 16];
  // rows layout at head_dim 64: 32-token tiles per loop step, and two LDS
  // stages of a step each
  constexpr int kTps = 1;
  constexpr int kLdsBytes = (ROWS && !kPipe) ? 2 * kTps * kStageBytes : 16;
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

  auto qk_tile = [&](const uint4 (&kr)[KS]) { return tile_qk<DT>(kr, qv); };
  auto softmax_scores = [&](int t0, f32x16_t sc, uint4& pb0, uint4& pb1, uint4& pl0,
                            uint4& pl1) {
    tile_softmax<DT>(sc, t0, hh, t0 + 32 <= min(l_tile_min, tok_end), lim, c, m_run, l_run, o,
                     pb0, pb1, pl0, pl1);
  };
  auto pv_block = [&](int db, const uint4& va0, const uint4& va1, const uint4& pb0,
                      const uint4& pb1, const uint4& pl0, const uint4& pl1) {
    tile_pv<DT>(o[db], va0, va1, pb0, pb1, pl0, pl1);
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

  if constexpr (kPipe) {
    // All four waves walk the workgroup's tiles tok0 + 32 i, i < nT, in step.
    // Tile i sits in stage i mod 4; each wave loads a quarter of it (two of
    // the eight load instructions of K and two of V, tile rows 8 wave ..
    // 8 wave + 7) three steps ahead.  Step i: wait for this wave's loads of
    // tile i (the eight issued after them, tiles i + 1 and i + 2, stay in
    // flight), a barrier (every wave's quarter has landed, and every wave is
    // past step i - 1, whose stage the loads of tile i + 3 then overwrite),
    // read this wave's operands, issue tile i + 3, compute.  Past the last
    // tile the loads repeat tile nT - 1 into a stage nobody reads again, so
    // every step issues the same loads and waits the same count.  The loop
    // bounds are workgroup-uniform, so every wave reaches every barrier; a
    // wave whose rows see no key of a tile skips its reads and compute.
    const TokenTileWalker<B> w{kbase, vbase, tblc, jlast, L, Hk, g, lane};
    const unsigned pipe0 = (unsigned)(size_t)(__attribute__((address_space(3))) char*)sm_pipe;
    unsigned koff[KS], voff[DB];
    w.lane_offsets(pipe0, koff, voff);
    // full tiles: this lane's byte offsets inside the block of its rows, for
    // load instruction j of this wave (row r = 8 wave + 4 j + lane / 16 of
    // the tile, at slot r mod B of block r / B; position lane % 16 holds
    // chunk (lane % 16) ^ (r mod 16) of K, (lane % 16) ^ 4 (r mod 4) of V)
    const int lrow = lane >> 4;
    const unsigned lck = (unsigned)((lane & 15) ^ lrow);
    const unsigned cv = (unsigned)(((lane & 15) ^ (4 * lrow)) << 4);
    const size_t head_off = (size_t)g * B * kRowBytes;
    const int nT = (wg_end - tok0 + 31) / 32;   // >= 1
    auto issue = [&](int i, char* st) {
      const int t0 = tok0 + 32 * min(i, nT - 1);
      if (t0 + 32 <= L) {   // workgroup-uniform: block ids and bases are scalar
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int r = 8 * wave + 4 * j;   // the instruction's first row
          const size_t boff = ((size_t)tblc[(t0 + r) / B] * Hk) * B * kRowBytes + head_off;
          const unsigned row = (unsigned)((r % B + lrow) * kRowBytes);
          const unsigned offk = row + ((lck ^ (unsigned)(r & 12)) << 4);
          char* dst = st + 1024 * (2 * wave + j);
          __builtin_amdgcn_global_load_lds(kbase + boff + offk,
                                           (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
          __builtin_amdgcn_global_load_lds(vbase + boff + row + cv,
                                           (__attribute__((address_space(3))) void*)(dst + 8192),
                                           16, 0, 0);
        }
      } else {
        w.template load_k_part<false, 2>(t0, st, 2 * wave);
        w.template load_v_part<false, 2>(t0, st + 8192, 2 * wave);
      }
    };
    // the query operands first (vmcnt(0)): with them still in flight at the
    // loop the compiler would wait for every load before entering it
    __builtin_amdgcn_s_waitcnt(0x0F70);
    issue(0, sm_pipe);
    issue(1, sm_pipe + kPipeStage);
    issue(2, sm_pipe + 2 * kPipeStage);
    auto step = [&](int i, auto stage) {
      constexpr int S = decltype(stage)::value;
      // s_waitcnt vmcnt(8), other counters untouched; then a bare barrier
      // (__syncthreads() also fences global memory, which would wait for
      // every load in flight)
      __builtin_amdgcn_s_waitcnt(0x0F78);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      const int t0 = tok0 + 32 * i;
      const bool mine = t0 < tok_end;   // wave-uniform
      uint4 kr[KS], va[DB][2];
      if (mine) w.template read_stage_asm<S * kPipeStage>(koff, voff, kr, va);
      __builtin_amdgcn_sched_barrier(0);
      issue(i + 3, sm_pipe + ((S + 3) % 4) * kPipeStage);
      __builtin_amdgcn_sched_barrier(0);
      if (mine) {
        uint4 pb0, pb1, pl0, pl1;
        softmax_scores(t0, qk_tile(kr), pb0, pb1, pl0, pl1);
#pragma unroll
        for (int db = 0; db < DB; ++db) pv_block(db, va[db][0], va[db][1], pb0, pb1, pl0, pl1);
      }
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;
    for (int i = 0; i < nT; i += 4) {
      step(i, S0{});
      if (i + 1 >= nT) break;
      step(i + 1, S1{});
      if (i + 2 >= nT) break;
      step(i + 2, S2{});
      if (i + 3 >= nT) break;
      step(i + 3, S3{});
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): no load into LDS outlives the wave
  } else if constexpr (ROWS) {
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
  } else if constexpr (kStaged) {
    // Each wave takes tiles tok0 + 32 wave, + 32 kWaves, ... through its own
    // K and V stages (cached loads: partitions of one sequence may share lines)
    const int t0 = tok0 + 32 * wave;
    if (t0 < tok_end) {
      const TokenTileWalker<B> w{kbase, vbase, tblc, jlast, L, Hk, g, lane};
      w.template walk<DT, false>(t0, tok_end, 32 * kWaves, qv, c, lim, min(l_tile_min, tok_end),
                                 sm_kst + wave * kVTile, sm_vst + wave * kVTile, o, m_run, l_run);
    }
  } else {
    // (head_dim 64) Each wave takes tiles tok0 + 32 wave, + 32 kWaves, ...
    // and loads them straight into registers in the operand layout (lane (mcol, hh) reads
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
    // (at head_dim 128 in the waves' K stages, once every wave is past them)
    typedef float MergeO[32][D + 4];
    __shared__ float sm_o_own[kStaged ? 1 : 32][kStaged ? 1 : D + 4];
    __shared__ float sm_m[32], sm_l[32];
    static_assert(!kStaged || sizeof(MergeO) <= kWaves * kVTile, "merge area");
    if constexpr (kStaged) __syncthreads();
    MergeO& sm_o = *reinterpret_cast<MergeO*>(kStaged ? (void*)sm_kst : (void*)sm_o_own);
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

// The two layouts as kernels, both at two waves per SIMD, which lets one
// wave's softmax and loads overlap the other's matrix products.  (The rows
// layout holds one staged chunk per thread; the token layout at head_dim 128
// keeps only K in registers and stages V in LDS.)
template <int DT, int D, int B>
__global__ __launch_bounds__(kThreads, 2) void multiq_mfma_kernel(const AttnArgs a) {
  multiq_mfma_body<DT, D, B, false>(a);
}

template <int DT, int D, int B>
__global__ __launch_bounds__(kThreads, 2) void multiq_mfma_rows_kernel(const AttnArgs a) {
  multiq_mfma_body<DT, D, B, true>(a);
}

// 8-bit E4M3 K/V at head_dim 128 (the decode of an 8-bit cache through the
// balanced split): the codes of a 32-token tile reach the wave's stages by
// direct-to-LDS loads (a wave instruction moves eight 128-byte rows) and are
// widened to f16 on their way into the operands (exact: every E4M3 value is an
// f16 value); the products run in f16 with fp32 accumulation.  Stages: the K
// codes (4 KiB) and the V codes (4 KiB) in one 8 KiB stage, and V widened to
// f16 in a second 8 KiB stage with the 16-bit layout, read by transpose reads.
template <int B>
struct Fp8TileWalker {
  static constexpr int kRowBytes = 128;   // 128 codes
  static constexpr int kTileBlocks = 32 / B;
  static constexpr int KS = 8, DB = 4;
  const char* kbase;
  const char* vbase;
  ConstI32Ptr tblc;   // the sequence's block table
  int jlast;          // its last block, (L - 1) / B
  int L, Hk, g, lane;

  __device__ __forceinline__ int phys_of(int t0, int t) const {
    const int jt = t / B - t0 / B;
    int phys = tblc[min(t0 / B, jlast)];
#pragma unroll
    for (int k = 1; k < kTileBlocks; ++k) {
      const int id = tblc[min(t0 / B + k, jlast)];
      phys = (jt == k) ? id : phys;
    }
    return phys;
  }
  __device__ __forceinline__ size_t row_off(int phys, int t) const {
    return (((size_t)phys * Hk + g) * B + (t % B)) * kRowBytes;
  }
  // instruction i: lane l writes stage bytes 1024 i + 16 l, i.e. row
  // r = 8 i + l / 8 at position l % 8, which holds 16-byte chunk
  // (l % 8) ^ ((r / 2) mod 8) of K, (l % 8) ^ ((r / 2) mod 4) of V
  template <bool NT, int MASK>
  __device__ __forceinline__ void load_codes(const char* base, int t0, char* stage) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 8 * i + (lane >> 3);
      const int t = min(t0 + r, L - 1);   // >= t0, since t0 < L
      const char* src = base + row_off(phys_of(t0, t), t) + (((lane & 7) ^ ((r >> 1) & MASK)) * 16);
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(stage + 1024 * i),
                                       16, 0, NT ? kCpolNt : 0);
    }
  }
  // eight codes (two words) -> eight f16 (one 16-byte operand)
  __device__ static __forceinline__ uint4 widen8(uint32_t w0, uint32_t w1) {
    const auto a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
    const auto b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
    const auto c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
    const auto d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
    return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                      __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d));
  }
  // K operands: lane (m, hh), k-step ks: codes 16 ks + 8 hh .. + 7 of row m
  // (chunk ks at position ks ^ ((m / 2) mod 8): the 16 rows of one lane half
  // fall on distinct banks)
  __device__ __forceinline__ void read_k(const char* stage, uint4 (&kr)[KS]) const {
    typedef unsigned int u2v __attribute__((ext_vector_type(2)));
    const int m = lane & 31, hh = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int pos = ks ^ ((m >> 1) & 7);
      const u2v x = *(__attribute__((address_space(3))) const u2v*)(
          __attribute__((address_space(3))) const char*)(stage + m * kRowBytes + pos * 16 + hh * 8);
      kr[ks] = widen8(x.x, x.y);
    }
  }
  // V codes -> f16 rows of 256 bytes, 16-byte chunk c of row r at position
  // c ^ 4 (r mod 4): lane l widens half l % 2 of row l / 2
  __device__ __forceinline__ void widen_v(const char* v8, char* v16) const {
    typedef unsigned int u4v __attribute__((ext_vector_type(4)));
    const int r = lane >> 1, h = lane & 1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = 4 * h + j;            // codes 16 c .. 16 c + 15
      const u4v x = *(__attribute__((address_space(3))) const u4v*)(
          __attribute__((address_space(3))) const char*)(v8 + r * kRowBytes + ((c ^ ((r >> 1) & 3)) * 16));
      const uint4 lo = widen8(x.x, x.y), hi = widen8(x.z, x.w);
      *(__attribute__((address_space(3))) u4v*)(__attribute__((address_space(3))) char*)(
          v16 + r * 256 + (((2 * c) ^ (4 * (r & 3))) * 16)) = u4v{lo.x, lo.y, lo.z, lo.w};
      *(__attribute__((address_space(3))) u4v*)(__attribute__((address_space(3))) char*)(
          v16 + r * 256 + (((2 * c + 1) ^ (4 * (r & 3))) * 16)) = u4v{hi.x, hi.y, hi.z, hi.w};
    }
  }
  // The tiles t0, t0 + stride, ... below t_end, as TokenTileWalker::walk:
  // each step reads its K operands and widens its V, then (once those LDS
  // accesses are back) loads the next tile's codes into the same stage.
  // kst: the K codes, then the V codes; v16: V in f16.
  template <bool NT>
  __device__ __forceinline__ void walk(int t0, int t_end, int stride, const uint4 (&qv)[KS],
                                       float c, int lim, int unmask_end, char* kst, char* v16,
                                       f32x16_t (&o)[DB], float& m_run, float& l_run) const {
    const int hh = lane >> 5;
    const TokenTileWalker<B> t16{nullptr, nullptr, tblc, jlast, L, Hk, g, lane};
    t_end = __builtin_amdgcn_readfirstlane(t_end);
    load_codes<NT, 7>(kbase, t0, kst);
    load_codes<NT, 3>(vbase, t0, kst + 4096);
    for (;;) {
      uint4 kr[KS];
      read_k(kst, kr);
      widen_v(kst + 4096, v16);
      uint4 va[DB][2];
      t16.read_vt(v16, va);
      const bool more = t0 + stride < t_end;   // wave-uniform
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): the stage is read
      __builtin_amdgcn_sched_barrier(0);
      if (more) {
        load_codes<NT, 7>(kbase, t0 + stride, kst);
        load_codes<NT, 3>(vbase, t0 + stride, kst + 4096);
      }
      const f32x16_t sc = tile_qk<PA_F16>(kr, qv);
      uint4 pb0, pb1, pl0, pl1;
      tile_softmax<PA_F16>(sc, t0, hh, t0 + 32 <= unmask_end, lim, c, m_run, l_run, o, pb0, pb1,
                           pl0, pl1);
#pragma unroll
      for (int db = 0; db < DB; ++db)
        tile_pv<PA_F16>(o[db], va[db][0], va[db][1], pb0, pb1, pl0, pl1);
      if (!more) break;
      t0 += stride;
    }
  }
};

// Q^T operand in f16 from bf16 queries (the 8-bit cache's queries): exact for
// |q| in f16's normal range; a negative scale flips the f16 sign bits.
__device__ __forceinline__ void load_q_operand_f16(const void* q, size_t out_row, int hh,
                                                   bool row_ok, float scale_log2,
                                                   uint4 (&qv)[8]) {
  constexpr int D = 128;
  const uint4* qp = reinterpret_cast<const uint4*>(q) + (out_row * D + hh * 8) / 8;
  auto cv = [](uint32_t w) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w << 16),
                                                                   __uint_as_float(w & 0xffff0000u)));
  };
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    const uint4 x = row_ok ? qp[2 * ks] : make_uint4(0, 0, 0, 0);
    qv[ks] = make_uint4(cv(x.x), cv(x.y), cv(x.z), cv(x.w));
    if (scale_log2 < 0.f) {
      qv[ks].x ^= 0x80008000u; qv[ks].y ^= 0x80008000u;
      qv[ks].z ^= 0x80008000u; qv[ks].w ^= 0x80008000u;
    }
  }
}

// ---------------------------------------------------------------------------
// balanced split (token layout, head_dim 128)
// ---------------------------------------------------------------------------
// Units are (sequence s, KV head g, row tile rt): R_s = ceil(n_s G / 32) row
// tiles per KV head.  Each unit of a sequence with n_s > 0 rows and L_s > 0
// keys costs c_s = nt_s + X items: its nt_s = ceil(L_s / 32) key
// tiles plus a fixed cost (the query load, the first tile's latency, the
// stores).  Items are numbered f = pre[s] + (g R_s + rt) c_s + k (pre:
// exclusive prefix sums of Hk R_s c_s); wave w takes f in [w chunk,
// (w + 1) chunk), item k >= X being key tile k - X (X = mq_seg_items(DT)).  So
// every wave does the same work whatever the mix of context lengths, with no
// partition size to choose.  A wave that covers all of a unit's tiles writes
// its rows' outputs; otherwise it leaves its piece (max, sum, unnormalised O
// of the unit's rows) in slot V + w, V = (s Hk + g) Rmax + rt, which
// mq_split_merge_kernel combines.  The waves of a workgroup are independent
// (each has its own K and V stages in LDS).  Workgroup 0 stores the plan for the
// merge: plan[0] = chunk, plan[1] = total items, plan[2 ..] = pre[0 .. S].
struct MqSeqShape {
  int L, n, R, nt;   // keys, rows (tokens), row tiles, key tiles (R = nt = 0: no work)
};
__device__ __forceinline__ MqSeqShape mq_seq_shape(const AttnArgs& a, ConstI32Ptr lens,
                                                   ConstI32Ptr qoff, int s) {
  MqSeqShape r;
  r.L = min(max(lens[s], 0), a.max_context_len);
  // (no query offsets: a decode, one query token per sequence)
  r.n = a.q_offsets ? min(max(qoff[s + 1] - qoff[s], 0), a.max_q_len) : 1;
  r.R = (r.n * a.group + 31) / 32;
  r.nt = (r.L + 31) / 32;
  if (r.R == 0 || r.nt == 0) r.R = r.nt = 0;
  return r;
}

// One wave's share of the split: items [f, f_end), starting r0 items into
// sequence s (NT: the loads carry the non-temporal hint).
template <int DT, int B, bool NT>
__device__ __forceinline__ void mq_split_wave(const AttnArgs& a, int s, int r0, int f, int f_end,
                                              int wid, char* st0, char* st1) {
  using Wk = TokenTileWalker<B>;
  constexpr int D = 128, KS = Wk::KS, DB = Wk::DB, X = mq_seg_items(DT);
  const int H = a.num_heads, Hk = a.num_kv_heads, G = a.group;
  const int Rmax = (a.max_q_len * G + 31) / 32;
  // rows per piece slot: a row tile, or for a decode the group's G rows
  const int prow = a.q_offsets ? 32 : G;
  const int lane = threadIdx.x & 63;
  const ConstI32Ptr lens = as_const(a.context_lens), qoff = as_const(a.q_offsets);
  MqSeqShape sh = mq_seq_shape(a, lens, qoff, s);
  int c = sh.nt + X;                   // items of each unit of s
  int ui = r0 / c, k = r0 % c;
  int g = ui / sh.R, rt = ui % sh.R;
  const int hh = lane >> 5, mcol = lane & 31;
  const float cs = fmaxf(fabsf(a.scale_log2), 1e-30f);
  const char* kbase = static_cast<const char*>(a.k_cache);
  const char* vbase = static_cast<const char*>(a.v_cache);

  while (f < f_end) {
    if (k < X) {                       // the unit's own cost: no tile
      f += X - k;
      k = X;
      if (f >= f_end) break;
    }
    const int j = k - X;               // first key tile of this piece
    const int n_here = min(sh.nt - j, f_end - f);
    const int L = sh.L, n = sh.n;
    const int n_rows = n * G;
    const int r = rt * 32 + mcol;
    const bool row_ok = r < n_rows;
    const int qi = row_ok ? r / G : 0;
    const int qh = row_ok ? r % G : 0;
    auto visible = [&](int i) { return a.causal ? max(0, min(L, L - n + i + 1)) : L; };
    const int lrow = row_ok ? visible(qi) : 0;
    const int l_tile_max = visible(min(rt * 32 + 31, n_rows - 1) / G);
    const int l_tile_min = visible((rt * 32) / G);
    const size_t out_row = (size_t)((a.q_offsets ? qoff[s] : s) + qi) * H + (size_t)g * G + qh;
    uint4 qv[KS];
    if constexpr (DT == PA_FP8_E4M3)
      load_q_operand_f16(a.q, out_row, hh, row_ok, a.scale_log2, qv);
    else
      load_q_operand<D>(a.q, out_row, hh, row_ok, a.scale_log2, qv);
    f32x16_t o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x16_t{};
    float m_run = kMaxInit, l_run = 0.f;
    const int seg_end = min(32 * (j + n_here), l_tile_max);
    if (32 * j < seg_end) {            // (a causal row tile may see fewer tiles)
      const ConstI32Ptr tbl = as_const(a.block_tables + (size_t)s * a.max_blocks_per_seq);
      if constexpr (DT == PA_FP8_E4M3) {
        const Fp8TileWalker<B> w{kbase, vbase, tbl, (L - 1) / B, L, Hk, g, lane};
        w.template walk<NT>(32 * j, seg_end, 32, qv, cs, min(lrow, seg_end),
                            min(l_tile_min, seg_end), st0, st1, o, m_run, l_run);
      } else {
        const Wk w{kbase, vbase, tbl, (L - 1) / B, L, Hk, g, lane};
        w.template walk<DT, NT>(32 * j, seg_end, 32, qv, cs, min(lrow, seg_end),
                                min(l_tile_min, seg_end), st0, st1, o, m_run, l_run);
      }
    }
    if (j == 0 && n_here == sh.nt) {   // the whole unit: final output
      if (row_ok) {
        const float inv = l_run > 0.f ? a.out_scale / l_run : 0.f;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            store_out(a.out, out_row * D + 32 * db + tile_token(v, hh), o[db][v] * inv,
                      a.out_dtype);
        if (a.lse && hh == 0) a.lse[out_row] = lse2_of(m_run, l_run);
      }
    } else if (row_ok) {               // a piece: partial for the merge
      const size_t slot = ((size_t)(s * Hk + g) * Rmax + rt + wid) * prow + mcol;
      float* po = a.ws_o + slot * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *reinterpret_cast<float4*>(po + 32 * db + 8 * q4 + 4 * hh) =
              make_float4(o[db][4 * q4], o[db][4 * q4 + 1], o[db][4 * q4 + 2], o[db][4 * q4 + 3]);
      if (hh == 0) {
        a.ws_ml[2 * slot] = m_run;
        a.ws_ml[2 * slot + 1] = l_run;
      }
    }
    f += n_here;
    k += n_here;
    if (k == c && f < f_end) {         // next row tile, KV head, or non-empty sequence
      k = 0;
      if (++rt == sh.R) {
        rt = 0;
        if (++g == Hk) {
          g = 0;
          do {
            ++s;
            sh = mq_seq_shape(a, lens, qoff, s);
          } while (sh.R == 0 && s + 1 < a.num_seqs);
          c = sh.nt + X;
        }
      }
    }
  }
}

template <int DT, int B>
__global__ __launch_bounds__(kThreads, 2) void multiq_split_kernel(const AttnArgs a) {
  using Wk = TokenTileWalker<B>;
  constexpr int X = mq_seg_items(DT);
  // the waves' K stages, then their V stages; before the walk the same LDS
  // holds the prefix sums (kMaxSplitSeqs + 1 ints fit)
  __shared__ __attribute__((aligned(16))) char sm_stage[2 * kWaves * Wk::kStageBytes];
  __shared__ int sm_wsum[kWaves], sm_went[kWaves];
  static_assert((kMaxSplitSeqs + 1) * sizeof(int) <= sizeof(sm_stage), "prefix sums fit");
  int* sm_pre = reinterpret_cast<int*>(sm_stage);
  const int S = a.num_seqs, Hk = a.num_kv_heads, G = a.group;
  const int Rmax = (a.max_q_len * G + 31) / 32;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const ConstI32Ptr lens = as_const(a.context_lens), qoff = as_const(a.q_offsets);

  // items per sequence and their prefix sums, 256 sequences per round: an
  // inclusive scan inside each wave (shuffles), then the wave totals through
  // LDS (two barriers per round)
  // The block-table entries that the units read are counted alongside.
  int carry = 0, entries = 0;
  if (tid == 0) sm_pre[0] = 0;
  for (int base = 0; base < S; base += kThreads) {
    const int s = base + tid;
    int v = 0, e = 0;
    if (s < S) {
      const MqSeqShape sh = mq_seq_shape(a, lens, qoff, s);
      v = Hk * sh.R * (sh.nt > 0 ? sh.nt + X : 0);
      e = sh.nt > 0 ? (sh.L + B - 1) / B : 0;
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(v, off, 64);
      v += lane >= off ? t : 0;
      e += __shfl_xor(e, off, 64);
    }
    if (lane == 63) {
      sm_wsum[wave] = v;
      sm_went[wave] = e;
    }
    __syncthreads();
    int before = carry;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int t = sm_wsum[w];
      before += w < wave ? t : 0;
      carry += t;
      entries += sm_went[w];
    }
    if (s < S) sm_pre[s + 1] = before + v;
    __syncthreads();
  }
  auto pre_at = [&](int i) { return __builtin_amdgcn_readfirstlane(sm_pre[i]); };
  const int total = pre_at(S);
  // With one row tile per (sequence, KV head) and no more table entries than
  // pool blocks, no K/V line is read twice (a block shared by sequences
  // needs more entries than blocks): the loads then carry the non-temporal
  // hint, which streams them past the caches.  Otherwise the lines are kept.
  const bool stream = Rmax == 1 && __builtin_amdgcn_readfirstlane(entries) <= a.pool_blocks;
  const int nwaves = gridDim.x * kWaves;
  const int chunk = max(1, (total + nwaves - 1) / nwaves);
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
  // the first item's sequence: pre[s] <= f < pre[s + 1] (found while the
  // prefix sums are still in LDS)
  int s = 0, r0 = 0;
  if (f < total) {
    int lo = 0, hi = S - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pre_at(mid) <= f) lo = mid;
      else hi = mid - 1;
    }
    s = lo;
    r0 = f - pre_at(s);
  }
  __syncthreads();   // from here the LDS holds V stages
  if (f >= total) return;

  char* st0 = sm_stage + wave * Wk::kStageBytes;   // K stage
  char* st1 = sm_stage + (kWaves + wave) * Wk::kStageBytes;   // V stage
  if (stream)
    mq_split_wave<DT, B, true>(a, s, r0, f, f_end, wid, st0, st1);
  else
    mq_split_wave<DT, B, false>(a, s, r0, f, f_end, wid, st0, st1);
}

// Merge of the split kernel's pieces: thread c owns 4 consecutive dims of one
// (query token, head) of sequence blockIdx.y.  Its row r = i G + h of KV head
// g is row r % 32 of row tile rt = r / 32; that unit's items are
// [a0, a0 + c) with a0 = pre[s] + (g R + rt) c, its tiles the last
// c - X (X: the fixed cost of the split kernel's K/V type), so the waves
// (a0 + X) / chunk ..
// (a0 + c - 1) / chunk covered it, wave w leaving its piece in slot
// (s Hk + g) Rmax + rt + w.  Sequences without keys get zero rows.
template <int D, int X>
__global__ __launch_bounds__(256) void mq_split_merge_kernel(const AttnArgs a) {
  constexpr int kChunks = D / 4;
  const int H = a.num_heads, Hk = a.num_kv_heads, G = a.group;
  const int Rmax = (a.max_q_len * G + 31) / 32;
  const int s = blockIdx.y;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int per_tok = H * kChunks;
  const int qi = idx / per_tok;
  const int hq = (idx % per_tok) / kChunks, d0 = (idx % kChunks) * 4;
  const ConstI32Ptr lens = as_const(a.context_lens), qoff = as_const(a.q_offsets);
  const MqSeqShape sh = mq_seq_shape(a, lens, qoff, s);
  if (qi >= sh.n) return;
  const size_t orow = (size_t)((a.q_offsets ? qoff[s] : s) + qi) * H + hq;
  const int prow = a.q_offsets ? 32 : G;   // rows per piece slot
  if (sh.L == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) store_out(a.out, orow * D + d0 + e, 0.f, a.out_dtype);
    if (a.lse && d0 == 0) a.lse[orow] = kNegInf;
    return;
  }
  const int g = hq / G, h = hq - g * G;
  const int r = qi * G + h, rt = r / 32, row = r % 32;
  const ConstI32Ptr plan = as_const(a.plan);
  const int chunk = plan[0];
  const int c = sh.nt + X;
  const int a0 = plan[2 + s] + (g * sh.R + rt) * c;
  const int w0 = (a0 + X) / chunk, w1 = (a0 + c - 1) / chunk;
  if (w0 == w1) return;                // written by its one wave
  const size_t base = (size_t)(s * Hk + g) * Rmax + rt;
  constexpr int kBatch = 8;
  float M = kNegInf, den = 0.f;
  float num[4] = {0.f, 0.f, 0.f, 0.f};
  for (int w = w0; w <= w1; w += kBatch) {
    float pm[kBatch], pl[kBatch];
    float4 pv[kBatch];
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const size_t sl = (base + min(w + q, w1)) * prow + row;   // past the last piece: weight 0
      pm[q] = a.ws_ml[2 * sl];
      pl[q] = a.ws_ml[2 * sl + 1];
      pv[q] = *reinterpret_cast<const float4*>(a.ws_o + sl * D + d0);
    }
    float mx = M;
#pragma unroll
    for (int q = 0; q < kBatch; ++q)
      if (w + q <= w1) mx = fmaxf(mx, pm[q]);
    const float ms = (mx == kNegInf) ? 0.f : mx;
    const float rs = fast_exp2(M - ms);
    den *= rs;
#pragma unroll
    for (int e = 0; e < 4; ++e) num[e] *= rs;
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const float wt = (w + q <= w1) ? fast_exp2(pm[q] - ms) : 0.f;
      num[0] = __builtin_fmaf(wt, pv[q].x, num[0]);
      num[1] = __builtin_fmaf(wt, pv[q].y, num[1]);
      num[2] = __builtin_fmaf(wt, pv[q].z, num[2]);
      num[3] = __builtin_fmaf(wt, pv[q].w, num[3]);
      den = __builtin_fmaf(wt, pl[q], den);
    }
    M = mx;
  }
  const float inv = den > 0.f ? a.out_scale / den : 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) store_out(a.out, orow * D + d0 + e, num[e] * inv, a.out_dtype);
  if (a.lse && d0 == 0) a.lse[orow] = lse2_of(M, den);
}

hipError_t launch_merge(int head_dim, int num_seqs, const AttnArgs& a, hipStream_t st);

template <int DT, int D, int B>
static hipError_t launch_mfma_t(int num_seqs, const AttnArgs& a, hipStream_t st,
                                const KernelEvents& ev) {
  if constexpr (D == 128) {
    if (a.plan) {   // balanced split (the host chose it for this shape)
      hipError_t e = launch_main(multiq_split_kernel<DT, B>, dim3(a.split_workgroups),
                                 dim3(kThreads), 0, st, ev, a);
      if (e != hipSuccess) return e;
      const int per_seq = a.max_q_len * a.num_heads * (D / 4);
      hipLaunchKernelGGL((mq_split_merge_kernel<D, mq_seg_items(DT)>),
                         dim3((per_seq + 255) / 256, num_seqs), dim3(256), 0, st, a);
      return hipGetLastError();
    }
  }
  if (a.plan) return hipErrorNotSupported;
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

// Resident workgroups per CU of the split kernel (occupancy query, cached;
// threads that race on the first query store the same value, atomically).
template <int DT, int B>
static int mq_split_wgs_per_cu() {
  static std::atomic<int> cached{0};
  int n = cached.load(std::memory_order_relaxed);
  if (!n) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &n, reinterpret_cast<const void*>(multiq_split_kernel<DT, B>), kThreads, 0) !=
            hipSuccess || n < 1)
      n = 1;
    cached.store(n, std::memory_order_relaxed);
  }
  return n;
}

// A decode at head_dim 128 through the split kernel (AttnArgs without query
// offsets: one query token per sequence, pieces in (S Hk + waves) x G slots)
// and its merge.  DT: the K/V type (the 8-bit cache runs its products in f16).
template <int DT, int B>
static hipError_t launch_split_decode_t(int num_seqs, const AttnArgs& a, hipStream_t st,
                                        const KernelEvents& ev) {
  hipError_t e = launch_main(multiq_split_kernel<DT, B>, dim3(a.split_workgroups),
                             dim3(kThreads), 0, st, ev, a);
  if (e != hipSuccess) return e;
  const int per_seq = a.num_heads * (128 / 4);
  hipLaunchKernelGGL((mq_split_merge_kernel<128, mq_seg_items(DT)>),
                     dim3((per_seq + 255) / 256, num_seqs), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_split_decode_b(int block_size, int num_seqs, const AttnArgs& a,
                                        hipStream_t st, const KernelEvents& ev) {
  switch (block_size) {
    case 8: return launch_split_decode_t<DT, 8>(num_seqs, a, st, ev);
    case 16: return launch_split_decode_t<DT, 16>(num_seqs, a, st, ev);
    default: return launch_split_decode_t<DT, 32>(num_seqs, a, st, ev);
  }
}

hipError_t launch_split_decode(int dtype, int block_size, int num_seqs, const AttnArgs& a,
                               hipStream_t st, const KernelEvents& ev) {
  if (dtype == PA_FP8_E4M3) return launch_split_decode_b<PA_FP8_E4M3>(block_size, num_seqs, a, st, ev);
  if (dtype == PA_F16) return launch_split_decode_b<PA_F16>(block_size, num_seqs, a, st, ev);
  return launch_split_decode_b<PA_BF16>(block_size, num_seqs, a, st, ev);
}

int multiq_split_workgroups_per_cu(int dtype, int block_size) {
  if (dtype == PA_FP8_E4M3) {
    switch (block_size) {
      case 8: return mq_split_wgs_per_cu<PA_FP8_E4M3, 8>();
      case 16: return mq_split_wgs_per_cu<PA_FP8_E4M3, 16>();
      default: return mq_split_wgs_per_cu<PA_FP8_E4M3, 32>();
    }
  }
  const bool f16 = dtype == PA_F16;
  switch (block_size) {
    case 8: return f16 ? mq_split_wgs_per_cu<PA_F16, 8>() : mq_split_wgs_per_cu<PA_BF16, 8>();
    case 16: return f16 ? mq_split_wgs_per_cu<PA_F16, 16>() : mq_split_wgs_per_cu<PA_BF16, 16>();
    default: return f16 ? mq_split_wgs_per_cu<PA_F16, 32>() : mq_split_wgs_per_cu<PA_BF16, 32>();
  }
}

hipError_t launch_multiq(int dtype, int head_dim, int block_size, int group, int num_seqs,
                         const AttnArgs& a, hipStream_t st, const KernelEvents& ev) {
  if (dtype == PA_BF16) return dispatch_mfma<PA_BF16>(head_dim, block_size, num_seqs, a, st, ev);
  if (dtype == PA_F16) return dispatch_mfma<PA_F16>(head_dim, block_size, num_seqs, a, st, ev);
  // fp32: vector-ALU path, each query row as a decode row over its visible length
  return launch_decode(dtype, head_dim, block_size, group, num_seqs, a, st, ev);
}

}  // namespace pa
