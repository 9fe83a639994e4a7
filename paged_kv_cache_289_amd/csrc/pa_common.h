// Device helpers shared by the gfx950 paged-attention kernels: element traits
// for the three storage types, 16-byte vector loads, bf16/f16 dot2 and
// conversions, and wave64 cross-lane reductions built on DPP.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {

// Launch of a call's main kernel.  When profiling events are given they are
// handed to hipExtLaunchKernel, which stamps them with the dispatch's own start
// and end (no separate marker packets around it), so they time the kernel as
// a kernel trace does.
template <typename K>
inline hipError_t launch_main(K kernel, dim3 grid, dim3 block, size_t smem, hipStream_t st,
                              const KernelEvents& ev, const AttnArgs& a) {
  if (ev.start || ev.stop) {
    void* args[] = {const_cast<AttnArgs*>(&a)};
    return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, smem, st,
                              ev.start, ev.stop, 0);
  }
  hipLaunchKernelGGL(kernel, grid, block, smem, st, a);
  return hipGetLastError();
}


typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;
// Online softmax: the running max moves only when a score beats it by more
// than this (log2 units), and it starts at a finite sentinel below any score.
constexpr float kRescaleLog2 = 8.f;
constexpr float kMaxInit = -1e30f;

// ---------------------------------------------------------------------------
// element traits: one 16-byte vector = kPerVec elements
// ---------------------------------------------------------------------------
template <int DT> struct Elem;

template <> struct Elem<PA_F32> {
  typedef uint4 Vec;    // a lane's share of one token row: one 16-byte vector
  typedef uint4 QVec;   // the query in the same type, one 16-byte vector
  __device__ static inline QVec load_q(const void* q, size_t idx) {
    return reinterpret_cast<const uint4*>(q)[idx / kPerVec];
  }
  __device__ static inline QVec zero_q() { return make_uint4(0, 0, 0, 0); }
  __device__ static inline void flip_q(QVec& v) {
    v.x ^= 0x80000000u; v.y ^= 0x80000000u; v.z ^= 0x80000000u; v.w ^= 0x80000000u;
  }
  static constexpr int kBytes = 4;
  static constexpr int kPerVec = 4;
  // partial dot product of the 4 elements held in one vector
  __device__ static inline float dot(const uint4& q, const uint4& k, float acc) {
    acc = __builtin_fmaf(__uint_as_float(q.x), __uint_as_float(k.x), acc);
    acc = __builtin_fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
    acc = __builtin_fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
    acc = __builtin_fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
    return acc;
  }
  __device__ static inline float dot0(const uint4& q, const uint4& k) {
    float acc = __uint_as_float(q.x) * __uint_as_float(k.x);
    acc = __builtin_fmaf(__uint_as_float(q.y), __uint_as_float(k.y), acc);
    acc = __builtin_fmaf(__uint_as_float(q.z), __uint_as_float(k.z), acc);
    acc = __builtin_fmaf(__uint_as_float(q.w), __uint_as_float(k.w), acc);
    return acc;
  }
  __device__ static inline void to_float(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
};

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <> struct Elem<PA_BF16> {
  typedef uint4 Vec;    // a lane's share of one token row: one 16-byte vector
  typedef uint4 QVec;   // the query in the same type, one 16-byte vector
  __device__ static inline QVec load_q(const void* q, size_t idx) {
    return reinterpret_cast<const uint4*>(q)[idx / kPerVec];
  }
  __device__ static inline QVec zero_q() { return make_uint4(0, 0, 0, 0); }
  __device__ static inline void flip_q(QVec& v) {
    v.x ^= 0x80008000u; v.y ^= 0x80008000u; v.z ^= 0x80008000u; v.w ^= 0x80008000u;
  }
  static constexpr int kBytes = 2;
  static constexpr int kPerVec = 8;
  __device__ static inline float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), acc, false);
  }
  __device__ static inline float dot(const uint4& q, const uint4& k, float acc) {
    acc = dot2(q.x, k.x, acc);
    acc = dot2(q.y, k.y, acc);
    acc = dot2(q.z, k.z, acc);
    acc = dot2(q.w, k.w, acc);
    return acc;
  }
  // dot(q, k, 0) with the first step in the three-operand form, which takes the
  // zero as an inline constant instead of a zeroed accumulator register
  __device__ static inline float dot0(const uint4& q, const uint4& k) {
    float acc;
    asm("v_dot2_f32_bf16 %0, %1, %2, 0" : "=v"(acc) : "v"(q.x), "v"(k.x));
    acc = dot2(q.y, k.y, acc);
    acc = dot2(q.z, k.z, acc);
    acc = dot2(q.w, k.w, acc);
    return acc;
  }
  __device__ static inline void to_float(const uint4& v, float* f) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
  }
};

template <> struct Elem<PA_F16> {
  typedef uint4 Vec;    // a lane's share of one token row: one 16-byte vector
  typedef uint4 QVec;   // the query in the same type, one 16-byte vector
  __device__ static inline QVec load_q(const void* q, size_t idx) {
    return reinterpret_cast<const uint4*>(q)[idx / kPerVec];
  }
  __device__ static inline QVec zero_q() { return make_uint4(0, 0, 0, 0); }
  __device__ static inline void flip_q(QVec& v) {
    v.x ^= 0x80008000u; v.y ^= 0x80008000u; v.z ^= 0x80008000u; v.w ^= 0x80008000u;
  }
  static constexpr int kBytes = 2;
  static constexpr int kPerVec = 8;
  __device__ static inline float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b),
                                  acc, false);
  }
  __device__ static inline float dot(const uint4& q, const uint4& k, float acc) {
    acc = dot2(q.x, k.x, acc);
    acc = dot2(q.y, k.y, acc);
    acc = dot2(q.z, k.z, acc);
    acc = dot2(q.w, k.w, acc);
    return acc;
  }
  __device__ static inline float dot0(const uint4& q, const uint4& k) {
    float acc;
    asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(acc) : "v"(q.x), "v"(k.x));
    acc = dot2(q.y, k.y, acc);
    acc = dot2(q.z, k.z, acc);
    acc = dot2(q.w, k.w, acc);
    return acc;
  }
  __device__ static inline void pair(uint32_t w, float* f) {
    f16x2_t h = __builtin_bit_cast(f16x2_t, w);
    f[0] = (float)h.x;
    f[1] = (float)h.y;
  }
  __device__ static inline void to_float(const uint4& v, float* f) {
    pair(v.x, f); pair(v.y, f + 2); pair(v.z, f + 4); pair(v.w, f + 6);
  }
};

// 8-bit E4M3 keys and values, with bf16 queries.  A lane holds 8 codes of a
// token row (an 8-byte vector), so a row of 128 codes is 16 lanes, one DPP
// row, as for the 16-bit types: the same reduce-scatter of the scores, and a
// lane's accumulators and query cover 8 dims.  gfx950 widens two codes per
// instruction: v_cvt_scalef32_pk_f16_fp8 to an f16 pair (every E4M3 value is
// exact in f16) for QK as v_dot2_f32_f16 against the query held as f16 pairs,
// and v_cvt_pk_f32_fp8 to two fp32 values for PV.  The NaN codes are not
// supported.
struct Fp8Q {
  uint32_t w[4];   // 8 query values as f16 pairs
};

template <> struct Elem<PA_FP8_E4M3> {
  static constexpr int kBytes = 1;
  static constexpr int kPerVec = 8;
  typedef uint2 Vec;
  typedef Fp8Q QVec;
  __device__ static inline float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b),
                                  acc, false);
  }
  // codes 0, 1 (hi = false) or 2, 3 (hi = true) of a dword as an f16 pair
  template <bool HI>
  __device__ static inline uint32_t f16_pair(uint32_t x) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, HI));
  }
  // (first step in the three-operand form with an inline zero, as for f16)
  __device__ static inline float dot0(const QVec& q, const uint2& k) {
    float acc;
    const uint32_t k0 = f16_pair<false>(k.x);
    asm("v_dot2_f32_f16 %0, %1, %2, 0" : "=v"(acc) : "v"(q.w[0]), "v"(k0));
    acc = dot2(q.w[1], f16_pair<true>(k.x), acc);
    acc = dot2(q.w[2], f16_pair<false>(k.y), acc);
    acc = dot2(q.w[3], f16_pair<true>(k.y), acc);
    return acc;
  }
  __device__ static inline void to_float(const uint2& v, float* f) {
    const uint32_t vw[2] = {v.x, v.y};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(vw[i], false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(vw[i], true);
      f[4 * i] = lo[0];
      f[4 * i + 1] = lo[1];
      f[4 * i + 2] = hi[0];
      f[4 * i + 3] = hi[1];
    }
  }
  // 8 bf16 query values starting at element `idx` (8-element aligned), as f16
  // pairs (rounded to nearest; bf16 values within f16's range convert exactly)
  __device__ static inline QVec load_q(const void* q, size_t idx) {
    const uint4 a = reinterpret_cast<const uint4*>(q)[idx / 8];
    const uint32_t src[4] = {a.x, a.y, a.z, a.w};
    QVec r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      typedef float f2_t __attribute__((ext_vector_type(2)));
      const f2_t f = {bf16_lo(src[i]), bf16_hi(src[i])};
      r.w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2_t));
    }
    return r;
  }
  __device__ static inline QVec zero_q() {
    QVec r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.w[i] = 0u;
    return r;
  }
  __device__ static inline void flip_q(QVec& q) {
#pragma unroll
    for (int i = 0; i < 4; ++i) q.w[i] ^= 0x80008000u;
  }
};

// ---------------------------------------------------------------------------
// output conversion (round to nearest even)
// ---------------------------------------------------------------------------
__device__ inline uint16_t f32_to_bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;  // NaN stays NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ inline void store_out(void* out, size_t idx, float x, int out_dtype) {
  if (out_dtype == PA_F32) {
    reinterpret_cast<float*>(out)[idx] = x;
  } else if (out_dtype == PA_BF16) {
    reinterpret_cast<uint16_t*>(out)[idx] = f32_to_bf16_rne(x);
  } else {
    reinterpret_cast<_Float16*>(out)[idx] = (_Float16)x;
  }
}

// ---------------------------------------------------------------------------
// cross-lane helpers (wave64)
// ---------------------------------------------------------------------------
// DPP control codes (GCN/CDNA encoding)
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// Every lane reads a lane of its own row, so bound_ctrl never matters; setting
// it lets the compiler fold the move into the consuming add (v_add_f32_dpp).
template <int CTRL>
__device__ inline float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Per-lane select: b where the lane's bit of mask is set, else a.
__device__ inline float lane_select(float a, float b, uint64_t mask) {
  float r;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(mask));
  return r;
}

// Value of lane n (0..15, a compile-time constant after unrolling) of this
// lane's 16-lane row (DPP row_newbcast).
__device__ inline float row_bcast(float x, int n) {
  switch (n) {
#define PA_ROW_BCAST(N) \
    case N: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x150 + N, 0xF, 0xF, false));
    PA_ROW_BCAST(0) PA_ROW_BCAST(1) PA_ROW_BCAST(2) PA_ROW_BCAST(3)
    PA_ROW_BCAST(4) PA_ROW_BCAST(5) PA_ROW_BCAST(6) PA_ROW_BCAST(7)
    PA_ROW_BCAST(8) PA_ROW_BCAST(9) PA_ROW_BCAST(10) PA_ROW_BCAST(11)
    PA_ROW_BCAST(12) PA_ROW_BCAST(13) PA_ROW_BCAST(14) PA_ROW_BCAST(15)
#undef PA_ROW_BCAST
    default: return x;
  }
}

// Value of the lane n places further along this lane's 16-lane row, wrapping
// (DPP row_ror; n in 1..15, a compile-time constant after unrolling).
__device__ inline float row_ror(float x, int n) {
  switch (n) {
#define PA_ROW_ROR(N) \
    case N: return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x120 + N, 0xF, 0xF, false));
    PA_ROW_ROR(1) PA_ROW_ROR(2) PA_ROW_ROR(4) PA_ROW_ROR(8)
#undef PA_ROW_ROR
    default: return x;
  }
}

// Sum over aligned groups of N lanes (N in {1,2,4,8,16,32}); every lane of a
// group receives the group's sum.  All 64 lanes must be active.
template <int N>
__device__ inline float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<kDppQuadXor1>(x);
  if constexpr (N >= 4) x += dpp<kDppQuadXor2>(x);
  if constexpr (N >= 8) x += dpp<kDppRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppRowMirror>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16, 64);
  return x;
}

// group_sum over a whole array: step by step across all entries, so every DPP
// read is far from the write that produced its operand.
template <int N, int K>
__device__ inline void group_sum_all(float (&x)[K]) {
  if constexpr (N >= 2) {
#pragma unroll
    for (int k = 0; k < K; ++k) x[k] += dpp<kDppQuadXor1>(x[k]);
  }
  if constexpr (N >= 4) {
#pragma unroll
    for (int k = 0; k < K; ++k) x[k] += dpp<kDppQuadXor2>(x[k]);
  }
  if constexpr (N >= 8) {
#pragma unroll
    for (int k = 0; k < K; ++k) x[k] += dpp<kDppRowHalfMirror>(x[k]);
  }
  if constexpr (N >= 16) {
#pragma unroll
    for (int k = 0; k < K; ++k) x[k] += dpp<kDppRowMirror>(x[k]);
  }
  if constexpr (N >= 32) {
#pragma unroll
    for (int k = 0; k < K; ++k) x[k] += __shfl_xor(x[k], 16, 64);
  }
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Log-sum-exp (log2 units) of a softmax state: running max m, sum l of 2^(z - m).
__device__ inline float lse2_of(float m, float l) { return l > 0.f ? m + log2f(l) : kNegInf; }

// Max / sum of a value and the one held by the lane 32 apart.  v_permlane32_swap
// exchanges the upper half of one register with the lower half of the other;
// applied to two copies of x, the two results hold x and its partner in every
// lane (in some order), so any symmetric combination of them is the answer.
__device__ inline float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// workgroup placement
// ---------------------------------------------------------------------------
// The eight XCDs of the device each have their own L2, and a launch deals its
// workgroups to them round-robin in launch order.  xcd_major(b, n) renumbers
// the n workgroups of a 1-D launch so that consecutive numbers run on the same
// XCD: workgroups that read the same data, given consecutive numbers, then
// share one L2 instead of fetching that data once per XCD.  (Only a placement
// hint: the numbering is a bijection of [0, n) whatever the hardware does.)
constexpr int kXcds = 8;
__device__ inline int xcd_major(int b, int n) {
  const int x = b % kXcds, q = b / kXcds;
  return x * (n / kXcds) + min(x, n % kXcds) + q;
}

// ---------------------------------------------------------------------------
// read-only metadata through the constant address space
// ---------------------------------------------------------------------------
// Block tables and context lengths are never written while a kernel runs;
// reading them through an address-space-4 pointer lets the compiler use scalar
// loads for wave-uniform indices even in kernels that store elsewhere.
typedef const __attribute__((address_space(4))) int32_t* ConstI32Ptr;

__device__ inline ConstI32Ptr as_const(const int32_t* p) { return (ConstI32Ptr)p; }

// ---------------------------------------------------------------------------
// raw buffer loads (SGPR descriptor + per-lane byte offset)
// ---------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t BufRsrc;
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

// Descriptor word 3 for untyped dword access on gfx9-family parts.
constexpr int kBufferWord3 = 0x00020000;
// Cache-policy operand of buffer loads: the nt bit.
constexpr int kCpolNt = 2;

// A descriptor covering nbytes from base; accesses at or past nbytes return
// zero without touching memory.
__device__ inline BufRsrc make_rsrc(const void* base, int nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nbytes,
                                           kBufferWord3);
}

// One lane vector (16 or 8 bytes) through a buffer descriptor, with or without
// the non-temporal hint.
template <typename V, bool NT> __device__ inline V buffer_load_vec(BufRsrc r, int off, int coff);
template <> __device__ inline uint4 buffer_load_vec<uint4, false>(BufRsrc r, int off, int coff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, coff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <> __device__ inline uint4 buffer_load_vec<uint4, true>(BufRsrc r, int off, int coff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, coff, kCpolNt);
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <> __device__ inline uint2 buffer_load_vec<uint2, false>(BufRsrc r, int off, int coff) {
  const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off, coff, 0);
  return make_uint2(v.x, v.y);
}
template <> __device__ inline uint2 buffer_load_vec<uint2, true>(BufRsrc r, int off, int coff) {
  const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, off, coff, kCpolNt);
  return make_uint2(v.x, v.y);
}

}  // namespace pa
