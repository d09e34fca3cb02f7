// Device helpers shared by the DMTP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dmtp.h"

namespace dmtp {

constexpr int kWave = 64;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bf16 ----
// bf16 values are handled as their 16-bit patterns.

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// Round-to-nearest-even float32 -> bf16 (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// x = hi + lo + r with |r| <= 2^-18 |x|: the two-term bf16 split that lets a
// bf16 x bf16 matrix core product reproduce a float32 operand.
__device__ __forceinline__ void split_bf16(float x, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16(x);
  lo = f32_to_bf16(x - bf16_to_f32(hi));
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two-plane split of two floats with the hardware round-to-nearest-even
// conversion (v_cvt_pk_bf16_f32): hi2 packs bf16(a), bf16(b); lo2 packs the
// bf16 of the remainders.  Same values as split_bf16 for finite inputs.
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi2, uint32_t& lo2) {
  const bf16x2_t h = {(__bf16)a, (__bf16)b};
  hi2 = __builtin_bit_cast(uint32_t, h);
  const bf16x2_t l = {(__bf16)(a - (float)h[0]), (__bf16)(b - (float)h[1])};
  lo2 = __builtin_bit_cast(uint32_t, l);
}

// Element i of a float32 activation stored as its two bf16 planes: the hi
// plane at p, the lo plane at p + pst.
__device__ __forceinline__ void store_planes(uint16_t* p, size_t pst, size_t i, float v) {
  uint16_t h, l;
  split_bf16(v, h, l);
  p[i] = h;
  p[pst + i] = l;
}

__device__ __forceinline__ uint32_t pack2(uint16_t a, uint16_t b) {
  return (uint32_t)a | ((uint32_t)b << 16);
}

// ---------------------------------------------------------------- MFMA ----
// D(16x16, f32) += A(16x32, bf16) * B(32x16, bf16).  Lane l supplies row
// (l % 16) of A and column (l % 16) of B, eight consecutive k values from the
// lane group l / 16; it receives D rows 4 * (l / 16) + i, column l % 16.
__device__ __forceinline__ f32x4_t mfma_16x16x32(const uint4& a, const uint4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// D(32x32, f32) += A(32x16, bf16) * B(16x32, bf16).  Lane l supplies row
// (l % 32) of A and column (l % 32) of B, eight consecutive k values from the
// lane half l / 32; it receives D[8 (i / 4) + 4 (l / 32) + (i % 4)][l % 32] in
// element i (i = 0..15).
typedef float f32x16_t __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16_t mfma_32x32x16(const uint4& a, const uint4& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// ----------------------------------------------------------- reductions ----
template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask) {
  return __shfl_xor(v, mask, kWave);
}

// Wave-wide sum and maximum by DPP moves, with no LDS round trip: pairs and
// pairs of pairs within each quad, the mirrors within each 8- and 16-lane
// row, then row 0's total into row 1 and row 2's into row 3, and lane 31's
// into rows 2 and 3; lane 63 then holds the whole wave's result, which is
// returned to every lane (a wave-uniform value).  Summation order: quads,
// eighths, rows, then (r0 + r1) + (r2 + r3).  Every lane of the wave must be
// active: the moves read the registers of all 64 lanes.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ int dpp_mov_i(int v, int old) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_mov(float v, float old) {
  return __builtin_bit_cast(float, dpp_mov_i<CTRL, ROWS>(__builtin_bit_cast(int, v), __builtin_bit_cast(int, old)));
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ double dpp_mov(double v, double old) {
  const int lo = dpp_mov_i<CTRL, ROWS>(__double2loint(v), __double2loint(old));
  const int hi = dpp_mov_i<CTRL, ROWS>(__double2hiint(v), __double2hiint(old));
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ float lane63(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ double lane63(double v) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), 63),
                          __builtin_amdgcn_readlane(__double2loint(v), 63));
}
template <class T>
__device__ __forceinline__ T wave_sum(T v) {
  v += dpp_mov<0xB1>(v, T(0));          // quad_perm [1, 0, 3, 2]
  v += dpp_mov<0x4E>(v, T(0));          // quad_perm [2, 3, 0, 1]
  v += dpp_mov<0x141>(v, T(0));         // row_half_mirror
  v += dpp_mov<0x140>(v, T(0));         // row_mirror
  v += dpp_mov<0x142, 0xA>(v, T(0));    // row_bcast15 into rows 1 and 3
  v += dpp_mov<0x143, 0xC>(v, T(0));    // row_bcast31 into rows 2 and 3
  return lane63(v);
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v, v));
  v = fmaxf(v, dpp_mov<0x4E>(v, v));
  v = fmaxf(v, dpp_mov<0x141>(v, v));
  v = fmaxf(v, dpp_mov<0x140>(v, v));
  v = fmaxf(v, dpp_mov<0x142, 0xA>(v, v));
  v = fmaxf(v, dpp_mov<0x143, 0xC>(v, v));
  return lane63(v);
}

// --------------------------------------------------------- Philox4x64-10 ----
// The counter-based generator of Salmon, Moraes, Dror and Shaw (SC'11): ten
// rounds, each multiplying counter words 0 and 2 by fixed odd constants and
// mixing both product halves with the other words and the round key; the key
// is advanced by two Weyl increments between rounds.
struct u64x4 {
  uint64_t x, y, z, w;
};

// hi:lo = a * m, the full 128-bit product, from four 32 x 32 -> 64 partial
// products (each a single multiply-add on the vector unit):
//   a m = p00 + 2^32 (a0 m1 + a1 m0) + 2^64 a1 m1, with the middle terms folded
//   one at a time so that no partial sum exceeds 64 bits.
__device__ __forceinline__ void mulhilo64(uint64_t a, uint64_t m, uint64_t& hi, uint64_t& lo) {
  const uint32_t a0 = (uint32_t)a, a1 = (uint32_t)(a >> 32);
  const uint32_t m0 = (uint32_t)m, m1 = (uint32_t)(m >> 32);
  const uint64_t p00 = (uint64_t)a0 * m0;
  const uint64_t p01 = (uint64_t)a0 * m1 + (p00 >> 32);
  const uint64_t p10 = (uint64_t)a1 * m0 + (uint32_t)p01;
  hi = (uint64_t)a1 * m1 + (p01 >> 32) + (p10 >> 32);
  lo = (p10 << 32) | (uint32_t)p00;
}

__device__ __forceinline__ u64x4 philox4x64_10(u64x4 c, uint64_t k0, uint64_t k1) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += W0;
      k1 += W1;
    }
    uint64_t hi0, lo0, hi1, lo1;
    mulhilo64(c.x, M0, hi0, lo0);
    mulhilo64(c.z, M1, hi1, lo1);
    c = u64x4{hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0};
  }
  return c;
}

// Gumbel(0, 1) variate of a 32-bit word x: t = (x + 1/2) 2^-32,
// E = -log(1 - t) = -log1p(-t) (Exp(1)), g = -log(E).
__device__ __forceinline__ float gumbel_of_word(uint32_t x) {
  const float t = fmaf((float)x, 2.3283064365386963e-10f, 1.1641532182693481e-10f);
  const float e = -log1pf(-t);
  return -logf(e);
}

// Base-2 logarithm and exponential of the hardware transcendental unit
// (v_log_f32 / v_exp_f32, about one ulp for normal arguments).
__device__ __forceinline__ float hw_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// gumbel_of_word with the hardware logarithm (absolute error below 1e-5 over
// the whole range).  1 - t is formed from the integer 2^32 - 1 - x, so it keeps
// full relative precision near t = 1; for t < 2^-7, E = -log(1 - t) is taken
// from its series t + t^2/2 + t^3/3 + t^4/4 (truncation below 2^-30 relative).
__device__ __forceinline__ float gumbel_fast(uint32_t x) {
  const float ln2 = 0.6931471805599453f;
  const float t = fmaf((float)x, 0x1p-32f, 0x1p-33f);
  const float om = fmaf((float)(0xFFFFFFFFu - x), 0x1p-32f, 0x1p-33f);
  const float e_series = t * fmaf(t, fmaf(t, fmaf(t, 0.25f, 0.33333334f), 0.5f), 1.f);
  const float e = t < 0x1p-7f ? e_series : -hw_log2(om) * ln2;
  return -hw_log2(e) * ln2;
}

// log(1 - e^d) for d <= 0 with the hardware log/exp (absolute error about
// 1e-6): 1 - e^d from the series of -expm1(d) when |d| < 2^-6, where the
// subtraction would cancel, directly otherwise.
__device__ __forceinline__ float log1m_exp(float d) {
  const float ln2 = 0.6931471805599453f, log2e = 1.4426950408889634f;
  const float em = -d * fmaf(d, fmaf(d, fmaf(d, 1.f / 24.f, 1.f / 6.f), 0.5f), 1.f);
  const float om = d > -0x1p-6f ? em : 1.f - hw_exp2(d * log2e);
  return hw_log2(om) * ln2;
}

// The eight 32-bit words of block (j >> 3) of noise level `level` of draw
// (seed, key): counter (block, key, level, 0), key (seed, 0).  Level 0 noise
// is indexed by vocabulary entry, level 1 by block of kDrawBlock entries.
__device__ __forceinline__ void philox_words8(uint64_t seed, uint64_t key, uint64_t block,
                                              uint32_t w[8], uint64_t level = 0) {
  const u64x4 o = philox4x64_10(u64x4{block, key, level, 0}, seed, 0);
  w[0] = (uint32_t)o.x; w[1] = (uint32_t)(o.x >> 32);
  w[2] = (uint32_t)o.y; w[3] = (uint32_t)(o.y >> 32);
  w[4] = (uint32_t)o.z; w[5] = (uint32_t)(o.z >> 32);
  w[6] = (uint32_t)o.w; w[7] = (uint32_t)(o.w >> 32);
}

// Entries per block of a two-level draw: a draw picks a block of kDrawBlock
// consecutive vocabulary entries by Gumbel-max over the blocks' log masses
// (level-1 noise), then an entry of that block by Gumbel-max over its log
// weights (level-0 noise).  The two noises are independent, so the entry is
// drawn with probability w_j / sum w, as by one Gumbel-max over all entries;
// only the entries of the chosen block need noise, so a draw over a
// vocabulary costs one memory-bound pass for the block masses.
constexpr int kDrawBlock = 128;

// 1 - e^d for d <= 0, accurate where the subtraction would cancel: the series
// of -expm1(d) when |d| < 2^-6, directly otherwise (hardware exp2).
__device__ __forceinline__ float one_minus_exp(float d) {
  const float log2e = 1.4426950408889634f;
  const float em = -d * fmaf(d, fmaf(d, fmaf(d, 1.f / 24.f, 1.f / 6.f), 0.5f), 1.f);
  return d > -0x1p-6f ? em : 1.f - hw_exp2(d * log2e);
}

// ----------------------------------------------------- running maximum ----
// Best-two tracker for argmax with a gap: (v1, i1) is the best value and its
// index (lowest index among equals), v2 the second-best value.
struct Top2 {
  float v1;
  int i1;
  float v2;
};

__device__ __forceinline__ Top2 top2_empty() { return Top2{-INFINITY, 0x7FFFFFFF, -INFINITY}; }

__device__ __forceinline__ void top2_push(Top2& t, float v, int i) {
  if (v > t.v1 || (v == t.v1 && i < t.i1)) {
    t.v2 = t.v1;
    t.v1 = v;
    t.i1 = i;
  } else if (v > t.v2) {
    t.v2 = v;
  }
}

__device__ __forceinline__ Top2 top2_merge(const Top2& a, const Top2& b) {
  Top2 r;
  if (b.v1 > a.v1 || (b.v1 == a.v1 && b.i1 < a.i1)) {
    r.v1 = b.v1;
    r.i1 = b.i1;
    r.v2 = fmaxf(a.v1, b.v2);
  } else {
    r.v1 = a.v1;
    r.i1 = a.i1;
    r.v2 = fmaxf(a.v2, b.v1);
  }
  return r;
}

// Running top-2 of a lane that sees its indices in increasing order: an equal
// value never displaces the earlier (lower) index, so no index compare is needed.
__device__ __forceinline__ void top2_push_inc(Top2& t, float v, int i) {
  const bool gt = v > t.v1;
  t.v2 = fmaxf(t.v2, fminf(v, t.v1));
  t.i1 = gt ? i : t.i1;
  t.v1 = gt ? v : t.v1;
}

__device__ __forceinline__ Top2 top2_shfl_xor(const Top2& t, int mask) {
  Top2 o;
  o.v1 = shfl_xor(t.v1, mask);
  o.i1 = shfl_xor(t.i1, mask);
  o.v2 = shfl_xor(t.v2, mask);
  return o;
}

// ---------------------------------------------------------- load helpers ----
template <int DT>
struct Elem;
template <>
struct Elem<DMTP_F32> {
  typedef float T;
  __device__ static float load(const void* p, size_t i) { return ((const float*)p)[i]; }
};
template <>
struct Elem<DMTP_BF16> {
  typedef uint16_t T;
  __device__ static float load(const void* p, size_t i) {
    return bf16_to_f32(((const uint16_t*)p)[i]);
  }
};

__device__ __forceinline__ float load_elem(const void* p, int dtype, size_t i) {
  return dtype == DMTP_BF16 ? bf16_to_f32(((const uint16_t*)p)[i]) : ((const float*)p)[i];
}

__device__ __forceinline__ void store_elem(void* p, int dtype, size_t i, float v) {
  if (dtype == DMTP_BF16)
    ((uint16_t*)p)[i] = f32_to_bf16(v);
  else
    ((float*)p)[i] = v;
}

// Context length of sequence b from the prefix sums, clamped so that rows
// cu_ctx[b] .. cu_ctx[b] + L - 1 lie inside [0, ctx_rows).
__device__ __forceinline__ int ctx_len_of(const int32_t* cu_ctx, int b, int ctx_rows) {
  const int lo = cu_ctx[b], hi = cu_ctx[b + 1];
  if (lo < 0 || lo >= ctx_rows || hi <= lo) return 0;
  return (hi > ctx_rows ? ctx_rows : hi) - lo;
}

}  // namespace dmtp
