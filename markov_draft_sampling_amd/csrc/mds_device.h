// Device-side building blocks shared by the sampling kernels (gfx950).
//
// Noise: Philox4x32-10 (Salmon et al., "Parallel random numbers: as easy as
// 1, 2, 3", SC'11) keyed by the request seed, counter (column>>2, position
// key, salt). The pages fix only the keying by (seed, position-1, column) and
// the draft salt 1<<30 (DSparkSpeculator API page, _sample_logits; PR #65007,
// Part 1 and its constants review thread); the counter layout is this
// library's definition and is stated in include/mds.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mds {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kStatusBadAnchor = 1u;
constexpr uint32_t kStatusBadDraft = 2u;
constexpr uint32_t kStatusBadIndex = 8u;
constexpr uint32_t kSaltDraft = 1u << 30;
constexpr uint32_t kSaltAccept = 1u;
constexpr uint32_t kSaltResample = 2u;

// ---------------------------------------------------------------- Philox --
struct Philox4 {
  uint32_t x0, x1, x2, x3;
};

// Ten rounds; each multiplies words 0 and 2 by the two round constants, keeps
// both product halves, and folds the high halves into words 1 and 3 with the
// round key; the key advances by the two Weyl constants between rounds.
__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                                 uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    // three-input XORs as single v_bitop3_b32 (truth table 0x96: odd parity)
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return Philox4{c0, c1, c2, c3};
}

// Uniform (2m+1) * 2^-24 from the top 23 bits m of a word: build 1 + m*2^-23
// from the bits, then subtract 1 - 2^-24 (both steps exact).
__device__ __forceinline__ float uniform24(uint32_t w) {
  const float f = __uint_as_float(0x3F800000u | (w >> 9));
  return f - 0x1.fffffep-1f;
}

// Standard Gumbel -log(-log u) with hardware base-2 logs:
// -ln(-ln u) = -ln(ln 2) - ln 2 * log2(-log2 u).
// E2 = -log2(u) > 0 of the word's uniform (u in (0, 1), normal)
__device__ __forceinline__ float neg_log2_uniform(uint32_t w) { return -__builtin_amdgcn_logf(uniform24(w)); }
__device__ __forceinline__ float gumbel_from_e2(float e2) {
  return __builtin_fmaf(-0x1.62e430p-1f, __builtin_amdgcn_logf(e2), 0x1.774f2ap-2f);
}
__device__ __forceinline__ float gumbel_from_word(uint32_t w) { return gumbel_from_e2(neg_log2_uniform(w)); }

// ---------------------------------------------------------- winner keys --
// Total order of the winner rule: NaN above every value, -0 == +0, and on
// equal values the lower column wins. key = ord(value) << 32 | ~column, so
// the largest key is the winner and 0 means "no candidate".
__device__ __forceinline__ uint32_t ord_f32(float x) {
  if (x != x) return 0xFFFFFFFFu;
  const uint32_t b = __float_as_uint(x + 0.0f);  // -0 -> +0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ uint64_t win_key(float x, uint32_t col) {
  return ((uint64_t)ord_f32(x) << 32) | (uint32_t)(~col);
}
__device__ __forceinline__ uint32_t win_col(uint64_t key) { return ~(uint32_t)key; }

// fp64 option: the same uniform, -ln(-ln u) and the score in float64. The
// cross-work-group key keeps the top 40 bits of the ordered float64 (2^-28
// relative) above the column's 24 bits, so candidates within that resolution
// go to the lower column.
__device__ __forceinline__ double gumbel64_from_word(uint32_t w) {
  const double u = (double)uniform24(w);  // exact: an odd multiple of 2^-24
  return -log(-log(u));
}
__device__ __forceinline__ uint64_t ord_f64(double x) {
  if (x != x) return ~0ull;
  const uint64_t b = (uint64_t)__double_as_longlong(x + 0.0);
  return (b >> 63) ? ~b : (b | (1ull << 63));
}
__device__ __forceinline__ uint64_t win_key64(double x, uint32_t col) {
  return (ord_f64(x) & ~0xFFFFFFull) | (0xFFFFFFu - col);
}
// column of a key in either format; key 0 (no candidate) gives -1
__device__ __forceinline__ int key_col(uint64_t key, bool f64) {
  if (!key) return -1;
  return f64 ? (int)(0xFFFFFFu - (uint32_t)(key & 0xFFFFFFu)) : (int)(~(uint32_t)key);
}

// In-order update of a running winner (columns arrive in increasing order).
template <typename S>
__device__ __forceinline__ void win_update(S& bv, int& bi, S s, int col) {
  const bool take = (s > bv) || ((s != s) && (bv == bv)) || (bi < 0);
  bv = take ? s : bv;
  bi = take ? col : bi;
}
__device__ __forceinline__ uint64_t win_key_of(float x, uint32_t col) { return win_key(x, col); }
__device__ __forceinline__ uint64_t win_key_of(double x, uint32_t col) { return win_key64(x, col); }

// ------------------------------------------------------------------ bf16 --
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// round to nearest, ties to even; NaN stays a quiet NaN
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t b = __float_as_uint(f);
  if (f != f) return (b >> 16) | 0x40u;
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// ------------------------------------------------------------ arithmetic --
// z / T from a precomputed reciprocal plus one residual correction; an
// infinite z keeps its sign (the correction would turn it into NaN).
__device__ __forceinline__ float div_t(float z, float T, float invT) {
  const float q = z * invT;
  const float r = __builtin_fmaf(-q, T, z);
  const float y = __builtin_fmaf(r, invT, q);
  return __builtin_isinf(q) ? q : y;
}

__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 0x1.715476p+0f); }

// (max, sum of exp(x - max)) pairs; an empty side has max = -inf, sum = 0.
// A NaN sum marks a row that held NaN and survives every merge.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) {
    s = s + s2;
  } else {
    s = s * __expf(m - M) + s2 * __expf(m2 - M);
  }
  m = M;
}

__device__ __forceinline__ void set_status(uint32_t* status, uint32_t bit) {
  if (status) atomicOr(status, bit);
}

// 64-bit max across the lanes l, l^16, l^32, l^48 of a wave
__device__ __forceinline__ uint64_t max_over_groups16(uint64_t k) {
  uint64_t o = (uint64_t)__shfl_xor((unsigned long long)k, 16);
  k = o > k ? o : k;
  o = (uint64_t)__shfl_xor((unsigned long long)k, 32);
  return o > k ? o : k;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t o = (uint64_t)__shfl_xor((unsigned long long)k, off);
    k = o > k ? o : k;
  }
  return k;
}

__device__ __forceinline__ void wave_lse_merge(float& m, float& s) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
    lse_merge(m, s, m2, s2);
  }
}

__device__ __forceinline__ float wave_max_f32(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

__device__ __forceinline__ float wave_sum_f32(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// Wave reductions without LDS permutes: DPP within each row of 16 lanes (the
// quad permutations, then rotations by 4 and 8 lanes, so every lane holds its
// row's result), then the four rows' results read as scalars and combined in
// a fixed order; every lane returns the same value. All 64 lanes must be
// active. For associative, commutative operations (max, the winner order);
// sums and log-sum-exp merges come out in one fixed order.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_val(float v) { return __uint_as_float(dpp32<CTRL>(__float_as_uint(v))); }
template <int CTRL>
__device__ __forceinline__ int dpp_val(int v) { return (int)dpp32<CTRL>((uint32_t)v); }
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_val(unsigned long long v) {
  return ((unsigned long long)dpp32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp32<CTRL>((uint32_t)v);
}
template <int CTRL>
__device__ __forceinline__ double dpp_val(double v) {
  return __longlong_as_double((long long)dpp_val<CTRL>((unsigned long long)__double_as_longlong(v)));
}
__device__ __forceinline__ int lane_val(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ float lane_val(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ unsigned long long lane_val(unsigned long long v, int l) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
  return ((unsigned long long)hi << 32) | lo;
}
__device__ __forceinline__ double lane_val(double v, int l) {
  return __longlong_as_double((long long)lane_val((unsigned long long)__double_as_longlong(v), l));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppRor4 = 0x124, kDppRor8 = 0x128;

__device__ __forceinline__ float wave_max_dpp(float x) {
  x = fmaxf(x, dpp_val<kDppXor1>(x));
  x = fmaxf(x, dpp_val<kDppXor2>(x));
  x = fmaxf(x, dpp_val<kDppRor4>(x));
  x = fmaxf(x, dpp_val<kDppRor8>(x));
  return fmaxf(fmaxf(lane_val(x, 0), lane_val(x, 16)), fmaxf(lane_val(x, 32), lane_val(x, 48)));
}
__device__ __forceinline__ float wave_sum_dpp(float x) {
  x += dpp_val<kDppXor1>(x);
  x += dpp_val<kDppXor2>(x);
  x += dpp_val<kDppRor4>(x);
  x += dpp_val<kDppRor8>(x);
  return (lane_val(x, 0) + lane_val(x, 16)) + (lane_val(x, 32) + lane_val(x, 48));
}
__device__ __forceinline__ unsigned long long wave_max_key(unsigned long long k) {
  unsigned long long o;
  o = dpp_val<kDppXor1>(k);
  k = o > k ? o : k;
  o = dpp_val<kDppXor2>(k);
  k = o > k ? o : k;
  o = dpp_val<kDppRor4>(k);
  k = o > k ? o : k;
  o = dpp_val<kDppRor8>(k);
  k = o > k ? o : k;
  unsigned long long r = lane_val(k, 0);
#pragma unroll
  for (int l = 16; l < 64; l += 16) {
    const unsigned long long x = lane_val(k, l);
    r = x > r ? x : r;
  }
  return r;
}
__device__ __forceinline__ void wave_lse_merge_dpp(float& m, float& s) {
  lse_merge(m, s, dpp_val<kDppXor1>(m), dpp_val<kDppXor1>(s));
  lse_merge(m, s, dpp_val<kDppXor2>(m), dpp_val<kDppXor2>(s));
  lse_merge(m, s, dpp_val<kDppRor4>(m), dpp_val<kDppRor4>(s));
  lse_merge(m, s, dpp_val<kDppRor8>(m), dpp_val<kDppRor8>(s));
  float rm = lane_val(m, 0), rs = lane_val(s, 0);
#pragma unroll
  for (int l = 16; l < 64; l += 16) lse_merge(rm, rs, lane_val(m, l), lane_val(s, l));
  m = rm;
  s = rs;
}

}  // namespace mds
