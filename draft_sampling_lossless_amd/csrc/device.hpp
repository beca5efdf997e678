// Device building blocks shared by the DSpark kernels (gfx950 / CDNA4).
//
//  * Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) and the uniform map
//    u = ((w >> 8) | 1) * 2^-24 (exact in fp32, never 0 or 1).
//  * The Gumbel-max key of the Markov sampler, in base-2 units.
//  * The portable log2 and exact comparison of the exponential race.
//  * bf16 vector types for the MFMA operands.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Philox counter tags (counter word 3).
constexpr uint32_t kTagDraft = 0;   // Gumbel noise of the Markov loop
constexpr uint32_t kTagAccept = 1;  // acceptance uniform of verify
constexpr uint32_t kTagResid = 2;   // residual resample race
constexpr uint32_t kTagBonus = 3;   // bonus race

struct u32x4 {
  uint32_t x, y, z, w;
};

// a ^ b ^ c in one gfx950 three-input bitwise instruction (truth table 0x96)
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

// Ten Philox4x32 rounds.  Each round multiplies counter words 0 and 2 by the two
// round constants (full 64-bit products), then mixes the halves with words 1, 3
// and the key; the key takes a Weyl step between rounds.
__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int rnd = 0; rnd < 10; ++rnd) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    c = u32x4{xor3(hi1, c.y, k0), lo1, xor3(hi0, c.w, k1), lo0};
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

__device__ __forceinline__ float uniform01(uint32_t w) {
  return (float)((w >> 8) | 1u) * 0x1.0p-24f;
}

// -log2(-log2(u)): Gumbel noise scaled by log2(e), up to an additive constant.
// argmax_j (l_j * log2(e)/T + g2(u_j)) is the Gumbel-max sample of softmax(l/T).
__device__ __forceinline__ float gumbel2(uint32_t w) {
  const float u = uniform01(w);
  return -__builtin_amdgcn_logf(-__builtin_amdgcn_logf(u));
}

// Portable float32 log2 built from IEEE add / multiply / divide only, in a fixed
// order, no contraction: u = m * 2^e with m in [sqrt2/2, sqrt2);
// log2 u = e + s * (c1 + z (c3 + z (c5 + z (c7 + z c9)))),  s = (m-1)/(m+1), z = s*s,
// c_k = fp32(2 / (k ln 2)).  Valid for positive normal u.
__device__ __forceinline__ float plog2(float u) {
#pragma clang fp contract(off)
  constexpr double kLn2 = 0.69314718055994530942;
  constexpr float c1 = (float)(2.0 / (1.0 * kLn2));
  constexpr float c3 = (float)(2.0 / (3.0 * kLn2));
  constexpr float c5 = (float)(2.0 / (5.0 * kLn2));
  constexpr float c7 = (float)(2.0 / (7.0 * kLn2));
  constexpr float c9 = (float)(2.0 / (9.0 * kLn2));
  const uint32_t bits = __float_as_uint(u);
  int e = (int)((bits >> 23) & 0xFFu) - 127;
  float m = __uint_as_float((bits & 0x7FFFFFu) | 0x3F800000u);
  if (m > __uint_as_float(0x3FB504F3u)) {  // float nearest below sqrt(2)
    m = m * 0.5f;
    e += 1;
  }
  const float s = __fdiv_rn(__fsub_rn(m, 1.0f), __fadd_rn(m, 1.0f));
  const float z = __fmul_rn(s, s);
  float p = c9;
  p = __fadd_rn(__fmul_rn(p, z), c7);
  p = __fadd_rn(__fmul_rn(p, z), c5);
  p = __fadd_rn(__fmul_rn(p, z), c3);
  p = __fadd_rn(__fmul_rn(p, z), c1);
  return __fadd_rn((float)e, __fmul_rn(s, p));
}

// Race candidate: weight r >= 0, exponential E > 0, index v.  a beats b iff
// r_a / E_a > r_b / E_b, compared exactly as r_a * E_b > r_b * E_a in double
// (a product of two floats is exact in double); ties go to the smaller index.
struct RaceCand {
  float r;
  float E;
  int v;
};

__device__ __forceinline__ bool race_beats(float ra, float Ea, int va, float rb, float Eb, int vb) {
  const double lhs = (double)ra * (double)Eb;
  const double rhs = (double)rb * (double)Ea;
  return lhs > rhs || (lhs == rhs && va < vb);
}

// Argmax candidate of the Markov sampler: larger key wins, ties to smaller id.
__device__ __forceinline__ bool key_beats(float ka, int ta, float kb, int tb) {
  return ka > kb || (ka == kb && ta < tb);
}

// Online log-sum-exp state in base-2 units: value = m + log2(s).
__device__ __forceinline__ void lse2_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;  // both empty
  s = s * __builtin_amdgcn_exp2f(m - mn) + s2 * __builtin_amdgcn_exp2f(m2 - mn);
  m = mn;
}

// Workgroup barrier without the memory fence of __syncthreads() (which makes every
// wave wait for all of its outstanding global loads): only this wave's LDS
// operations are completed first.  Used where asynchronous global->LDS loads must
// stay in flight across the barrier; their completion is awaited explicitly.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---- cross-lane moves without the LDS crossbar
// A butterfly over a 64-lane wave: four DPP moves inside each 16-lane row (swap
// neighbours, swap pairs, mirror within 8, mirror within 16), then the gfx950
// permlane swaps, which hand every lane the value of the same lane in the other
// row of its row pair (16) and in the other half of the wave (32).  After a stage
// both partners hold the merge of their two inputs (up to the rounding order of
// a floating-point merge), so every lane of the group ends with the group's result.
template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0u, v, kCtrl, 0xF, 0xF, false);
}
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<kCtrl>(__float_as_uint(v)));
}
constexpr int kDppSwap1 = 0xB1, kDppSwap2 = 0x4E, kDppMirror8 = 0x141, kDppMirror16 = 0x140;

// {value in the even row, value in the odd row} of this lane's row pair
__device__ __forceinline__ void rows_pair(uint32_t v, uint32_t& even, uint32_t& odd) {
  const auto s = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  even = s[0];
  odd = s[1];
}
// {value in the lower half, value in the upper half} of the wave
__device__ __forceinline__ void halves_pair(uint32_t v, uint32_t& lo, uint32_t& hi) {
  const auto s = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  lo = s[0];
  hi = s[1];
}

// sum over aligned groups of `width` lanes (1, 2, 4, ..., 64; uniform)
__device__ __forceinline__ float group_sum(float v, int width) {
  if (width >= 2) v += dpp_f32<kDppSwap1>(v);
  if (width >= 4) v += dpp_f32<kDppSwap2>(v);
  if (width >= 8) v += dpp_f32<kDppMirror8>(v);
  if (width >= 16) v += dpp_f32<kDppMirror16>(v);
  if (width >= 32) {
    uint32_t a, b;
    rows_pair(__float_as_uint(v), a, b);
    v = __uint_as_float(a) + __uint_as_float(b);
  }
  if (width >= 64) {
    uint32_t a, b;
    halves_pair(__float_as_uint(v), a, b);
    v = __uint_as_float(a) + __uint_as_float(b);
  }
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, dpp_f32<kDppSwap1>(v));
  v = fmaxf(v, dpp_f32<kDppSwap2>(v));
  v = fmaxf(v, dpp_f32<kDppMirror8>(v));
  v = fmaxf(v, dpp_f32<kDppMirror16>(v));
  uint32_t a, b;
  rows_pair(__float_as_uint(v), a, b);
  v = fmaxf(__uint_as_float(a), __uint_as_float(b));
  halves_pair(__float_as_uint(v), a, b);
  return fmaxf(__uint_as_float(a), __uint_as_float(b));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<kDppSwap1>(v));
  v = max(v, dpp_u32<kDppSwap2>(v));
  v = max(v, dpp_u32<kDppMirror8>(v));
  v = max(v, dpp_u32<kDppMirror16>(v));
  uint32_t a, b;
  rows_pair(v, a, b);
  v = max(a, b);
  halves_pair(v, a, b);
  return max(a, b);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

}  // namespace dspark
