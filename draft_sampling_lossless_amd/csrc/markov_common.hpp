// Pieces shared by the two implementations of the Markov loop (markov.hip: one
// launch per step for many requests; markov_few.hip: one cooperative launch for
// few requests).
#pragma once

#include <math.h>

#include "device.hpp"

namespace dspark {
namespace mk {

constexpr int kReqPerWave = 16;
constexpr int kReqPerWG = 64;
constexpr int kChunk = 64;       // vocabulary entries per MFMA chunk
constexpr int kMaxKSteps = 8;    // r <= 256 in steps of 32

struct MarkovPartial {
  float key;   // best Gumbel key (base-2 units; T == 0: the logit)
  int tok;     // its target id
  float m, s;  // log-sum-exp state: log2 sum 2^y = m + log2 s, y = l * log2(e) / T (T == 0: y = l)
};

inline int cu_count_markov() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

__device__ __forceinline__ bf16x8 zero8() { return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0)); }

__device__ __forceinline__ void wg_coords(int CH, int nvs, int nbt, int& vs, int& bt) {
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  vs = (local / nbt) * 8 + xcd;
  bt = local % nbt;
}

// argmax (key desc, id asc) and log-sum-exp merges of a (key, tok, m, s) state
__device__ __forceinline__ void state_merge(float& key, int& tok, float& m, float& s, float k2, int t2, float m2,
                                            float s2) {
  if (key_beats(k2, t2, key, tok)) {
    key = k2;
    tok = t2;
  }
  lse2_merge(m, s, m2, s2);
}
template <int kCtrl>
__device__ __forceinline__ void state_stage(float& key, int& tok, float& m, float& s) {
  state_merge(key, tok, m, s, dpp_f32<kCtrl>(key), (int)dpp_u32<kCtrl>((uint32_t)tok), dpp_f32<kCtrl>(m),
              dpp_f32<kCtrl>(s));
}
// merge over each 16-lane row
__device__ __forceinline__ void row_state_merge(float& key, int& tok, float& m, float& s) {
  state_stage<kDppSwap1>(key, tok, m, s);
  state_stage<kDppSwap2>(key, tok, m, s);
  state_stage<kDppMirror8>(key, tok, m, s);
  state_stage<kDppMirror16>(key, tok, m, s);
}
// merge over the wave (every lane ends with the same state)
__device__ __forceinline__ void wave_state_merge(float& key, int& tok, float& m, float& s) {
  row_state_merge(key, tok, m, s);
  uint32_t k0, k1, t0, t1, m0, m1, s0, s1;
  rows_pair(__float_as_uint(key), k0, k1);
  rows_pair((uint32_t)tok, t0, t1);
  rows_pair(__float_as_uint(m), m0, m1);
  rows_pair(__float_as_uint(s), s0, s1);
  key = __uint_as_float(k0);
  tok = (int)t0;
  m = __uint_as_float(m0);
  s = __uint_as_float(s0);
  state_merge(key, tok, m, s, __uint_as_float(k1), (int)t1, __uint_as_float(m1), __uint_as_float(s1));
  halves_pair(__float_as_uint(key), k0, k1);
  halves_pair((uint32_t)tok, t0, t1);
  halves_pair(__float_as_uint(m), m0, m1);
  halves_pair(__float_as_uint(s), s0, s1);
  key = __uint_as_float(k0);
  tok = (int)t0;
  m = __uint_as_float(m0);
  s = __uint_as_float(s0);
  state_merge(key, tok, m, s, __uint_as_float(k1), (int)t1, __uint_as_float(m1), __uint_as_float(s1));
}

template <int kCtrl>
__device__ __forceinline__ void argmax_stage(float& key, int& tok) {
  const float k2 = dpp_f32<kCtrl>(key);
  const int t2 = (int)dpp_u32<kCtrl>((uint32_t)tok);
  if (key_beats(k2, t2, key, tok)) {
    key = k2;
    tok = t2;
  }
}
// argmax (key desc, id asc) over each 16-lane row
__device__ __forceinline__ void row_argmax(float& key, int& tok) {
  argmax_stage<kDppSwap1>(key, tok);
  argmax_stage<kDppSwap2>(key, tok);
  argmax_stage<kDppMirror8>(key, tok);
  argmax_stage<kDppMirror16>(key, tok);
}
// argmax (key desc, id asc) over the wave
__device__ __forceinline__ void wave_argmax(float& key, int& tok) {
  row_argmax(key, tok);
  uint32_t k0, k1, t0, t1;
  rows_pair(__float_as_uint(key), k0, k1);
  rows_pair((uint32_t)tok, t0, t1);
  key = __uint_as_float(k0);
  tok = (int)t0;
  if (key_beats(__uint_as_float(k1), (int)t1, key, tok)) {
    key = __uint_as_float(k1);
    tok = (int)t1;
  }
  halves_pair(__float_as_uint(key), k0, k1);
  halves_pair((uint32_t)tok, t0, t1);
  key = __uint_as_float(k0);
  tok = (int)t0;
  if (key_beats(__uint_as_float(k1), (int)t1, key, tok)) {
    key = __uint_as_float(k1);
    tok = (int)t1;
  }
}
template <int kCtrl>
__device__ __forceinline__ void lse_stage(float& m, float& s) {
  lse2_merge(m, s, dpp_f32<kCtrl>(m), dpp_f32<kCtrl>(s));
}
// log-sum-exp merge over each 16-lane row
__device__ __forceinline__ void row_lse_merge(float& m, float& s) {
  lse_stage<kDppSwap1>(m, s);
  lse_stage<kDppSwap2>(m, s);
  lse_stage<kDppMirror8>(m, s);
  lse_stage<kDppMirror16>(m, s);
}

// Cross-workgroup traffic of the persistent kernel goes through device-scope
// atomic stores and loads: on this chip they bypass the per-XCD L2 caches, so the
// barrier needs no L2 write-back / invalidate (which would cost far more than the
// few partials exchanged per step).
__device__ __forceinline__ void store_partial(MarkovPartial* p, const MarkovPartial& v) {
  __hip_atomic_store(&p->key, v.key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(&p->tok, v.tok, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(&p->m, v.m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(&p->s, v.s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ MarkovPartial load_partial(const MarkovPartial* p) {
  MarkovPartial v;
  v.key = __hip_atomic_load(&p->key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  v.tok = __hip_atomic_load(&p->tok, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  v.m = __hip_atomic_load(&p->m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  v.s = __hip_atomic_load(&p->s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return v;
}

// Merge every workgroup's partial of request b (one wave; all lanes get the result).
__device__ __forceinline__ MarkovPartial wave_merge(const MarkovPartial* __restrict__ part, int count, int lane) {
  float key = -INFINITY, m = -INFINITY, s = 0.0f;
  int tok = 0x7FFFFFFF;
  for (int p = lane; p < count; p += 64) {
    const MarkovPartial q = load_partial(part + p);
    state_merge(key, tok, m, s, q.key, q.tok, q.m, q.s);
  }
  wave_state_merge(key, tok, m, s);
  return MarkovPartial{key, tok, m, s};
}

__device__ __forceinline__ float log_z_of(const MarkovPartial& q, float T) {
  return (T > 0.0f) ? (q.m + log2f(q.s)) * 0.69314718055994531f : q.m;
}


// sum of the products of eight bf16 pairs (two 16-byte pieces)
__device__ __forceinline__ float dot_bf16x8(const uint4& a, const uint4& b) {
  const uint32_t x[4] = {a.x, a.y, a.z, a.w}, y[4] = {b.x, b.y, b.z, b.w};
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    s += __uint_as_float(x[q] << 16) * __uint_as_float(y[q] << 16);
    s += __uint_as_float(x[q] & 0xFFFF0000u) * __uint_as_float(y[q] & 0xFFFF0000u);
  }
  return s;
}

// the confidence head's probability from its logit parts
__device__ __forceinline__ float conf_prob(float hdot, float edot, float bias, float tau) {
  return 1.0f / (1.0f + expf(-(hdot + edot + bias) / tau));
}

}  // namespace mk
}  // namespace dspark
