// Context-KV precompute ["DSpark 的实现和测评", section Context KV 预计算]: the draft
// KV cache of new context tokens is filled from the target's intermediate hidden states
// in one pass instead of a layer-by-layer target forward:
//
//   ctx     = aux . fc_w^T (+ fc_b)                  [M, H_d]     the draft-logit GEMM
//   normed  = bf16(RMSNorm(ctx) * hnorm_w)           [M, H_d]     ctx_rmsnorm
//   all_kv  = normed . kv_w^T                        [M, L*2*kv]  the draft-logit GEMM
//   per token, layer l, head h (all layers in one launch):
//     K = RoPE(RMSNorm(all_kv[l, 0, h] + b) * knorm_w[l], pos)  -> k_cache[l, slot, h]
//     V = all_kv[l, 1, h] + b                                    -> v_cache[l, slot, h]
//                                                                    ctx_kv_finish
//
// The two products are MFMA GEMMs (the draft-logit kernels).  With heads of 128 and
// more than 64 tokens the K/V product finishes each output tile itself (bias, K norm,
// RoPE, bf16, slot writes; kv_epilogue_half in gemm.hip), so all_kv never reaches
// memory; otherwise it writes all_kv in fp32 and ctx_kv_finish reads it.  Angles of the
// rotary embedding are formed in double per token and shared by every layer and head:
// in ctx_kv_finish, or for the fused epilogue as a float table [cos x 64, sin x 64] per
// token (ctx_rope_table).
#include <math.h>

#include "device.hpp"
#include "kernels.hpp"

namespace dspark {

namespace {

// float32 -> bf16 bits, round to nearest, ties to even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float block_sum(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = 0.0f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += red[w];
  __syncthreads();
  return t;
}

// the rotary table for heads of 128: rope[m, i] = cos, rope[m, 64 + i] = sin of
// positions[m] * theta^(-2 i / 128), formed in double; one thread per (token, i)
__global__ __launch_bounds__(256) void ctx_rope_table(const int32_t* __restrict__ positions, float* __restrict__ rope,
                                                      int M, double theta) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (int64_t)M * 64) return;
  const int64_t m = t >> 6;
  const int i = (int)(t & 63);
  const double ang = (double)positions[m] * pow(theta, -2.0 * (double)i / 128.0);
  double s_, c_;
  sincos(ang, &s_, &c_);
  rope[(size_t)m * 128 + i] = (float)c_;
  rope[(size_t)m * 128 + 64 + i] = (float)s_;
}

// one workgroup per row: x (+ bias) -> x / sqrt(mean(x^2) + eps) * w -> bf16
__global__ __launch_bounds__(256) void ctx_rmsnorm(const float* __restrict__ x, const uint16_t* __restrict__ bias,
                                                   const uint16_t* __restrict__ w, uint16_t* __restrict__ out, int Hd,
                                                   float eps) {
  __shared__ float red[4];
  const float* row = x + (size_t)blockIdx.x * Hd;
  float ss = 0.0f;
  for (int j = threadIdx.x; j < Hd; j += 256) {
    const float v = row[j] + (bias ? bf16_to_f32(bias[j]) : 0.0f);
    ss = fmaf(v, v, ss);
  }
  const float inv = 1.0f / sqrtf(block_sum(ss, red) / (float)Hd + eps);
  uint16_t* orow = out + (size_t)blockIdx.x * Hd;
  for (int j = threadIdx.x; j < Hd; j += 256) {
    const float v = row[j] + (bias ? bf16_to_f32(bias[j]) : 0.0f);
    orow[j] = f32_to_bf16(v * inv * bf16_to_f32(w[j]));
  }
}

// one workgroup per row, H_d <= 1024 x kRowVec: the row in registers as float4, one pass
constexpr int kRowVec = 16;
__global__ __launch_bounds__(256) void ctx_rmsnorm_vec(const float* __restrict__ x, const uint16_t* __restrict__ bias,
                                                       const uint16_t* __restrict__ w, uint16_t* __restrict__ out,
                                                       int Hd, float eps) {
  __shared__ float red[4];
  const float4* row = reinterpret_cast<const float4*>(x + (size_t)blockIdx.x * Hd);
  const int n4 = Hd / 4;
  float4 v[kRowVec];
  float ss = 0.0f;
#pragma unroll
  for (int t = 0; t < kRowVec; ++t) {
    const int j = threadIdx.x + 256 * t;
    v[t] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (j < n4) {
      v[t] = row[j];
      if (bias) {
        const uint2 bb = reinterpret_cast<const uint2*>(bias)[j];
        v[t].x += bf16_to_f32(bb.x & 0xFFFF);
        v[t].y += bf16_to_f32(bb.x >> 16);
        v[t].z += bf16_to_f32(bb.y & 0xFFFF);
        v[t].w += bf16_to_f32(bb.y >> 16);
      }
      ss = fmaf(v[t].x, v[t].x, fmaf(v[t].y, v[t].y, fmaf(v[t].z, v[t].z, fmaf(v[t].w, v[t].w, ss))));
    }
  }
  const float inv = 1.0f / sqrtf(block_sum(ss, red) / (float)Hd + eps);
  uint2* orow = reinterpret_cast<uint2*>(out + (size_t)blockIdx.x * Hd);
#pragma unroll
  for (int t = 0; t < kRowVec; ++t) {
    const int j = threadIdx.x + 256 * t;
    if (j < n4) {
      const uint2 ww = reinterpret_cast<const uint2*>(w)[j];
      const uint32_t a = f32_to_bf16(v[t].x * inv * bf16_to_f32(ww.x & 0xFFFF));
      const uint32_t b = f32_to_bf16(v[t].y * inv * bf16_to_f32(ww.x >> 16));
      const uint32_t c = f32_to_bf16(v[t].z * inv * bf16_to_f32(ww.y & 0xFFFF));
      const uint32_t d = f32_to_bf16(v[t].w * inv * bf16_to_f32(ww.y >> 16));
      orow[j] = make_uint2(a | (b << 16), c | (d << 16));
    }
  }
}

constexpr int kMaxHd = 256;

// one workgroup per token; wave w takes the (layer, head) pairs w, w + 4, ...; lane i
// holds the rotary pairs (i + 64 t, i + 64 t + hd/2) of a head's hd values
__global__ __launch_bounds__(256) void ctx_kv_finish(const float* __restrict__ allkv, const uint16_t* __restrict__ kv_b,
                                                     const uint16_t* __restrict__ knorm_w,
                                                     const int32_t* __restrict__ positions,
                                                     const int64_t* __restrict__ slots, uint16_t* __restrict__ kc,
                                                     uint16_t* __restrict__ vc, int L, int nkv, int hd,
                                                     int64_t num_slots, float eps, double theta) {
  __shared__ float cs[kMaxHd / 2], sn[kMaxHd / 2];
  const int m = blockIdx.x;
  const int half = hd / 2;
  const int64_t slot = slots[m];
  if (slot < 0 || slot >= num_slots) return;  // (uniform) a slot outside the cache is skipped
  const double pos = (double)positions[m];
  for (int i = threadIdx.x; i < half; i += 256) {
    const double ang = pos * pow(theta, -2.0 * (double)i / (double)hd);
    double s, c;
    sincos(ang, &s, &c);
    cs[i] = (float)c;
    sn[i] = (float)s;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kv = nkv * hd;
  const float* row = allkv + (size_t)m * L * 2 * kv;
  for (int p = wave; p < L * nkv; p += 4) {
    const int l = p / nkv, h = p % nkv;
    const int ko = (2 * l) * kv + h * hd, vo = (2 * l + 1) * kv + h * hd;
    // K: bias, RMSNorm over hd with the layer's weight, rotate-half RoPE
    float a[kMaxHd / 128], b[kMaxHd / 128];
    float ss = 0.0f;
#pragma unroll
    for (int t = 0; t < kMaxHd / 128; ++t) {
      const int i = lane + 64 * t;
      a[t] = b[t] = 0.0f;
      if (i < half) {
        a[t] = row[ko + i] + bf16_to_f32(kv_b[ko + i]);
        b[t] = row[ko + i + half] + bf16_to_f32(kv_b[ko + i + half]);
        ss = fmaf(a[t], a[t], fmaf(b[t], b[t], ss));
      }
    }
    for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    const float inv = 1.0f / sqrtf(ss / (float)hd + eps);
    const uint16_t* kw = knorm_w + (size_t)l * hd;
    uint16_t* kdst = kc + (((size_t)l * num_slots + slot) * nkv + h) * hd;
    uint16_t* vdst = vc + (((size_t)l * num_slots + slot) * nkv + h) * hd;
#pragma unroll
    for (int t = 0; t < kMaxHd / 128; ++t) {
      const int i = lane + 64 * t;
      if (i < half) {
        const float x1 = a[t] * inv * bf16_to_f32(kw[i]);
        const float x2 = b[t] * inv * bf16_to_f32(kw[i + half]);
        kdst[i] = f32_to_bf16(x1 * cs[i] - x2 * sn[i]);
        kdst[i + half] = f32_to_bf16(x2 * cs[i] + x1 * sn[i]);
      }
    }
    // V: bias only
    for (int i = lane; i < hd; i += 64) vdst[i] = f32_to_bf16(row[vo + i] + bf16_to_f32(kv_b[vo + i]));
  }
}

// hd = 128: one workgroup per token, one (layer, head) per wave and iteration; lanes
// 0-31 do the head's K (lane q: entries 2q, 2q+1 and their rotary partners 2q+64,
// 2q+65), lanes 32-63 its V (four consecutive entries each); paired loads and stores
__global__ __launch_bounds__(256) void ctx_kv_finish128(const float* __restrict__ allkv,
                                                        const uint16_t* __restrict__ kv_b,
                                                        const uint16_t* __restrict__ knorm_w,
                                                        const int32_t* __restrict__ positions,
                                                        const int64_t* __restrict__ slots,
                                                        uint16_t* __restrict__ kc, uint16_t* __restrict__ vc, int L,
                                                        int nkv, int64_t num_slots, float eps, double theta) {
  constexpr int hd = 128, half = 64;
  __shared__ float cs[half], sn[half];
  const int m = blockIdx.x;
  const int64_t slot = slots[m];
  if (slot < 0 || slot >= num_slots) return;  // (uniform) a slot outside the cache is skipped
  if (threadIdx.x < half) {
    const double ang = (double)positions[m] * pow(theta, -2.0 * (double)threadIdx.x / (double)hd);
    double s_, c_;
    sincos(ang, &s_, &c_);
    cs[threadIdx.x] = (float)c_;
    sn[threadIdx.x] = (float)s_;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kv = nkv * hd;
  const float* row = allkv + (size_t)m * L * 2 * kv;
  for (int p = wave; p < L * nkv; p += 4) {
    const int l = p / nkv, h = p % nkv;
    const size_t cbase = (((size_t)l * num_slots + slot) * nkv + h) * hd;
    if (lane < 32) {
      const int i = 2 * lane, ko = (2 * l) * kv + h * hd;
      const float2 x = *reinterpret_cast<const float2*>(row + ko + i);
      const float2 y = *reinterpret_cast<const float2*>(row + ko + i + half);
      const uint32_t bx = *reinterpret_cast<const uint32_t*>(kv_b + ko + i);
      const uint32_t by = *reinterpret_cast<const uint32_t*>(kv_b + ko + i + half);
      const float a0 = x.x + bf16_to_f32(bx & 0xFFFF), a1 = x.y + bf16_to_f32(bx >> 16);
      const float b0 = y.x + bf16_to_f32(by & 0xFFFF), b1 = y.y + bf16_to_f32(by >> 16);
      float ss = fmaf(a0, a0, fmaf(a1, a1, fmaf(b0, b0, b1 * b1)));
      for (int o = 16; o > 0; o >>= 1) ss += __shfl_xor(ss, o);   // (within lanes 0-31)
      const float inv = 1.0f / sqrtf(ss / (float)hd + eps);
      const uint16_t* kw = knorm_w + (size_t)l * hd;
      const uint32_t wx = *reinterpret_cast<const uint32_t*>(kw + i);
      const uint32_t wy = *reinterpret_cast<const uint32_t*>(kw + i + half);
      const float x0 = a0 * inv * bf16_to_f32(wx & 0xFFFF), x1 = a1 * inv * bf16_to_f32(wx >> 16);
      const float y0 = b0 * inv * bf16_to_f32(wy & 0xFFFF), y1 = b1 * inv * bf16_to_f32(wy >> 16);
      const float c0 = cs[i], s0 = sn[i], c1 = cs[i + 1], s1 = sn[i + 1];
      const uint32_t lo = (uint32_t)f32_to_bf16(x0 * c0 - y0 * s0) | ((uint32_t)f32_to_bf16(x1 * c1 - y1 * s1) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16(y0 * c0 + x0 * s0) | ((uint32_t)f32_to_bf16(y1 * c1 + x1 * s1) << 16);
      *reinterpret_cast<uint32_t*>(kc + cbase + i) = lo;
      *reinterpret_cast<uint32_t*>(kc + cbase + i + half) = hi;
    } else {
      const int i = 4 * (lane - 32), vo = (2 * l + 1) * kv + h * hd;
      const float4 x = *reinterpret_cast<const float4*>(row + vo + i);
      const uint2 bb = *reinterpret_cast<const uint2*>(kv_b + vo + i);
      const uint32_t a = f32_to_bf16(x.x + bf16_to_f32(bb.x & 0xFFFF));
      const uint32_t b = f32_to_bf16(x.y + bf16_to_f32(bb.x >> 16));
      const uint32_t c = f32_to_bf16(x.z + bf16_to_f32(bb.y & 0xFFFF));
      const uint32_t d = f32_to_bf16(x.w + bf16_to_f32(bb.y >> 16));
      *reinterpret_cast<uint2*>(vc + cbase + i) = make_uint2(a | (b << 16), c | (d << 16));
    }
  }
}

}  // namespace

// workspace: the fc product (fp32), the normalised states (bf16), then either the rotary
// table (fused epilogue) or all_kv (fp32)
size_t context_kv_workspace_bytes(int M, int Hd, int L, int nkv, int hd) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t tail = kv_product_fused(M, Hd, hd) ? al((size_t)M * 128 * sizeof(float))
                                                  : al((size_t)M * L * 2 * nkv * hd * sizeof(float));
  return al((size_t)M * Hd * sizeof(float)) + al((size_t)M * Hd * sizeof(uint16_t)) + tail;
}

hipError_t launch_context_kv(const uint16_t* aux, const uint16_t* fc_w, const uint16_t* fc_b, const uint16_t* hnorm_w,
                             const uint16_t* kv_w, const uint16_t* kv_b, const uint16_t* knorm_w,
                             const int32_t* positions, const int64_t* slots, uint16_t* k_cache, uint16_t* v_cache,
                             int M, int H_in, int Hd, int L, int nkv, int hd, int64_t num_slots, float eps,
                             float theta, void* workspace, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  char* w = static_cast<char*>(workspace);
  float* ctx = reinterpret_cast<float*>(w);
  w += al((size_t)M * Hd * sizeof(float));
  uint16_t* normed = reinterpret_cast<uint16_t*>(w);
  w += al((size_t)M * Hd * sizeof(uint16_t));
  float* tail = reinterpret_cast<float*>(w);
  const bool fused = kv_product_fused(M, Hd, hd);
  float* rope = fused ? tail : nullptr;
  if (fused)
    hipLaunchKernelGGL(ctx_rope_table, dim3((unsigned)(((int64_t)M * 64 + 255) / 256)), dim3(256), 0, stream,
                       positions, rope, M, (double)theta);
  hipError_t e = launch_draft_logits(aux, fc_w, ctx, M, H_in, Hd, nullptr, nullptr, stream);
  if (e != hipSuccess) return e;
  if (Hd <= 1024 * kRowVec)
    hipLaunchKernelGGL(ctx_rmsnorm_vec, dim3(M), dim3(256), 0, stream, ctx, fc_b, hnorm_w, normed, Hd, eps);
  else
    hipLaunchKernelGGL(ctx_rmsnorm, dim3(M), dim3(256), 0, stream, ctx, fc_b, hnorm_w, normed, Hd, eps);
  if (fused) {
    KvEpilogue ep;
    ep.kv_b = kv_b;
    ep.knorm_w = knorm_w;
    ep.rope = rope;
    ep.slots = slots;
    ep.kc = k_cache;
    ep.vc = v_cache;
    ep.nkv = nkv;
    ep.num_slots = num_slots;
    ep.eps = eps;
    return launch_kv_product(normed, kv_w, M, Hd, L * 2 * nkv * hd, ep, stream);
  }
  float* allkv = tail;
  e = launch_draft_logits(normed, kv_w, allkv, M, Hd, L * 2 * nkv * hd, nullptr, nullptr, stream);
  if (e != hipSuccess) return e;
  if (hd == 128)
    hipLaunchKernelGGL(ctx_kv_finish128, dim3(M), dim3(256), 0, stream, allkv, kv_b, knorm_w, positions, slots,
                       k_cache, v_cache, L, nkv, num_slots, eps, (double)theta);
  else
    hipLaunchKernelGGL(ctx_kv_finish, dim3(M), dim3(256), 0, stream, allkv, kv_b, knorm_w, positions, slots,
                       k_cache, v_cache, L, nkv, hd, num_slots, eps, (double)theta);
  return hipGetLastError();
}

}  // namespace dspark
