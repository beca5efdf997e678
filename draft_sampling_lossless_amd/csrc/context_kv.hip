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
// The two products are MFMA GEMMs (the draft-logit kernels, fp32 out); the two small
// passes are memory-bound and read what the products wrote.  Angles of the rotary
// embedding are formed in double per token and shared by every layer and head.
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

}  // namespace

size_t context_kv_workspace_bytes(int M, int Hd, int L, int nkv, int hd) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  return al((size_t)M * Hd * sizeof(float)) + al((size_t)M * Hd * sizeof(uint16_t)) +
         al((size_t)M * L * 2 * nkv * hd * sizeof(float));
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
  float* allkv = reinterpret_cast<float*>(w);
  hipError_t e = launch_draft_logits(aux, fc_w, ctx, M, H_in, Hd, nullptr, nullptr, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ctx_rmsnorm, dim3(M), dim3(256), 0, stream, ctx, fc_b, hnorm_w, normed, Hd, eps);
  e = launch_draft_logits(normed, kv_w, allkv, M, Hd, L * 2 * nkv * hd, nullptr, nullptr, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(ctx_kv_finish, dim3(M), dim3(256), 0, stream, allkv, kv_b, knorm_w, positions, slots, k_cache,
                     v_cache, L, nkv, hd, num_slots, eps, (double)theta);
  return hipGetLastError();
}

}  // namespace dspark
