// Stage 2: the N-step low-rank Markov (bigram) sampling loop.
//
// Step i of request b: e = W1[prev_b] (r values), bias = W2 . e (one value per
// draft token), l = base[b, i] + bias (written back in place), x = Gumbel-max
// sample of softmax(l / T_b) mapped to a target id, prev_b = x.  The step's
// argmax spans the whole vocabulary, so each step is one grid-wide pass:
//
//   markov_step   workgroup = 64 requests x (CH * 64) vocabulary entries.
//                 The bias tile is a dense [64 x r] x [r x 64] product per
//                 64-wide chunk: MFMA 16x16x32 bf16 with the gathered W1 rows
//                 (A operand) held in registers for the whole pass and the W2
//                 chunk (B operand) staged in LDS and shared by the 4 waves.
//                 The MFMA column of fragment f, lane n is vocabulary entry
//                 4n + f of the chunk, so each lane ends up holding 4
//                 consecutive entries of 4 requests: one float4 of base logits
//                 per request and one Philox block (4 words) per float4.
//                 Per lane and request a running best (key, target id) and a
//                 base-2 log-sum-exp (m, s) are kept; they are reduced over the
//                 16 lanes of a request group and written as one partial per
//                 (request, vocabulary slice).
//   markov_merge  one wave per request reduces the slice partials, writes the
//                 token and log Z.  The next step's kernel reads that token.
//
//   markov_small  few requests (B <= 16): the per-step work is small and the two
//                 launches per step are latency.  One cooperative workgroup per CU
//                 owns a fixed vocabulary slice for all N steps and keeps that
//                 slice of W2 in LDS; a grid barrier separates the steps, and every
//                 workgroup reduces the previous step's partials itself to learn the
//                 sampled tokens (workgroup 0 also writes them out).  The next step's
//                 base logits are loaded before the barrier.
//
// Workgroup order is XCD-aware: the workgroups of one vocabulary slice (one per
// request tile) go to the same XCD one after another, so the slice of W2 they
// all read is fetched from HBM once and then served by that XCD's L2.
#include <math.h>

#include <algorithm>

#include "device.hpp"
#include "kernels.hpp"
#include "markov_common.hpp"

namespace dspark {

namespace {

using namespace mk;

__global__ __launch_bounds__(256) void markov_step(float* __restrict__ logits, const uint16_t* __restrict__ w1,
                                                   const uint16_t* __restrict__ w2, const int64_t* __restrict__ d2t,
                                                   const int32_t* __restrict__ prev_tok, int prev_stride,
                                                   const float* __restrict__ temperature,
                                                   const uint32_t* __restrict__ request_id, uint32_t key0,
                                                   uint32_t key1, MarkovPartial* __restrict__ partial, int step,
                                                   int B, int N, int V, int Vd, int r, int CH, int nvs, int nbt) {
  extern __shared__ __attribute__((aligned(16))) char lds[];  // 64 rows x (2r + 16) bytes
  int vs, bt;
  wg_coords(CH, nvs, nbt, vs, bt);
  if (vs >= nvs) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int ksteps = (r + 31) / 32;
  const int row_bytes = 2 * r + 16;
  const int rq0 = bt * kReqPerWG + wave * kReqPerWave;
  const bool wave_active = rq0 < B;

  // A fragments: W1 rows of this wave's 16 requests (lane row n), all k steps.
  bf16x8 efrag[kMaxKSteps];
  {
    const int b = rq0 + n;
    // clamp: an out-of-range anchor (or a row with no finite key) must not read outside W1
    const int prev = (b < B) ? min(max(prev_tok[(size_t)b * prev_stride], 0), V - 1) : 0;
    const uint16_t* er = w1 + (size_t)prev * r;
#pragma unroll
    for (int s = 0; s < kMaxKSteps; ++s) {
      const int k = s * 32 + 8 * g;
      efrag[s] = (s < ksteps && k < r && b < B) ? __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(er + k))
                                                : zero8();
    }
  }

  // Epilogue requests of this lane: rq0 + 4g + i.
  float c2[4];
  bool noisy[4], rvalid[4];
  uint32_t rid[4];
  float bkey[4], bm[4], bs[4];
  int btok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int b = rq0 + 4 * g + i;
    rvalid[i] = b < B;
    const float T = rvalid[i] ? temperature[b] : 1.0f;
    noisy[i] = T > 0.0f;
    c2[i] = noisy[i] ? (1.0f / T) * 1.4426950408889634f : 1.0f;
    rid[i] = rvalid[i] ? request_id[b] : 0u;
    bkey[i] = -INFINITY;
    btok[i] = 0x7FFFFFFF;
    bm[i] = -INFINITY;
    bs[i] = 0.0f;
  }

  const int vbase = vs * CH * kChunk;
  const int kchunks16 = r / 8;  // 16-byte pieces per W2 row
  for (int c = 0; c < CH; ++c) {
    const int jc = vbase + c * kChunk;
    if (jc >= Vd) break;
    __syncthreads();
    // Stage W2 rows jc .. jc+63 into LDS; row rho goes to slot (rho % 4) * 16 + rho / 4
    // so that fragment f, lane n reads vocabulary entry 4n + f.
    for (int p = tid; p < kChunk * kchunks16; p += 256) {
      const int rho = p / kchunks16, piece = p % kchunks16;
      const int j = jc + rho;
      const uint4 v = (j < Vd) ? *reinterpret_cast<const uint4*>(w2 + (size_t)j * r + piece * 8) : make_uint4(0, 0, 0, 0);
      const int slot = (rho & 3) * 16 + (rho >> 2);
      *reinterpret_cast<uint4*>(lds + slot * row_bytes + piece * 16) = v;
    }
    __syncthreads();
    if (!wave_active) continue;

    floatx4 acc[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      acc[f] = floatx4{0.f, 0.f, 0.f, 0.f};
      const char* rowp = lds + (f * 16 + n) * row_bytes;
#pragma unroll
      for (int s = 0; s < kMaxKSteps; ++s) {
        if (s < ksteps) {
          const int k = s * 32 + 8 * g;
          const bf16x8 bfr = (k < r) ? __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(rowp + k * 2)) : zero8();
          acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(efrag[s], bfr, acc[f], 0, 0, 0);
        }
      }
    }

    const int jb = jc + 4 * n;  // this lane's 4 vocabulary entries jb .. jb+3
    if (jb >= Vd) continue;
    int tgt[4];
    if (d2t) {
      const longlong2 d01 = *reinterpret_cast<const longlong2*>(d2t + jb);
      const longlong2 d23 = *reinterpret_cast<const longlong2*>(d2t + jb + 2);
      tgt[0] = jb + (int)d01.x;
      tgt[1] = jb + 1 + (int)d01.y;
      tgt[2] = jb + 2 + (int)d23.x;
      tgt[3] = jb + 3 + (int)d23.y;
    } else {
#pragma unroll
      for (int f = 0; f < 4; ++f) tgt[f] = jb + f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (!rvalid[i]) continue;
      const int b = rq0 + 4 * g + i;
      float4* rowp = reinterpret_cast<float4*>(logits + ((size_t)b * N + step) * Vd + jb);
      float4 v = *rowp;
      v.x += acc[0][i];
      v.y += acc[1][i];
      v.z += acc[2][i];
      v.w += acc[3][i];
      *rowp = v;
      const float l[4] = {v.x, v.y, v.z, v.w};
      float y[4], key[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) y[f] = l[f] * c2[i];
      if (noisy[i]) {
        const u32x4 w = philox4x32_10(u32x4{(uint32_t)jb >> 2, (uint32_t)step, rid[i], kTagDraft}, key0, key1);
        key[0] = y[0] + gumbel2(w.x);
        key[1] = y[1] + gumbel2(w.y);
        key[2] = y[2] + gumbel2(w.z);
        key[3] = y[3] + gumbel2(w.w);
      } else {
#pragma unroll
        for (int f = 0; f < 4; ++f) key[f] = l[f];
      }
#pragma unroll
      for (int f = 0; f < 4; ++f)
        if (key_beats(key[f], tgt[f], bkey[i], btok[i])) {
          bkey[i] = key[f];
          btok[i] = tgt[f];
        }
      const float mx = fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3]));
      const float mn = fmaxf(bm[i], mx);
      float s = bs[i] * __builtin_amdgcn_exp2f(bm[i] - mn);
#pragma unroll
      for (int f = 0; f < 4; ++f) s += __builtin_amdgcn_exp2f(y[f] - mn);
      bs[i] = s;
      bm[i] = mn;
    }
  }
  if (!wave_active) return;

  // Reduce over the 16 lanes (n) of each request group g.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const float ok = __shfl_xor(bkey[i], off, 16);
      const int ot = __shfl_xor(btok[i], off, 16);
      const float om = __shfl_xor(bm[i], off, 16);
      const float os = __shfl_xor(bs[i], off, 16);
      if (key_beats(ok, ot, bkey[i], btok[i])) {
        bkey[i] = ok;
        btok[i] = ot;
      }
      lse2_merge(bm[i], bs[i], om, os);
    }
    const int b = rq0 + 4 * g + i;
    if (n == 0 && b < B) partial[(size_t)b * nvs + vs] = MarkovPartial{bkey[i], btok[i], bm[i], bs[i]};
  }
}

__global__ __launch_bounds__(256) void markov_merge(const MarkovPartial* __restrict__ partial,
                                                    const float* __restrict__ temperature,
                                                    int32_t* __restrict__ draft_tokens, float* __restrict__ log_z,
                                                    int step, int B, int N, int nvs) {
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (b >= B) return;
  float key = -INFINITY, m = -INFINITY, s = 0.0f;
  int tok = 0x7FFFFFFF;
  for (int p = lane; p < nvs; p += 64) {
    const MarkovPartial q = partial[(size_t)b * nvs + p];
    if (key_beats(q.key, q.tok, key, tok)) {
      key = q.key;
      tok = q.tok;
    }
    lse2_merge(m, s, q.m, q.s);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float ok = __shfl_xor(key, off);
    const int ot = __shfl_xor(tok, off);
    const float om = __shfl_xor(m, off);
    const float os = __shfl_xor(s, off);
    if (key_beats(ok, ot, key, tok)) {
      key = ok;
      tok = ot;
    }
    lse2_merge(m, s, om, os);
  }
  if (lane == 0) {
    draft_tokens[(size_t)b * N + step] = tok;
    const float T = temperature[b];
    log_z[(size_t)b * N + step] = (T > 0.0f) ? (m + __log2f(s)) * 0.69314718055994531f : m;
  }
}

__global__ void inverse_fill(int32_t* __restrict__ inv, int V) {
  const int v = blockIdx.x * blockDim.x + threadIdx.x;
  if (v < V) inv[v] = -1;
}

__global__ void inverse_scatter(const int64_t* __restrict__ d2t, int Vd, int V, int32_t* __restrict__ inv) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= Vd) return;
  const int64_t t = (int64_t)j + d2t[j];
  if (t >= 0 && t < V) inv[t] = j;
}

}  // namespace

MarkovPlan plan_markov(int B, int N, int Vd, int r, int cus) {
  MarkovPlan p{};
  p.few = plan_markov_few(B, N, Vd, r, cus);
  p.btiles = (B + kReqPerWG - 1) / kReqPerWG;
  const int chunks = (Vd + kChunk - 1) / kChunk;
  int ch = 16;
  while (ch > 1 && (long)((chunks + ch - 1) / ch) * p.btiles < 1024) ch >>= 1;
  p.chunks_per_wg = ch;
  p.vslices = (chunks + ch - 1) / ch;
  p.partial_bytes = (size_t)B * p.vslices * sizeof(MarkovPartial);
  // the query (cus == 0) must cover whichever path a launch picks
  if (p.few.bytes > p.partial_bytes) p.partial_bytes = p.few.bytes;
  return p;
}

hipError_t launch_markov_sample(float* logits, const uint16_t* w1, const uint16_t* w2, const int64_t* d2t,
                                const int32_t* anchor, const float* temperature, const uint32_t* request_id,
                                uint64_t seed, int32_t* draft_tokens, float* log_z, int B, int N, int V, int Vd,
                                int r, void* workspace, hipStream_t stream) {
  const MarkovPlan p = plan_markov(B, N, Vd, r, cu_count_markov());
  if (p.few.use)
    return launch_markov_few(p.few, logits, w1, w2, d2t, anchor, temperature, request_id, seed, draft_tokens, log_z,
                             B, N, V, Vd, r, workspace, stream);
  MarkovPartial* partial = static_cast<MarkovPartial*>(workspace);
  const int nvs8 = (p.vslices + 7) / 8 * 8;
  const dim3 grid(nvs8 * p.btiles), block(256);
  const size_t lds = (size_t)kChunk * (2 * r + 16);
  const uint32_t k0 = (uint32_t)(seed & 0xFFFFFFFFu), k1 = (uint32_t)(seed >> 32);
  for (int i = 0; i < N; ++i) {
    const int32_t* prev = (i == 0) ? anchor : draft_tokens + (i - 1);
    const int stride = (i == 0) ? 1 : N;
    hipLaunchKernelGGL(markov_step, grid, block, lds, stream, logits, w1, w2, d2t, prev, stride, temperature,
                       request_id, k0, k1, partial, i, B, N, V, Vd, r, p.chunks_per_wg, p.vslices, p.btiles);
    hipLaunchKernelGGL(markov_merge, dim3((B + 3) / 4), block, 0, stream, partial, temperature, draft_tokens,
                       log_z, i, B, N, p.vslices);
  }
  return hipGetLastError();
}

hipError_t launch_build_inverse_map(const int64_t* d2t, int Vd, int V, int32_t* inv_map, hipStream_t stream) {
  hipLaunchKernelGGL(inverse_fill, dim3((V + 255) / 256), dim3(256), 0, stream, inv_map, V);
  hipLaunchKernelGGL(inverse_scatter, dim3((Vd + 255) / 256), dim3(256), 0, stream, d2t, Vd, V, inv_map);
  return hipGetLastError();
}

}  // namespace dspark
