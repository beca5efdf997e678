// Stage 2: the N-step low-rank Markov (bigram) sampling loop.
//
// Step i of request b: e = W1[prev_b] (r values), bias = W2 . e (one value per
// draft token), l = base[b, i] + bias (written back in place), x = Gumbel-max
// sample of softmax(l / T_b) mapped to a target id, prev_b = x.  The step's
// argmax spans the whole vocabulary, so each step is one grid-wide pass:
//
//   markov_step   workgroup = 64 requests (16 per wave) x a strided set of
//                 64-wide vocabulary chunks.  The bias of a chunk is a dense
//                 [64 x r] x [r x 16] product per wave: MFMA 16x16x32 bf16 with
//                 the W2 chunk as the A operand (staged in LDS by global->LDS DMA,
//                 shared by the 4 waves) and the gathered W1 rows of the wave's
//                 16 requests as the B operand, held in registers for the whole
//                 pass.  A rows are ordered so that lane (n, g) of the result
//                 holds request n and the 16 consecutive entries 16g .. 16g+15 of
//                 the chunk: four float4 of base logits and four Philox blocks
//                 per lane and chunk.  The next chunk's W2 and base logits are
//                 requested before this chunk's epilogue runs.  Per lane a
//                 running best (key, target id) and a base-2 log-sum-exp (m, s)
//                 are kept; the four lanes of a request merge them and write one
//                 partial per (request, workgroup).
//   markov_merge  one wave per request reduces the partials, writes the token
//                 and log Z.  The next step's kernel reads that token.
//
// Few requests use markov_few.hip instead.
//
// Workgroup order is XCD-aware: the workgroups of the request tiles that walk the
// same vocabulary chunks go to the same XCD one after another, so each W2 chunk is
// fetched from HBM once and then served by that XCD's L2.
#include <float.h>
#include <math.h>

#include <algorithm>

#include "device.hpp"
#include "kernels.hpp"
#include "markov_common.hpp"

namespace dspark {

namespace {

using namespace mk;

constexpr int kSlots = 1024;     // workgroups the grid is sized for: 4 per CU on 256 CUs
constexpr float kLseSlack = 64;  // the running reference may trail the maximum by this much (base 2)
constexpr uint32_t kPhiloxM0 = 0xD2511F53u, kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kWeyl0 = 0x9E3779B9u, kWeyl1 = 0xBB67AE85u;

// s_waitcnt immediates (gfx9 encoding): wait for every vector-memory operation,
// resp. every LDS operation, and nothing else
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitLgkm0 = 0xC07F;

// Rounds 1..9 of Philox4x32-10 (round 0 is applied by the caller, whose counter
// words 2 and 3 are loop-invariant here).  k0, k1: the key before round 0.
__device__ __forceinline__ u32x4 philox_rounds_1_9(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int rnd = 1; rnd < 10; ++rnd) {
    k0 += kWeyl0;
    k1 += kWeyl1;
    const uint64_t p0 = (uint64_t)kPhiloxM0 * c.x;
    const uint64_t p1 = (uint64_t)kPhiloxM1 * c.z;
    c = u32x4{xor3((uint32_t)(p1 >> 32), c.y, k0), (uint32_t)p1, xor3((uint32_t)(p0 >> 32), c.w, k1), (uint32_t)p0};
  }
  return c;
}

// log2(-log2(u)), u = ((w >> 8) | 1) * 2^-24: the negated base-2 Gumbel variate of
// one Philox word.  u is formed without an integer conversion: the float with
// exponent 0 and mantissa w >> 9 is 1 + (w >> 9) 2^-23, and subtracting
// 1 - 2^-24 leaves (2 (w >> 9) + 1) 2^-24, exactly ((w >> 8) | 1) 2^-24.
__device__ __forceinline__ float neg_gumbel2(uint32_t w) {
  const float f = __uint_as_float(__builtin_amdgcn_alignbit(0x7Fu, w, 9u));
  const float u = f - 0x1.fffffep-1f;
  return __builtin_amdgcn_logf(-__builtin_amdgcn_logf(u));
}

}  // namespace

// (templates outside the anonymous namespace: the launch stubs of their instances
// must be emitted for the host-side switch below)
// LDS layout of one W2 chunk (64 rows of P = 4 KS 16-byte pieces).  Rows sit in P
// groups of 64 / P rows; a group is 1 KB, written by one global->LDS DMA
// instruction, and groups are 1040 bytes apart.  A-fragment f, row m lives in
// group grp(f, m), position pos(f, m) of it.  The 16 rows that one MFMA fragment
// reads at a k offset land in 16 distinct 16-byte bank groups, and every lane
// reaches all its fragments and k steps from one base address plus immediates.
template <int P>
struct ChunkLds {
  static constexpr int kRows = 64 / P;  // rows per group
  static constexpr int kPer = P >= 16 ? 1 : 16 / P;  // (P < 16) positions per fragment
  static constexpr int kGroup = 1040;   // bytes from one group to the next
  static constexpr int kBytes = P * kGroup;
  __host__ __device__ static constexpr int grp(int f, int m) { return P >= 16 ? (f / kRows) * 16 + m : m % P; }
  __host__ __device__ static constexpr int pos(int f, int m) { return P >= 16 ? f % kRows : f * kPer + m / P; }
  __host__ __device__ static constexpr int offset(int f, int m) { return grp(f, m) * kGroup + pos(f, m) * P * 16; }
  // chunk row (vocabulary offset) that group p, position h holds; fragment f row m
  // is vocabulary offset 16 (m >> 2) + 4 f + (m & 3)
  __host__ __device__ static constexpr int vocab(int p, int h) {
    const int f = P >= 16 ? (p / 16) * kRows + h : h / kPer;
    const int m = P >= 16 ? p % 16 : (h % kPer) * P + p;
    return 16 * (m >> 2) + 4 * f + (m & 3);
  }
};

// one 16-byte global->LDS DMA per lane (lane i writes lds_base + 16 i); a plain
// function, so the kernel template below stays instantiable by the host compiler
__device__ __forceinline__ void dma16(const uint16_t* src, char* lds_base) {
  __builtin_amdgcn_global_load_lds(src, lds_base, 16, 0, 0);
}

template <int KS, bool kReduced>
__global__ __launch_bounds__(256) void markov_step(float* __restrict__ logits, const uint16_t* __restrict__ w1,
                                                   const uint16_t* __restrict__ w2, const int32_t* __restrict__ tgt_of,
                                                   const int32_t* __restrict__ prev_tok, int prev_stride,
                                                   const float* __restrict__ temperature,
                                                   const uint32_t* __restrict__ request_id, uint32_t key0,
                                                   uint32_t key1, MarkovPartial* __restrict__ partial, int step,
                                                   int B, int N, int V, int Vd, int r, int nvs, int nbt) {
  constexpr int P = 4 * KS;
  using Lay = ChunkLds<P>;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  int vs, bt;
  wg_coords(0, nvs, nbt, vs, bt);
  if (vs >= nvs) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int nchunks = (Vd + kChunk - 1) / kChunk;
  const int kc = r / 8;  // W2 pieces per row that hold data (the rest of a row is zero)
  const int rq0 = bt * kReqPerWG + wave * kReqPerWave;
  const bool wave_active = rq0 < B;
  const bool lane_ok = rq0 + n < B;
  const int b = min(rq0 + n, B - 1);

  if (kc != P) {  // rank not a multiple of 32: the padding pieces must read as zero
    for (int p = tid; p < Lay::kBytes / 16; p += 256) reinterpret_cast<uint4*>(lds)[p] = make_uint4(0, 0, 0, 0);
    __syncthreads();
  }

  // B fragments: W1 row of request n, k = 32 s + 8 g .. +7 (zero past r)
  bf16x8 efrag[KS];
  {
    const int prev = min(max(prev_tok[(size_t)b * prev_stride], 0), V - 1);
    const uint16_t* er = w1 + (size_t)prev * r;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int k = s * 32 + 8 * g;
      const uint4 v = *reinterpret_cast<const uint4*>(er + min(k, r - 8));
      efrag[s] = __builtin_bit_cast(bf16x8, k < r ? v : make_uint4(0, 0, 0, 0));
    }
  }

  const float T = temperature[b];
  const bool noisy = T > 0.0f;
  const float c2 = noisy ? (1.0f / T) * 1.4426950408889634f : 1.0f;
  const float gs = noisy ? 1.0f : 0.0f;  // greedy rows take key = l
  const bool any_noisy = __ballot(noisy) != 0;
  // Philox round 0 of counter (j >> 2, step, request, draft tag): words 2 and 3 do
  // not depend on the vocabulary index
  const uint64_t pr = (uint64_t)kPhiloxM1 * request_id[b];
  const uint32_t x1 = (uint32_t)(pr >> 32) ^ (uint32_t)step ^ key0, y1 = (uint32_t)pr;

  float bkey = -INFINITY, bm = -FLT_MAX, bthr = -FLT_MAX, bs = 0.0f;
  // Without a target map ids grow along a lane, so the running best is kept per
  // block of 4 (strict comparison: an earlier block wins ties) and the entry inside
  // the winning block is found again after the pass.  bblk: first id of that block
  // minus 16 g (uniform per chunk and block); the lane's first block stands in.
  int bblk = vs * kChunk;
  int btok = 0x7FFFFFFF;  // with a target map: the best target id so far

  // DMA of chunk c: instruction t of this wave fills group 4 t + wave; lane L takes
  // piece L % P of position L / P.  The chunk row of (t, wave, L) splits into
  // vocab(4 t, 0) + wave + vocab(0, L / P), so a full chunk needs one lane offset.
  const int dma_piece = lane % P;
  const bool dma_ok = dma_piece < kc;
  const int dma_row = Lay::vocab(0, lane / P);
  const int dma_off = dma_row * r + dma_piece * 8;
  auto issue_w2 = [&](int c) {
    const int jc = c * kChunk;
    if (jc + kChunk <= Vd) {
      const uint16_t* src = w2 + (size_t)(jc + wave) * r;
#pragma unroll
      for (int t = 0; t < KS; ++t)
        if (dma_ok)
          dma16(src + (size_t)Lay::vocab(4 * t, 0) * r + dma_off, lds + (t * 4 + wave) * Lay::kGroup);
    } else {  // the last, partial chunk: rows past Vd load row Vd - 1 (never used)
#pragma unroll
      for (int t = 0; t < KS; ++t) {
        const int j = min(jc + wave + Lay::vocab(4 * t, 0) + dma_row, Vd - 1);
        if (dma_ok)
          dma16(w2 + (size_t)j * r + dma_piece * 8, lds + (t * 4 + wave) * Lay::kGroup);
      }
    }
  };
  float* const row = logits + ((size_t)b * N + step) * Vd + 16 * g;  // this lane's 16 entries of a chunk
  const int32_t* const trow = kReduced ? tgt_of + 16 * g : nullptr;
  auto load_base = [&](int c, float4 (&bv)[4], int4 (&tv)[4]) {
    const int jc = c * kChunk;
    if (jc + kChunk <= Vd) {
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        bv[f] = *reinterpret_cast<const float4*>(row + jc + 4 * f);
        if (kReduced) tv[f] = *reinterpret_cast<const int4*>(trow + jc + 4 * f);
      }
    } else {
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const int o = min(jc + 16 * g + 4 * f, Vd - 4) - 16 * g;
        bv[f] = *reinterpret_cast<const float4*>(row + o);
        if (kReduced) tv[f] = *reinterpret_cast<const int4*>(trow + o);
      }
    }
  };
  // noise of the Philox block of entries j .. j+3 (j a multiple of 4)
  auto noise = [&](int j, float (&lg)[4]) {
    const uint64_t p0 = (uint64_t)kPhiloxM0 * (uint32_t)(j >> 2);
    const u32x4 w =
        philox_rounds_1_9(u32x4{x1, y1, (uint32_t)(p0 >> 32) ^ kTagDraft ^ key1, (uint32_t)p0}, key0, key1);
    lg[0] = neg_gumbel2(w.x);
    lg[1] = neg_gumbel2(w.y);
    lg[2] = neg_gumbel2(w.z);
    lg[3] = neg_gumbel2(w.w);
  };

  // one chunk: bias on MFMA, then the epilogue over this lane's 16 entries; the
  // next chunk's W2 pieces and base logits go out first (into `nb`, `nt`)
  auto chunk = [&](int c, float4 (&cb)[4], int4 (&ct)[4], float4 (&nb)[4], int4 (&nt)[4]) {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);    // this wave's DMA pieces of chunk c (and its base logits)
    asm volatile("s_barrier" ::: "memory");  // every wave's pieces
    floatx4 acc[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      acc[f] = floatx4{0.f, 0.f, 0.f, 0.f};
      if (wave_active) {
        const char* arow = lds + Lay::offset(f, n) + 16 * g;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(arow + 64 * s));
          acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, efrag[s], acc[f], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    asm volatile("s_barrier" ::: "memory");  // the chunk buffer is free again
    const int cn = c + nvs;
    if (cn < nchunks) {
      issue_w2(cn);
      load_base(cn, nb, nt);
    }
    if (!wave_active) return;
    const int jc = c * kChunk, j0 = jc + 16 * g;
    float l[4][4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      l[f][0] = cb[f].x + acc[f][0];
      l[f][1] = cb[f].y + acc[f][1];
      l[f][2] = cb[f].z + acc[f][2];
      l[f][3] = cb[f].w + acc[f][3];
      if (lane_ok && j0 + 4 * f < Vd)
        *reinterpret_cast<float4*>(row + jc + 4 * f) = make_float4(l[f][0], l[f][1], l[f][2], l[f][3]);
    }
    if (jc + kChunk > Vd) {  // the last, partial chunk: entries past Vd never win nor count
#pragma unroll
      for (int f = 0; f < 4; ++f)
        if (j0 + 4 * f >= Vd) l[f][0] = l[f][1] = l[f][2] = l[f][3] = -INFINITY;
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      float lg[4];
      if (any_noisy) {
        noise(j0 + 4 * f, lg);
      } else {
        lg[0] = lg[1] = lg[2] = lg[3] = 0.0f;
      }
      float y[4], key[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y[i] = __fmul_rn(l[f][i], c2);
        key[i] = fmaf(lg[i], -gs, y[i]);
      }
      const float mx = fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3]));
      const bool grow = mx > bthr;
      if (__ballot(grow)) {  // rare after a lane's first block
        const float sc = __builtin_amdgcn_exp2f(bm - mx);
        bs = grow ? bs * sc : bs;
        bm = grow ? mx : bm;
        bthr = grow ? mx + kLseSlack : bthr;
      }
      bs += (__builtin_amdgcn_exp2f(y[0] - bm) + __builtin_amdgcn_exp2f(y[1] - bm)) +
            (__builtin_amdgcn_exp2f(y[2] - bm) + __builtin_amdgcn_exp2f(y[3] - bm));
      if (kReduced) {
        const int t[4] = {ct[f].x, ct[f].y, ct[f].z, ct[f].w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (key_beats(key[i], t[i], bkey, btok)) {
            bkey = key[i];
            btok = t[i];
          }
      } else {
        const float km = fmaxf(fmaxf(key[0], key[1]), fmaxf(key[2], key[3]));
        if (km > bkey) {
          bkey = km;
          bblk = jc + 4 * f;
        }
      }
      // one block at a time: interleaving the four blocks' Philox chains buys nothing
      // here (other waves fill the pipeline) and would hold four times the registers
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  float4 ba[4], bb[4];
  int4 ta[4], tb[4];
  issue_w2(vs);
  load_base(vs, ba, ta);
  for (int c = vs; c < nchunks; c += 2 * nvs) {  // unrolled by two: the prefetch buffers alternate
    chunk(c, ba, ta, bb, tb);
    if (c + nvs >= nchunks) break;
    chunk(c + nvs, bb, tb, ba, ta);
  }

  if (!kReduced && wave_active) {
    // the entry of the winning block that holds bkey (the keys are recomputed with the
    // same operations from the processed logits this lane stored); no winner: the
    // block's first id, which is also what a strict argmax over all -inf keys returns
    const int jb = bblk + 16 * g;
    btok = jb;
    if (bkey > -INFINITY) {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      const float4 v = *reinterpret_cast<const float4*>(row + bblk);  // block jb, stored by this lane
      const float lv[4] = {v.x, v.y, v.z, v.w};
      float lg[4] = {0.f, 0.f, 0.f, 0.f};
      if (any_noisy) noise(jb, lg);
      int hit = 3;
#pragma unroll
      for (int i = 3; i >= 0; --i)
        if (fmaf(lg[i], -gs, __fmul_rn(lv[i], c2)) == bkey) hit = i;
      btok = jb + hit;
    }
  }
  if (!wave_active) return;

  // merge the four lanes (g) of request n: partners n ^ 16, then n ^ 32
  {
    uint32_t k0, k1, t0, t1, m0, m1, s0, s1;
    rows_pair(__float_as_uint(bkey), k0, k1);
    rows_pair((uint32_t)btok, t0, t1);
    rows_pair(__float_as_uint(bm), m0, m1);
    rows_pair(__float_as_uint(bs), s0, s1);
    bkey = __uint_as_float(k0);
    btok = (int)t0;
    bm = __uint_as_float(m0);
    bs = __uint_as_float(s0);
    state_merge(bkey, btok, bm, bs, __uint_as_float(k1), (int)t1, __uint_as_float(m1), __uint_as_float(s1));
    halves_pair(__float_as_uint(bkey), k0, k1);
    halves_pair((uint32_t)btok, t0, t1);
    halves_pair(__float_as_uint(bm), m0, m1);
    halves_pair(__float_as_uint(bs), s0, s1);
    bkey = __uint_as_float(k0);
    btok = (int)t0;
    bm = __uint_as_float(m0);
    bs = __uint_as_float(s0);
    state_merge(bkey, btok, bm, bs, __uint_as_float(k1), (int)t1, __uint_as_float(m1), __uint_as_float(s1));
  }
  if (g == 0 && lane_ok) partial[(size_t)b * nvs + vs] = MarkovPartial{bkey, btok, bm, bs};
}

namespace {

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
    state_merge(key, tok, m, s, q.key, q.tok, q.m, q.s);
  }
  wave_state_merge(key, tok, m, s);
  if (lane == 0) {
    draft_tokens[(size_t)b * N + step] = tok;
    // T == 0: the key is the logit itself, and log Z is defined as the largest one
    log_z[(size_t)b * N + step] = (temperature[b] > 0.0f) ? (m + __log2f(s)) * 0.69314718055994531f : key;
  }
}

__global__ void target_table(const int64_t* __restrict__ d2t, int Vd, int32_t* __restrict__ tgt) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j < Vd) tgt[j] = j + (int)d2t[j];
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

int ksteps_of(int r) {  // MFMA k steps of 32, rounded up to a power of two
  const int k = (r + 31) / 32;
  return k <= 1 ? 1 : k <= 2 ? 2 : k <= 4 ? 4 : 8;
}

template <int KS>
hipError_t launch_steps(bool reduced, dim3 grid, float* logits, const uint16_t* w1, const uint16_t* w2,
                        const int32_t* tgt, const int32_t* anchor, const float* temperature,
                        const uint32_t* request_id, uint32_t k0, uint32_t k1, MarkovPartial* partial,
                        int32_t* draft_tokens, float* log_z, int B, int N, int V, int Vd, int r, int nvs, int nbt,
                        hipStream_t stream) {
  const size_t lds = ChunkLds<4 * KS>::kBytes;
  for (int i = 0; i < N; ++i) {
    const int32_t* prev = (i == 0) ? anchor : draft_tokens + (i - 1);
    const int stride = (i == 0) ? 1 : N;
    if (reduced)
      hipLaunchKernelGGL(HIP_KERNEL_NAME(markov_step<KS, true>), grid, dim3(256), lds, stream, logits, w1, w2, tgt, prev, stride,
                         temperature, request_id, k0, k1, partial, i, B, N, V, Vd, r, nvs, nbt);
    else
      hipLaunchKernelGGL(HIP_KERNEL_NAME(markov_step<KS, false>), grid, dim3(256), lds, stream, logits, w1, w2, tgt, prev, stride,
                         temperature, request_id, k0, k1, partial, i, B, N, V, Vd, r, nvs, nbt);
    hipLaunchKernelGGL(markov_merge, dim3((B + 3) / 4), dim3(256), 0, stream, partial, temperature, draft_tokens,
                       log_z, i, B, N, nvs);
  }
  return hipGetLastError();
}

}  // namespace

MarkovPlan plan_markov(int B, int N, int Vd, int r, int cus) {
  MarkovPlan p{};
  p.few = plan_markov_few(B, N, Vd, r, cus);
  p.btiles = (B + kReqPerWG - 1) / kReqPerWG;
  const int chunks = (Vd + kChunk - 1) / kChunk;
  // workgroups per request tile: enough to fill the chip, at most one per chunk
  const int want = std::min(chunks, (kSlots + p.btiles - 1) / p.btiles);
  p.vslices = want;
  p.chunks_per_wg = (chunks + want - 1) / want;
  p.partial_bytes = (size_t)B * p.vslices * sizeof(MarkovPartial);
  p.partial_bytes = (p.partial_bytes + 255) / 256 * 256;
  p.tgt_offset = p.partial_bytes;
  p.partial_bytes += (size_t)Vd * sizeof(int32_t);
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
  int32_t* tgt = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + p.tgt_offset);
  const bool reduced = d2t != nullptr;
  if (reduced) hipLaunchKernelGGL(target_table, dim3((Vd + 255) / 256), dim3(256), 0, stream, d2t, Vd, tgt);
  const int nvs8 = (p.vslices + 7) / 8 * 8;
  const dim3 grid(nvs8 * p.btiles);
  const uint32_t k0 = (uint32_t)(seed & 0xFFFFFFFFu), k1 = (uint32_t)(seed >> 32);
  switch (ksteps_of(r)) {
    case 1:
      return launch_steps<1>(reduced, grid, logits, w1, w2, tgt, anchor, temperature, request_id, k0, k1, partial,
                             draft_tokens, log_z, B, N, V, Vd, r, p.vslices, p.btiles, stream);
    case 2:
      return launch_steps<2>(reduced, grid, logits, w1, w2, tgt, anchor, temperature, request_id, k0, k1, partial,
                             draft_tokens, log_z, B, N, V, Vd, r, p.vslices, p.btiles, stream);
    case 4:
      return launch_steps<4>(reduced, grid, logits, w1, w2, tgt, anchor, temperature, request_id, k0, k1, partial,
                             draft_tokens, log_z, B, N, V, Vd, r, p.vslices, p.btiles, stream);
    default:
      return launch_steps<8>(reduced, grid, logits, w1, w2, tgt, anchor, temperature, request_id, k0, k1, partial,
                             draft_tokens, log_z, B, N, V, Vd, r, p.vslices, p.btiles, stream);
  }
}

hipError_t launch_build_inverse_map(const int64_t* d2t, int Vd, int V, int32_t* inv_map, hipStream_t stream) {
  hipLaunchKernelGGL(inverse_fill, dim3((V + 255) / 256), dim3(256), 0, stream, inv_map, V);
  hipLaunchKernelGGL(inverse_scatter, dim3((Vd + 255) / 256), dim3(256), 0, stream, d2t, Vd, V, inv_map);
  return hipGetLastError();
}

}  // namespace dspark
