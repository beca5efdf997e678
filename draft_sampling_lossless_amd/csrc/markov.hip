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
//                 pass.  Fragment f covers entries 16 f .. 16 f + 15, so lane
//                 (n, g) holds request n, entries 16 f + 4 g .. +3: one float4 of
//                 base logits and one Philox block per fragment, and the four lanes
//                 of a request read 64 contiguous bytes per load instruction.  The
//                 processed logits go back through a per-wave LDS block and out
//                 by rows (256 contiguous bytes per request per instruction).  The
//                 next chunk's W2 and base logits are requested before this chunk's
//                 epilogue runs; every lane issues the same memory operations, so
//                 nothing waits on them until the next chunk.  Per lane a running
//                 best (key, block) and a base-2 log-sum-exp (m, s) are kept; the
//                 four lanes of a request merge them and write one partial per
//                 (request, workgroup).  Modes (StepMode below): store the processed
//                 logits, keep the base logits and record each partial's winning
//                 logit instead (with one request tile, two LDS chunk buffers), or
//                 rebuild one listed row per request.
//   markov_merge  one wave per request reduces the partials, writes the token
//                 and log Z (keep modes: and the winner's processed logit).  The
//                 next step's kernel reads that token.
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

constexpr int kMaxSlots = 2048;  // resident workgroups a launch may count on (8 per CU on 256 CUs)
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
// LDS layout of one W2 chunk (64 rows of P = 4 KS 16-byte pieces) in P groups of
// 64 / P rows; a group is 1 KB, written by one global->LDS DMA instruction (lane L:
// position L / P, slot L % P).  A-fragment f, row m lives in group grp(f, m), position
// pos(f, m), and logical piece q of it (k = 8 q .. 8 q + 7) at slot piece(q, m).  A
// 16-byte LDS read on gfx950 is free of bank conflicts for these patterns (each lane
// (n, g) of a fragment read takes row n, piece 4 s + g), as measured with a read probe:
//  * P >= 16: a fragment's rows are consecutive groups, 1056 bytes apart (1040 left
//    the reads two-way conflicted); pieces in order;
//  * P < 16: a fragment's 16 rows are contiguous (one or two groups, no padding), and
//    the pieces of a row are permuted by row pairs: P = 8 (128-byte rows) q ^ ((m >> 1)
//    & 7), P = 4 (64-byte rows) (q + (m >> 1)) & 3.  Rows in group order with pieces in
//    order read at half the rate whatever the group stride.
// Every lane reaches all its fragments from one base address per k step plus immediates.
template <int P>
struct ChunkLds {
  static constexpr int kRows = 64 / P;  // rows per group
  static constexpr int kPer = P >= 16 ? 1 : 16 / kRows;  // (P < 16) groups per fragment
  static constexpr int kGroup = P >= 16 ? 1056 : 1024;  // bytes from one group to the next
  static constexpr int kBytes = P * kGroup;
  __host__ __device__ static constexpr int grp(int f, int m) { return P >= 16 ? (f / kRows) * 16 + m : f * kPer + m / kRows; }
  __host__ __device__ static constexpr int pos(int f, int m) { return P >= 16 ? f % kRows : m % kRows; }
  __host__ __device__ static constexpr int offset(int f, int m) { return grp(f, m) * kGroup + pos(f, m) * P * 16; }
  __host__ __device__ static constexpr int piece(int q, int m) {
    return P >= 16 ? q : P == 8 ? (q ^ ((m >> 1) & 7)) : ((q + (m >> 1)) & 3);
  }
  // chunk row (vocabulary offset) that group p, position h holds; fragment f row m
  // is vocabulary offset 16 f + m
  __host__ __device__ static constexpr int vocab(int p, int h) {
    return P >= 16 ? 16 * ((p / 16) * kRows + h) + p % 16 : p * kRows + h;
  }
  // the logical piece that slot s of group p, position h holds
  __host__ __device__ static constexpr int logical(int s, int p, int h) {
    const int m = P >= 16 ? 0 : (p % kPer) * kRows + h;  // the row within its fragment
    return P >= 16 ? s : P == 8 ? (s ^ ((m >> 1) & 7)) : ((s - (m >> 1)) & 3);
  }
};
static_assert(ChunkLds<8>::logical(ChunkLds<8>::piece(5, 11), 3, 3) == 5, "slot map inverts (P = 8)");
static_assert(ChunkLds<4>::logical(ChunkLds<4>::piece(2, 13), 0, 13) == 2, "slot map inverts (P = 4)");
static_assert(ChunkLds<8>::vocab(3, 3) == 16 * 1 + 11 && ChunkLds<8>::offset(1, 11) == 3 * 1024 + 3 * 128,
              "group 3 position 3 is fragment 1 row 11 (P = 8)");
static_assert(ChunkLds<4>::vocab(3, 5) == 16 * 3 + 5 && ChunkLds<4>::offset(3, 5) == 3 * 1024 + 5 * 64 &&
                  ChunkLds<4>::offset(3, 15) + 64 <= ChunkLds<4>::kBytes,
              "group 3 position 5 is fragment 3 row 5, inside the chunk (P = 4)");
static_assert(ChunkLds<8>::offset(3, 15) + 128 <= ChunkLds<8>::kBytes &&
                  ChunkLds<16>::offset(3, 15) + 256 <= ChunkLds<16>::kBytes &&
                  ChunkLds<32>::offset(3, 15) + 512 <= ChunkLds<32>::kBytes,
              "every fragment row lies inside the chunk");
static_assert(ChunkLds<32>::vocab(17, 1) == 16 * 3 + 1 && ChunkLds<32>::offset(3, 1) == 17 * 1056 + 1 * 512,
              "group 17 position 1 is fragment 3 row 1 (P = 32)");

// four floats this thread stored earlier in the kernel (device-coherent loads, so a
// stale vector-L1 line of the values loaded before the store is never returned)
__device__ __forceinline__ void load_stored4(const float* p, float (&v)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __hip_atomic_load(p + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// one 16-byte global->LDS DMA per lane (lane i writes lds_base + 16 i); a plain
// function, so the kernel template below stays instantiable by the host compiler
__device__ __forceinline__ void dma16(const uint16_t* src, char* lds_base) {
  __builtin_amdgcn_global_load_lds(src, lds_base, 16, 0, 0);
}

constexpr int kTurnRow = 272, kTurnBytes = 16 * kTurnRow;  // per wave: 16 requests x 64 entries

// Modes of the per-step kernel.  kStore: sample and store the processed logits in
// place.  kKeep: sample, leave the base logits untouched and record, per (request,
// workgroup), the processed logit of the workgroup's winner (io.lw).  kReplay: store
// the processed logits of one row per request (io.rows[b], -1: none) in place, with the
// same chunk, fragment and MFMA sequence as the sampling modes, so they equal what
// kStore would have stored bit for bit.  kKeep2: kKeep with two chunk buffers: the
// next chunk's W2 rows and base logits are requested right after the barrier that
// opens a chunk, so they arrive under its MFMAs and epilogue, and one barrier per
// chunk suffices (faster with one request tile, where there are few workgroups to
// hide each other's waits; with more, the halved residency costs more than it saves).
enum StepMode { kStore = 0, kKeep = 1, kReplay = 2, kKeep2 = 3 };
struct StepIO {
  float* lw;             // kKeep: [B x nvs]
  const int32_t* rows;   // kReplay: [B]
};
template <int KS, bool kReduced, int kMode>
__global__ __launch_bounds__(256) void markov_step(float* __restrict__ logits, const uint16_t* __restrict__ w1,
                                                   const uint16_t* __restrict__ w2, const int32_t* __restrict__ tgt_of,
                                                   float* __restrict__ spill_row, const int32_t* __restrict__ prev_tok,
                                                   int prev_stride, const float* __restrict__ temperature,
                                                   const uint32_t* __restrict__ request_id, uint32_t key0,
                                                   uint32_t key1, MarkovPartial* __restrict__ partial, int step,
                                                   int B, int N, int V, int Vd, int r, int nvs, int nbt,
                                                   ConfArgs conf, StepIO io) {
  constexpr int P = 4 * KS;
  constexpr bool kKeeps = kMode == kKeep || kMode == kKeep2;
  using Lay = ChunkLds<P>;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  int vs, bt;
  wg_coords(0, nvs, nbt, vs, bt);
  if (vs >= nvs) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int nchunks = (Vd + kChunk - 1) / kChunk;
  const int kc = r / 8;  // W2 pieces per row that hold data
  if (kMode == kReplay) {
    // a request tile without a row to rebuild has nothing to do (uniform over the workgroup)
    const int q = bt * kReqPerWG + tid;
    if (!__syncthreads_or(tid < kReqPerWG && q < B && io.rows[q] >= 0)) return;
  }
  const int rq0 = bt * kReqPerWG + wave * kReqPerWave;
  const bool wave_active = rq0 < B;
  const bool lane_ok = rq0 + n < B;
  const int b = min(rq0 + n, B - 1);

  // DMA of chunk c: instruction t of this wave fills group 4 t + wave; lane L takes
  // piece L % P of position L / P.  The chunk row of (t, wave, L) splits into
  // vocab(4 t, 0) + wave + vocab(0, L / P), so a full chunk needs one lane offset.
  // With a rank below 32 KS the pieces past the rank repeat the row's last piece:
  // finite values that meet the zero B operand there.  Every wave issues exactly KS
  // DMA instructions per chunk, so the vector-memory counter is known at each wait.
  // (the row and piece map of group 4 t + wave depends on the wave's parity only, as
  // 4 t is even: group 4 t + wave holds rows vocab(4 t, 0) + vocab(wave, 0) + vocab(0, h))
  const int dma_piece = min(Lay::logical(lane % P, wave, lane / P), kc - 1);
  const int dma_row = Lay::vocab(0, lane / P);
  const int dma_off = dma_row * r + dma_piece * 8;
  const int wrow = Lay::vocab(wave, 0);
  auto issue_w2 = [&](int c) {
    // kKeep2: chunk c into buffer ((c - vs) / nvs) & 1
    char* const lbuf = lds + (kMode == kKeep2 ? (((c - vs) / nvs) & 1) * Lay::kBytes : 0);
    const int jc = c * kChunk;
    if (jc + kChunk <= Vd) {
      const uint16_t* src = w2 + (size_t)(jc + wrow) * r;
#pragma unroll
      for (int t = 0; t < KS; ++t)
        dma16(src + (size_t)Lay::vocab(4 * t, 0) * r + dma_off, lbuf + (t * 4 + wave) * Lay::kGroup);
    } else {  // the last, partial chunk: rows past Vd load row Vd - 1 (never used)
#pragma unroll
      for (int t = 0; t < KS; ++t) {
        const int j = min(jc + wrow + Lay::vocab(4 * t, 0) + dma_row, Vd - 1);
        dma16(w2 + (size_t)j * r + dma_piece * 8, lbuf + (t * 4 + wave) * Lay::kGroup);
      }
    }
  };

  if (!wave_active) {
    // a wave without requests (the last request tile) still stages its share of W2
    for (int c = vs; c < nchunks; c += nvs) {
      if (c == vs) issue_w2(c);
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      asm volatile("s_barrier" ::: "memory");
      if (kMode != kKeep2) asm volatile("s_barrier" ::: "memory");
      if (c + nvs < nchunks) issue_w2(c + nvs);
    }
    return;
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
  // confidence head of this step (first workgroup of each request tile): the embedding
  // part w_e . W1[prev] from the fragments above, the four lanes of a request summed
  if (conf.out != nullptr && vs == 0) {
    float d = 0.0f;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int k = s * 32 + 8 * g;
      if (k < r) d += dot_bf16x8(__builtin_bit_cast(uint4, efrag[s]), *reinterpret_cast<const uint4*>(conf.we + k));
    }
    d += __shfl_xor(d, 16);
    d += __shfl_xor(d, 32);
    if (g == 0 && lane_ok) {
      const size_t row = (size_t)b * N + step;
      conf.out[row] = conf_prob(conf.hdot[row], d, conf.bias, conf.tau[step]);
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
  // The running best is kept per block of 4 entries: the block's largest key, compared
  // strictly (an earlier block keeps a tie), and bblk = the block's first id minus 4 g.
  // After the pass the entry inside the winning block is found again from the stored
  // logits.  Without a target map ids grow along a lane, so this is the argmax with
  // ties to the smallest id.  With one, ties are broken by target id: a tie between
  // two blocks (or a lane with no finite key) sends the lane to an exact rescan.
  int bblk = vs * kChunk;
  bool tie = false;
  float bl[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};  // kKeep: logits of the best block

  // This lane's logits row as float4 (Vd is a multiple of 4).  Loads clamp to the
  // row; stores of entries that do not exist (past Vd, or a lane without a request)
  // go to a spill row in the workspace, so every lane issues the same loads and
  // stores and the vector-memory counter stays exact.
  const int vd4 = Vd / 4;
  // the row this step reads (kReplay: the request's own row; a request without one
  // reads the spill row, which stays in L2, and stores nothing)
  const int rowb = (kMode == kReplay) ? io.rows[b] : step;
  float4* const spill4 = reinterpret_cast<float4*>(spill_row);
  float4* const row4 = rowb >= 0 ? reinterpret_cast<float4*>(logits + ((size_t)b * N + rowb) * Vd) : spill4;
  // stores go out by rows: store instruction k of a chunk writes requests 4 k .. 4 k + 3
  // of the wave, lane L entries 4 (L % 16) .. +3 of request 4 k + L / 16 (256 contiguous
  // bytes per request); the chunk's logits are turned around in this wave's LDS block
  // (16 rows of 272 bytes: the 16 rows one fragment writes fall into 16 bank groups)
  char* const turn = lds + Lay::kBytes + wave * kTurnBytes;
  float4* srow[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int bq = rq0 + 4 * k + (lane >> 4);
    const int rq = (kMode == kReplay && bq < B) ? io.rows[bq] : step;
    srow[k] = (bq < B && rq >= 0) ? reinterpret_cast<float4*>(logits + ((size_t)bq * N + rq) * Vd) : nullptr;
  }
  auto load_base = [&](int c, float4 (&bv)[4]) {
    const int j4 = c * (kChunk / 4) + g;
#pragma unroll
    for (int f = 0; f < 4; ++f) bv[f] = row4[min(j4 + 4 * f, vd4 - 1)];
  };
  // noise of the Philox block of entries j .. j+3 (j a multiple of 4)
  auto noise = [&](int j, float (&lg)[4]) {
    if (any_noisy) {
      const uint64_t p0 = (uint64_t)kPhiloxM0 * (uint32_t)(j >> 2);
      const u32x4 w =
          philox_rounds_1_9(u32x4{x1, y1, (uint32_t)(p0 >> 32) ^ kTagDraft ^ key1, (uint32_t)p0}, key0, key1);
      lg[0] = neg_gumbel2(w.x);
      lg[1] = neg_gumbel2(w.y);
      lg[2] = neg_gumbel2(w.z);
      lg[3] = neg_gumbel2(w.w);
    } else {
      lg[0] = lg[1] = lg[2] = lg[3] = 0.0f;
    }
  };
  // y = l log2(e) / T and key = y + Gumbel (T == 0: key = y = l); the final search
  // repeats exactly these operations on the stored logits
  auto keys_of = [&](const float (&lg)[4], const float (&l)[4], float (&y)[4], float (&key)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      y[i] = __fmul_rn(l[i], c2);
      key[i] = fmaf(lg[i], -gs, y[i]);
    }
  };

  // One chunk.  The W2 DMA and base logits of the next chunk, then this chunk's
  // stores, are issued at the start of the epilogue, so the wait at the top of the
  // next chunk finds them complete unless the epilogue was shorter than the memory
  // latency.
  auto chunk = [&](int c, float4 (&cb)[4], float4 (&nb)[4]) {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);    // DMA pieces and base logits of chunk c
    asm volatile("s_barrier" ::: "memory");  // every wave's pieces
    const int cn = c + nvs;
    if (kMode == kKeep2 && cn < nchunks) {    // the other buffer: last read by chunk c - nvs
      issue_w2(cn);
      load_base(cn, nb);
    }
    const char* const cbuf = lds + (kMode == kKeep2 ? (((c - vs) / nvs) & 1) * Lay::kBytes : 0);
    floatx4 acc[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      acc[f] = floatx4{0.f, 0.f, 0.f, 0.f};
      const char* arow = cbuf + Lay::offset(f, n);
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 a =
            __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(arow + 16 * Lay::piece(4 * s + g, n)));
        acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, efrag[s], acc[f], 0, 0, 0);
      }
    }
    if (kMode != kKeep2) {
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      asm volatile("s_barrier" ::: "memory");  // the chunk buffer is free again
      if (cn < nchunks) {
        issue_w2(cn);
        load_base(cn, nb);
      }
    }
    const int jc = c * kChunk, j0 = jc + 4 * g, j4 = j0 / 4;  // block f: entries j0 + 16 f .. +3
    float l[4][4];
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      l[f][0] = cb[f].x + acc[f][0];
      l[f][1] = cb[f].y + acc[f][1];
      l[f][2] = cb[f].z + acc[f][2];
      l[f][3] = cb[f].w + acc[f][3];
      if (!kKeeps)
        *reinterpret_cast<float4*>(turn + n * kTurnRow + (16 * f + 4 * g) * 4) =
            make_float4(l[f][0], l[f][1], l[f][2], l[f][3]);
    }
    if (!kKeeps) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int e = lane & 15, jj4 = jc / 4 + e;
        const float4 v = *reinterpret_cast<const float4*>(turn + (4 * k + (lane >> 4)) * kTurnRow + e * 16);
        float4* dst = (srow[k] != nullptr && jj4 < vd4) ? srow[k] + jj4 : spill4 + jj4;
        *dst = v;
      }
    }
    if (kMode == kReplay) return;
    if (jc + kChunk > Vd) {  // the last, partial chunk: entries past Vd never win nor count
#pragma unroll
      for (int f = 0; f < 4; ++f)
        if (j0 + 16 * f >= Vd) l[f][0] = l[f][1] = l[f][2] = l[f][3] = -INFINITY;
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      float lg[4], y[4], key[4];
      noise(j0 + 16 * f, lg);
      keys_of(lg, l[f], y, key);
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
      const float km = fmaxf(fmaxf(key[0], key[1]), fmaxf(key[2], key[3]));
      if (kReduced) tie = tie || (km == bkey && km > -INFINITY);
      if (km > bkey) {
        bkey = km;
        bblk = jc + 16 * f;
        if (kKeeps) {
#pragma unroll
          for (int i = 0; i < 4; ++i) bl[i] = l[f][i];
        }
      }
      // one block at a time: interleaving the four blocks' Philox chains buys nothing
      // here (other waves fill the pipeline) and would hold four times the registers
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  float4 ba[4], bb[4];
  issue_w2(vs);
  load_base(vs, ba);
  for (int c = vs; c < nchunks; c += 2 * nvs) {  // unrolled by two: the prefetch buffers alternate
    chunk(c, ba, bb);
    if (c + nvs >= nchunks) break;
    chunk(c + nvs, bb, ba);
  }

  if (kMode == kReplay) return;
  // the entry of the winning block: its keys again from the logits this lane stored
  // (kKeep: from the copy in registers)
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  int btok;
  float lwin = -INFINITY;  // kKeep: processed logit of this lane's winner
  {
    const int jb = bblk + 4 * g;
    float lv[4];
    if (kKeeps) {
#pragma unroll
      for (int i = 0; i < 4; ++i) lv[i] = bl[i];
    } else {
      load_stored4(reinterpret_cast<const float*>(row4) + min(jb, Vd - 4), lv);
    }
    float lg[4], y[4], key[4];
    noise(jb, lg);
    keys_of(lg, lv, y, key);
    if (!kReduced) {
      // no winner (every key -inf): the block's first id, as a strict argmax would give
      int hit = 0;
#pragma unroll
      for (int i = 3; i >= 0; --i)
        if (key[i] == bkey) hit = i;
      btok = jb + hit;
      lwin = lv[0];
#pragma unroll
      for (int i = 1; i < 4; ++i)
        if (hit == i) lwin = lv[i];
    } else {
      const int4 tv = *reinterpret_cast<const int4*>(tgt_of + min(jb, Vd - 4));
      const int t[4] = {tv.x, tv.y, tv.z, tv.w};
      btok = 0x7FFFFFFF;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (key[i] == bkey) btok = min(btok, t[i]);
    }
  }
  if (kReduced) {
    const bool rescan = tie || !(bkey > -INFINITY);
    if (__ballot(rescan)) {  // rare: the exact argmax over this lane's entries, ties to the smaller target
      if (rescan) {
        bkey = -INFINITY;
        btok = 0x7FFFFFFF;
        for (int c = vs; c < nchunks; c += nvs) {
          const int jc = c * kChunk;
#pragma unroll
          for (int f = 0; f < 4; ++f) {
            const int j = jc + 16 * f + 4 * g;
            if (j >= Vd) continue;
            float lv[4];
            load_stored4(reinterpret_cast<const float*>(row4) + j, lv);
            const int4 tv = *reinterpret_cast<const int4*>(tgt_of + j);
            const int t[4] = {tv.x, tv.y, tv.z, tv.w};
            float lg[4], y[4], key[4];
            noise(j, lg);
            keys_of(lg, lv, y, key);
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (key_beats(key[i], t[i], bkey, btok)) {
                bkey = key[i];
                btok = t[i];
              }
          }
        }
      }
    }
  }

  // merge the four lanes (g) of request n: partners n ^ 16, then n ^ 32
  const int btok_own = btok;
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
  // (the lanes of a request hold disjoint entries: exactly one of them owns the winner)
  if (kKeeps && lane_ok && btok_own == btok) io.lw[(size_t)b * nvs + vs] = lwin;
}

namespace {

__global__ __launch_bounds__(256) void markov_merge(const MarkovPartial* __restrict__ partial,
                                                    const float* __restrict__ temperature,
                                                    int32_t* __restrict__ draft_tokens, float* __restrict__ log_z,
                                                    int step, int B, int N, int nvs, const float* __restrict__ lw,
                                                    float* __restrict__ win) {
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (b >= B) return;
  float key = -INFINITY, m = -INFINITY, s = 0.0f, v = -INFINITY;
  int tok = 0x7FFFFFFF;
  const bool keep = win != nullptr;
  // up to 8 partials per lane in flight at once
  for (int p0 = 0; p0 < nvs; p0 += 512) {
    MarkovPartial q[8];
    float qv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int p = p0 + 64 * j + lane;
      q[j] = p < nvs ? partial[(size_t)b * nvs + p] : MarkovPartial{-INFINITY, 0x7FFFFFFF, -INFINITY, 0.0f};
      qv[j] = keep && p < nvs ? lw[(size_t)b * nvs + p] : -INFINITY;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if (key_beats(q[j].key, q[j].tok, key, tok)) v = qv[j];
      state_merge(key, tok, m, s, q[j].key, q[j].tok, q[j].m, q[j].s);
    }
  }
  const int lane_tok = tok;
  wave_state_merge(key, tok, m, s);
  if (keep) {
    // the winner's processed logit: the lane whose own best is the winner holds it
    // (the workgroups of a request cover disjoint entries)
    const uint64_t hit = __ballot(lane_tok == tok);
    v = __shfl(v, hit ? (int)__builtin_ctzll(hit) : 0);
    if (lane == 0) win[(size_t)b * N + step] = v;
  }
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

// workgroups per request tile: the resident capacity of the chip spread over the
// request tiles (a multiple of 8 for the XCD order), at most one per chunk
int markov_slices(int chunks, int nbt, int slots) {
  const int per = std::max(8, slots / nbt / 8 * 8);
  return std::min(chunks, per);
}

template <int KS, bool kReduced, int kMode>
int resident_per_cu(size_t lds) {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (!cached[dev]) {
    int occ = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &occ, reinterpret_cast<const void*>(&markov_step<KS, kReduced, kMode>), 256, lds) != hipSuccess || occ <= 0)
      occ = 1;
    cached[dev] = occ;
  }
  return cached[dev];
}

template <int KS, bool kReduced, int kMode>
int step_slices(int chunks, int nbt, int max_slices, size_t lds) {
  const int slots = std::min(kMaxSlots, resident_per_cu<KS, kReduced, kMode>(lds) * cu_count_markov());
  return std::min(max_slices, markov_slices(chunks, nbt, slots));
}

template <int KS, bool kReduced, int kMode>
hipError_t launch_steps(float* logits, const uint16_t* w1, const uint16_t* w2, const int32_t* tgt,
                        float* spill, const int32_t* anchor, const float* temperature, const uint32_t* request_id, uint32_t k0,
                        uint32_t k1, MarkovPartial* partial, int32_t* draft_tokens, float* log_z, int B, int N, int V,
                        int Vd, int r, int nbt, int max_slices, const ConfArgs& conf, float* lw, float* win,
                        hipStream_t stream) {
  const size_t lds = (kMode == kKeep2) ? 2 * ChunkLds<4 * KS>::kBytes : ChunkLds<4 * KS>::kBytes + 4 * kTurnBytes;
  if (lds > 65536) {  // past the default dynamic LDS limit (once per device)
    static bool attr_set[64] = {false};
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (dev >= 0 && dev < 64 && !attr_set[dev]) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&markov_step<KS, kReduced, kMode>),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e != hipSuccess) return e;
      attr_set[dev] = true;
    }
  }
  const int chunks = (Vd + kChunk - 1) / kChunk;
  const int nvs = step_slices<KS, kReduced, kMode>(chunks, nbt, max_slices, lds);
  const dim3 grid((nvs + 7) / 8 * 8 * nbt);
  const StepIO io{lw, nullptr};
  for (int i = 0; i < N; ++i) {
    const int32_t* prev = (i == 0) ? anchor : draft_tokens + (i - 1);
    const int stride = (i == 0) ? 1 : N;
    hipLaunchKernelGGL(HIP_KERNEL_NAME(markov_step<KS, kReduced, kMode>), grid, dim3(256), lds, stream, logits, w1,
                       w2, tgt, spill, prev, stride, temperature, request_id, k0, k1, partial, i, B, N, V, Vd, r, nvs,
                       nbt, conf, io);
    hipLaunchKernelGGL(markov_merge, dim3((B + 3) / 4), dim3(256), 0, stream, partial, temperature, draft_tokens,
                       log_z, i, B, N, nvs, lw, win);
  }
  return hipGetLastError();
}

template <int KS>
hipError_t launch_ks(bool reduced, bool keep, float* logits, const uint16_t* w1, const uint16_t* w2,
                     const int32_t* tgt, float* spill, const int32_t* anchor, const float* temperature,
                     const uint32_t* request_id, uint32_t k0, uint32_t k1, MarkovPartial* partial,
                     int32_t* draft_tokens, float* log_z, int B, int N, int V, int Vd, int r, int nbt, int max_slices,
                     const ConfArgs& conf, float* lw, float* win, hipStream_t stream) {
  if (keep && nbt == 1)  // (no target map: checked by the caller)
    return launch_steps<KS, false, kKeep2>(logits, w1, w2, tgt, spill, anchor, temperature, request_id, k0, k1,
                                           partial, draft_tokens, log_z, B, N, V, Vd, r, nbt, max_slices, conf, lw,
                                           win, stream);
  if (keep)
    return launch_steps<KS, false, kKeep>(logits, w1, w2, tgt, spill, anchor, temperature, request_id, k0, k1,
                                          partial, draft_tokens, log_z, B, N, V, Vd, r, nbt, max_slices, conf, lw,
                                          win, stream);
  return reduced ? launch_steps<KS, true, kStore>(logits, w1, w2, tgt, spill, anchor, temperature, request_id, k0, k1,
                                                  partial, draft_tokens, log_z, B, N, V, Vd, r, nbt, max_slices, conf,
                                                  nullptr, nullptr, stream)
                 : launch_steps<KS, false, kStore>(logits, w1, w2, tgt, spill, anchor, temperature, request_id, k0,
                                                   k1, partial, draft_tokens, log_z, B, N, V, Vd, r, nbt, max_slices,
                                                   conf, nullptr, nullptr, stream);
}

template <int KS>
hipError_t launch_replay_ks(float* logits, const uint16_t* w1, const uint16_t* w2, float* spill, const int32_t* rows,
                            const int32_t* prev, const float* temperature, const uint32_t* request_id, int B, int N,
                            int V, int Vd, int r, int nbt, int max_slices, hipStream_t stream) {
  const size_t lds = ChunkLds<4 * KS>::kBytes + 4 * kTurnBytes;
  const int chunks = (Vd + kChunk - 1) / kChunk;
  const int nvs = step_slices<KS, false, kReplay>(chunks, nbt, max_slices, lds);
  const dim3 grid((nvs + 7) / 8 * 8 * nbt);
  const StepIO io{nullptr, rows};
  hipLaunchKernelGGL(HIP_KERNEL_NAME(markov_step<KS, false, kReplay>), grid, dim3(256), lds, stream, logits, w1, w2,
                     nullptr, spill, prev, 1, temperature, request_id, 0u, 0u, nullptr, 0, B, N, V, Vd, r, nvs, nbt,
                     ConfArgs{}, io);
  return hipGetLastError();
}

}  // namespace

MarkovPlan plan_markov(int B, int N, int Vd, int r, int cus) {
  MarkovPlan p{};
  p.few = plan_markov_few(B, N, Vd, r, cus);
  p.btiles = (B + kReqPerWG - 1) / kReqPerWG;
  const int chunks = (Vd + kChunk - 1) / kChunk;
  // the most workgroups per request tile any launch uses (the workspace holds one
  // partial per request and workgroup)
  p.vslices = markov_slices(chunks, p.btiles, kMaxSlots);
  p.chunks_per_wg = (chunks + p.vslices - 1) / p.vslices;
  p.partial_bytes = (size_t)B * p.vslices * sizeof(MarkovPartial);
  p.partial_bytes = (p.partial_bytes + 255) / 256 * 256;
  p.tgt_offset = p.partial_bytes;
  p.partial_bytes += ((size_t)Vd * sizeof(int32_t) + 255) / 256 * 256;
  p.spill_offset = p.partial_bytes;  // a logits row for stores of entries that do not exist
  p.partial_bytes += (size_t)chunks * kChunk * sizeof(float);
  p.lw_offset = p.partial_bytes;     // winner logits of the partials (kept base logits)
  p.partial_bytes += ((size_t)B * p.vslices * sizeof(float) + 255) / 256 * 256;
  // the query (cus == 0) must cover whichever path a launch picks
  if (p.few.bytes > p.partial_bytes) p.partial_bytes = p.few.bytes;
  return p;
}

hipError_t launch_markov_sample(float* logits, const uint16_t* w1, const uint16_t* w2, const int64_t* d2t,
                                const int32_t* anchor, const float* temperature, const uint32_t* request_id,
                                uint64_t seed, int32_t* draft_tokens, float* log_z, int B, int N, int V, int Vd,
                                int r, void* workspace, const ConfArgs& conf, float* win, hipStream_t stream) {
  const MarkovPlan p = plan_markov(B, N, Vd, r, cu_count_markov());
  const bool keep = win != nullptr;
  if (keep && d2t != nullptr) return hipErrorInvalidValue;  // kept base logits: no target map
  // (the few-request kernel stores the processed logits: kept base logits take the per-step path)
  if (p.few.use && !keep)
    return launch_markov_few(p.few, logits, w1, w2, d2t, anchor, temperature, request_id, seed, draft_tokens, log_z,
                             B, N, V, Vd, r, workspace, conf, stream);
  MarkovPartial* partial = static_cast<MarkovPartial*>(workspace);
  int32_t* tgt = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + p.tgt_offset);
  float* spill = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.spill_offset);
  float* lw = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.lw_offset);
  const bool reduced = d2t != nullptr;
  if (reduced) hipLaunchKernelGGL(target_table, dim3((Vd + 255) / 256), dim3(256), 0, stream, d2t, Vd, tgt);
  const uint32_t k0 = (uint32_t)(seed & 0xFFFFFFFFu), k1 = (uint32_t)(seed >> 32);
  switch (ksteps_of(r)) {
    case 1:
      return launch_ks<1>(reduced, keep, logits, w1, w2, tgt, spill, anchor, temperature, request_id, k0, k1, partial,
                          draft_tokens, log_z, B, N, V, Vd, r, p.btiles, p.vslices, conf, lw, win, stream);
    case 2:
      return launch_ks<2>(reduced, keep, logits, w1, w2, tgt, spill, anchor, temperature, request_id, k0, k1, partial,
                          draft_tokens, log_z, B, N, V, Vd, r, p.btiles, p.vslices, conf, lw, win, stream);
    case 4:
      return launch_ks<4>(reduced, keep, logits, w1, w2, tgt, spill, anchor, temperature, request_id, k0, k1, partial,
                          draft_tokens, log_z, B, N, V, Vd, r, p.btiles, p.vslices, conf, lw, win, stream);
    default:
      return launch_ks<8>(reduced, keep, logits, w1, w2, tgt, spill, anchor, temperature, request_id, k0, k1, partial,
                          draft_tokens, log_z, B, N, V, Vd, r, p.btiles, p.vslices, conf, lw, win, stream);
  }
}

size_t markov_replay_spill_bytes(int Vd) {
  const int chunks = (Vd + kChunk - 1) / kChunk;
  return (size_t)chunks * kChunk * sizeof(float);
}

hipError_t launch_markov_replay(float* logits, const uint16_t* w1, const uint16_t* w2, const int32_t* rows,
                                const int32_t* prev, const float* temperature, const uint32_t* request_id, int B,
                                int N, int V, int Vd, int r, float* spill, hipStream_t stream) {
  const int nbt = (B + kReqPerWG - 1) / kReqPerWG;
  const int chunks = (Vd + kChunk - 1) / kChunk;
  const int max_slices = markov_slices(chunks, nbt, kMaxSlots);
  switch (ksteps_of(r)) {
    case 1:
      return launch_replay_ks<1>(logits, w1, w2, spill, rows, prev, temperature, request_id, B, N, V, Vd, r, nbt,
                                 max_slices, stream);
    case 2:
      return launch_replay_ks<2>(logits, w1, w2, spill, rows, prev, temperature, request_id, B, N, V, Vd, r, nbt,
                                 max_slices, stream);
    case 4:
      return launch_replay_ks<4>(logits, w1, w2, spill, rows, prev, temperature, request_id, B, N, V, Vd, r, nbt,
                                 max_slices, stream);
    default:
      return launch_replay_ks<8>(logits, w1, w2, spill, rows, prev, temperature, request_id, B, N, V, Vd, r, nbt,
                                 max_slices, stream);
  }
}

hipError_t launch_build_inverse_map(const int64_t* d2t, int Vd, int V, int32_t* inv_map, hipStream_t stream) {
  hipLaunchKernelGGL(inverse_fill, dim3((V + 255) / 256), dim3(256), 0, stream, inv_map, V);
  hipLaunchKernelGGL(inverse_scatter, dim3((Vd + 255) / 256), dim3(256), 0, stream, d2t, Vd, V, inv_map);
  return hipGetLastError();
}

}  // namespace dspark
