// Stage 2 for few requests (B <= 16): the whole N-step Markov loop in one
// persistent launch, with the sequential part reduced to a few candidates.
//
// With few requests a step is a tiny amount of work spread over the whole chip,
// so a step-by-step loop pays a grid-wide synchronisation per step.  Here the
// steps are decoupled instead.  Step i samples
//     x_i = t(argmax_j key_ij + c * bias_j(x_{i-1})),   key_ij = c * base_ij + G_ij
// (c = log2(e)/T; T == 0: c = 1 and no noise).  By Cauchy-Schwarz,
//     |bias_j(p)| = |W2[j] . W1[p]| <= ||W1[p]|| ||W2[j]|| <= n1 ||W2[j]||
// with n1 a bound on the norm of every W1 row that can be a previous token, so
// entry j's full key lies within c * n1 * ||W2[j]|| of its bias-free key.  The
// argmax lies among the entries whose upper end reaches the largest lower end.
// Bias-free keys do not depend on the previous token, so every step's candidates
// are found at once, in parallel; only the chain through them is sequential, and
// it touches a handful of rows.
//
// Every workgroup owns a slice of the draft vocabulary (at most 1024 entries):
//   phase A  (all workgroups)  the W2 slice into LDS (kept for the whole kernel)
//            and the norm of each of its rows; its loads are in flight while the
//            first row batch's keys of phase B are computed.
//   phase B  (all)   bias-free keys of every (request, step) row of the slice; the
//            slice's best two entries of each row are recorded with ||W2[j]|| and
//            ||W1[t(j)]|| (the row j would use as a previous token).  Every entry
//            the slice did not record is at most the second recorded key.  A
//            previous token is the anchor or a chosen (so recorded) entry of the
//            step before, so n1 is the largest of these W1 norms.  Then the base
//            logits of the first phase-D tile are prefetched.
//   -- grid barrier --
//   phase C  (one workgroup per request)  n1; per step (one wave each) the largest
//            lower end LB over the recorded entries and the survivors: recorded
//            entries whose upper end reaches LB.  The set is complete unless some
//            slice's second recorded key, raised by c * n1 times the slice's
//            largest W2 row norm, also reaches LB (the slice might hold more): from
//            the first such step on, the request goes to the per-step pass.
//            Survivor weight rows are staged in LDS, the bias of every (previous
//            survivor, survivor) pair is computed at once, and one lane walks the
//            chain through that table.  The W1 rows of the chosen previous tokens
//            are published for phase D.
//   -- grid barrier --
//   per-step pass (all, only from a step whose survivor set was incomplete): bias
//            for every entry, grid-wide argmax, one step at a time.
//   phase D  (all)   processed logits base + bias for every step, written in
//            place, and per-workgroup log-sum-exp partials; the last workgroup
//            to finish merges them into log Z.
//
// The result is the same sampling rule as the per-step path; only the order of
// the floating-point work differs (the bounds carry a margin for that rounding).
// Data crossing workgroups (norms, recorded entries, partials, tokens, rows) uses
// device-scope atomic loads and stores, which bypass the per-XCD L2 caches.
//
// Launch: an ordinary launch of one workgroup per slice (at most one per CU, by
// its LDS size).  The grid barriers need every workgroup resident at once, which
// an idle device gives but nothing guarantees.  Every workgroup runs phases A and
// B of its own slice, which need no other workgroup; at the first barrier the
// first workgroup to take an arrival number checks that all of them arrive within
// a short window.  If they do, the phases go on as above; if not (the device is
// busy elsewhere), that workgroup runs every phase for every slice by itself and
// the others return.  Either way no workgroup ever waits for one that has not
// started.  The barrier counters are one of the library's counter sets, which
// every launch leaves cleared (see kCtrSets).
#include <math.h>
#include <stdlib.h>

#include <algorithm>
#include <atomic>

#include "device.hpp"
#include "kernels.hpp"
#include "markov_common.hpp"

namespace dspark {

namespace {

using namespace mk;

constexpr int kTop = 2;          // entries recorded per (row, slice)
constexpr int kMaxRows = 1024;   // B * N
constexpr int kMaxSlice = 1024;  // draft entries per workgroup (one 4-entry group per thread)
constexpr int kMaxSlices = 256;  // workgroups: a step's recorded entries fit 8 per lane
constexpr int kPerLane = 8;      // recorded entries of one step per lane in phase C
constexpr int kMaxCPW = 4;       // 64-entry chunks per wave in phase D (kMaxSlice / 64 / 4 waves)
constexpr int kRowBatch = 8;     // rows whose keys phase B computes together
constexpr int kFly = 24;         // 16-byte loads in flight per thread in phase A
constexpr int kStage = 4;        // 16-byte loads in flight per thread when staging survivor rows
constexpr int kPairs = 2048;     // (previous survivor, survivor) biases phase C can tabulate
constexpr int kMisc = 512;       // ints of per-workgroup bookkeeping in LDS
constexpr int kFixedScratch = 256 + 1024 + 4 * kMisc + 4 * kMaxSlice + 4 * kMaxSlices;  // + row / slice W2 norms
constexpr uint64_t kArriveTicks = 5000;  // start-up window: 50 us of the 100 MHz real-time counter

// Counters (32-bit words).  Words 0..3: grid barrier (groups arrived), workgroups
// done (groups finished), arrivals, departures (solo mode only).  Workgroup w
// belongs to group w % kGroups; each group has its own barrier and done counters,
// 128 bytes apart, so that no single address takes an atomic from every workgroup
// (same-address atomics are served one at a time, ~20 ns each).
// A launch takes one of kCtrSets counter sets that the library keeps in device
// memory (zero when the library is loaded) and leaves it zero when it ends: the
// last workgroup to use the counters clears them.  So no launch has to clear
// them first, and the caller's workspace holds no counters.
constexpr int kGroups = 16;
constexpr int kCtrWords = 32 + 32 * 2 * kGroups;
constexpr int kCtrSets = 64;
__device__ __forceinline__ unsigned* ctr_group(unsigned* ctr, int kind, int grp) {
  return ctr + 32 + 32 * (kind * kGroups + grp);
}
__device__ __forceinline__ unsigned group_size(int G, int grp) { return (unsigned)((G - grp + kGroups - 1) / kGroups); }
__device__ __forceinline__ unsigned group_count(int G) { return (unsigned)min(G, kGroups); }
constexpr int kWaitVm0 = 0x0F70;  // s_waitcnt vmcnt(0) (gfx9 encoding)

// misc layout (ints)
constexpr int kMsCnt = 0, kMsInc = 64, kMsOff = 128, kMsSel = 192, kMsPre = 256;  // [64] each ([65] for kMsPre)
constexpr int kMsFs = 336, kMsFit = 337, kMsPairs = 338, kMsTot = 339, kMsRole = 340, kMsTicket = 341;
constexpr int kMsLastOut = 342, kMsRows = 343, kMsBarrierOk = 344;
constexpr int kMsRoff = 448;  // [64] first (previous survivor) row of each step in phase C
constexpr int kMsPrev = 352, kMsFst = 368;  // [16] each (per-step pass)
constexpr int kMsN1 = 384;                  // [16] floats: largest recorded W1 norm per request (phase B)
constexpr int kMsT = 400, kMsRid = 416, kMsAnc = 432;  // [16] each: temperature, request id, anchor per request

// A recorded entry is one word: key bits << 32 | ||W2[j]|| rounded up to bf16
// << 16 | j - (first draft index of its slice) (0xFFFF: none).  A candidate in
// phase C carries the draft index itself: key bits << 32 | j.
constexpr uint64_t kEmptySlot = ((uint64_t)0xFF800000u << 32) | 0xFFFFull;
__device__ __forceinline__ float slot_key(uint64_t s) { return __uint_as_float((uint32_t)(s >> 32)); }
__device__ __forceinline__ float rec_w2n(uint64_t s) { return __uint_as_float((uint32_t)s & 0xFFFF0000u); }
__device__ __forceinline__ int rec_jl(uint64_t s) { return (int)((uint32_t)s & 0xFFFFu); }
__device__ __forceinline__ int slot_j(uint64_t s) { return (int)(uint32_t)s; }
// bf16 bits of the smallest bf16 >= x (x >= 0; inf and NaN stay)
__device__ __forceinline__ uint32_t bf16_up(float x) {
  const uint32_t b = __float_as_uint(x);
  if ((b & 0x7F800000u) == 0x7F800000u) return b >> 16;
  return (b + 0xFFFFu) >> 16;
}
static_assert(kMaxSlice <= 0xFFFF, "slice-local draft index must fit 16 bits");

struct FewWs {
  float* norms;           // [G] largest squared W2 row norm of each slice
  float* n1;              // [B][G] largest W1 norm of each request's possible previous tokens, per slice
  uint64_t* rec;          // [B*N][G][kTop] recorded entries
  int* fstep;             // [B] first step left to the per-step pass (N if none)
  MarkovPartial* partF;   // [2][B][G] per-step partials of that pass
  MarkovPartial* partD;   // [B*N][G] log-sum-exp partials of the processed rows
  uint32_t* rows;         // [B*N][r/2] W1 row (bf16 pairs) of each step's previous token
  unsigned* ctr;          // [kCtrWords] this launch's counter set (see ctr_group)
};

struct FewArgs {
  float* logits;
  const uint16_t* w1;
  const uint16_t* w2;
  const int64_t* d2t;
  const int32_t* anchor;
  const float* temperature;
  const uint32_t* request_id;
  int32_t* draft_tokens;
  float* log_z;
  FewWs ws;
  uint32_t key0, key1;
  int B, N, V, Vd, r, CH, cap, force_solo;
  ConfArgs conf;          // fused confidence head (conf.out == nullptr: none)
  unsigned* status;       // the device's sticky error word (bit 0: a grid barrier gave up)
  int force_give_up;      // test mode: every grid barrier reports a give-up after it completes
};

// layout of the phase-C region of LDS (also used by the host plan)
struct CRegion {
  size_t cands, w2c, w1c, tgt, fk, bytes;
};
__host__ __device__ inline CRegion cregion(int N, int cap, int r) {
  CRegion o;
  const size_t m = (size_t)N * cap;
  size_t off = 0;
  o.cands = off;
  off += (m * 8 + 15) & ~(size_t)15;
  o.w2c = off;
  off += m * 2 * r;
  o.w1c = off;
  off += (m + 1) * 2 * r;
  o.tgt = off;
  off += (m * 4 + 15) & ~(size_t)15;
  o.fk = off;
  off += (size_t)kPairs * 4;
  o.bytes = off;
  return o;
}

struct Lds {
  char* w2s;          // [S] W2 rows of the slice, slot-permuted per 64-chunk, row_bytes apart
  float* w2n;         // [kMaxSlice] squared norms of those rows
  float* n2s;         // [kMaxSlices] largest W2 row norm of each slice (phase C)
  float* thr;         // [64] survivor thresholds (largest lower end) of the request in phase C
  float* redf;        // reduction scratch (1 KB)
  int* misc;          // bookkeeping
  uint64_t* cands;    // [N][cap] survivors (first word of the recorded entry)
  uint16_t* w2c;      // [N*cap][r] their W2 rows
  uint16_t* w1c;      // [1 + N*cap][r] W1 rows: the anchor, then each survivor's target
  int* tgt;           // [N*cap] target ids of the survivors
  float* fk;          // [kPairs] full keys of (previous survivor, survivor) pairs
};

// per-request parameters (copied into LDS after phase B)
__device__ __forceinline__ float req_temperature(const Lds& L, int b) { return reinterpret_cast<const float*>(L.misc)[kMsT + b]; }
__device__ __forceinline__ uint32_t req_id(const Lds& L, int b) { return reinterpret_cast<const uint32_t*>(L.misc)[kMsRid + b]; }
__device__ __forceinline__ int req_anchor(const Lds& L, int b) { return L.misc[kMsAnc + b]; }

// every launch's counter sets, kCtrWords words each (zero-initialised when loaded)
__device__ __attribute__((aligned(256))) unsigned g_few_counters[kCtrSets * kCtrWords];
// sticky error word of this device: set when a grid barrier's bounded wait gives up;
// read and cleared by the host (dspark_markov_check)
__device__ __attribute__((aligned(256))) unsigned g_few_status[64];

// half-width of a full key's interval around the bias-free key, per unit of W2
// row norm, and an absolute slack: room for the float rounding of norms, dots
// and keys on both sides
__device__ __forceinline__ float bias_bound(float c, float n1) { return c * n1 * (1.0f + 1.0f / 256.0f); }
constexpr float kKeySlack = 1.0f / 2048.0f;

__device__ __forceinline__ void st_i(int* p, int v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ int ld_i(const int* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_u(uint32_t* p, uint32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ uint32_t ld_u(const uint32_t* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_f(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ float ld_f(const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_u64(uint64_t* p, uint64_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ uint64_t ld_u64(const uint64_t* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

// order-preserving map of a key to unsigned (NaN -> 0: below every key)
__device__ __forceinline__ uint32_t ord_of(float k) {
  const uint32_t b = __float_as_uint(k);
  if (k != k) return 0u;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float key_of(uint32_t o) { return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o); }

__device__ __forceinline__ uint64_t slot_of_rank(uint64_t v) {
  const uint32_t o = (uint32_t)(v >> 32);
  if (o == 0u) return kEmptySlot;
  return ((uint64_t)__float_as_uint(key_of(o)) << 32) | (uint32_t)~(uint32_t)v;
}
// merge two descending best-two lists of ranks (key order, then smaller index)
__device__ __forceinline__ void merge2(uint64_t& a1, uint64_t& a2, uint64_t b1, uint64_t b2) {
  const uint64_t hi = a1 > b1 ? a1 : b1, lo = a1 > b1 ? b1 : a1;
  const uint64_t m2 = a2 > b2 ? a2 : b2;
  a1 = hi;
  a2 = lo > m2 ? lo : m2;
}

// lanes below this one whose bit is set in m
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// block-wide max over 256 threads (red: >= 4 floats of LDS)
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max_f32(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Batched loads are unconditional, from an index clamped into the array: a load
// under a branch (or a select the compiler turns into one) is waited for inside
// the branch, which serialises the batch.  A piece past the end reads the same
// piece of the last row, so such padding duplicates a real row.
__device__ __forceinline__ uint4 load_clamped(const uint4* src, int idx, int n, int row_pieces) {
  return src[idx < n ? idx : n - row_pieces + (idx & (row_pieces - 1))];
}

// (bf16 pair dot products: the norms only bound biases, with a relative slack far
// above their rounding)
__device__ __forceinline__ float sumsq8(const uint4& v) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  float ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, v.x), __builtin_bit_cast(b2, v.x), 0.0f, false);
  ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, v.y), __builtin_bit_cast(b2, v.y), ss, false);
  ss = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, v.z), __builtin_bit_cast(b2, v.z), ss, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, v.w), __builtin_bit_cast(b2, v.w), ss, false);
}

__device__ __forceinline__ float row_norm2(const uint16_t* row, int r) {
  float ss = 0.0f;
  for (int k = 0; k < r; k += 8) ss += sumsq8(*reinterpret_cast<const uint4*>(row + k));
  return ss;
}

__device__ __forceinline__ float dot_bf16(const uint16_t* a, const uint16_t* b, int r) {
  float acc = 0.0f;
  for (int k = 0; k < r; k += 8) {
    const uint4 x = *reinterpret_cast<const uint4*>(a + k);
    const uint4 y = *reinterpret_cast<const uint4*>(b + k);
    const uint32_t xa[4] = {x.x, x.y, x.z, x.w}, ya[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc += __uint_as_float(xa[q] << 16) * __uint_as_float(ya[q] << 16);
      acc += __uint_as_float(xa[q] & 0xFFFF0000u) * __uint_as_float(ya[q] & 0xFFFF0000u);
    }
  }
  return acc;
}

// bias-free keys of 4 consecutive draft entries j..j+3 of (request, step)
__device__ __forceinline__ void keys4(const float4& base, bool noisy, float c, int j, int step, uint32_t rid,
                                      uint32_t key0, uint32_t key1, float (&key)[4]) {
  const float l[4] = {base.x, base.y, base.z, base.w};
  if (noisy) {
    const u32x4 w = philox4x32_10(u32x4{(uint32_t)j >> 2, (uint32_t)step, rid, kTagDraft}, key0, key1);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int f = 0; f < 4; ++f) key[f] = l[f] * c + gumbel2(ws[f]);
  } else {
#pragma unroll
    for (int f = 0; f < 4; ++f) key[f] = l[f];
  }
}

__device__ __forceinline__ int target_of(const int64_t* d2t, int j) { return d2t ? j + (int)d2t[j] : j; }
__device__ __forceinline__ float temp_scale(float T) { return (T > 0.0f) ? (1.0f / T) * 1.4426950408889634f : 1.0f; }

// bias of a 64-entry chunk for the 16 MFMA rows held in efrag (rows: lane n's A row);
// lane (n, g) gets rows 4g+i of entries 4n+f of the chunk in acc[f][i]
__device__ __forceinline__ void chunk_bias(const char* chunk_rows, int row_bytes, int ksteps, int r,
                                           const bf16x8 (&efrag)[kMaxKSteps], int n, int g, floatx4 (&acc)[4]) {
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    acc[f] = floatx4{0.f, 0.f, 0.f, 0.f};
    const char* rowp = chunk_rows + (size_t)(f * 16 + n) * row_bytes;
#pragma unroll
    for (int s = 0; s < kMaxKSteps; ++s) {
      if (s < ksteps) {
        const int k = s * 32 + 8 * g;
        const bf16x8 bfr = (k < r) ? __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(rowp + k * 2)) : zero8();
        acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(efrag[s], bfr, acc[f], 0, 0, 0);
      }
    }
  }
}

// The same for r == 32 * KS: every k is in range, so all B fragments of the chunk
// are read first and the four entry groups' products run back to back.
template <int KS>
__device__ __forceinline__ void chunk_bias_k(const char* chunk_rows, int row_bytes, const bf16x8 (&efrag)[kMaxKSteps],
                                             int n, int g, floatx4 (&acc)[4]) {
  bf16x8 bfr[4][KS];
#pragma unroll
  for (int f = 0; f < 4; ++f) {
    const char* rowp = chunk_rows + (size_t)(f * 16 + n) * row_bytes;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      bfr[f][s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(rowp + (s * 32 + 8 * g) * 2));
  }
  __builtin_amdgcn_sched_barrier(0);  // (every read issued before the first product)
#pragma unroll
  for (int f = 0; f < 4; ++f) acc[f] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KS; ++s)
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(efrag[s], bfr[f][s], acc[f], 0, 0, 0);
}
__device__ __forceinline__ void chunk_bias_any(const char* chunk_rows, int row_bytes, int ksteps, int r,
                                               const bf16x8 (&efrag)[kMaxKSteps], int n, int g, floatx4 (&acc)[4]) {
  if (r == 64)
    chunk_bias_k<2>(chunk_rows, row_bytes, efrag, n, g, acc);
  else if (r == 32)
    chunk_bias_k<1>(chunk_rows, row_bytes, efrag, n, g, acc);
  else if (r == 128)
    chunk_bias_k<4>(chunk_rows, row_bytes, efrag, n, g, acc);
  else
    chunk_bias(chunk_rows, row_bytes, ksteps, r, efrag, n, g, acc);
}

// A operand from W1 row `prev` (read-only weights)
__device__ __forceinline__ void load_efrag(const uint16_t* w1, int prev, bool valid, int V, int r, int ksteps, int g,
                                           bf16x8 (&efrag)[kMaxKSteps]) {
  const int p = valid ? min(max(prev, 0), V - 1) : 0;
  const uint16_t* er = w1 + (size_t)p * r;
#pragma unroll
  for (int s = 0; s < kMaxKSteps; ++s) {
    const int k = s * 32 + 8 * g;
    efrag[s] = (s < ksteps && k < r && valid) ? __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(er + k))
                                              : zero8();
  }
}

// A operand from a published row (written by another workgroup in this launch)
__device__ __forceinline__ void load_efrag_published(const uint32_t* row, bool valid, int r, int ksteps, int g,
                                                     bf16x8 (&efrag)[kMaxKSteps]) {
  const uint64_t* rp = reinterpret_cast<const uint64_t*>(row);
#pragma unroll
  for (int s = 0; s < kMaxKSteps; ++s) {
    const int k = s * 32 + 8 * g;
    if (s < ksteps) {
      const int kc = min(k, r - 8) / 4;  // 8 bf16 = two 64-bit words
      const uint64_t lo = ld_u64(rp + kc), hi = ld_u64(rp + kc + 1);
      efrag[s] = (k < r && valid)
                     ? __builtin_bit_cast(bf16x8, make_uint4((uint32_t)lo, (uint32_t)(lo >> 32), (uint32_t)hi,
                                                             (uint32_t)(hi >> 32)))
                     : zero8();
    } else {
      efrag[s] = zero8();
    }
  }
}

// A operand from the W1 row that phase C staged in this workgroup's LDS for the
// previous token of `step` (step 0: the anchor; step i: survivor sel[i-1] of step
// i-1); only after a staged chain that covers every step
__device__ __forceinline__ void load_efrag_lds(const Lds& L, int step, bool valid, int r, int ksteps, int g, int cap,
                                               bf16x8 (&efrag)[kMaxKSteps]) {
  const int* sel = L.misc + kMsSel;
  const int row = (step == 0) ? 0 : 1 + (step - 1) * cap + sel[step - 1];
  const uint16_t* src = L.w1c + (size_t)row * r;
#pragma unroll
  for (int s = 0; s < kMaxKSteps; ++s) {
    const int k = s * 32 + 8 * g;
    efrag[s] = (s < ksteps && k < r && valid) ? __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(src + k))
                                              : zero8();
  }
}

// base logits of phase-D tile t (request t / tpr, steps 16 * (t % tpr) ..) that lane
// (n, g) of `wave` combines with its MFMA results: chunk wave + 4u, entries 4n..4n+3,
// steps 4g + i (indices clamped; lanes outside the tile never use the value)
__device__ __forceinline__ void load_tile(float4 (&dst)[kMaxCPW][4], const float* logits, int t, int tpr, int B, int N,
                                          int Vd, int vbase, int wave, int n, int g) {
  const int b = t / tpr, st0 = (t - b * tpr) * 16;
#pragma unroll
  for (int u = 0; u < kMaxCPW; ++u) {
    const int jb = vbase + (wave + 4 * u) * kChunk + 4 * n;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int step = st0 + 4 * g + i;
      dst[u][i] = *reinterpret_cast<const float4*>(logits + ((size_t)min(b, B - 1) * N + min(step, N - 1)) * Vd +
                                                   min(jb, Vd - 4));
    }
  }
}

struct Slice {
  int vbase, nvalid, nch;
};
__device__ __forceinline__ Slice slice_of(const FewArgs& a, int vwg) {
  Slice s;
  s.vbase = vwg * a.CH * kChunk;
  s.nvalid = max(0, min(a.CH * kChunk, a.Vd - s.vbase));  // a multiple of 4
  s.nch = (s.nvalid + kChunk - 1) / kChunk;
  return s;
}

// W2 rows of a slice into LDS (slot-permuted per 64-chunk for the MFMA B operand);
// with kNorm, also the largest squared row norm of the slice
template <bool kNorm>
__device__ __forceinline__ float load_slice(const FewArgs& a, const Lds& L, const Slice& sl) {
  const int tid = threadIdx.x, r = a.r, kc = r / 8, row_bytes = 2 * r + 16;
  const int pieces = sl.nch * kChunk * kc;  // 16-byte pieces, padded to whole chunks
  float n2 = 0.0f;
  if ((kc & (kc - 1)) == 0) {
    // a contiguous byte range; a row's kc pieces sit in consecutive lanes
    const int lg = __builtin_ctz(kc);
    const int valid = sl.nvalid * kc;
    const uint4* src = reinterpret_cast<const uint4*>(a.w2 + (size_t)sl.vbase * r);
    for (int p0 = 0; p0 < pieces; p0 += 256 * kFly) {
      uint4 v[kFly];
#pragma unroll
      for (int u = 0; u < kFly; ++u) v[u] = load_clamped(src, p0 + tid + 256 * u, valid, kc);
#pragma unroll
      for (int u = 0; u < kFly; ++u) {
        const int p = p0 + tid + 256 * u;
        if (p < pieces) {  // uniform per wave
          const int rho_all = p >> lg, piece = p & (kc - 1);
          if (kNorm) {
            const float ss = group_sum(sumsq8(v[u]), kc);
            n2 = fmaxf(n2, ss);
            if (piece == 0) L.w2n[rho_all] = ss;
          }
          const int c = rho_all >> 6, rho = rho_all & (kChunk - 1);
          const int slot = c * kChunk + (rho & 3) * 16 + (rho >> 2);
          *reinterpret_cast<uint4*>(L.w2s + (size_t)slot * row_bytes + piece * 16) = v[u];
        }
      }
    }
  } else {
    for (int p = tid; p < pieces; p += 256) {
      const int rho_all = p / kc, piece = p % kc;
      const int j = sl.vbase + min(rho_all, sl.nvalid - 1);
      const uint4 v = *reinterpret_cast<const uint4*>(a.w2 + (size_t)j * r + piece * 8);
      const int c = rho_all / kChunk, rho = rho_all % kChunk;
      const int slot = c * kChunk + (rho & 3) * 16 + (rho >> 2);
      *reinterpret_cast<uint4*>(L.w2s + (size_t)slot * row_bytes + piece * 16) = v;
    }
    if (kNorm)
      for (int q = tid; q < sl.nch * kChunk; q += 256) {
        const float ss = row_norm2(a.w2 + (size_t)(sl.vbase + min(q, sl.nvalid - 1)) * r, r);
        n2 = fmaxf(n2, ss);
        L.w2n[q] = ss;
      }
  }
  __syncthreads();
  return n2;
}

// ------------------------------------------------------------------------ phases A, B
// One batch of a slice's W2 pieces (power-of-two kc): the loads, issued on their own
// so that other work can run while they are in flight ...
__device__ __forceinline__ void w2_issue(const FewArgs& a, const Slice& sl, int p0, uint4 (&v)[kFly]) {
  const int kc = a.r / 8;
  const uint4* src = reinterpret_cast<const uint4*>(a.w2 + (size_t)sl.vbase * a.r);
#pragma unroll
  for (int u = 0; u < kFly; ++u) v[u] = load_clamped(src, p0 + (int)threadIdx.x + 256 * u, sl.nvalid * kc, kc);
}

// ... and their use: into LDS (slot-permuted per 64-chunk for the MFMA B operand),
// each row's squared norm into w2n; returns this thread's largest squared row
// norm.  KC: pieces per row when fixed at compile time (0: a.r / 8 at run time).
template <int KC>
__device__ __forceinline__ float w2_consume(const FewArgs& a, const Lds& L, const Slice& sl, int p0,
                                            const uint4 (&v)[kFly]) {
  const int kc = KC ? KC : a.r / 8, lg = __builtin_ctz(kc), row_bytes = 16 * (kc + 1);
  const int pieces = sl.nch * kChunk * kc;
  float n2 = 0.0f;
#pragma unroll
  for (int u = 0; u < kFly; ++u) {
    const int p = p0 + (int)threadIdx.x + 256 * u;
    if (p < pieces) {  // uniform per wave
      const int rho_all = p >> lg, piece = p & (kc - 1);
      const float ss = group_sum(sumsq8(v[u]), kc);
      n2 = fmaxf(n2, ss);
      if (piece == 0) L.w2n[rho_all] = ss;
      const int c = rho_all >> 6, rho = rho_all & (kChunk - 1);
      const int slot = c * kChunk + (rho & 3) * 16 + (rho >> 2);
      *reinterpret_cast<uint4*>(L.w2s + (size_t)slot * row_bytes + piece * 16) = v[u];
    }
  }
  return n2;
}
// (rank 64, eight pieces per row, has its own copy with the lane sums unrolled)
__device__ __forceinline__ float w2_consume_any(const FewArgs& a, const Lds& L, const Slice& sl, int p0,
                                                const uint4 (&v)[kFly]) {
  return (a.r == 64) ? w2_consume<8>(a, L, sl, p0, v) : w2_consume<0>(a, L, sl, p0, v);
}

// Rows row0 .. row0+kRowBatch-1: base logits at this thread's four entries, and
// each row's temperature and request id.  Every load is issued here, unguarded
// (clamped indices: invalid lanes and rows never use the value), so that one wait
// covers them all.
struct RowBatch {
  float4 bv[kRowBatch];
  float T[kRowBatch];
  uint32_t rid[kRowBatch];
};
// (The per-row values are loaded per lane: as wave-uniform values the compiler
// would move each into a scalar register at once, waiting for every load before.)
__device__ __forceinline__ void load_rows(const FewArgs& a, const Slice& sl, int row0, RowBatch& rb) {
  const int rows = a.B * a.N, jq = sl.vbase + 4 * (int)threadIdx.x;
  int lane_zero = 0;
  asm volatile("" : "+v"(lane_zero));
#pragma unroll
  for (int rr = 0; rr < kRowBatch; ++rr) {
    const int row = min(row0 + rr, rows - 1);
    rb.bv[rr] = *reinterpret_cast<const float4*>(a.logits + (size_t)row * a.Vd + min(jq, sl.vbase + sl.nvalid - 4));
    rb.T[rr] = a.temperature[row / a.N + lane_zero];
    rb.rid[rr] = a.request_id[row / a.N + lane_zero];
  }
}

// bias-free keys of a row batch; every wave's best two entries of each row into
// red64[(row * 4 + wave) * kTop ..]
__device__ __forceinline__ void keys_batch(const FewArgs& a, const Slice& sl, int row0, const RowBatch& rb,
                                           uint64_t* red64) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = a.N, rows = a.B * a.N;
  const bool qv = 4 * tid < sl.nvalid;  // this thread's entries jq .. jq+3
  const int jq = sl.vbase + 4 * tid;
#pragma unroll
  for (int rr = 0; rr < kRowBatch; ++rr) {
    const int row = row0 + rr;
    if (row >= rows) break;  // uniform
    // this lane's best two entries (ties: smaller index), then the wave's: the
    // lowest lane holding the maximum has the smallest index among equal keys
    uint32_t o[4] = {0u, 0u, 0u, 0u};
    const float T = rb.T[rr];
    const uint32_t rid = rb.rid[rr];
    if (qv) {
      const int i = row - (row / N) * N;
      float key[4];
      keys4(rb.bv[rr], T > 0.0f, temp_scale(T), jq, i, rid, a.key0, a.key1, key);
#pragma unroll
      for (int f = 0; f < 4; ++f) o[f] = ord_of(key[f]);
    }
    int f1 = 0;
#pragma unroll
    for (int f = 1; f < 4; ++f)
      if (o[f] > o[f1]) f1 = f;
    int f2 = (f1 == 0) ? 1 : 0;
#pragma unroll
    for (int f = 1; f < 4; ++f)
      if (f != f1 && o[f] > o[f2]) f2 = f;
    const uint32_t own1 = o[f1], own2 = o[f2];
    const uint32_t m1 = wave_max_u32(own1);
    const int l1 = __builtin_ctzll(__ballot(own1 == m1));
    const int j1 = __builtin_amdgcn_readlane(jq + f1, l1);
    const uint32_t cand = (lane == l1) ? own2 : own1;
    const int cj = (lane == l1) ? jq + f2 : jq + f1;
    const uint32_t m2 = wave_max_u32(cand);
    const int l2 = __builtin_ctzll(__ballot(cand == m2));
    const int j2 = __builtin_amdgcn_readlane(cj, l2);
    if (lane == 0) {
      red64[(rr * 4 + wave) * kTop] = m1 ? (((uint64_t)m1 << 32) | (uint32_t)~j1) : 0ull;
      red64[(rr * 4 + wave) * kTop + 1] = m2 ? (((uint64_t)m2 << 32) | (uint32_t)~j2) : 0ull;
    }
  }
}

// the slice's best two entries of each row of the batch (from the waves' in
// red64, written before the last barrier), and their records: key and index,
// ||W2[j]|| (from LDS) and ||W1[t(j)]|| (kc lanes per entry)
__device__ __forceinline__ void records_batch(const FewArgs& a, const Lds& L, const Slice& sl, int vwg, int G, int row0,
                                              uint64_t* red64, float* n1r) {
  const int tid = threadIdx.x;
  const int r = a.r, kc = r / 8, N = a.N, rows = a.B * a.N;
  const bool pow2 = (kc & (kc - 1)) == 0;
  const int lg = __builtin_ctz(kc);
  uint64_t* best = red64 + kRowBatch * 4 * kTop;  // [kRowBatch][kTop] ranks of the slice
  if (tid < kRowBatch && row0 + tid < rows) {
    uint64_t t1 = 0, t2 = 0;
    for (int w = 0; w < 4; ++w) merge2(t1, t2, red64[(tid * 4 + w) * kTop], red64[(tid * 4 + w) * kTop + 1]);
    best[tid * kTop] = t1;
    best[tid * kTop + 1] = t2;
  }
  __syncthreads();
  const int ne = kRowBatch * kTop;
  for (int p = tid; p < ne * kc; p += 256) {  // (whole groups of kc lanes)
    const int e = pow2 ? (p >> lg) : p / kc, piece = p - e * kc;
    const int row = row0 + e / kTop;
    const uint64_t rk = best[e];
    const bool ok = row < rows && (rk >> 32) != 0;
    const int j = ok ? (int)~(uint32_t)rk : sl.vbase;
    const int t = min(max(target_of(a.d2t, j), 0), a.V - 1);
    float ss;
    if (pow2) {
      ss = group_sum(sumsq8(*reinterpret_cast<const uint4*>(a.w1 + (size_t)t * r + piece * 8)), kc);
    } else {
      ss = row_norm2(a.w1 + (size_t)t * r, r);  // (every lane of the entry; one stores)
    }
    if (piece == 0 && row < rows) {
      uint64_t w0 = kEmptySlot;
      if (ok) {
        const float n1e = sqrtf(ss);
        w0 = ((uint64_t)__float_as_uint(key_of((uint32_t)(rk >> 32))) << 32) |
             (bf16_up(sqrtf(L.w2n[j - sl.vbase])) << 16) | (uint32_t)(j - sl.vbase);
        const int b = row / N;
        if (row - b * N < N - 1) atomicMax(reinterpret_cast<int*>(n1r) + b, __float_as_int(n1e));
      }
      st_u64(a.ws.rec + ((size_t)row * G + vwg) * kTop + (e % kTop), w0);
    }
  }
  __syncthreads();
}

// thread 0: this workgroup's arrival number (the first workgroup to take one gets 0)
__device__ __forceinline__ unsigned take_arrival_now(const FewArgs& a, bool take) {
  unsigned arrival = 1u;
  if (take && threadIdx.x == 0) {
    // (a lane-varying address keeps the atomic to this lane, without the wave-wide
    // reduction the compiler would otherwise wrap it in, which waits for the result)
    int zero = 0;
    asm volatile("" : "+v"(zero));
    arrival = __hip_atomic_fetch_add(a.ws.ctr + 2 + zero, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  return arrival;
}

// Phases A and B of one slice.  The first row batch's base logits and the first
// W2 batch are requested together, and that row batch's keys are computed while
// the W2 rows are still in flight.  With take_arrival, thread 0 also takes this
// workgroup's arrival number (returned; 1 elsewhere), right after those loads:
// vector memory operations complete in issue order, so an atomic issued before
// them would hold up every wait on them while the other workgroups' atomics on
// the same counter are served.
__device__ __forceinline__ unsigned phase_ab(const FewArgs& a, const Lds& L, int vwg, int G, bool take_arrival) {
  const int tid = threadIdx.x;
  const int r = a.r, kc = r / 8, rows = a.B * a.N;
  const bool pow2 = (kc & (kc - 1)) == 0;
  const int lg = __builtin_ctz(kc);
  const Slice sl = slice_of(a, vwg);
  float* n1r = reinterpret_cast<float*>(L.misc + kMsN1);  // per request (non-negative: int order = float order)
  uint64_t* red64 = reinterpret_cast<uint64_t*>(L.redf);  // [kRowBatch][4 waves][kTop], then [kRowBatch][kTop]
  float* red_n2 = L.redf + 192;                           // (past both)
  if (tid < 16) n1r[tid] = 0.0f;
  RowBatch rb;
  load_rows(a, sl, 0, rb);
  unsigned arrival = 1u;
  float n2 = 0.0f;
  if (pow2) {
    const int pieces = sl.nch * kChunk * kc;
    uint4 v[kFly];
    __builtin_amdgcn_sched_barrier(0);  // (every load issued before the keys use any)
    w2_issue(a, sl, 0, v);
    __builtin_amdgcn_sched_barrier(0);
    arrival = take_arrival_now(a, take_arrival);
    keys_batch(a, sl, 0, rb, red64);
    n2 = w2_consume_any(a, L, sl, 0, v);
    for (int p0 = 256 * kFly; p0 < pieces; p0 += 256 * kFly) {
      w2_issue(a, sl, p0, v);
      n2 = fmaxf(n2, w2_consume_any(a, L, sl, p0, v));
    }
    __syncthreads();
  } else {
    arrival = take_arrival_now(a, take_arrival);
    keys_batch(a, sl, 0, rb, red64);
    n2 = load_slice<true>(a, L, sl);
  }
  n2 = block_max(n2, red_n2);
  if (tid == 0) st_f(a.ws.norms + vwg, n2);
  // the anchors' W1 norms (slice 0 only: each request's bound needs them once)
  if (vwg == 0) {
    if (pow2) {
      for (int p = tid; p < a.B * kc; p += 256) {  // (whole groups of kc lanes)
        const int b = p >> lg, piece = p & (kc - 1);
        const int t = min(max(a.anchor[b], 0), a.V - 1);
        const float ss = group_sum(sumsq8(*reinterpret_cast<const uint4*>(a.w1 + (size_t)t * r + piece * 8)), kc);
        if (piece == 0) atomicMax(reinterpret_cast<int*>(n1r) + b, __float_as_int(sqrtf(ss)));
      }
    } else if (tid < a.B) {
      const int t = min(max(a.anchor[tid], 0), a.V - 1);
      atomicMax(reinterpret_cast<int*>(n1r) + tid, __float_as_int(sqrtf(row_norm2(a.w1 + (size_t)t * r, r))));
    }
  }
  records_batch(a, L, sl, vwg, G, 0, red64, n1r);
  for (int row0 = kRowBatch; row0 < rows; row0 += kRowBatch) {
    load_rows(a, sl, row0, rb);
    keys_batch(a, sl, row0, rb, red64);
    __syncthreads();
    records_batch(a, L, sl, vwg, G, row0, red64, n1r);
  }
  if (tid < a.B) st_f(a.ws.n1 + (size_t)tid * G + vwg, n1r[tid]);
  return arrival;
}

// last index i in [0, n) of a strictly increasing table with tab[i] <= x
__device__ __forceinline__ int search_le(const int* tab, int n, int x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tab[mid] <= x)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// W1 row of token t (clamped to the vocabulary) as the published row of (b, step)
__device__ __forceinline__ void publish_row_from(const FewArgs& a, int b, int step, int t, int first, int stride) {
  const int half = a.r / 2;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(a.w1 + (size_t)min(max(t, 0), a.V - 1) * a.r);
  for (int x = first; x < half; x += stride) st_u(a.ws.rows + (size_t)(b * a.N + step) * half + x, src[x]);
}

// ------------------------------------------------------------------------ phase C
// writer: this workgroup stores the request's outputs (tokens, first per-step
// step, published rows); other workgroups that run the phase only keep its results
__device__ __forceinline__ void phase_c(const FewArgs& a, const Lds& L, int b, int G, bool writer) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int N = a.N, r = a.r, cap = a.cap, kc = r / 8, half = r / 2;
  const int per = G * kTop;  // recorded entries of one step (<= 64 * kPerLane)
  const uint64_t* recb = a.ws.rec + (size_t)b * N * per;
  const int sw = a.CH * kChunk;  // draft entries per slice
  int* cnt = L.misc + kMsCnt;
  int* inc = L.misc + kMsInc;
  int* offp = L.misc + kMsOff;
  int* sel = L.misc + kMsSel;
  int* pre = L.misc + kMsPre;
  // recorded entries of steps i0 and i0 + 4 (this wave's steps of one round)
  uint64_t h[2][kPerLane];
  auto load_recs = [&](int i0) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int i = min(i0 + 4 * st, N - 1);
#pragma unroll
      for (int u = 0; u < kPerLane; ++u) h[st][u] = ld_u64(recb + (size_t)i * per + min(lane + 64 * u, per - 1));
    }
  };
  // the first round's records are requested together with the norms below
  load_recs(wave);
  // n1 for this request and every slice's largest W2 row norm
  float n1 = 0.0f;
  for (int q = tid; q < G; q += 256) {
    n1 = fmaxf(n1, ld_f(a.ws.n1 + (size_t)b * G + q));
    L.n2s[q] = sqrtf(ld_f(a.ws.norms + q));
  }
  const float c = temp_scale(req_temperature(L, b));
  n1 = block_max(n1, L.redf);  // (its barriers also publish n2s)
  const float cb = bias_bound(c, n1);
  // the widest bias of each of this lane's entries' slices (the same for every step)
  float cbn[kPerLane];
#pragma unroll
  for (int u = 0; u < kPerLane; ++u) cbn[u] = cb * L.n2s[min(lane + 64 * u, per - 1) / kTop];
  // survivors of every step: one wave per step, two steps per round; compaction by
  // ballot into the step's own LDS region
  for (int i0 = wave; i0 < N; i0 += 8) {
    if (i0 != wave) load_recs(i0);
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int i = i0 + 4 * st;
      if (i >= N) break;  // uniform per wave
      // largest lower end of a full key (empty records: -inf)
      float lb = -INFINITY;
#pragma unroll
      for (int u = 0; u < kPerLane; ++u)
        if (lane + 64 * u < per) lb = fmaxf(lb, slot_key(h[st][u]) - cb * rec_w2n(h[st][u]) - kKeySlack);
      lb = wave_max_f32(lb);
      // nothing above -inf recorded, or no usable bound: leave the step to the per-step pass
      const bool bad = !(lb > -INFINITY);
      uint64_t cov = 0, m[kPerLane];
      bool sv[kPerLane];
#pragma unroll
      for (int u = 0; u < kPerLane; ++u) {
        const int e = lane + 64 * u;
        const float k = slot_key(h[st][u]);
        sv[u] = e < per && k + cb * rec_w2n(h[st][u]) + kKeySlack >= lb;
        m[u] = __ballot(sv[u]);
        // a slice whose unrecorded entries could still reach the bound
        cov |= __ballot(e < per && (e % kTop) == kTop - 1 && k + cbn[u] + kKeySlack >= lb);
      }
      int total = 0;
#pragma unroll
      for (int u = 0; u < kPerLane; ++u) {
        const int e = lane + 64 * u, pos = total + lanes_below(m[u]);
        if (sv[u] && pos < cap)
          L.cands[i * cap + pos] = (h[st][u] & 0xFFFFFFFF00000000ull) | (uint32_t)((e / kTop) * sw + rec_jl(h[st][u]));
        total += __popcll(m[u]);
      }
      if (lane == 0) {
        cnt[i] = total;
        inc[i] = (bad || cov != 0) ? 1 : 0;
        L.thr[i] = lb;
      }
    }
  }
  __syncthreads();
  // the plan (wave 0, lane i = step i; N <= 64): the first step left to the per-step
  // pass (fs), each step's staged survivors nq and (previous, current) pairs, and
  // their offsets by prefix sums (every step before fs has at least one survivor)
  if (wave == 0) {
    const int i = lane;
    const bool act = i < N;
    const int ci = act ? cnt[i] : 0;
    const uint64_t incm = __ballot(act && inc[i] != 0);
    const int fs = incm ? (int)__builtin_ctzll(incm) : N;
    const bool in = i < fs;
    const int nq = in ? min(ci, cap) : 0;
    const int cprev = __shfl_up(ci, 1);
    const int pr = in ? ((i == 0) ? 1 : min(cprev, cap)) * nq : 0;
    const int np = in ? ((i == 0) ? 1 : min(cprev, cap)) : 0;  // previous survivors of step i
    const bool overflow = __ballot(in && ci > cap) != 0;
    int sq = nq, sp = pr, sr = np;  // inclusive prefix sums over the steps
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int aq = __shfl_up(sq, off), ap = __shfl_up(sp, off), ar = __shfl_up(sr, off);
      if (lane >= off) {
        sq += aq;
        sp += ap;
        sr += ar;
      }
    }
    if (in) {
      pre[i] = sq - nq;
      offp[i] = sp - pr;
      L.misc[kMsRoff + i] = sr - np;
    }
    const int tot = __shfl(sq, 63), pairs = __shfl(sp, 63), nrows = __shfl(sr, 63);
    if (lane == 0) {
      L.misc[kMsFs] = fs;
      L.misc[kMsFit] = (!overflow && pairs <= kPairs) ? 1 : 0;
      L.misc[kMsPairs] = pairs;
      L.misc[kMsTot] = tot;
      L.misc[kMsRows] = nrows;
    }
  }
  __syncthreads();
  const int fs = L.misc[kMsFs], pairs = L.misc[kMsPairs], tot = L.misc[kMsTot];
  if (__builtin_expect(L.misc[kMsFit] != 0, 1)) {
    // stage: W1[anchor] -> w1c row 0; survivor (i, q) (compact index pre[i] + q): its
    // W2 row -> w2c row i*cap+q, the W1 row of its target -> w1c row 1+i*cap+q
    const int np = kc * (1 + 2 * tot);
    const int anc = min(max(req_anchor(L, b), 0), a.V - 1);
    for (int p0 = 0; p0 < np; p0 += 256 * kStage) {
      uint4 v[kStage];
      uint16_t* dst[kStage];
#pragma unroll
      for (int u = 0; u < kStage; ++u) {
        const int p = min(p0 + tid + 256 * u, np - 1);
        const int row = p / kc, piece = p - row * kc;
        const uint16_t* src;
        if (row == 0) {
          src = a.w1 + (size_t)anc * r;
          dst[u] = L.w1c;
        } else {
          const int ci = (row - 1) >> 1;
          const int i = search_le(pre, fs, ci), q = ci - pre[i];
          const int slot = i * cap + q;
          const int j = slot_j(L.cands[slot]);
          if (((row - 1) & 1) == 0) {
            src = a.w2 + (size_t)j * r;
            dst[u] = L.w2c + (size_t)slot * r;
          } else {
            const int t = target_of(a.d2t, j);
            if (piece == 0) L.tgt[slot] = t;
            src = a.w1 + (size_t)min(max(t, 0), a.V - 1) * r;
            dst[u] = L.w1c + (size_t)(1 + slot) * r;
          }
        }
        v[u] = *reinterpret_cast<const uint4*>(src + piece * 8);
        dst[u] += piece * 8;
      }
#pragma unroll
      for (int u = 0; u < kStage; ++u)
        if (p0 + tid + 256 * u < np) *reinterpret_cast<uint4*>(dst[u]) = v[u];
    }
    __syncthreads();
    // the bias of every (previous survivor, survivor) pair of consecutive steps
    for (int t = tid; t < pairs; t += 256) {
      const int i = search_le(offp, fs, t);
      const int nq = min(cnt[i], cap);
      const int pi = (t - offp[i]) / nq, q = (t - offp[i]) - pi * nq;
      const uint16_t* e1 = L.w1c + (size_t)((i == 0) ? 0 : 1 + (i - 1) * cap + pi) * r;
      const uint16_t* e2 = L.w2c + (size_t)(i * cap + q) * r;
      L.fk[t] = slot_key(L.cands[i * cap + q]) + c * dot_bf16(e1, e2, r);
    }
    __syncthreads();
    // each step's winner for every previous survivor: the best (key, token) of the
    // row, its index written over the row's first key (-1: no key beats the
    // empty one)
    const int* roff = L.misc + kMsRoff;
    int* fki = reinterpret_cast<int*>(L.fk);
    for (int x = tid; x < L.misc[kMsRows]; x += 256) {
      const int i = search_le(roff, fs, x), pi = x - roff[i];
      const int nq = min(cnt[i], cap), base = offp[i] + pi * nq;
      float bk = -INFINITY;
      int bt = 0x7FFFFFFF, bq = -1;
      for (int q = 0; q < nq; ++q) {
        const float k = L.fk[base + q];
        const int t = L.tgt[i * cap + q];
        if (key_beats(k, t, bk, bt)) {
          bk = k;
          bt = t;
          bq = q;
        }
      }
      fki[base] = bq;
    }
    __syncthreads();
    if (tid == 0) {  // the chain through those winners
      int p = 0;
      for (int i = 0; i < fs; ++i) {
        const int bq = fki[offp[i] + p * min(cnt[i], cap)];
        sel[i] = max(bq, 0);
        if (writer) st_i(a.draft_tokens + (size_t)b * N + i, (bq < 0) ? 0 : L.tgt[i * cap + bq]);
        p = max(bq, 0);
      }
    }
    __syncthreads();
    // publish the W1 rows of each step's previous token (step 0: the anchor)
    for (int x = writer ? tid : fs * half; x < fs * half; x += 256) {
      const int i = x / half, k2 = x - i * half;
      const uint16_t* src = L.w1c + (size_t)((i == 0) ? 0 : 1 + (i - 1) * cap + sel[i - 1]) * r;
      st_u(a.ws.rows + (size_t)(b * N + i) * half + k2, reinterpret_cast<const uint32_t*>(src)[k2]);
    }
  } else {
    // too many survivors to stage or tabulate: lanes take recorded entries and
    // read weight rows from global memory, one step at a time
    if (wave == 0) {
      int prev = req_anchor(L, b);
      for (int i = 0; i < fs; ++i) {
        const uint16_t* e1 = a.w1 + (size_t)min(max(prev, 0), a.V - 1) * r;
        float bk = -INFINITY;
        int bt = 0x7FFFFFFF;
        for (int q = lane; q < per; q += 64) {
          const uint64_t s = ld_u64(recb + (size_t)i * per + q);
          const float k = slot_key(s);
          if (!(k + cb * rec_w2n(s) + kKeySlack >= L.thr[i])) continue;
          const int j = (q / kTop) * sw + rec_jl(s);
          const float full = k + c * dot_bf16(e1, a.w2 + (size_t)j * r, r);
          const int t = target_of(a.d2t, j);
          if (key_beats(full, t, bk, bt)) {
            bk = full;
            bt = t;
          }
        }
        wave_argmax(bk, bt);
        prev = (bt != 0x7FFFFFFF) ? bt : 0;
        if (lane == 0) {
          if (writer) st_i(a.draft_tokens + (size_t)b * N + i, prev);
          sel[i] = prev;
        }
      }
    }
    __syncthreads();
    if (writer)
      for (int i = 0; i < fs; ++i) publish_row_from(a, b, i, (i == 0) ? req_anchor(L, b) : sel[i - 1], tid, 256);
  }
  if (writer && tid == 0) st_i(a.ws.fstep + b, fs);
  __syncthreads();
}

// ------------------------------------------------------------------------ per-step pass
// this slice's partial argmax of step s for every request resolved here (prevs known)
__device__ __forceinline__ void step_partial(const FewArgs& a, const Lds& L, const Slice& sl, int vwg, int G, int s,
                                             const int* fstl, const bf16x8 (&efrag)[kMaxKSteps]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int r = a.r, ksteps = (r + 31) / 32, row_bytes = 2 * r + 16, B = a.B, N = a.N;
  MarkovPartial* redp = reinterpret_cast<MarkovPartial*>(L.redf);
  float bkey[4];
  int btok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bkey[i] = -INFINITY;
    btok[i] = 0x7FFFFFFF;
  }
  for (int cidx = wave; cidx < sl.nch; cidx += 4) {
    floatx4 acc[4];
    chunk_bias_any(L.w2s + (size_t)cidx * kChunk * row_bytes, row_bytes, ksteps, r, efrag, n, g, acc);
    const int jb = sl.vbase + cidx * kChunk + 4 * n;
    if (jb >= a.Vd) continue;
    int tgt[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) tgt[f] = target_of(a.d2t, jb + f);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int b = 4 * g + i;
      if (b >= B || fstl[b] > s) continue;
      const float T = req_temperature(L, b);
      float4 v = *reinterpret_cast<const float4*>(a.logits + ((size_t)b * N + s) * a.Vd + jb);
      v.x += acc[0][i];
      v.y += acc[1][i];
      v.z += acc[2][i];
      v.w += acc[3][i];
      float key[4];
      keys4(v, T > 0.0f, temp_scale(T), jb, s, req_id(L, b), a.key0, a.key1, key);
#pragma unroll
      for (int f = 0; f < 4; ++f)
        if (key_beats(key[f], tgt[f], bkey[i], btok[i])) {
          bkey[i] = key[f];
          btok[i] = tgt[f];
        }
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    row_argmax(bkey[i], btok[i]);
    if (n == 0) redp[wave * 16 + 4 * g + i] = MarkovPartial{bkey[i], btok[i], -INFINITY, 0.0f};
  }
  __syncthreads();
  if (tid < B) {
    MarkovPartial m = redp[tid];
    for (int w = 1; w < 4; ++w) {
      const MarkovPartial q = redp[w * 16 + tid];
      if (key_beats(q.key, q.tok, m.key, m.tok)) {
        m.key = q.key;
        m.tok = q.tok;
      }
    }
    store_partial(a.ws.partF + (size_t)(s & 1) * B * G + (size_t)tid * G + vwg, m);
  }
  __syncthreads();
}

// previous token of step s for every request the per-step pass resolves at s; the
// writer also stores the token of step s-1 and publishes the row of step s
__device__ __forceinline__ void step_prevs(const FewArgs& a, int G, int s, const int* fstl, int* prevs, bool writer) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, N = a.N;
  for (int b = wave; b < a.B; b += 4) {
    if (fstl[b] > s) continue;
    int p;
    if (s == fstl[b]) {
      p = (s == 0) ? a.anchor[b] : ld_i(a.draft_tokens + (size_t)b * N + s - 1);
    } else {
      const MarkovPartial q = wave_merge(a.ws.partF + (size_t)((s - 1) & 1) * a.B * G + (size_t)b * G, G, lane);
      p = (q.tok == 0x7FFFFFFF) ? 0 : q.tok;
      if (writer && lane == 0) st_i(a.draft_tokens + (size_t)b * N + s - 1, p);
    }
    if (lane == 0) prevs[b] = p;
    if (writer && s < N) publish_row_from(a, b, s, p, lane, 64);
  }
  __syncthreads();
}

// ------------------------------------------------------------------------ phase D
__device__ __forceinline__ void phase_d(const FewArgs& a, const Lds& L, const Slice& sl, int vwg, int G,
                                        float4 (&pre)[kMaxCPW][4], bool rows_in_lds) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int r = a.r, ksteps = (r + 31) / 32, row_bytes = 2 * r + 16, B = a.B, N = a.N, half = r / 2;
  const int tpr = (N + 15) / 16, ntiles = B * tpr;
  MarkovPartial* redp = reinterpret_cast<MarkovPartial*>(L.redf);
  for (int t = 0; t < ntiles; ++t) {
    float4 cur[kMaxCPW][4];
#pragma unroll
    for (int u = 0; u < kMaxCPW; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) cur[u][i] = pre[u][i];
    if (t + 1 < ntiles) load_tile(pre, a.logits, t + 1, tpr, B, N, a.Vd, sl.vbase, wave, n, g);
    const int b = t / tpr, st0 = (t - b * tpr) * 16;
    const float c = temp_scale(req_temperature(L, b));
    // MFMA rows = steps st0 .. st0+15 of request b; lane row n is step st0 + n
    const int sn = st0 + n;
    bf16x8 efrag[kMaxKSteps];
    if (rows_in_lds)
      load_efrag_lds(L, min(sn, N - 1), sn < N, r, ksteps, g, a.cap, efrag);
    else
      load_efrag_published(a.ws.rows + (size_t)(b * N + min(sn, N - 1)) * half, sn < N, r, ksteps, g, efrag);
    float bm[4], bs[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bm[i] = -INFINITY;
      bs[i] = 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kMaxCPW; ++u) {
      const int cidx = wave + 4 * u;
      if (cidx >= sl.nch) break;  // uniform per wave
      floatx4 acc[4];
      chunk_bias_any(L.w2s + (size_t)cidx * kChunk * row_bytes, row_bytes, ksteps, r, efrag, n, g, acc);
      const int jb = sl.vbase + cidx * kChunk + 4 * n;
      if (jb >= a.Vd) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int step = st0 + 4 * g + i;
        if (step >= N) continue;
        float4 v = cur[u][i];
        v.x += acc[0][i];
        v.y += acc[1][i];
        v.z += acc[2][i];
        v.w += acc[3][i];
        *reinterpret_cast<float4*>(a.logits + ((size_t)b * N + step) * a.Vd + jb) = v;
        const float y[4] = {v.x * c, v.y * c, v.z * c, v.w * c};
        const float mn = fmaxf(bm[i], fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3])));
        float sacc = bs[i] * __builtin_amdgcn_exp2f(bm[i] - mn);
#pragma unroll
        for (int f = 0; f < 4; ++f) sacc += __builtin_amdgcn_exp2f(y[f] - mn);
        bs[i] = sacc;
        bm[i] = mn;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      row_lse_merge(bm[i], bs[i]);
      if (n == 0) redp[wave * 16 + 4 * g + i] = MarkovPartial{0.0f, 0, bm[i], bs[i]};
    }
    __syncthreads();
    if (tid < 16 && st0 + tid < N) {
      MarkovPartial m = redp[tid];
      for (int w = 1; w < 4; ++w) lse2_merge(m.m, m.s, redp[w * 16 + tid].m, redp[w * 16 + tid].s);
      store_partial(a.ws.partD + (size_t)(b * N + st0 + tid) * G + vwg, m);
    }
    __syncthreads();
  }
}

// Arrival at grid barrier `round` (1, 2, ...).  Every thread first waits for its
// own stores, so that whatever this workgroup published before the barrier is in
// memory when the barrier counts it; the last workgroup of each group to arrive
// counts the group.
__device__ __forceinline__ void barrier_arrive(unsigned* ctr, unsigned round, int G) {
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int grp = (int)blockIdx.x % kGroups;
    const unsigned old = __hip_atomic_fetch_add(ctr_group(ctr, 0, grp), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1u == round * group_size(G, grp))
      __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// thread 0: whether every group has arrived at barrier `round`
__device__ __forceinline__ bool barrier_done(unsigned* ctr, unsigned round, int G) {
  return ld_u(ctr) >= round * group_count(G);
}

// The wait is bounded (about 0.1 s) so that a broken launch can never hang the device.
// Returns false (the whole workgroup) when the bound ran out before every workgroup
// arrived; the sticky status word then records it, and the caller consumes nothing
// that other workgroups were to publish before this barrier.  (force_give_up: the
// test mode reports a give-up after a barrier that did complete.)
__device__ __forceinline__ bool grid_barrier(const FewArgs& a, unsigned round, int G, int* misc) {
  barrier_arrive(a.ws.ctr, round, G);
  if (threadIdx.x == 0) {
    bool done = false;
    for (int spin = 0; spin < (1 << 22); ++spin) {
      if ((done = barrier_done(a.ws.ctr, round, G))) break;
      __builtin_amdgcn_s_sleep(1);
    }
    if (!done || a.force_give_up) __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    misc[kMsBarrierOk] = done && !a.force_give_up;
  }
  __syncthreads();
  return misc[kMsBarrierOk] != 0;
}

// Role of this workgroup at the first barrier: 0 return at once, 1 go on with its
// slice, 2 run every slice alone.  The first workgroup to start (`first`) waits
// for every group within a window; if the window ends first, it closes the
// barrier (a flag bit in the group count) unless the count has just completed,
// and runs alone.  Every workgroup goes on once the count is complete and returns
// once the barrier is closed, so no workgroup ever waits for one that has not
// started.  With `force_solo` the first workgroup closes the barrier before it
// arrives itself, so the count can never complete.
constexpr unsigned kClosed = 0x80000000u;
__device__ __forceinline__ void close_first_barrier(unsigned* ctr) {
  __hip_atomic_fetch_or(ctr, kClosed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int first_barrier_role(const FewArgs& a, int G, bool first, int* misc) {
  unsigned* ctr = a.ws.ctr;
  if (threadIdx.x == 0) {
    const unsigned target = group_count(G);
    int role = 0;
    if (first && a.force_solo) {
      role = 2;
    } else if (first) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      for (;;) {
        if (ld_u(ctr) >= target) {
          role = 1;
          break;
        }
        if (__builtin_amdgcn_s_memrealtime() - t0 > kArriveTicks) {
          const unsigned old = __hip_atomic_fetch_or(ctr, kClosed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          role = (old >= target) ? 1 : 2;  // (old has no flag: only this workgroup sets it)
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    } else {
      // the first workgroup settles it within its window; the bound only guards a broken
      // launch, and running out of it is recorded in the sticky status word
      bool settled = false;
      for (int spin = 0; spin < (1 << 22); ++spin) {
        const unsigned v = ld_u(ctr);
        if (v & kClosed) {
          settled = true;
          break;
        }
        if (v >= target) {
          role = 1;
          settled = true;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (!settled) __hip_atomic_fetch_or(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    misc[kMsRole] = role;
  }
  __syncthreads();
  return misc[kMsRole];
}

// Clears the counter set (the whole workgroup; uniform `last`).  Called only by the
// last workgroup to use the counters, once every other workgroup's counter
// operations are done.
__device__ __forceinline__ void clear_counters(unsigned* ctr, bool last) {
  if (last)
    for (int q = threadIdx.x; q < kCtrWords; q += blockDim.x) st_u(ctr + q, 0u);
}

// Solo mode: every workgroup counts its departure once its counter operations are
// done; the last of all gridDim.x workgroups clears the counters (a workgroup that
// starts late still departs, so the count always completes).
__device__ __forceinline__ void depart(unsigned* ctr, int* misc) {
  if (threadIdx.x == 0) {
    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // this workgroup's counter atomics are done
    misc[kMsLastOut] =
        __hip_atomic_fetch_add(ctr + 3, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u == gridDim.x;
  }
  __syncthreads();
  clear_counters(ctr, misc[kMsLastOut] != 0);
}

// Whether this workgroup is the last one to finish (the counts of every group).
__device__ __forceinline__ bool last_to_finish(unsigned* ctr, int G, int* misc) {
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int grp = (int)blockIdx.x % kGroups;
    int last = 0;
    const unsigned old = __hip_atomic_fetch_add(ctr_group(ctr, 1, grp), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1u == group_size(G, grp))
      last = __hip_atomic_fetch_add(ctr + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u == group_count(G);
    misc[kMsTicket] = last;
  }
  __syncthreads();
  return misc[kMsTicket] != 0;
}

__global__ __launch_bounds__(256) void markov_few(FewArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int G = gridDim.x, wg = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int r = a.r, ksteps = (r + 31) / 32, B = a.B, N = a.N, rows = B * N;
  const int S = a.CH * kChunk, row_bytes = 2 * r + 16;
  Lds L;
  L.w2s = lds;
  L.thr = reinterpret_cast<float*>(lds + (size_t)S * row_bytes);
  L.redf = L.thr + 64;
  L.misc = reinterpret_cast<int*>(L.redf + 256);
  L.w2n = reinterpret_cast<float*>(L.misc + kMisc);
  L.n2s = L.w2n + kMaxSlice;
  char* creg = reinterpret_cast<char*>(L.n2s + kMaxSlices);
  const CRegion cr = cregion(N, a.cap, r);
  L.cands = reinterpret_cast<uint64_t*>(creg + cr.cands);
  L.w2c = reinterpret_cast<uint16_t*>(creg + cr.w2c);
  L.w1c = reinterpret_cast<uint16_t*>(creg + cr.w1c);
  L.tgt = reinterpret_cast<int*>(creg + cr.tgt);
  L.fk = reinterpret_cast<float*>(creg + cr.fk);

  // per-request parameters, kept in LDS for the later phases (unguarded loads from a
  // clamped index, stored once phase B no longer waits on anything)
  const int pq = min(tid, B - 1);
  const float p_t = a.temperature[pq];
  const uint32_t p_rid = a.request_id[pq];
  const int p_anc = a.anchor[pq];
  // arrival order (the first to take a number decides the mode at the first barrier)
  unsigned arrival = phase_ab(a, L, wg, G, true);
  asm volatile("" : "+v"(arrival));  // (first read here, after phase B)
  if (tid < B) {
    reinterpret_cast<float*>(L.misc)[kMsT + tid] = p_t;
    reinterpret_cast<uint32_t*>(L.misc)[kMsRid + tid] = p_rid;
    L.misc[kMsAnc + tid] = p_anc;
  }
  if (tid == 0 && arrival == 0u && a.force_solo) close_first_barrier(a.ws.ctr);
  barrier_arrive(a.ws.ctr, 1u, G);
  float4 pre[kMaxCPW][4];  // base logits of the first phase-D tile, read while the chain runs
  load_tile(pre, a.logits, 0, (N + 15) / 16, B, N, a.Vd, slice_of(a, wg).vbase, wave, n, g);
  const int role = first_barrier_role(a, G, arrival == 0u, L.misc);
  if (__builtin_expect(role == 0, 0)) {  // (only in solo mode)
    depart(a.ws.ctr, L.misc);
    return;
  }
  const bool solo = role == 2;
  const int v0 = solo ? 0 : wg, v1 = solo ? G : wg + 1;  // slices this workgroup runs
  unsigned round = 1;
  if (__builtin_expect(solo, 0))
    for (int vwg = 0; vwg < G; ++vwg)
      if (vwg != wg) phase_ab(a, L, vwg, G, false);

  // With one request every workgroup runs phase C itself (workgroup 0 stores the
  // outputs): when its staged chain covers every step, phase D takes the W1 rows
  // from this workgroup's LDS, and neither the second barrier nor the published
  // rows are needed.  (Every workgroup reaches the same decision: the same records,
  // the same arithmetic.)
  const bool redundant = !solo && B == 1;
  if (redundant)
    phase_c(a, L, 0, G, wg == 0);
  else
    for (int b = solo ? 0 : wg; b < B; b += solo ? 1 : G) phase_c(a, L, b, G, true);
  const bool rows_in_lds = redundant && L.misc[kMsFs] == N && L.misc[kMsFit] != 0;
  // A grid barrier whose bounded wait gave up leaves this workgroup "broken": it reads
  // nothing more that other workgroups publish and goes straight to the final count
  // (every later barrier of the others then gives up too), and the last workgroup
  // replaces the outputs by -1 tokens and NaN log Z.
  bool broken = false;
  if (!solo && !rows_in_lds) broken = !grid_barrier(a, ++round, G, L.misc);

  // per-step pass from the first incomplete step of any request
  int* prevs = L.misc + kMsPrev;
  int* fstl = L.misc + kMsFst;
  if (tid < B) fstl[tid] = (rows_in_lds || broken) ? N : ld_i(a.ws.fstep + tid);
  __syncthreads();
  int fmin = N;
  for (int b = 0; b < B; ++b) fmin = min(fmin, fstl[b]);
  const bool writer = solo || wg == 0;
  if (__builtin_expect(fmin < N, 0)) {
    for (int s = fmin; s < N && !broken; ++s) {
      step_prevs(a, G, s, fstl, prevs, writer);
      bf16x8 efrag[kMaxKSteps];
      load_efrag(a.w1, (n < B) ? prevs[n] : 0, n < B && fstl[n] <= s, a.V, r, ksteps, g, efrag);
      for (int vwg = v0; vwg < v1; ++vwg) {
        const Slice sl = slice_of(a, vwg);
        if (solo) load_slice<false>(a, L, sl);
        step_partial(a, L, sl, vwg, G, s, fstl, efrag);
      }
      if (!solo) broken = !grid_barrier(a, ++round, G, L.misc);
    }
    if (!broken) {
      // tokens of the last step (s == N: nothing is published)
      step_prevs(a, G, N, fstl, prevs, writer);
      if (!solo) broken = !grid_barrier(a, ++round, G, L.misc);
    }
  }

  for (int vwg = v0; vwg < v1 && !broken; ++vwg) {
    const Slice sl = slice_of(a, vwg);
    if (__builtin_expect(solo, 0)) {
      load_slice<false>(a, L, sl);
      load_tile(pre, a.logits, 0, (N + 15) / 16, B, N, a.Vd, sl.vbase, wave, n, g);
    }
    phase_d(a, L, sl, vwg, G, pre, rows_in_lds);
  }

  // log Z: the last workgroup to finish its partials merges them.  In normal mode
  // every other workgroup's last counter operation has been counted by then, so
  // that workgroup clears the counters; in solo mode the last to depart does.
  const bool merge = solo || last_to_finish(a.ws.ctr, G, L.misc);
  if (solo)
    depart(a.ws.ctr, L.misc);
  else
    clear_counters(a.ws.ctr, merge);
  if (merge) {
    // a grid barrier of this launch (or of an earlier one not yet checked) gave up:
    // no output is trustworthy, so none is left looking valid
    if (tid == 0) L.misc[kMsBarrierOk] = ld_u(a.status) == 0u;
    __syncthreads();
    if (L.misc[kMsBarrierOk]) {
      for (int row = wave; row < rows; row += 4) {
        const MarkovPartial q = wave_merge(a.ws.partD + (size_t)row * G, G, lane);
        if (lane == 0) a.log_z[row] = log_z_of(q, req_temperature(L, row / N));
      }
      // confidence head of every position, now that the chains are final: one wave per
      // row, w_e . W1[previous token] over 16-byte pieces
      if (a.conf.out != nullptr)
        for (int row = wave; row < rows; row += 4) {
          const int b = row / N, k = row - b * N;
          const int prev = (k == 0) ? req_anchor(L, b) : ld_i(a.draft_tokens + row - 1);
          const uint4* er = reinterpret_cast<const uint4*>(a.w1 + (size_t)min(max(prev, 0), a.V - 1) * r);
          const uint4* we = reinterpret_cast<const uint4*>(a.conf.we);
          float d = 0.0f;
          for (int p = lane; p < r / 8; p += 64) d += dot_bf16x8(er[p], we[p]);
          d = group_sum(d, 64);
          if (lane == 0) a.conf.out[row] = conf_prob(a.conf.hdot[row], d, a.conf.bias, a.conf.tau[k]);
        }
    } else {
      for (int row = tid; row < rows; row += blockDim.x) {
        st_i(a.draft_tokens + row, -1);
        a.log_z[row] = __builtin_nanf("");
        if (a.conf.out != nullptr) a.conf.out[row] = __builtin_nanf("");
      }
    }
  }
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

// test hooks (dspark_markov_test_mode): 1 every slice in one workgroup, 2 every grid
// barrier reports a give-up after it completes
std::atomic<int> g_markov_test_mode{0};

FewPlan plan_markov_few(int B, int N, int Vd, int r, int cus) {
  FewPlan p{};
  const int chunks = (Vd + kChunk - 1) / kChunk;
  const int grid = std::min(std::min(cus > 0 ? cus : 256, kMaxSlices), chunks);
  const int ch = (chunks + grid - 1) / grid;
  const size_t slice = (size_t)ch * kChunk * (2 * r + 16);
  const size_t budget = 160 * 1024;
  p.grid = (chunks + ch - 1) / ch;
  p.ch = ch;
  const long room = (long)budget - (long)slice - kFixedScratch;
  int cap = 0;
  if (room > 0 && N > 0) {
    cap = (int)std::max<long>(0, (room - 2 * r - 64 - 4L * kPairs) / ((long)N * (8 + 4 * r + 4)));
    while (cap > 0 && (long)cregion(N, cap, r).bytes > room) --cap;
  }
  p.cap = std::min(cap, 64);
  p.lds = slice + kFixedScratch + cregion(N, p.cap, r).bytes;
  p.use = B <= 16 && B * N <= kMaxRows && N <= 64 && slice <= 120 * 1024 && p.cap >= 2 &&
          ch * kChunk <= kMaxSlice && p.grid <= kMaxSlices;
  // workspace layout, sized for any grid up to gmax workgroups so that it never
  // depends on the device
  p.gmax = std::min(chunks, kMaxSlices);
  p.use = p.use && p.grid <= p.gmax;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t rowsN = (size_t)B * N, G = (size_t)p.gmax;
  p.off_norms = take(G * sizeof(float));
  p.off_n1 = take((size_t)B * G * sizeof(float));
  p.off_rec = take(rowsN * G * kTop * sizeof(uint64_t));
  p.off_fstep = take((size_t)B * sizeof(int));
  p.off_partF = take(2 * (size_t)B * G * sizeof(MarkovPartial));
  p.off_partD = take(rowsN * G * sizeof(MarkovPartial));
  p.off_rows = take(rowsN * (size_t)r * 2);
  p.bytes = (B <= 16) ? off : 0;
  return p;
}

hipError_t launch_markov_few(const FewPlan& p, float* logits, const uint16_t* w1, const uint16_t* w2,
                             const int64_t* d2t, const int32_t* anchor, const float* temperature,
                             const uint32_t* request_id, uint64_t seed, int32_t* draft_tokens, float* log_z, int B,
                             int N, int V, int Vd, int r, void* workspace, const ConfArgs& conf, hipStream_t stream) {
  static bool attr_set[64] = {false};
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev >= 0 && dev < 64 && !attr_set[dev]) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(markov_few),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set[dev] = true;
  }
  char* w = static_cast<char*>(workspace);
  FewArgs a;
  a.logits = logits;
  a.w1 = w1;
  a.w2 = w2;
  a.d2t = d2t;
  a.anchor = anchor;
  a.temperature = temperature;
  a.request_id = request_id;
  a.draft_tokens = draft_tokens;
  a.log_z = log_z;
  a.conf = conf;
  a.ws.norms = reinterpret_cast<float*>(w + p.off_norms);
  a.ws.n1 = reinterpret_cast<float*>(w + p.off_n1);
  a.ws.rec = reinterpret_cast<uint64_t*>(w + p.off_rec);
  a.ws.fstep = reinterpret_cast<int*>(w + p.off_fstep);
  a.ws.partF = reinterpret_cast<MarkovPartial*>(w + p.off_partF);
  a.ws.partD = reinterpret_cast<MarkovPartial*>(w + p.off_partD);
  a.ws.rows = reinterpret_cast<uint32_t*>(w + p.off_rows);
  // this launch's counter set: the next of the library's sets on this device
  static std::atomic<unsigned*> ctr_base[64];
  static std::atomic<unsigned> next_set[64];
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  unsigned* base = ctr_base[dev].load(std::memory_order_relaxed);
  if (!base) {  // (concurrent first calls store the same address)
    void* sym = nullptr;
    const hipError_t e = hipGetSymbolAddress(&sym, HIP_SYMBOL(g_few_counters));
    if (e != hipSuccess) return e;
    base = static_cast<unsigned*>(sym);
    ctr_base[dev].store(base, std::memory_order_relaxed);
  }
  a.ws.ctr = base + (size_t)(next_set[dev].fetch_add(1u, std::memory_order_relaxed) % kCtrSets) * kCtrWords;
  static std::atomic<unsigned*> status_of[64];
  unsigned* status = status_of[dev].load(std::memory_order_relaxed);
  if (!status) {
    void* sym = nullptr;
    const hipError_t e = hipGetSymbolAddress(&sym, HIP_SYMBOL(g_few_status));
    if (e != hipSuccess) return e;
    status = static_cast<unsigned*>(sym);
    status_of[dev].store(status, std::memory_order_relaxed);
  }
  a.status = status;
  a.key0 = (uint32_t)(seed & 0xFFFFFFFFu);
  a.key1 = (uint32_t)(seed >> 32);
  a.B = B;
  a.N = N;
  a.V = V;
  a.Vd = Vd;
  a.r = r;
  a.CH = p.ch;
  a.cap = p.cap;
  const int mode = g_markov_test_mode.load(std::memory_order_relaxed);
  a.force_solo = mode == 1;
  a.force_give_up = mode == 2;
  hipLaunchKernelGGL(markov_few, dim3(p.grid), dim3(256), p.lds, stream, a);
  return hipGetLastError();
}

void set_markov_test_mode(int mode) { g_markov_test_mode.store(mode, std::memory_order_relaxed); }

hipError_t markov_check(hipStream_t stream, bool* gave_up) {
  *gave_up = false;
  hipError_t e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return e;
  void* sym = nullptr;
  if ((e = hipGetSymbolAddress(&sym, HIP_SYMBOL(g_few_status))) != hipSuccess) return e;
  unsigned v = 0;
  if ((e = hipMemcpy(&v, sym, sizeof(v), hipMemcpyDeviceToHost)) != hipSuccess) return e;
  if (v == 0u) return hipSuccess;
  *gave_up = true;
  // a launch that gave up may have left its counter set uncleared: reset every set
  void* ctr = nullptr;
  if ((e = hipGetSymbolAddress(&ctr, HIP_SYMBOL(g_few_counters))) != hipSuccess) return e;
  if ((e = hipMemset(ctr, 0, sizeof(unsigned) * kCtrSets * kCtrWords)) != hipSuccess) return e;
  if ((e = hipMemset(sym, 0, sizeof(unsigned))) != hipSuccess) return e;
  return hipDeviceSynchronize();
}

}  // namespace dspark
