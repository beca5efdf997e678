// Stage 3: lossless rejection-sampling verification.
//
// For request b with verify length L and drafted target ids x_k: accept x_k iff
// u_k * p_d(x_k) < p_t(x_k) (double products of float32 values: exact), stop at
// the first rejection k and resample from max(0, p_t - p_d) there, or, with all
// L accepted, draw a bonus token from target row L.  Both draws are exponential
// races: argmax_v r_v / E_v with E_v = -plog2(u_v), compared exactly.  On request
// the per-position acceptance probability alpha_k = sum_v min(p_t, p_d) is also
// produced for k < L.
//
// Kernels:
//   rowstats   logits mode only.  Row statistics of target rows k <= L: base-2
//              log-sum-exp of l / T (T > 0) or the argmax (T == 0), per
//              (row, chunk) partial.  Above kFusedMaxB requests without alpha the
//              rows are lazy: rows 0-1 first, the others only for requests the
//              acceptance on those rows leaves undecided (two launches each).
//   accept     one workgroup per request: merges every row's partials at once,
//              tests all L positions in parallel (one lane each) and takes the
//              first rejection; writes the accepted prefix, the merged row
//              statistics and a sampling job.
//   replay     (kept base logits) the first-rejection row rebuilt in place by the
//              Markov step kernel, before the sampling pass reads it.
//   sample     (request, row, chunk) workgroups stream the job row: the target
//              row and, for a residual, the draft row gathered through the inverse
//              map; per-chunk race winners for the residual and for its fallback
//              (p_t itself, used only if the residual is zero everywhere).  With
//              alpha requested, rows k < L are streamed too for their partial sums.
//              The last workgroup of a request (a ticket counter the accept kernel
//              cleared) merges the partials and writes y and alpha.
#include <float.h>
#include <math.h>

#include <algorithm>
#include <atomic>

#include "dspark.h"
#include "device.hpp"
#include "kernels.hpp"

namespace dspark {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaitVm0 = 0x0F70;  // s_waitcnt vmcnt(0) (gfx9 encoding)

struct RowStat {
  float m, s;     // base-2 log-sum-exp state of y = l * log2(e) / T
  float amax;     // argmax value (T == 0 rows)
  int aidx;       // argmax index (smallest on ties)
};

enum { kJobDone = 0, kJobResid = 1, kJobBonus = 2 };

struct Job {
  int mode;       // kJobDone / kJobResid / kJobBonus
  int row;        // position a of the sampling row
  int L;          // verify length
  int parts;      // sampling workgroups of the request (ticket target)
  int hot;        // probabilities are not point masses (T > 0 or probability input)
  int pad[3];
};

struct RacePartial {
  float r, E;
  int v;
  float fr, fE;   // fallback race over p_t
  int fv;
  int pad[2];
};

__device__ __forceinline__ bool amax_beats(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

__device__ __forceinline__ void stat_merge(float& m, float& s, float& av, int& ai, float m2, float s2, float av2,
                                           int ai2) {
  lse2_merge(m, s, m2, s2);
  if (amax_beats(av2, ai2, av, ai)) {
    av = av2;
    ai = ai2;
  }
}

template <int kCtrl>
__device__ __forceinline__ void stat_stage(float& m, float& s, float& av, int& ai) {
  stat_merge(m, s, av, ai, dpp_f32<kCtrl>(m), dpp_f32<kCtrl>(s), dpp_f32<kCtrl>(av), (int)dpp_u32<kCtrl>((uint32_t)ai));
}

// merge of (log-sum-exp, argmax) states over the wave (lane 0 holds the result)
__device__ __forceinline__ void wave_stat_merge(float& m, float& s, float& av, int& ai) {
  stat_stage<kDppSwap1>(m, s, av, ai);
  stat_stage<kDppSwap2>(m, s, av, ai);
  stat_stage<kDppMirror8>(m, s, av, ai);
  stat_stage<kDppMirror16>(m, s, av, ai);
  uint32_t a0, a1, b0, b1, c0, c1, d0, d1;
  rows_pair(__float_as_uint(m), a0, a1);
  rows_pair(__float_as_uint(s), b0, b1);
  rows_pair(__float_as_uint(av), c0, c1);
  rows_pair((uint32_t)ai, d0, d1);
  m = __uint_as_float(a0);
  s = __uint_as_float(b0);
  av = __uint_as_float(c0);
  ai = (int)d0;
  stat_merge(m, s, av, ai, __uint_as_float(a1), __uint_as_float(b1), __uint_as_float(c1), (int)d1);
  halves_pair(__float_as_uint(m), a0, a1);
  halves_pair(__float_as_uint(s), b0, b1);
  halves_pair(__float_as_uint(av), c0, c1);
  halves_pair((uint32_t)ai, d0, d1);
  m = __uint_as_float(a0);
  s = __uint_as_float(b0);
  av = __uint_as_float(c0);
  ai = (int)d0;
  stat_merge(m, s, av, ai, __uint_as_float(a1), __uint_as_float(b1), __uint_as_float(c1), (int)d1);
}

// The value as the compiler must materialise it: keeps a clamped, unconditional
// load from being sunk under the branch that decides whether it is used (which
// would serialise a batch of loads).
__device__ __forceinline__ float opaque(float v) {
  asm volatile("" : "+v"(v));
  return v;
}
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ void st_f(float* p, float v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ float ld_f(const float* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ void st_i(int* p, int v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
__device__ __forceinline__ int ld_i(const int* p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }

__device__ __forceinline__ void store_race(RacePartial* p, const RacePartial& v) {
  st_f(&p->r, v.r);
  st_f(&p->E, v.E);
  st_i(&p->v, v.v);
  st_f(&p->fr, v.fr);
  st_f(&p->fE, v.fE);
  st_i(&p->fv, v.fv);
}
__device__ __forceinline__ RacePartial load_race(const RacePartial* p) {
  RacePartial v;
  v.r = ld_f(&p->r);
  v.E = ld_f(&p->E);
  v.v = ld_i(&p->v);
  v.fr = ld_f(&p->fr);
  v.fE = ld_f(&p->fE);
  v.fv = ld_i(&p->fv);
  return v;
}

// ------------------------------------------------------------------ row statistics

// This workgroup's partial statistics of chunk c of target row `row` (request b);
// every thread calls it, thread 0 gets the result.
__device__ __forceinline__ RowStat rowstats_part(const float* __restrict__ target, const float* __restrict__ temperature,
                                                 int row, int b, int c, int V, int chunk) {
  const float T = temperature[b];
  const bool hot = T > 0.0f;
  const float c2 = hot ? (1.0f / T) * kLog2e : 1.0f;
  const float4* r4 = reinterpret_cast<const float4*>(target + (size_t)row * V);
  const int lo4 = c * (chunk / 4), hi4 = min(V, c * chunk + chunk) / 4;
  const int tid = threadIdx.x;
  constexpr int kB = 8;  // float4 loads per thread in flight

  // T > 0: base-2 log-sum-exp with a lazily raised reference m (every y seen is at
  // most m + 64, so no term overflows); T == 0: the argmax, ties to the smaller index.
  float m = -FLT_MAX, thr = -FLT_MAX, s = 0.0f, av = -INFINITY;
  int ai = lo4 * 4 + 4 * tid;  // this thread's first index (a strict argmax over all -inf keeps it)
  for (int i0 = lo4 + tid; i0 < hi4; i0 += 256 * kB) {
    float4 q[kB];
#pragma unroll
    for (int u = 0; u < kB; ++u) q[u] = r4[min(i0 + 256 * u, hi4 - 1)];
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const bool ok = i0 + 256 * u < hi4;
      const float l[4] = {ok ? q[u].x : -INFINITY, ok ? q[u].y : -INFINITY, ok ? q[u].z : -INFINITY,
                          ok ? q[u].w : -INFINITY};
      if (hot) {
        float y[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) y[f] = l[f] * c2;
        const float mx = fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3]));
        const bool grow = mx > thr;
        if (__ballot(grow)) {
          const float sc = __builtin_amdgcn_exp2f(m - mx);
          s = grow ? s * sc : s;
          m = grow ? mx : m;
          thr = grow ? mx + 64.0f : thr;
        }
        s += (__builtin_amdgcn_exp2f(y[0] - m) + __builtin_amdgcn_exp2f(y[1] - m)) +
             (__builtin_amdgcn_exp2f(y[2] - m) + __builtin_amdgcn_exp2f(y[3] - m));
      } else {
        const int v = (i0 + 256 * u) * 4;
#pragma unroll
        for (int f = 0; f < 4; ++f)
          if (l[f] > av) {
            av = l[f];
            ai = v + f;
          }
      }
    }
  }
  wave_stat_merge(m, s, av, ai);
  __shared__ RowStat red[4];
  const int wave = tid >> 6;
  if ((tid & 63) == 0) red[wave] = RowStat{m, s, av, ai};
  __syncthreads();
  RowStat a = red[0];
  if (tid == 0)
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) stat_merge(a.m, a.s, a.amax, a.aidx, red[w].m, red[w].s, red[w].amax, red[w].aidx);
  return a;
}

// Target rows k0 .. k0 + nk - 1 of every request (rows past the request's verify length
// exit at once); with cont set, only the requests whose cont flag is set.
__global__ __launch_bounds__(256) void verify_rowstats(const float* __restrict__ target,
                                                       const int32_t* __restrict__ verify_len,
                                                       const float* __restrict__ temperature,
                                                       RowStat* __restrict__ stats, int B, int N, int V,
                                                       int nchunks, int chunk, int k0, int nk,
                                                       const int32_t* __restrict__ cont) {
  const int rr = blockIdx.x / nchunks, c = blockIdx.x % nchunks;
  const int b = rr / nk, k = k0 + rr % nk;
  const int L = verify_len ? min(max(verify_len[b], 0), N) : N;
  if (k > L || (cont && !cont[b])) return;
  const int row = b * (N + 1) + k;
  const RowStat a = rowstats_part(target, temperature, row, b, c, V, chunk);
  if (threadIdx.x == 0) stats[(size_t)row * nchunks + c] = a;
}

// ------------------------------------------------------------------ acceptance

// The acceptance of request b by one 256-thread workgroup.  kCoherent: the
// partial statistics were written by other workgroups of the same launch (loads
// at device scope).
// Kept base logits (deferred draft rows): p_d of the drafted token at position k is
// win[b, k], and the acceptance pass names the row the sampling pass will read
// (rows[b]: the first rejection, -1 when no draft row is read) and the token before it
// (prev[b]) for the replay that recomputes that row.
struct AcceptDef {
  const float* win = nullptr;
  const int32_t* anchor = nullptr;
  int32_t* rows = nullptr;
  int32_t* prev = nullptr;
};

// Lazy row statistics: the statistics of the first `avail` target rows are computed
// first, and the acceptance runs on them.  A request whose first rejection (or whose
// bonus row L) falls among those rows is decided there.  A request whose first
// min(L, avail) positions are all accepted, with L >= avail, is undecided: cont_out[b] =
// 1 and nothing else is written.  The rest of its rows are computed next, and a second
// acceptance pass (avail = N + 1, cont_in) runs only the undecided requests.
struct AcceptLazy {
  int avail = DSPARK_MAX_N + 1;
  int32_t* cont_out = nullptr;
  const int32_t* cont_in = nullptr;
};

template <bool kCoherent>
__device__ __forceinline__ void accept_body(int b, int input_kind, const float* __restrict__ target,
                                            const float* __restrict__ draft, const float* __restrict__ draft_log_z,
                                            const int32_t* __restrict__ draft_tokens,
                                            const int32_t* __restrict__ inv_map,
                                            const int32_t* __restrict__ verify_len,
                                            const float* __restrict__ temperature,
                                            const uint32_t* __restrict__ request_id, uint32_t key0, uint32_t key1,
                                            const RowStat* __restrict__ stats, float2* __restrict__ rstat,
                                            Job* __restrict__ jobs, unsigned* __restrict__ tickets,
                                            int32_t* __restrict__ accepted, int32_t* __restrict__ out_tokens,
                                            float* __restrict__ accept_prob, int N, int V, int Vd, int nchunks,
                                            int sample_chunks, AcceptDef def, AcceptLazy lz) {
  if (lz.cont_in && !lz.cont_in[b]) return;  // (uniform) decided by the first pass
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = verify_len ? min(max(verify_len[b], 0), N) : N;
  const int tested = min(L, lz.avail);  // positions whose target row has statistics
  const uint32_t req = request_id[b];
  const bool probs = input_kind == DSPARK_INPUT_PROBS;
  const float T = probs ? 1.0f : temperature[b];
  const bool hot = probs || T > 0.0f;
  const float c2 = (!probs && hot) ? (1.0f / T) * kLog2e : 1.0f;

  // The accept test's inputs (wave 3, lane k < L: the drafted id, its draft index,
  // the target and draft values) are requested first; their chain of dependent
  // loads runs while waves 0-2 merge the row statistics.
  int x = 0, xj = -1;
  float lt = 0.0f, ld = 0.0f, ldz = 0.0f;
  if (wave == 3 && L > 0) {
    const int k = min(lane, L - 1);
    x = draft_tokens[(size_t)b * N + k];
    const int xs = (x >= 0 && x < V) ? x : 0;
    xj = inv_map ? inv_map[xs] : xs;
    lt = target[((size_t)b * (N + 1) + k) * V + xs];
    ld = def.win ? def.win[(size_t)b * N + k] : draft[((size_t)b * N + k) * Vd + max(xj, 0)];
    if (!probs) ldz = draft_log_z[(size_t)b * N + k];
  }

  // Merged statistics of target rows k <= L (logits mode): eight lanes of waves
  // 0-2 per row, each merging a strided share of the row's partials (all loads of
  // a share at once), then the eight lanes by DPP.
  __shared__ float row_m[DSPARK_MAX_N + 1], row_s[DSPARK_MAX_N + 1];
  __shared__ int row_amax[DSPARK_MAX_N + 1];
  __shared__ int s_a;
  if (!probs && wave < 3) {
    constexpr int kU = 20;  // partials per lane and round
    const int rows = min(L + 1, lz.avail), sub = tid & 7;
    for (int k0 = 0; k0 < rows; k0 += 24) {
      const int k = k0 + (tid >> 3);
      float m = -INFINITY, s = 0.0f, av = -INFINITY;
      int ai = 0x7FFFFFFF;
      const RowStat* rp = stats + ((size_t)b * (N + 1) + min(k, rows - 1)) * nchunks;
      for (int c0 = sub; c0 < nchunks; c0 += 8 * kU) {
        RowStat q[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const RowStat* e = rp + min(c0 + 8 * u, nchunks - 1);
          if (kCoherent)
            q[u] = RowStat{ld_f(&e->m), ld_f(&e->s), ld_f(&e->amax), ld_i(&e->aidx)};
          else
            q[u] = *e;
        }
#pragma unroll
        for (int u = 0; u < kU; ++u)
          if (c0 + 8 * u < nchunks)
            stat_merge(m, s, av, ai, opaque(q[u].m), opaque(q[u].s), opaque(q[u].amax), opaque(q[u].aidx));
      }
      stat_stage<kDppSwap1>(m, s, av, ai);
      stat_stage<kDppSwap2>(m, s, av, ai);
      stat_stage<kDppMirror8>(m, s, av, ai);
      if (sub == 0 && k < rows) {
        row_m[k] = m;
        row_s[k] = s;
        row_amax[k] = ai;
        rstat[(size_t)b * (N + 1) + k] = make_float2(m, 1.0f / s);
      }
    }
  }
  __syncthreads();

  // All L positions at once, one lane each; the first rejection decides.
  if (wave == 3) {
    bool rej = false;
    float greedy_alpha = 0.0f;
    if (lane < tested) {
      const int k = lane;
      const bool valid = x >= 0 && x < V;  // not a target id: rejected without using anything
      float pt, pd;
      if (probs) {
        pt = lt;
        pd = (xj >= 0) ? ld : 0.0f;
      } else if (hot) {
        pt = __builtin_amdgcn_exp2f(lt * c2 - row_m[k]) / row_s[k];
        pd = (xj >= 0) ? __builtin_amdgcn_exp2f(ld * c2 - ldz * kLog2e) : 0.0f;
      } else {
        pt = (x == row_amax[k]) ? 1.0f : 0.0f;
        pd = 1.0f;
        greedy_alpha = pt;
      }
      const u32x4 w = philox4x32_10(u32x4{0u, (uint32_t)k, req, kTagAccept}, key0, key1);
      const float u = uniform01(w.x);
      rej = !valid || !((double)u * (double)pd < (double)pt);
    }
    const uint64_t mask = __ballot(rej);
    // no rejection among the tested positions: the bonus row L when its statistics are
    // there (L < avail), else undecided (-1)
    const int a = mask ? __builtin_ctzll(mask) : (L < lz.avail ? L : -1);
    if (lane == 0) s_a = a;
    // greedy: alpha is 1 where the draft token is the target argmax (computed here)
    if (accept_prob && !hot && lane < N)
      accept_prob[(size_t)b * N + lane] = (lane < L) ? greedy_alpha : __builtin_nanf("");
  }
  __syncthreads();
  const int a = s_a;
  if (lz.cont_out && tid == 0) lz.cont_out[b] = (a < 0) ? 1 : 0;
  if (a < 0) return;

  // Outputs: accepted prefix, -1 padding, the sampling job.
  for (int k = tid; k <= N; k += 256) {
    int32_t o = -1;
    if (k < a) o = draft_tokens[(size_t)b * N + k];
    out_tokens[(size_t)b * (N + 1) + k] = o;
  }
  if (tid == 0) {
    accepted[b] = a;
    Job jb;
    jb.row = a;
    jb.L = L;
    jb.hot = hot ? 1 : 0;
    jb.mode = (a < L) ? kJobResid : kJobBonus;
    if (!hot) {
      // greedy: the residual and the bonus are both the point mass on the argmax
      out_tokens[(size_t)b * (N + 1) + a] = row_amax[a];
      jb.mode = kJobDone;
    }
    // sampling rows: the job row, and with alpha every row k < L of a non-greedy request
    int rows = (jb.mode == kJobDone) ? 0 : 1;
    if (accept_prob && hot) rows = L + ((a == L) ? 1 : 0);
    jb.parts = rows * sample_chunks;
    jobs[b] = jb;
    if (def.rows) {
      def.rows[b] = (jb.mode == kJobResid) ? a : -1;
      def.prev[b] = (a == 0) ? def.anchor[b] : draft_tokens[(size_t)b * N + a - 1];
    }
    tickets[b] = 0u;
    if (probs) rstat[(size_t)b * (N + 1)] = make_float2(0.0f, 1.0f);
  }
}

__global__ __launch_bounds__(256) void verify_accept(int input_kind, const float* __restrict__ target,
                                                     const float* __restrict__ draft,
                                                     const float* __restrict__ draft_log_z,
                                                     const int32_t* __restrict__ draft_tokens,
                                                     const int32_t* __restrict__ inv_map,
                                                     const int32_t* __restrict__ verify_len,
                                                     const float* __restrict__ temperature,
                                                     const uint32_t* __restrict__ request_id, uint32_t key0,
                                                     uint32_t key1, const RowStat* __restrict__ stats,
                                                     float2* __restrict__ rstat, Job* __restrict__ jobs,
                                                     unsigned* __restrict__ tickets, int32_t* __restrict__ accepted,
                                                     int32_t* __restrict__ out_tokens, float* __restrict__ accept_prob,
                                                     int N, int V, int Vd, int nchunks, int sample_chunks,
                                                     AcceptDef def, AcceptLazy lz) {
  accept_body<false>(blockIdx.x, input_kind, target, draft, draft_log_z, draft_tokens, inv_map, verify_len,
                     temperature, request_id, key0, key1, stats, rstat, jobs, tickets, accepted, out_tokens,
                     accept_prob, N, V, Vd, nchunks, sample_chunks, def, lz);
}

// Statistics and acceptance in one launch (logits input, B <= kFusedMaxB): the
// (row, chunk) workgroups of the statistics pass write their partials, and the
// last of a request's workgroups to finish (tickets taken once every thread's
// stores have completed) runs that request's acceptance.  Same-address atomics are
// served one at a time, so a request's workgroups count in kTGroups groups (local
// index mod kTGroups, counters 128 bytes apart) and the last of each group counts
// the group at the request's top counter.  The tickets are the launch's set of the
// library's per-device sets, zero when the library loads; the last workgroup of a
// request puts that request's counters back to zero (every other workgroup of the
// request has counted by then), so every launch leaves its set as it found it.
constexpr int kFusedMaxB = 16, kTicketSets = 64, kTGroups = 16;
// target rows whose statistics the lazy first pass computes (most requests reject
// within the first two positions)
constexpr int kLazyRows = 2;
constexpr int kTStride = 32;                              // words between counters (128 bytes)
constexpr int kTWordsPerReq = (kTGroups + 1) * kTStride;  // [top, group 0 .. group 15]
__device__ __attribute__((aligned(256))) unsigned g_stat_tickets[kTicketSets * kFusedMaxB * kTWordsPerReq];

__global__ __launch_bounds__(256) void verify_stats_accept(
    const float* __restrict__ target, const float* __restrict__ draft, const float* __restrict__ draft_log_z,
    const int32_t* __restrict__ draft_tokens, const int32_t* __restrict__ inv_map,
    const int32_t* __restrict__ verify_len, const float* __restrict__ temperature,
    const uint32_t* __restrict__ request_id, uint32_t key0, uint32_t key1, RowStat* __restrict__ stats,
    float2* __restrict__ rstat, Job* __restrict__ jobs, unsigned* __restrict__ tickets,
    int32_t* __restrict__ accepted, int32_t* __restrict__ out_tokens, float* __restrict__ accept_prob,
    unsigned* __restrict__ stat_tickets, int N, int V, int Vd, int nchunks, int chunk, int sample_chunks,
    AcceptDef def) {
  const int row = blockIdx.x / nchunks, c = blockIdx.x % nchunks;
  const int b = row / (N + 1), k = row % (N + 1);
  const int L = verify_len ? min(max(verify_len[b], 0), N) : N;
  if (k <= L) {  // (uniform: rows past L are not read, but their workgroups still count)
    const RowStat a = rowstats_part(target, temperature, row, b, c, V, chunk);
    if (threadIdx.x == 0) {
      RowStat* e = stats + (size_t)row * nchunks + c;
      st_f(&e->m, a.m);
      st_f(&e->s, a.s);
      st_f(&e->amax, a.amax);
      st_i(&e->aidx, a.aidx);
    }
  }
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  unsigned* rt = stat_tickets + (size_t)b * kTWordsPerReq;  // [0]: top; [(1 + g) * kTStride]: group g
  const int total = (N + 1) * nchunks, li = k * nchunks + c, grp = li % kTGroups;
  if (threadIdx.x == 0) {
    int last = 0;
    const unsigned old =
        __hip_atomic_fetch_add(rt + (1 + grp) * kTStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (old + 1u == (unsigned)((total - grp + kTGroups - 1) / kTGroups))
      last = __hip_atomic_fetch_add(rt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u ==
             (unsigned)min(total, kTGroups);
    s_last = last;
  }
  __syncthreads();
  if (!s_last) return;
  if (threadIdx.x <= kTGroups)  // (every workgroup of b has counted)
    __hip_atomic_store(rt + threadIdx.x * kTStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  accept_body<true>(b, DSPARK_INPUT_LOGITS, target, draft, draft_log_z, draft_tokens, inv_map, verify_len,
                    temperature, request_id, key0, key1, stats, rstat, jobs, tickets, accepted, out_tokens,
                    accept_prob, N, V, Vd, nchunks, sample_chunks, def, AcceptLazy{});
}

// ------------------------------------------------------------------ sampling rows

__device__ __forceinline__ void race_update(float r, float E, int v, float& br, float& bE, int& bv) {
  if (race_beats(r, E, v, br, bE, bv)) {
    br = r;
    bE = E;
    bv = v;
  }
}


// A pruning threshold for the exponential race: the exact (r, E) of one real candidate,
// the lane best with the largest approximate key r / E in this wave (uniform).  Any
// entry with r * tE < tr * E_lo (E_lo a lower bound of its E) loses strictly to that
// candidate, so it can never be the race's winner.
__device__ __forceinline__ void race_threshold(float br, float bE, float& tr, float& tE) {
  const float key = br * __builtin_amdgcn_rcpf(bE);  // r = 0 ("nobody"): key 0
  const float kmax = wave_max_f32(key);
  const uint64_t hit = __ballot(key == kmax);
  const int src = hit ? (int)__builtin_ctzll(hit) : 0;
  tr = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(br), src));
  tE = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(bE), src));
}

// E = -plog2(u) >= -log2(u) (1 - 2^-20) >= (1 - u) / ln 2 (1 - 2^-20): -ln u >= 1 - u, and
// the portable log2 is within a few ulp of log2.  kEloScale is 1/ln 2 rounded down,
// times (1 - 2^-16); kPrune absorbs the rounding of the two products of the test.
constexpr float kEloScale = 1.4426949f * (1.0f - 0x1p-16f);
constexpr float kPrune = 1.0f - 0x1p-20f;

__global__ __launch_bounds__(256) void verify_sample(int input_kind, const float* __restrict__ target,
                                                     const float* __restrict__ draft,
                                                     const float* __restrict__ draft_log_z,
                                                     const int32_t* __restrict__ inv_map,
                                                     const float* __restrict__ temperature,
                                                     const uint32_t* __restrict__ request_id, uint32_t key0,
                                                     uint32_t key1, const Job* __restrict__ jobs,
                                                     const float2* __restrict__ rstat, RacePartial* __restrict__ race,
                                                     float* __restrict__ apart, unsigned* __restrict__ tickets,
                                                     const int32_t* __restrict__ accepted,
                                                     int32_t* __restrict__ out_tokens, float* __restrict__ accept_prob,
                                                     int B, int N, int V, int Vd, int R, int nchunks, int chunk) {
  const int b = blockIdx.x / (R * nchunks), rr = (blockIdx.x / nchunks) % R, c = blockIdx.x % nchunks;
  const Job jb = jobs[b];
  const bool alpha = accept_prob != nullptr && jb.hot;
  const int k = (R > 1) ? rr : jb.row;
  const bool do_race = jb.mode != kJobDone && k == jb.row;
  const bool do_alpha = alpha && k < jb.L;
  if (!do_race && !do_alpha) return;  // (exactly jb.parts workgroups of the request pass here)
  const int tid = threadIdx.x, wave = tid >> 6;
  const bool probs = input_kind == DSPARK_INPUT_PROBS;
  const bool need_draft = do_alpha || jb.mode == kJobResid;
  const uint32_t req = request_id[b];
  const uint32_t tag = (jb.mode == kJobResid) ? kTagResid : kTagBonus;
  const float c2 = probs ? 1.0f : (1.0f / temperature[b]) * kLog2e;
  const float dlz2 = (!probs && need_draft && k < N) ? draft_log_z[(size_t)b * N + k] * kLog2e : 0.0f;
  const float2 st = rstat[(size_t)b * (N + 1) + (probs ? 0 : k)];
  const float* trow = target + ((size_t)b * (N + 1) + k) * V;
  const float* drow = draft + ((size_t)b * N + min(k, N - 1)) * Vd;
  const float4* t4 = reinterpret_cast<const float4*>(trow);
  const int lo4 = c * (chunk / 4), hi4 = min(V, c * chunk + chunk) / 4;
  constexpr int kB = 4;  // float4 of the target row per thread in flight

  // Race candidates start as "nobody": r = 0 with E = 1 at index INT_MAX loses
  // to everything with r > 0, and index order decides among r = 0.
  float br = 0.0f, bE = 1.0f, fr = 0.0f, fE = 1.0f, asum = 0.0f;
  int bv = 0x7FFFFFFF, fv = 0x7FFFFFFF;
  float tr = 0.0f, tE = 1.0f, tfr = 0.0f, tfE = 1.0f;  // wave thresholds (nobody: prunes nothing)
  for (int i0 = lo4 + tid; i0 < hi4; i0 += 256 * kB) {
    // every load of the batch first (clamped indices), then the arithmetic
    float4 q[kB];
    float dv[kB][4];
    int jv[kB][4];
    unsigned dmask = 0xFFFFu;  // bit 4 u + f: target id in the draft vocabulary
    // (one loop per case: a branch inside the batch would split it into blocks and
    // make the loads wait for each other)
    if (!need_draft) {
#pragma unroll
      for (int u = 0; u < kB; ++u) q[u] = t4[min(i0 + 256 * u, hi4 - 1)];
    } else if (inv_map) {
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int i = min(i0 + 256 * u, hi4 - 1);
        q[u] = t4[i];
        const int4 jj = reinterpret_cast<const int4*>(inv_map)[i];
        jv[u][0] = jj.x;
        jv[u][1] = jj.y;
        jv[u][2] = jj.z;
        jv[u][3] = jj.w;
      }
    } else {
#pragma unroll
      for (int u = 0; u < kB; ++u) {
        const int i = min(i0 + 256 * u, hi4 - 1);
        q[u] = t4[i];
        const float4 d = reinterpret_cast<const float4*>(drow)[i];
        dv[u][0] = d.x;
        dv[u][1] = d.y;
        dv[u][2] = d.z;
        dv[u][3] = d.w;
      }
    }
    if (need_draft && inv_map) {  // the gathers of the whole batch, unconditional (clamped)
#pragma unroll
      for (int u = 0; u < kB; ++u)
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          dv[u][f] = drow[max(jv[u][f], 0)];
          if (jv[u][f] < 0) dmask &= ~(1u << (4 * u + f));
        }
    }
#pragma unroll
    for (int u = 0; u < kB; ++u) {
      const int v = (i0 + 256 * u) * 4;
      if (i0 + 256 * u >= hi4) continue;  // (the batch's tail past the chunk)
      float pt[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
      if (!probs) {
#pragma unroll
        for (int f = 0; f < 4; ++f) pt[f] = __builtin_amdgcn_exp2f(pt[f] * c2 - st.x) * st.y;
      }
      float pd[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (need_draft) {
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const float d = dv[u][f];
          pd[f] = !((dmask >> (4 * u + f)) & 1u) ? 0.0f : (probs ? d : __builtin_amdgcn_exp2f(d * c2 - dlz2));
        }
      }
      if (do_alpha) {
#pragma unroll
        for (int f = 0; f < 4; ++f) asum += fminf(pt[f], pd[f]);
      }
      if (do_race) {
        const u32x4 w = philox4x32_10(u32x4{(uint32_t)v >> 2, (uint32_t)k, req, tag}, key0, key1);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const float u01 = uniform01(ws[f]);
          const float elo = (1.0f - u01) * kEloScale;
          const float rr = (jb.mode == kJobResid) ? fmaxf(0.0f, __fsub_rn(pt[f], pd[f])) : pt[f];
          // (a threshold product near the denormal range never prunes)
          const float lim = (tr * elo) * kPrune, limf = (tfr * elo) * kPrune;
          const bool need = !(lim > 0x1p-100f && rr * tE < lim);
          const bool needf = jb.mode == kJobResid && !(limf > 0x1p-100f && pt[f] * tfE < limf);
          if (need || needf) {  // the exact log2 only for entries that can still win
            const float E = -plog2(u01);
            if (need) race_update(rr, E, v + f, br, bE, bv);
            if (needf) race_update(pt[f], E, v + f, fr, fE, fv);
          }
        }
      }
    }
    if (do_race) {  // refresh the thresholds from this wave's bests
      race_threshold(br, bE, tr, tE);
      if (jb.mode == kJobResid) race_threshold(fr, fE, tfr, tfE);
    }
  }
  __shared__ RacePartial red[4];
  __shared__ float ared[4];
  __shared__ unsigned s_ticket;
  if (do_race) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float o_r = __shfl_xor(br, off), o_E = __shfl_xor(bE, off);
      const int o_v = __shfl_xor(bv, off);
      const float o_fr = __shfl_xor(fr, off), o_fE = __shfl_xor(fE, off);
      const int o_fv = __shfl_xor(fv, off);
      race_update(o_r, o_E, o_v, br, bE, bv);
      race_update(o_fr, o_fE, o_fv, fr, fE, fv);
    }
    if ((tid & 63) == 0) red[wave] = RacePartial{br, bE, bv, fr, fE, fv, {0, 0}};
  }
  if (do_alpha) {
    asum = group_sum(asum, 64);
    if ((tid & 63) == 0) ared[wave] = asum;
  }
  __syncthreads();
  const int slot = (b * R + (R > 1 ? k : 0)) * nchunks + c;
  if (tid == 0) {
    if (do_race) {
      RacePartial a = red[0];
      for (int w2 = 1; w2 < 4; ++w2) {
        race_update(red[w2].r, red[w2].E, red[w2].v, a.r, a.E, a.v);
        race_update(red[w2].fr, red[w2].fE, red[w2].fv, a.fr, a.fE, a.fv);
      }
      store_race(race + slot, a);
    }
    if (do_alpha) st_f(apart + slot, (ared[0] + ared[1]) + (ared[2] + ared[3]));
  }
  // the request's last workgroup merges: every thread's stores complete before the
  // barrier, and the ticket is taken after it
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  if (tid == 0) s_ticket = __hip_atomic_fetch_add(tickets + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (s_ticket != (unsigned)jb.parts - 1) return;
  const int lane = tid & 63;
  if (jb.mode != kJobDone && wave == 0) {
    float r0 = 0.0f, E0 = 1.0f, r1 = 0.0f, E1 = 1.0f;
    int v0 = 0x7FFFFFFF, v1 = 0x7FFFFFFF;
    const RacePartial* rp = race + (size_t)(b * R + (R > 1 ? jb.row : 0)) * nchunks;
    for (int cc = lane; cc < nchunks; cc += 64) {
      const RacePartial q = load_race(rp + cc);
      race_update(q.r, q.E, q.v, r0, E0, v0);
      race_update(q.fr, q.fE, q.fv, r1, E1, v1);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float o_r = __shfl_xor(r0, off), o_E = __shfl_xor(E0, off);
      const int o_v = __shfl_xor(v0, off);
      const float o_fr = __shfl_xor(r1, off), o_fE = __shfl_xor(E1, off);
      const int o_fv = __shfl_xor(v1, off);
      race_update(o_r, o_E, o_v, r0, E0, v0);
      race_update(o_fr, o_fE, o_fv, r1, E1, v1);
    }
    // an all-zero residual leaves r == 0 at the winner: fall back to p_t
    if (lane == 0) out_tokens[(size_t)b * (N + 1) + jb.row] = (jb.mode == kJobResid && r0 == 0.0f) ? v1 : v0;
  }
  if (alpha) {
    for (int kk = wave; kk < N; kk += 4) {
      float sum = 0.0f;
      if (kk < jb.L)
        for (int cc = lane; cc < nchunks; cc += 64) sum += ld_f(apart + (size_t)(b * R + kk) * nchunks + cc);
      sum = group_sum(sum, 64);
      if (lane == 0) accept_prob[(size_t)b * N + kk] = (kk < jb.L) ? sum : __builtin_nanf("");
    }
  }
}

int pick_chunks(long rows, int V, long target = 2048) {
  // aim for >= target workgroups, chunks of >= 1024 elements, multiple of 4
  long want = (target + rows - 1) / rows;
  long maxc = (V + 1023) / 1024;
  if (want > maxc) want = maxc;
  if (want < 1) want = 1;
  return (int)want;
}

}  // namespace

VerifyPlan plan_verify(int B, int N, int V) {
  VerifyPlan p{};
  // rows past a request's verify length exit at once, so the live rows alone must
  // fill the chip: chunks of at most 16K entries whatever the row count.  With few
  // rows, about one workgroup per CU (more, smaller chunks only add launch work and
  // partials for the acceptance kernel to merge: 28.0 -> 24.4 us for the whole
  // verify stage at one request of N = 8, V = 151936)
  p.stat_chunks = std::max(pick_chunks((long)B * (N + 1), V, 256), (V + 16383) / 16384);
  p.stat_chunk = ((V + p.stat_chunks - 1) / p.stat_chunks + 3) / 4 * 4;
  p.sample_chunks = pick_chunks(B, V);
  p.sample_chunk = ((V + p.sample_chunks - 1) / p.sample_chunks + 3) / 4 * 4;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t rows = (size_t)B * (N + 1);
  p.stats_bytes = al(rows * p.stat_chunks * sizeof(RowStat));
  p.jobs_bytes = al((size_t)B * sizeof(Job)) + al(rows * sizeof(float2)) + 2 * al((size_t)B * sizeof(unsigned));
  // race and alpha partials for every (request, row, chunk): the rows dimension is
  // used only when alpha is requested, but the size must not depend on the call
  p.race_bytes = al(rows * p.sample_chunks * sizeof(RacePartial)) + al(rows * p.sample_chunks * sizeof(float));
  p.total_bytes = p.stats_bytes + p.jobs_bytes + p.race_bytes;
  return p;
}

namespace {
hipError_t verify_impl(int input_kind, const float* target, const float* draft, const float* draft_log_z,
                       const int32_t* draft_tokens, const int32_t* inv_map, const int32_t* verify_len,
                       const float* temperature, const uint32_t* request_id, uint64_t seed, int32_t* accepted,
                       int32_t* out_tokens, float* accept_prob, int B, int N, int V, int Vd, void* workspace,
                       const DeferredArgs* dfr, hipStream_t stream) {
  const VerifyPlan p = plan_verify(B, N, V);
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t rows = (size_t)B * (N + 1);
  char* ws = static_cast<char*>(workspace);
  RowStat* stats = reinterpret_cast<RowStat*>(ws);
  char* w = ws + p.stats_bytes;
  Job* jobs = reinterpret_cast<Job*>(w);
  w += al((size_t)B * sizeof(Job));
  float2* rstat = reinterpret_cast<float2*>(w);
  w += al(rows * sizeof(float2));
  unsigned* tickets = reinterpret_cast<unsigned*>(w);
  w += al((size_t)B * sizeof(unsigned));
  int32_t* cont = reinterpret_cast<int32_t*>(w);
  w += al((size_t)B * sizeof(int32_t));
  RacePartial* race = reinterpret_cast<RacePartial*>(w);
  w += al(rows * p.sample_chunks * sizeof(RacePartial));
  float* apart = reinterpret_cast<float*>(w);
  AcceptDef def;
  float* spill = nullptr;
  if (dfr) {  // after the plan's bytes: rows [B], prev [B], the replay's spill row
    char* x = ws + p.total_bytes;
    def.win = dfr->win;
    def.anchor = dfr->anchor;
    def.rows = reinterpret_cast<int32_t*>(x);
    x += al((size_t)B * sizeof(int32_t));
    def.prev = reinterpret_cast<int32_t*>(x);
    x += al((size_t)B * sizeof(int32_t));
    spill = reinterpret_cast<float*>(x);
  }
  const uint32_t k0 = (uint32_t)(seed & 0xFFFFFFFFu), k1 = (uint32_t)(seed >> 32);
  const bool probs = input_kind == DSPARK_INPUT_PROBS;
  const unsigned stat_grid = (unsigned)((long)B * (N + 1) * p.stat_chunks);
  if (!probs && B <= kFusedMaxB) {
    // statistics and acceptance in one launch, with this launch's ticket set
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    static std::atomic<unsigned*> set_base[64];
    static std::atomic<unsigned> next_set[64];
    unsigned* base = set_base[dev].load(std::memory_order_relaxed);
    if (!base) {  // (concurrent first calls store the same address)
      void* sym = nullptr;
      const hipError_t e = hipGetSymbolAddress(&sym, HIP_SYMBOL(g_stat_tickets));
      if (e != hipSuccess) return e;
      base = static_cast<unsigned*>(sym);
      set_base[dev].store(base, std::memory_order_relaxed);
    }
    unsigned* st = base + (size_t)(next_set[dev].fetch_add(1u, std::memory_order_relaxed) % kTicketSets) *
                              kFusedMaxB * kTWordsPerReq;
    hipLaunchKernelGGL(verify_stats_accept, dim3(stat_grid), dim3(256), 0, stream, target, draft, draft_log_z,
                       draft_tokens, inv_map, verify_len, temperature, request_id, k0, k1, stats, rstat, jobs,
                       tickets, accepted, out_tokens, accept_prob, st, N, V, Vd, p.stat_chunks, p.stat_chunk,
                       p.sample_chunks, def);
  } else if (!probs && !accept_prob && N + 1 > kLazyRows) {
    // lazy row statistics: rows 0 .. kLazyRows - 1 and the acceptance on them, then the
    // remaining rows of the requests still undecided and their acceptance
    const unsigned grid_a = (unsigned)((long)B * kLazyRows * p.stat_chunks);
    const unsigned grid_b = (unsigned)((long)B * (N + 1 - kLazyRows) * p.stat_chunks);
    AcceptLazy first, second;
    first.avail = kLazyRows;
    first.cont_out = cont;
    second.cont_in = cont;
    hipLaunchKernelGGL(verify_rowstats, dim3(grid_a), dim3(256), 0, stream, target, verify_len, temperature, stats,
                       B, N, V, p.stat_chunks, p.stat_chunk, 0, kLazyRows, static_cast<const int32_t*>(nullptr));
    hipLaunchKernelGGL(verify_accept, dim3(B), dim3(256), 0, stream, input_kind, target, draft, draft_log_z,
                       draft_tokens, inv_map, verify_len, temperature, request_id, k0, k1, stats, rstat, jobs,
                       tickets, accepted, out_tokens, accept_prob, N, V, Vd, p.stat_chunks, p.sample_chunks, def,
                       first);
    hipLaunchKernelGGL(verify_rowstats, dim3(grid_b), dim3(256), 0, stream, target, verify_len, temperature, stats,
                       B, N, V, p.stat_chunks, p.stat_chunk, kLazyRows, N + 1 - kLazyRows,
                       static_cast<const int32_t*>(cont));
    hipLaunchKernelGGL(verify_accept, dim3(B), dim3(256), 0, stream, input_kind, target, draft, draft_log_z,
                       draft_tokens, inv_map, verify_len, temperature, request_id, k0, k1, stats, rstat, jobs,
                       tickets, accepted, out_tokens, accept_prob, N, V, Vd, p.stat_chunks, p.sample_chunks, def,
                       second);
  } else {
    if (!probs)
      hipLaunchKernelGGL(verify_rowstats, dim3(stat_grid), dim3(256), 0, stream, target, verify_len, temperature,
                         stats, B, N, V, p.stat_chunks, p.stat_chunk, 0, N + 1, static_cast<const int32_t*>(nullptr));
    hipLaunchKernelGGL(verify_accept, dim3(B), dim3(256), 0, stream, input_kind, target, draft, draft_log_z,
                       draft_tokens, inv_map, verify_len, temperature, request_id, k0, k1, stats, rstat, jobs,
                       tickets, accepted, out_tokens, accept_prob, N, V, Vd, p.stat_chunks, p.sample_chunks, def,
                       AcceptLazy{});
  }
  if (dfr) {
    // the rows the sampling pass reads, from the base logits (the caller's buffer)
    const hipError_t e =
        launch_markov_replay(const_cast<float*>(draft), dfr->w1, dfr->w2, def.rows, def.prev, temperature,
                             request_id, B, N, V, Vd, dfr->r, spill, stream);
    if (e != hipSuccess) return e;
  }
  const int R = accept_prob ? N + 1 : 1;
  hipLaunchKernelGGL(verify_sample, dim3((unsigned)((long)B * R * p.sample_chunks)), dim3(256), 0, stream,
                     input_kind, target, draft, draft_log_z, inv_map, temperature, request_id, k0, k1, jobs, rstat,
                     race, apart, tickets, accepted, out_tokens, accept_prob, B, N, V, Vd, R, p.sample_chunks,
                     p.sample_chunk);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_verify(int input_kind, const float* target, const float* draft, const float* draft_log_z,
                         const int32_t* draft_tokens, const int32_t* inv_map, const int32_t* verify_len,
                         const float* temperature, const uint32_t* request_id, uint64_t seed, int32_t* accepted,
                         int32_t* out_tokens, float* accept_prob, int B, int N, int V, int Vd, void* workspace,
                         hipStream_t stream) {
  return verify_impl(input_kind, target, draft, draft_log_z, draft_tokens, inv_map, verify_len, temperature,
                     request_id, seed, accepted, out_tokens, accept_prob, B, N, V, Vd, workspace, nullptr, stream);
}

size_t verify_deferred_extra_bytes(int B, int V) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  return 2 * al((size_t)B * sizeof(int32_t)) + al(markov_replay_spill_bytes(V));
}

hipError_t launch_verify_deferred(const float* target, float* draft_base, const float* draft_log_z,
                                  const int32_t* draft_tokens, const int32_t* verify_len, const float* temperature,
                                  const uint32_t* request_id, uint64_t seed, int32_t* accepted, int32_t* out_tokens,
                                  int B, int N, int V, const DeferredArgs& d, void* workspace, hipStream_t stream) {
  return verify_impl(DSPARK_INPUT_LOGITS, target, draft_base, draft_log_z, draft_tokens, nullptr, verify_len,
                     temperature, request_id, seed, accepted, out_tokens, nullptr, B, N, V, V, workspace, &d, stream);
}

// ---------------------------------------------------------------- no-allocation variant
// The workspace of launch_verify as a file-scope device array, for callers that cannot
// allocate.  Each device holds its own copy at its own address; host code uses the
// address hipGetSymbolAddress returns for the current device, never the array's name.
// Every call on a device shares that device's copy, so calls that overlap on one
// device race.  launch_verify needs no initialised workspace content.
__device__ __attribute__((aligned(256))) char scratch[kVerifyScratchBytes];

hipError_t launch_verify_noalloc(int input_kind, const float* target, const float* draft, const float* draft_log_z,
                                 const int32_t* draft_tokens, const int32_t* inv_map, const int32_t* verify_len,
                                 const float* temperature, const uint32_t* request_id, uint64_t seed,
                                 int32_t* accepted, int32_t* out_tokens, float* accept_prob, int B, int N, int V,
                                 int Vd, hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  static std::atomic<void*> ptr_of[64];
  void* ptr = ptr_of[dev].load(std::memory_order_acquire);
  if (!ptr) {  // first call on this device, with the device current (concurrent first calls store the same address)
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptr_of[dev].store(ptr, std::memory_order_release);
  }
  return launch_verify(input_kind, target, draft, draft_log_z, draft_tokens, inv_map, verify_len, temperature,
                       request_id, seed, accepted, out_tokens, accept_prob, B, N, V, Vd, ptr, stream);
}

}  // namespace dspark
