// Stage 3: lossless rejection-sampling verification.
//
// For request b with verify length L and drafted target ids x_k: accept x_k iff
// u_k * p_d(x_k) < p_t(x_k) (double products of float32 values: exact), stop at
// the first rejection k and resample from max(0, p_t - p_d) there, or, with all
// L accepted, draw a bonus token from target row L.  Both draws are exponential
// races: argmax_v r_v / E_v with E_v = -plog2(u_v), compared exactly.
//
// Kernels (one pass each, grid-wide where a row is long):
//   rowstats   logits mode only.  Row statistics of target rows k <= L: base-2
//              log-sum-exp of l / T (T > 0) or the argmax (T == 0), per
//              (row, chunk) partial.
//   accept     one wave per request: merges the row partials, runs the sequential
//              acceptance test (one element per row of each side), writes the
//              accepted prefix and a sampling job (row, residual or bonus).
//   sample     (request, chunk) workgroups stream the job row(s): target row, and
//              for a residual the draft row (gathered through the inverse map);
//              per-chunk race winner for the residual and for its fallback
//              (p_t itself, used only if the residual is zero everywhere).
//   finalize   one wave per request reduces the race partials and writes y.
#include <math.h>

#include "dspark.h"
#include "device.hpp"
#include "kernels.hpp"

namespace dspark {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

struct RowStat {
  float m, s;     // base-2 log-sum-exp state of y = l * log2(e) / T
  float amax;     // argmax value (T == 0 rows)
  int aidx;       // argmax index (smallest on ties)
};

enum { kJobDone = 0, kJobResid = 1, kJobBonus = 2 };

struct Job {
  int mode;       // kJobDone / kJobResid / kJobBonus
  int row;        // position k of the sampling row
  float m, invs;  // target row statistics (logits mode): p_t = 2^(y - m) * invs
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

// ------------------------------------------------------------------ row statistics

__global__ __launch_bounds__(256) void verify_rowstats(const float* __restrict__ target,
                                                       const int32_t* __restrict__ verify_len,
                                                       const float* __restrict__ temperature,
                                                       RowStat* __restrict__ stats, int B, int N, int V,
                                                       int nchunks, int chunk) {
  const int row = blockIdx.x / nchunks, c = blockIdx.x % nchunks;
  const int b = row / (N + 1), k = row % (N + 1);
  const int L = verify_len ? min(max(verify_len[b], 0), N) : N;
  if (k > L) return;
  const float T = temperature[b];
  const bool hot = T > 0.0f;
  const float c2 = hot ? (1.0f / T) * kLog2e : 1.0f;
  const float* rowp = target + (size_t)row * V;
  const int lo = c * chunk, hi = min(V, lo + chunk);

  float m = -INFINITY, s = 0.0f, av = -INFINITY;
  int ai = 0x7FFFFFFF;
  for (int v = lo + 4 * threadIdx.x; v < hi; v += 4 * blockDim.x) {
    const float4 q = *reinterpret_cast<const float4*>(rowp + v);
    const float l[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int f = 0; f < 4; ++f)
      if (amax_beats(l[f], v + f, av, ai)) {
        av = l[f];
        ai = v + f;
      }
    if (hot) {
      float y[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) y[f] = l[f] * c2;
      const float mn = fmaxf(m, fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3])));
      float acc = s * __builtin_amdgcn_exp2f(m - mn);
#pragma unroll
      for (int f = 0; f < 4; ++f) acc += __builtin_amdgcn_exp2f(y[f] - mn);
      s = acc;
      m = mn;
    }
  }
  // block reduction: waves, then LDS
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float om = __shfl_xor(m, off), os = __shfl_xor(s, off), ov = __shfl_xor(av, off);
    const int oi = __shfl_xor(ai, off);
    lse2_merge(m, s, om, os);
    if (amax_beats(ov, oi, av, ai)) {
      av = ov;
      ai = oi;
    }
  }
  __shared__ RowStat red[4];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = RowStat{m, s, av, ai};
  __syncthreads();
  if (threadIdx.x == 0) {
    RowStat a = red[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) {
      lse2_merge(a.m, a.s, red[w].m, red[w].s);
      if (amax_beats(red[w].amax, red[w].aidx, a.amax, a.aidx)) {
        a.amax = red[w].amax;
        a.aidx = red[w].aidx;
      }
    }
    stats[(size_t)row * nchunks + c] = a;
  }
}

// ------------------------------------------------------------------ acceptance

__global__ __launch_bounds__(64) void verify_accept(int input_kind, const float* __restrict__ target,
                                                    const float* __restrict__ draft,
                                                    const float* __restrict__ draft_log_z,
                                                    const int32_t* __restrict__ draft_tokens,
                                                    const int32_t* __restrict__ inv_map,
                                                    const int32_t* __restrict__ verify_len,
                                                    const float* __restrict__ temperature,
                                                    const uint32_t* __restrict__ request_id, uint32_t key0,
                                                    uint32_t key1, const RowStat* __restrict__ stats,
                                                    Job* __restrict__ jobs, int32_t* __restrict__ accepted,
                                                    int32_t* __restrict__ out_tokens, int B, int N, int V,
                                                    int Vd, int nchunks) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int L = verify_len ? min(max(verify_len[b], 0), N) : N;
  const uint32_t req = request_id[b];
  const bool probs = input_kind == DSPARK_INPUT_PROBS;
  const float T = probs ? 1.0f : temperature[b];
  const bool hot = probs || T > 0.0f;
  const float c2 = (!probs && hot) ? (1.0f / T) * kLog2e : 1.0f;

  // Merged statistics of target rows k <= L (logits mode), kept in LDS.
  __shared__ float row_m[DSPARK_MAX_N + 1], row_s[DSPARK_MAX_N + 1];
  __shared__ int row_amax[DSPARK_MAX_N + 1];
  if (!probs) {
    for (int k = 0; k <= L; ++k) {
      float m = -INFINITY, s = 0.0f, av = -INFINITY;
      int ai = 0x7FFFFFFF;
      const RowStat* rp = stats + ((size_t)b * (N + 1) + k) * nchunks;
      for (int c = lane; c < nchunks; c += 64) {
        const RowStat q = rp[c];
        lse2_merge(m, s, q.m, q.s);
        if (amax_beats(q.amax, q.aidx, av, ai)) {
          av = q.amax;
          ai = q.aidx;
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float om = __shfl_xor(m, off), os = __shfl_xor(s, off), ov = __shfl_xor(av, off);
        const int oi = __shfl_xor(ai, off);
        lse2_merge(m, s, om, os);
        if (amax_beats(ov, oi, av, ai)) {
          av = ov;
          ai = oi;
        }
      }
      if (lane == 0) {
        row_m[k] = m;
        row_s[k] = s;
        row_amax[k] = ai;
      }
    }
  }
  __syncthreads();

  // Sequential acceptance test (every lane computes it; lane k supplies row k's stats).
  int a = L;
  for (int k = 0; k < L; ++k) {
    const int x = draft_tokens[(size_t)b * N + k];
    if (x < 0 || x >= V) {  // not a target id: reject without reading anything
      a = k;
      break;
    }
    const int j = inv_map ? inv_map[x] : x;
    float pt, pd;
    if (probs) {
      pt = target[((size_t)b * (N + 1) + k) * V + x];
      pd = (j >= 0) ? draft[((size_t)b * N + k) * Vd + j] : 0.0f;
    } else {
      const float m = row_m[k], s = row_s[k];
      const int ai = row_amax[k];
      if (hot) {
        const float lt = target[((size_t)b * (N + 1) + k) * V + x];
        pt = __builtin_amdgcn_exp2f(lt * c2 - m) / s;
        if (j >= 0) {
          const float ld = draft[((size_t)b * N + k) * Vd + j];
          pd = __builtin_amdgcn_exp2f(ld * c2 - draft_log_z[(size_t)b * N + k] * kLog2e);
        } else {
          pd = 0.0f;
        }
      } else {
        pt = (x == ai) ? 1.0f : 0.0f;
        pd = 1.0f;
      }
    }
    const u32x4 w = philox4x32_10(u32x4{0u, (uint32_t)k, req, kTagAccept}, key0, key1);
    const float u = uniform01(w.x);
    if (!((double)u * (double)pd < (double)pt)) {
      a = k;
      break;
    }
  }

  // Outputs: accepted prefix, -1 padding, the sampling job.
  for (int k = lane; k <= N; k += 64) {
    int32_t o = -1;
    if (k < a) o = draft_tokens[(size_t)b * N + k];
    out_tokens[(size_t)b * (N + 1) + k] = o;
  }
  if (lane == 0) accepted[b] = a;
  const int row = a;  // residual row (a < L) or bonus row (a == L)
  if (lane == 0) {
    const float m = probs ? 0.0f : row_m[row], s = probs ? 1.0f : row_s[row];
    const int ai = probs ? 0 : row_amax[row];
    Job jb;
    jb.row = row;
    jb.mode = (a < L) ? kJobResid : kJobBonus;
    jb.m = m;
    jb.invs = probs ? 1.0f : 1.0f / s;
    if (!probs && !hot) {
      // greedy: the residual and the bonus are both the point mass on the argmax
      out_tokens[(size_t)b * (N + 1) + a] = ai;
      jb.mode = kJobDone;
    }
    jobs[b] = jb;
  }
}

// ------------------------------------------------------------------ sampling row

__device__ __forceinline__ void race_update(float r, float E, int v, float& br, float& bE, int& bv) {
  if (race_beats(r, E, v, br, bE, bv)) {
    br = r;
    bE = E;
    bv = v;
  }
}

__global__ __launch_bounds__(256) void verify_sample(int input_kind, const float* __restrict__ target,
                                                     const float* __restrict__ draft,
                                                     const float* __restrict__ draft_log_z,
                                                     const int32_t* __restrict__ inv_map,
                                                     const float* __restrict__ temperature,
                                                     const uint32_t* __restrict__ request_id, uint32_t key0,
                                                     uint32_t key1, const Job* __restrict__ jobs,
                                                     RacePartial* __restrict__ race, int B, int N, int V, int Vd,
                                                     int nchunks, int chunk) {
  const int b = blockIdx.x / nchunks, c = blockIdx.x % nchunks;
  const Job jb = jobs[b];
  if (jb.mode == kJobDone) return;
  const bool probs = input_kind == DSPARK_INPUT_PROBS;
  const bool resid = jb.mode == kJobResid;
  const int k = jb.row;
  const uint32_t req = request_id[b];
  const uint32_t tag = resid ? kTagResid : kTagBonus;
  const float c2 = probs ? 1.0f : (1.0f / temperature[b]) * kLog2e;
  const float dlz2 = (!probs && resid) ? draft_log_z[(size_t)b * N + k] * kLog2e : 0.0f;
  const float* trow = target + ((size_t)b * (N + 1) + k) * V;
  const float* drow = resid ? draft + ((size_t)b * N + k) * Vd : nullptr;
  const int lo = c * chunk, hi = min(V, lo + chunk);

  // Race candidates start as "nobody": r = 0 with E = 1 at index INT_MAX loses
  // to everything with r > 0, and index order decides among r = 0.
  float br = 0.0f, bE = 1.0f, fr = 0.0f, fE = 1.0f;
  int bv = 0x7FFFFFFF, fv = 0x7FFFFFFF;
  for (int v = lo + 4 * threadIdx.x; v < hi; v += 4 * blockDim.x) {
    const float4 q = *reinterpret_cast<const float4*>(trow + v);
    float pt[4] = {q.x, q.y, q.z, q.w};
    if (!probs) {
#pragma unroll
      for (int f = 0; f < 4; ++f) pt[f] = __builtin_amdgcn_exp2f(pt[f] * c2 - jb.m) * jb.invs;
    }
    const u32x4 w = philox4x32_10(u32x4{(uint32_t)v >> 2, (uint32_t)k, req, tag}, key0, key1);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      const float E = -plog2(uniform01(ws[f]));
      if (resid) {
        const int j = inv_map ? inv_map[v + f] : v + f;
        float pd = 0.0f;
        if (j >= 0) {
          const float d = drow[j];
          pd = probs ? d : __builtin_amdgcn_exp2f(d * c2 - dlz2);
        }
        const float r = fmaxf(0.0f, __fsub_rn(pt[f], pd));
        race_update(r, E, v + f, br, bE, bv);
        race_update(pt[f], E, v + f, fr, fE, fv);
      } else {
        race_update(pt[f], E, v + f, br, bE, bv);
      }
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float o_r = __shfl_xor(br, off), o_E = __shfl_xor(bE, off);
    const int o_v = __shfl_xor(bv, off);
    const float o_fr = __shfl_xor(fr, off), o_fE = __shfl_xor(fE, off);
    const int o_fv = __shfl_xor(fv, off);
    race_update(o_r, o_E, o_v, br, bE, bv);
    race_update(o_fr, o_fE, o_fv, fr, fE, fv);
  }
  __shared__ RacePartial red[4];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = RacePartial{br, bE, bv, fr, fE, fv, {0, 0}};
  __syncthreads();
  if (threadIdx.x == 0) {
    RacePartial a = red[0];
    for (int w2 = 1; w2 < (int)(blockDim.x >> 6); ++w2) {
      race_update(red[w2].r, red[w2].E, red[w2].v, a.r, a.E, a.v);
      race_update(red[w2].fr, red[w2].fE, red[w2].fv, a.fr, a.fE, a.fv);
    }
    race[(size_t)b * nchunks + c] = a;
  }
}

__global__ __launch_bounds__(64) void verify_finalize(const Job* __restrict__ jobs,
                                                      const RacePartial* __restrict__ race,
                                                      const int32_t* __restrict__ accepted,
                                                      int32_t* __restrict__ out_tokens, int N, int nchunks) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const Job jb = jobs[b];
  if (jb.mode == kJobDone) return;
  float br = 0.0f, bE = 1.0f, fr = 0.0f, fE = 1.0f;
  int bv = 0x7FFFFFFF, fv = 0x7FFFFFFF;
  for (int c = lane; c < nchunks; c += 64) {
    const RacePartial q = race[(size_t)b * nchunks + c];
    race_update(q.r, q.E, q.v, br, bE, bv);
    race_update(q.fr, q.fE, q.fv, fr, fE, fv);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float o_r = __shfl_xor(br, off), o_E = __shfl_xor(bE, off);
    const int o_v = __shfl_xor(bv, off);
    const float o_fr = __shfl_xor(fr, off), o_fE = __shfl_xor(fE, off);
    const int o_fv = __shfl_xor(fv, off);
    race_update(o_r, o_E, o_v, br, bE, bv);
    race_update(o_fr, o_fE, o_fv, fr, fE, fv);
  }
  if (lane == 0) {
    // an all-zero residual leaves r == 0 at the winner: fall back to p_t
    const int y = (jb.mode == kJobResid && br == 0.0f) ? fv : bv;
    out_tokens[(size_t)b * (N + 1) + accepted[b]] = y;
  }
}

int pick_chunks(long rows, int V) {
  // aim for >= 2048 workgroups, chunks of >= 1024 elements, multiple of 4
  long want = (2048 + rows - 1) / rows;
  long maxc = (V + 1023) / 1024;
  if (want > maxc) want = maxc;
  if (want < 1) want = 1;
  return (int)want;
}

}  // namespace

VerifyPlan plan_verify(int B, int N, int V) {
  VerifyPlan p{};
  p.stat_chunks = pick_chunks((long)B * (N + 1), V);
  p.stat_chunk = ((V + p.stat_chunks - 1) / p.stat_chunks + 3) / 4 * 4;
  p.sample_chunks = pick_chunks(B, V);
  p.sample_chunk = ((V + p.sample_chunks - 1) / p.sample_chunks + 3) / 4 * 4;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  p.stats_bytes = al((size_t)B * (N + 1) * p.stat_chunks * sizeof(RowStat));
  p.jobs_bytes = al((size_t)B * sizeof(Job));
  p.race_bytes = al((size_t)B * p.sample_chunks * sizeof(RacePartial));
  p.total_bytes = p.stats_bytes + p.jobs_bytes + p.race_bytes;
  return p;
}

hipError_t launch_verify(int input_kind, const float* target, const float* draft, const float* draft_log_z,
                         const int32_t* draft_tokens, const int32_t* inv_map, const int32_t* verify_len,
                         const float* temperature, const uint32_t* request_id, uint64_t seed, int32_t* accepted,
                         int32_t* out_tokens, int B, int N, int V, int Vd, void* workspace, hipStream_t stream) {
  const VerifyPlan p = plan_verify(B, N, V);
  char* ws = static_cast<char*>(workspace);
  RowStat* stats = reinterpret_cast<RowStat*>(ws);
  Job* jobs = reinterpret_cast<Job*>(ws + p.stats_bytes);
  RacePartial* race = reinterpret_cast<RacePartial*>(ws + p.stats_bytes + p.jobs_bytes);
  const uint32_t k0 = (uint32_t)(seed & 0xFFFFFFFFu), k1 = (uint32_t)(seed >> 32);
  const bool probs = input_kind == DSPARK_INPUT_PROBS;
  if (!probs) {
    hipLaunchKernelGGL(verify_rowstats, dim3((unsigned)((long)B * (N + 1) * p.stat_chunks)), dim3(256), 0, stream,
                       target, verify_len, temperature, stats, B, N, V, p.stat_chunks, p.stat_chunk);
  }
  hipLaunchKernelGGL(verify_accept, dim3(B), dim3(64), 0, stream, input_kind, target, draft, draft_log_z,
                     draft_tokens, inv_map, verify_len, temperature, request_id, k0, k1, stats, jobs, accepted,
                     out_tokens, B, N, V, Vd, p.stat_chunks);
  hipLaunchKernelGGL(verify_sample, dim3((unsigned)((long)B * p.sample_chunks)), dim3(256), 0, stream, input_kind,
                     target, draft, draft_log_z, inv_map, temperature, request_id, k0, k1, jobs, race, B, N, V, Vd,
                     p.sample_chunks, p.sample_chunk);
  hipLaunchKernelGGL(verify_finalize, dim3(B), dim3(64), 0, stream, jobs, race, accepted, out_tokens, N,
                     p.sample_chunks);
  return hipGetLastError();
}

}  // namespace dspark
