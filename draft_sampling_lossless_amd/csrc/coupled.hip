// Gumbel-coupled verification: the target verifies with the same Gumbel noise the
// draft sampled with (DSpark 的实现和测评 §5), so the emitted tokens are the
// target's own Gumbel-max draws and no draft probabilities are needed.
//
// Row k of request b: key(v) = l_t[k](v) * log2(e) / T + G2(v), where G2 is the
// base-2 Gumbel variate of the same Philox word stage 2 used for the draft entry
// that is target id v (counter (j >> 2, k, request, 0), word j & 3, j = inv[v] or
// v); an id outside the draft vocabulary draws its own word (tag 4, keyed on v).
// T == 0: key = l_t (no noise).  y_k = argmax key (ties to the smaller v).
// Accept x_k while y_k == x_k; the first mismatch k < L, or row L, emits y_k.
//
// Kernels: coupled_rows streams rows k <= L in (row, chunk) workgroups and writes
// per-chunk argmax partials; coupled_finalize (one workgroup per request) merges
// them row by row and applies the prefix rule.  With more than 16 requests the rows
// are taken lazily: rows 0-1 of every request first, and a finalize pass that decides
// every request whose first mismatch (or row L) lies there; then the remaining rows
// of the undecided requests and a second finalize pass for them.
#include <math.h>

#include <algorithm>

#include "device.hpp"
#include "kernels.hpp"
#include "markov_common.hpp"

namespace dspark {

namespace {

using namespace mk;

constexpr uint32_t kTagTarget = 4;  // noise of a target id outside the draft vocabulary

struct ArgPartial {
  float key;
  int v;
};

__global__ __launch_bounds__(256) void coupled_rows(const float* __restrict__ target,
                                                   const int32_t* __restrict__ inv_map,
                                                   const int32_t* __restrict__ verify_len,
                                                   const float* __restrict__ temperature,
                                                   const uint32_t* __restrict__ request_id, uint32_t key0,
                                                   uint32_t key1, ArgPartial* __restrict__ part, int N, int V,
                                                   int nchunks, int chunk, int k0, int nk,
                                                   const int32_t* __restrict__ cont) {
  // rows k0 .. k0 + nk - 1 of every request (with cont: of the requests still undecided)
  const int rr = blockIdx.x / nchunks, c = blockIdx.x % nchunks;
  const int b = rr / nk, k = k0 + rr % nk;
  const int L = verify_len ? min(max(verify_len[b], 0), N) : N;
  if (k > L || (cont && !cont[b])) return;
  const int row = b * (N + 1) + k;
  const float T = temperature[b];
  const bool noisy = T > 0.0f;
  const float c2 = noisy ? (1.0f / T) * 1.4426950408889634f : 1.0f;
  const uint32_t req = request_id[b];
  const float* rowp = target + (size_t)row * V;
  const int lo = c * chunk, hi = min(V, lo + chunk);
  float bk = -INFINITY;
  int bv = 0x7FFFFFFF;
  for (int v = lo + 4 * threadIdx.x; v < hi; v += 4 * blockDim.x) {
    const float4 q = *reinterpret_cast<const float4*>(rowp + v);
    float key[4] = {q.x * c2, q.y * c2, q.z * c2, q.w * c2};
    if (noisy) {
      if (inv_map == nullptr) {
        const u32x4 w = philox4x32_10(u32x4{(uint32_t)v >> 2, (uint32_t)k, req, kTagDraft}, key0, key1);
        key[0] += gumbel2(w.x);
        key[1] += gumbel2(w.y);
        key[2] += gumbel2(w.z);
        key[3] += gumbel2(w.w);
      } else {
        const int4 jj = *reinterpret_cast<const int4*>(inv_map + v);
        const int j[4] = {jj.x, jj.y, jj.z, jj.w};
        // one block for the ids outside the draft vocabulary (they share a counter)
        const u32x4 wo = philox4x32_10(u32x4{(uint32_t)v >> 2, (uint32_t)k, req, kTagTarget}, key0, key1);
        const uint32_t own[4] = {wo.x, wo.y, wo.z, wo.w};
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          uint32_t word = own[f];
          if (j[f] >= 0) {
            const u32x4 wd = philox4x32_10(u32x4{(uint32_t)j[f] >> 2, (uint32_t)k, req, kTagDraft}, key0, key1);
            const uint32_t ws[4] = {wd.x, wd.y, wd.z, wd.w};
            word = ws[j[f] & 3];
          }
          key[f] += gumbel2(word);
        }
      }
    }
#pragma unroll
    for (int f = 0; f < 4; ++f)
      if (key_beats(key[f], v + f, bk, bv)) {
        bk = key[f];
        bv = v + f;
      }
  }
  wave_argmax(bk, bv);
  __shared__ ArgPartial red[4];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = ArgPartial{bk, bv};
  __syncthreads();
  if (threadIdx.x == 0) {
    ArgPartial a = red[0];
    for (int w = 1; w < 4; ++w)
      if (key_beats(red[w].key, red[w].v, a.key, a.v)) a = red[w];
    part[(size_t)row * nchunks + c] = a;
  }
}

__global__ __launch_bounds__(256) void coupled_finalize(const ArgPartial* __restrict__ part,
                                                        const int32_t* __restrict__ draft_tokens,
                                                        const int32_t* __restrict__ verify_len,
                                                        int32_t* __restrict__ accepted,
                                                        int32_t* __restrict__ out_tokens, int N, int nchunks,
                                                        int avail, int32_t* __restrict__ cont_out,
                                                        const int32_t* __restrict__ cont_in) {
  // rows 0 .. avail - 1 have partials; with cont_out, a request whose first min(L, avail)
  // positions all match while L >= avail is undecided (cont_out = 1, nothing written);
  // with cont_in only the requests so marked run
  const int b = blockIdx.x, tid = threadIdx.x;
  if (cont_in && !cont_in[b]) return;
  const int L = verify_len ? min(max(verify_len[b], 0), N) : N;
  const int rows = min(L + 1, avail), tpr = 256 / rows;
  const int tested = min(L, avail);
  const int k = tid / tpr, sub = tid - k * tpr;
  __shared__ float pk[256];
  __shared__ int pv[256];
  __shared__ int y[65];
  __shared__ int s_a;
  float bk = -INFINITY;
  int bv = 0x7FFFFFFF;
  if (k < rows) {
    const ArgPartial* rp = part + ((size_t)b * (N + 1) + k) * nchunks;
    for (int c = sub; c < nchunks; c += tpr) {
      const ArgPartial q = rp[c];
      if (key_beats(q.key, q.v, bk, bv)) {
        bk = q.key;
        bv = q.v;
      }
    }
  }
  pk[tid] = bk;
  pv[tid] = bv;
  __syncthreads();
  if (tid < rows) {
    float k2 = -INFINITY;
    int v2 = 0x7FFFFFFF;
    for (int t = tid * tpr; t < (tid + 1) * tpr; ++t)
      if (key_beats(pk[t], pv[t], k2, v2)) {
        k2 = pk[t];
        v2 = pv[t];
      }
    y[tid] = (v2 == 0x7FFFFFFF) ? 0 : v2;  // (a row of NaN keys only)
  }
  __syncthreads();
  if (tid < 64) {  // the first mismatch, one lane per position
    const bool miss = tid < tested && draft_tokens[(size_t)b * N + tid] != y[tid];
    const uint64_t m = __ballot(miss);
    if (tid == 0) s_a = m ? __builtin_ctzll(m) : (L < avail ? L : -1);
  }
  __syncthreads();
  const int a = s_a;
  if (cont_out && tid == 0) cont_out[b] = (a < 0) ? 1 : 0;
  if (a < 0) return;
  for (int kk = tid; kk <= N; kk += 256)
    out_tokens[(size_t)b * (N + 1) + kk] = (kk < a) ? draft_tokens[(size_t)b * N + kk] : (kk == a ? y[a] : -1);
  if (tid == 0) accepted[b] = a;
}

int coupled_chunks(long rows, int V) {
  long want = (2048 + rows - 1) / rows;
  long maxc = (V + 1023) / 1024;
  return (int)std::max(1L, std::min(want, maxc));
}

// rows whose partials the lazy first pass computes; lazy above 16 requests
constexpr int kLazyRows = 2;
bool coupled_lazy(int B, int N) { return B > 16 && N + 1 > kLazyRows; }
// chunks per row: sized for the live rows of the (first) pass
int coupled_nchunks(int B, int N, int V) {
  return coupled_chunks(coupled_lazy(B, N) ? (long)B * kLazyRows : (long)B * (N + 1), V);
}

}  // namespace

size_t coupled_workspace_bytes(int B, int N, int V) {
  const long rows = (long)B * (N + 1);
  const size_t parts = (size_t)rows * coupled_nchunks(B, N, V) * sizeof(ArgPartial);
  return (parts + 255) / 256 * 256 + (size_t)B * sizeof(int32_t);   // + the continue flags
}

hipError_t launch_verify_coupled(const float* target, const int32_t* draft_tokens, const int32_t* inv_map,
                                 const int32_t* verify_len, const float* temperature, const uint32_t* request_id,
                                 uint64_t seed, int32_t* accepted, int32_t* out_tokens, int B, int N, int V,
                                 void* workspace, hipStream_t stream) {
  const long rows = (long)B * (N + 1);
  const int nchunks = coupled_nchunks(B, N, V);
  const int chunk = ((V + nchunks - 1) / nchunks + 3) / 4 * 4;
  ArgPartial* part = static_cast<ArgPartial*>(workspace);
  int32_t* cont = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                             ((size_t)rows * nchunks * sizeof(ArgPartial) + 255) / 256 * 256);
  const uint32_t k0 = (uint32_t)(seed & 0xFFFFFFFFu), k1 = (uint32_t)(seed >> 32);
  const int32_t* none = nullptr;
  if (coupled_lazy(B, N)) {
    const int nk = N + 1 - kLazyRows;
    hipLaunchKernelGGL(coupled_rows, dim3((unsigned)((long)B * kLazyRows * nchunks)), dim3(256), 0, stream, target,
                       inv_map, verify_len, temperature, request_id, k0, k1, part, N, V, nchunks, chunk, 0,
                       kLazyRows, none);
    hipLaunchKernelGGL(coupled_finalize, dim3(B), dim3(256), 0, stream, part, draft_tokens, verify_len, accepted,
                       out_tokens, N, nchunks, kLazyRows, cont, none);
    hipLaunchKernelGGL(coupled_rows, dim3((unsigned)((long)B * nk * nchunks)), dim3(256), 0, stream, target, inv_map,
                       verify_len, temperature, request_id, k0, k1, part, N, V, nchunks, chunk, kLazyRows, nk,
                       static_cast<const int32_t*>(cont));
    hipLaunchKernelGGL(coupled_finalize, dim3(B), dim3(256), 0, stream, part, draft_tokens, verify_len, accepted,
                       out_tokens, N, nchunks, N + 1, static_cast<int32_t*>(nullptr),
                       static_cast<const int32_t*>(cont));
  } else {
    hipLaunchKernelGGL(coupled_rows, dim3((unsigned)(rows * nchunks)), dim3(256), 0, stream, target, inv_map,
                       verify_len, temperature, request_id, k0, k1, part, N, V, nchunks, chunk, 0, N + 1, none);
    hipLaunchKernelGGL(coupled_finalize, dim3(B), dim3(256), 0, stream, part, draft_tokens, verify_len, accepted,
                       out_tokens, N, nchunks, N + 1, static_cast<int32_t*>(nullptr), none);
  }
  return hipGetLastError();
}

}  // namespace dspark
