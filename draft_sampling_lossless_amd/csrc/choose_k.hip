// Throughput-optimal verification budget K (推测解码：从零到DSpark §6, §7): pool
// every request's draft candidates, order them by survival, and pick the K that
// maximises (expected tokens per batch) x (steps per second at that batch):
//   objective(K) = (B + S_K) * sps[B + K],  S_K = sum of the K largest survivals,
// scanned over every K (the SPS curve is jagged, so no early stop); the smallest K
// of the largest objective wins.
//
// One workgroup of 1024 threads: a bitonic sort of the pooled survivals in LDS
// (descending; equal values are interchangeable for the sums), an fp64 prefix sum
// (per-thread segments, then a block scan of the segment totals), the objective of
// every K and a block argmax.
#include <math.h>

#include "device.hpp"
#include "kernels.hpp"

namespace dspark {

namespace {

constexpr int kThreads = 1024;

__device__ __forceinline__ bool obj_beats(double a, int ka, double b, int kb) {
  return a > b || (a == b && ka < kb);
}

__global__ __launch_bounds__(1024) void choose_k_kernel(const float* __restrict__ survival, int M, int B,
                                                        const float* __restrict__ sps, int S, int P,
                                                        int32_t* __restrict__ k_out, double* __restrict__ obj_out) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  double* part = reinterpret_cast<double*>(smem);             // [kThreads] segment totals, then prefixes
  double* bo = part + kThreads;                                // [kThreads / 64] per-wave best objective
  int* bk = reinterpret_cast<int*>(bo + kThreads / 64);        // [kThreads / 64] its K
  float* key = reinterpret_cast<float*>(bk + kThreads / 64);   // [P] survivals, sorted in place
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < P; i += kThreads) key[i] = (i < M) ? survival[i] : -INFINITY;
  __syncthreads();
  // bitonic sort, descending
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int t = tid; t < P / 2; t += kThreads) {
        const int i = 2 * stride * (t / stride) + (t % stride), j = i + stride;
        const float a = key[i], b = key[j];
        const bool down = (i & size) == 0;  // this block ends up descending
        if (down ? (a < b) : (a > b)) {
          key[i] = b;
          key[j] = a;
        }
      }
      __syncthreads();
    }
  }
  // fp64 prefix sums: thread t owns sorted positions [t Q, t Q + Q)
  const int Q = (M + kThreads - 1) / kThreads;
  const int lo = min(M, tid * Q), hi = min(M, lo + Q);
  double sum = 0.0;
  for (int i = lo; i < hi; ++i) sum += (double)key[i];
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < kThreads; off <<= 1) {  // inclusive scan of the segment totals
    const double add = (tid >= off) ? part[tid - off] : 0.0;
    __syncthreads();
    part[tid] += add;
    __syncthreads();
  }
  const int kmax = min(M, S - 1 - B);
  double run = (tid > 0) ? part[tid - 1] : 0.0;  // S_K before this segment
  double best = -INFINITY;
  int bestk = 0x7FFFFFFF;
  if (tid == 0) {  // K = 0
    best = (double)B * (double)sps[B];
    bestk = 0;
  }
  for (int i = lo; i < hi; ++i) {
    run += (double)key[i];
    const int K = i + 1;
    if (K > kmax) break;
    const double o = ((double)B + run) * (double)sps[B + K];
    if (obj_beats(o, K, best, bestk)) {
      best = o;
      bestk = K;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const double ob = __shfl_xor(best, off);
    const int okk = __shfl_xor(bestk, off);
    if (obj_beats(ob, okk, best, bestk)) {
      best = ob;
      bestk = okk;
    }
  }
  if (lane == 0) {
    bo[wave] = best;
    bk[wave] = bestk;
  }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kThreads / 64; ++w)
      if (obj_beats(bo[w], bk[w], best, bestk)) {
        best = bo[w];
        bestk = bk[w];
      }
    k_out[0] = bestk;
    if (obj_out) obj_out[0] = best;
  }
}

}  // namespace

hipError_t launch_choose_k(const float* survival, int B, int N, const float* sps, int S, int32_t* k_out,
                           double* obj_out, hipStream_t stream) {
  const int M = B * N;
  int P = 1;
  while (P < M) P <<= 1;
  const size_t lds = (size_t)kThreads * 8 + (kThreads / 64) * 12 + (size_t)P * 4;
  if (lds > 64 * 1024) {
    static bool attr_set[64] = {false};
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (dev >= 0 && dev < 64 && !attr_set[dev]) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(choose_k_kernel),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
      if (e != hipSuccess) return e;
      attr_set[dev] = true;
    }
  }
  hipLaunchKernelGGL(choose_k_kernel, dim3(1), dim3(kThreads), lds, stream, survival, M, B, sps, S, P, k_out,
                     obj_out);
  return hipGetLastError();
}

}  // namespace dspark
