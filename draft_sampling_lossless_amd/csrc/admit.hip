// Stage 4: confidence-scheduled admission.
//
// survival[b, k] = running float32 product of c[b, 0..k]; the B*N candidates are
// ordered by (survival descending, k ascending, b ascending) and the first K are
// admitted.  One workgroup does it all in LDS:
//   * each candidate gets a unique 64-bit key whose ascending order is that order:
//       key = (~bits(survival)) << 32 | k << 16 | b
//     (bits of a non-negative float are monotone in its value);
//   * the K-th smallest key is found by an MSB-first radix select (8 passes of
//     8-bit digits, 256-bin LDS histogram, one-wave scan per pass);
//   * (b, k) is admitted iff its key <= that key; admit_len[b] counts them.
#include "dspark.h"
#include "device.hpp"
#include "kernels.hpp"

namespace dspark {

namespace {

constexpr int kAdmitThreads = 1024;

__global__ __launch_bounds__(kAdmitThreads) void admit_kernel(const float* __restrict__ c, int B, int N, int K,
                                                            float* __restrict__ survival,
                                                            int32_t* __restrict__ admit_len) {
  extern __shared__ uint64_t keys[];  // [B * N]
  __shared__ unsigned hist[256];
  __shared__ uint64_t sel_prefix;
  __shared__ int sel_rank;
  const int tid = threadIdx.x;
  const int BN = B * N;

  for (int b = tid; b < B; b += kAdmitThreads) {
    float s = 1.0f;
    for (int k = 0; k < N; ++k) {
      const float ck = c[(size_t)b * N + k];
      s = (k == 0) ? ck : __fmul_rn(s, ck);
      survival[(size_t)b * N + k] = s;
      keys[b * N + k] = ((uint64_t)(~__float_as_uint(s)) << 32) | ((uint64_t)k << 16) | (uint64_t)b;
    }
  }
  if (K >= BN || K <= 0) {
    for (int b = tid; b < B; b += kAdmitThreads) admit_len[b] = (K <= 0) ? 0 : N;
    return;
  }
  if (tid == 0) {
    sel_prefix = 0;
    sel_rank = K - 1;
  }
  __syncthreads();

  uint64_t mask = 0;
  for (int d = 7; d >= 0; --d) {
    for (int i = tid; i < 256; i += kAdmitThreads) hist[i] = 0;
    __syncthreads();
    const uint64_t prefix = sel_prefix;
    const int shift = 8 * d;
    for (int e = tid; e < BN; e += kAdmitThreads) {
      const uint64_t key = keys[e];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 0xFF], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      const int rank = sel_rank;
      unsigned h[4];
      unsigned tot = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        h[q] = hist[4 * tid + q];
        tot += h[q];
      }
      unsigned incl = tot;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const unsigned o = __shfl_up(incl, off);
        if (tid >= off) incl += o;
      }
      const unsigned excl = incl - tot;
      if (excl <= (unsigned)rank && (unsigned)rank < incl) {
        unsigned cum = excl;
        int q = 0;
        while (cum + h[q] <= (unsigned)rank) {
          cum += h[q];
          ++q;
        }
        sel_prefix = prefix | ((uint64_t)(4 * tid + q) << shift);
        sel_rank = rank - (int)cum;
      }
    }
    mask |= (uint64_t)0xFF << shift;
    __syncthreads();
  }
  const uint64_t theta = sel_prefix;
  for (int b = tid; b < B; b += kAdmitThreads) {
    int cnt = 0;
    for (int k = 0; k < N; ++k) cnt += (keys[b * N + k] <= theta) ? 1 : 0;
    admit_len[b] = cnt;
  }
}

}  // namespace

hipError_t launch_admit(const float* cond_accept, int B, int N, int K, float* survival, int32_t* admit_len,
                        hipStream_t stream) {
  const size_t lds = (size_t)B * N * sizeof(uint64_t);
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(admit_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(admit_kernel, dim3(1), dim3(kAdmitThreads), lds, stream, cond_accept, B, N, K, survival,
                     admit_len);
  return hipGetLastError();
}

}  // namespace dspark
