// Raw access to the path's random numbers, for bit-exact checks of the generator
// (Philox4x32-10 blocks) and of the stage-3 race variates (-plog2 of the uniform).
#include "device.hpp"
#include "kernels.hpp"

namespace dspark {

namespace {

__global__ void philox_blocks(const uint4* __restrict__ counters, uint32_t k0, uint32_t k1, uint4* __restrict__ out,
                              int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint4 c = counters[i];
  const u32x4 w = philox4x32_10(u32x4{c.x, c.y, c.z, c.w}, k0, k1);
  out[i] = make_uint4(w.x, w.y, w.z, w.w);
}

__global__ void race_exps(uint32_t k0, uint32_t k1, uint32_t position, uint32_t request_id, uint32_t tag,
                          float* __restrict__ out, int64_t n) {
  const int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (v >= n) return;
  const u32x4 w = philox4x32_10(u32x4{(uint32_t)(v >> 2), position, request_id, tag}, k0, k1);
  const uint32_t words[4] = {w.x, w.y, w.z, w.w};
  out[v] = -plog2(uniform01(words[v & 3]));
}

}  // namespace

hipError_t launch_philox_blocks(const uint32_t* counters, uint64_t seed, uint32_t* out, int64_t n,
                                hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(philox_blocks, dim3((unsigned)blocks), dim3(256), 0, stream,
                     reinterpret_cast<const uint4*>(counters), (uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32),
                     reinterpret_cast<uint4*>(out), n);
  return hipGetLastError();
}

hipError_t launch_race_exponentials(uint64_t seed, uint32_t position, uint32_t request_id, uint32_t tag,
                                    float* out, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(race_exps, dim3((unsigned)blocks), dim3(256), 0, stream, (uint32_t)(seed & 0xFFFFFFFFu),
                     (uint32_t)(seed >> 32), position, request_id, tag, out, n);
  return hipGetLastError();
}

}  // namespace dspark
