// End of a round ("DSpark 的实现和测评" §2.1: the anchor of a request is the token
// its previous step verified): every request's next anchor is the last token verify
// emitted for it, out_tokens[b, accepted[b]] (the correction or bonus token), and a
// running per-request count of emitted tokens (accepted drafts plus that token) lets
// a multi-round driver measure the tokens per round.
#include "kernels.hpp"

namespace dspark {

namespace {

__global__ __launch_bounds__(256) void advance_kernel(const int32_t* __restrict__ accepted,
                                                      const int32_t* __restrict__ out_tokens,
                                                      int32_t* __restrict__ anchor, int64_t* __restrict__ emitted,
                                                      int B, int N) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int a = min(max(accepted[b], 0), N);  // (verify writes 0 .. N)
  anchor[b] = out_tokens[(size_t)b * (N + 1) + a];
  if (emitted) emitted[b] += a + 1;
}

}  // namespace

hipError_t launch_advance(const int32_t* accepted, const int32_t* out_tokens, int32_t* anchor, int64_t* emitted,
                          int B, int N, hipStream_t stream) {
  hipLaunchKernelGGL(advance_kernel, dim3((B + 255) / 256), dim3(256), 0, stream, accepted, out_tokens, anchor,
                     emitted, B, N);
  return hipGetLastError();
}

}  // namespace dspark
