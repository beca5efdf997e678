// Confidence head (推测解码：从零到DSpark §6): each position's conditional
// acceptance probability from a linear projection of the backbone hidden state and
// the Markov embedding of the previous token, calibrated per position:
//   c[b, k] = 1 / (1 + exp(-(w_h . h[b*N + k] + w_e . W1[x_{k-1}] + bias) / tau[k]))
// with x_{-1} = the anchor.  Its output feeds admission (survival = running product).
//
// One wave per (request, position) row, four rows per workgroup: lanes take
// 16-byte pieces of the hidden row and of w_h (all loads of a batch in flight),
// then the embedding row; a DPP sum reduces the wave.
#include <math.h>

#include "device.hpp"
#include "kernels.hpp"

namespace dspark {

namespace {

constexpr int kBatch = 8;  // 16-byte pieces per lane in flight

__device__ __forceinline__ float dot8(const uint4& a, const uint4& b) {
  const uint32_t x[4] = {a.x, a.y, a.z, a.w}, y[4] = {b.x, b.y, b.z, b.w};
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    s += __uint_as_float(x[q] << 16) * __uint_as_float(y[q] << 16);
    s += __uint_as_float(x[q] & 0xFFFF0000u) * __uint_as_float(y[q] & 0xFFFF0000u);
  }
  return s;
}

__global__ __launch_bounds__(256) void confidence_kernel(const uint16_t* __restrict__ hidden,
                                                         const uint16_t* __restrict__ w1,
                                                         const int32_t* __restrict__ draft_tokens,
                                                         const int32_t* __restrict__ anchor,
                                                         const uint16_t* __restrict__ w, float bias,
                                                         const float* __restrict__ tau, float* __restrict__ c_out,
                                                         int rows, int N, int H, int V, int r) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // (whole waves)
  const int b = row / N, k = row - b * N;
  const int hp = H / 8, rp = r / 8;  // 16-byte pieces
  const uint4* hrow = reinterpret_cast<const uint4*>(hidden + (size_t)row * H);
  const uint4* wh = reinterpret_cast<const uint4*>(w);
  float acc = 0.0f;
  for (int p0 = 0; p0 < hp; p0 += 64 * kBatch) {
    uint4 x[kBatch], y[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int p = min(p0 + lane + 64 * u, hp - 1);  // clamped; extra pieces are not summed
      x[u] = hrow[p];
      y[u] = wh[p];
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float d = dot8(x[u], y[u]);
      acc += (p0 + lane + 64 * u < hp) ? d : 0.0f;
    }
  }
  const int prev = (k == 0) ? anchor[b] : draft_tokens[(size_t)b * N + k - 1];
  const uint4* erow = reinterpret_cast<const uint4*>(w1 + (size_t)min(max(prev, 0), V - 1) * r);
  const uint4* we = reinterpret_cast<const uint4*>(w + H);
  for (int p = lane; p < rp; p += 64) acc += dot8(erow[p], we[p]);
  acc = group_sum(acc, 64);
  if (lane == 0) c_out[row] = 1.0f / (1.0f + expf(-(acc + bias) / tau[k]));
}

}  // namespace

hipError_t launch_confidence(const uint16_t* hidden, const uint16_t* w1, const int32_t* draft_tokens,
                             const int32_t* anchor, const uint16_t* w, float bias, const float* tau, float* c_out,
                             int B, int N, int H, int V, int r, hipStream_t stream) {
  const int rows = B * N;
  hipLaunchKernelGGL(confidence_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream, hidden, w1, draft_tokens, anchor,
                     w, bias, tau, c_out, rows, N, H, V, r);
  return hipGetLastError();
}

}  // namespace dspark
