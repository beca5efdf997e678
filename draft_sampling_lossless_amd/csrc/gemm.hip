// Stage 1: draft base logits, logits[m, j] = sum_h hidden[m, h] * lm_head[j, h]
// (bf16 in, fp32 accumulate and out) on gfx950 MFMA (v_mfma_f32_16x16x32_bf16).
//
// Two tilings, picked by M (= B * N, the number of draft positions):
//  * skinny (M <= 64): the product is bound by streaming the LM head from HBM
//    (2 * Vd * H bytes, read once).  Each wave owns 16*FR vocabulary rows and
//    streams them straight from global memory into MFMA B fragments; the few
//    hidden rows (A fragments) come from L1/L2.  No LDS.
//  * tiled (M > 64): MFMA-bound.  128 x 128 output tiles, BK = 64, both operands
//    staged through double-buffered LDS; 4 waves, each a 64 x 64 block of 16x16
//    MFMA fragments.
//
// MFMA 16x16x32 fragment layout (64 lanes, lane = 16 * g + n):
//   A: lane holds 8 consecutive k of row n;  B: 8 consecutive k of column n;
//   the k block of a lane is 8 * g within each 32-wide k step (the same mapping
//   on both operands, which is all the reduction needs);
//   C/D: lane holds rows 4 * g + i (i = 0..3) of column n.
#include "device.hpp"
#include "kernels.hpp"

namespace dspark {

namespace {

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ bf16x8 zero_bf16x8() { return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0)); }

// ------------------------------------------------------------------ skinny

template <int FR, int MT>
__global__ __launch_bounds__(256) void k1_skinny(const uint16_t* __restrict__ A,
                                                 const uint16_t* __restrict__ W,
                                                 float* __restrict__ C, int M, int H, int Vd) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int j0 = wave * (16 * FR);
  if (j0 >= Vd) return;  // whole wave
  const int n = lane & 15, g = lane >> 4;

  const uint16_t* wrow[FR];
  bool wok[FR];
#pragma unroll
  for (int f = 0; f < FR; ++f) {
    const int j = j0 + 16 * f + n;
    wok[f] = j < Vd;
    wrow[f] = W + (size_t)(wok[f] ? j : 0) * H;
  }
  const uint16_t* arow[MT];
  bool aok[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = 16 * t + n;
    aok[t] = m < M;
    arow[t] = A + (size_t)(aok[t] ? m : 0) * H;
  }

  floatx4 acc[MT][FR];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int f = 0; f < FR; ++f) acc[t][f] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int steps = (H + 31) / 32;
  constexpr int U = 4;  // k steps whose loads are in flight together
  for (int s0 = 0; s0 < steps; s0 += U) {
    bf16x8 b[U][FR], a[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = (s0 + u) * 32 + 8 * g;
      const bool kok = (s0 + u) < steps && k < H;
#pragma unroll
      for (int f = 0; f < FR; ++f) b[u][f] = (kok && wok[f]) ? load_bf16x8(wrow[f] + k) : zero_bf16x8();
#pragma unroll
      for (int t = 0; t < MT; ++t) a[u][t] = (kok && aok[t]) ? load_bf16x8(arow[t] + k) : zero_bf16x8();
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int f = 0; f < FR; ++f)
          acc[t][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][t], b[u][f], acc[t][f], 0, 0, 0);
  }

#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int f = 0; f < FR; ++f) {
      const int j = j0 + 16 * f + n;
      if (j >= Vd) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * t + 4 * g + i;
        if (m < M) C[(size_t)m * Vd + j] = acc[t][f][i];
      }
    }
}

// ------------------------------------------------------------------ tiled

constexpr int TBM = 128, TBN = 128, TBK = 64;
constexpr int TLDS_ROW = TBK * 2 + 16;  // bytes per LDS row (16-byte pad)

__device__ __forceinline__ void tile_global_load(uint4 (&regs)[4], const uint16_t* __restrict__ src,
                                                 int row0, int nrows, int k0, int H, int tid) {
  // 128 rows x 64 bf16 = 1024 chunks of 16 bytes; thread takes chunks tid + 256 * p
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int c = tid + 256 * p;
    const int row = c >> 3, col = (c & 7) * 8;
    const int gr = row0 + row, gk = k0 + col;
    regs[p] = (gr < nrows && gk < H) ? *reinterpret_cast<const uint4*>(src + (size_t)gr * H + gk)
                                     : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void tile_lds_store(char* lds, const uint4 (&regs)[4], int tid) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int c = tid + 256 * p;
    const int row = c >> 3, col = (c & 7);
    *reinterpret_cast<uint4*>(lds + row * TLDS_ROW + col * 16) = regs[p];
  }
}

__global__ __launch_bounds__(256) void k1_tiled(const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
                                                float* __restrict__ C, int M, int H, int Vd, int mtiles,
                                                int ntiles) {
  __shared__ __attribute__((aligned(16))) char lds[2][2][TBM * TLDS_ROW];  // [buf][A|W]
  // XCD-aware order: blocks are dispatched round-robin over 8 XCDs; give each XCD
  // a contiguous run of output tiles so neighbouring tiles share LM-head rows in L2.
  const int total = mtiles * ntiles;
  const int per_xcd = (total + 7) / 8;
  const int lin = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (lin >= total) return;
  const int nt = lin / mtiles, mt = lin % mtiles;
  const int m0 = mt * TBM, n0 = nt * TBN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n = lane & 15, g = lane >> 4;

  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int ksteps = (H + TBK - 1) / TBK;
  uint4 ra[4], rw[4];
  tile_global_load(ra, A, m0, M, 0, H, tid);
  tile_global_load(rw, W, n0, Vd, 0, H, tid);
  tile_lds_store(lds[0][0], ra, tid);
  tile_lds_store(lds[0][1], rw, tid);
  __syncthreads();

  for (int ks = 0; ks < ksteps; ++ks) {
    const int cur = ks & 1;
    const bool more = ks + 1 < ksteps;
    if (more) {
      tile_global_load(ra, A, m0, M, (ks + 1) * TBK, H, tid);
      tile_global_load(rw, W, n0, Vd, (ks + 1) * TBK, H, tid);
    }
    const char* la = lds[cur][0];
    const char* lw = lds[cur][1];
#pragma unroll
    for (int s = 0; s < TBK / 32; ++s) {
      bf16x8 af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(la + (wm * 64 + 16 * i + n) * TLDS_ROW + s * 64 + g * 16));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(lw + (wn * 64 + 16 * j + n) * TLDS_ROW + s * 64 + g * 16));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      tile_lds_store(lds[cur ^ 1][0], ra, tid);
      tile_lds_store(lds[cur ^ 1][1], rw, tid);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 64 + 16 * j + n;
      if (col >= Vd) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = m0 + wm * 64 + 16 * i + 4 * g + q;
        if (row < M) C[(size_t)row * Vd + col] = acc[i][j][q];
      }
    }
}

}  // namespace

hipError_t launch_draft_logits(const uint16_t* hidden, const uint16_t* lm_head, float* logits, int M, int H,
                               int Vd, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  if (M <= 64) {
    constexpr int FR = 2;
    const int waves = (Vd + 16 * FR - 1) / (16 * FR);
    const dim3 grid((waves + 3) / 4), block(256);
    if (M <= 16)
      hipLaunchKernelGGL((k1_skinny<FR, 1>), grid, block, 0, stream, hidden, lm_head, logits, M, H, Vd);
    else if (M <= 32)
      hipLaunchKernelGGL((k1_skinny<FR, 2>), grid, block, 0, stream, hidden, lm_head, logits, M, H, Vd);
    else
      hipLaunchKernelGGL((k1_skinny<FR, 4>), grid, block, 0, stream, hidden, lm_head, logits, M, H, Vd);
  } else {
    const int mtiles = (M + TBM - 1) / TBM, ntiles = (Vd + TBN - 1) / TBN;
    const int total = mtiles * ntiles;
    const int per_xcd = (total + 7) / 8;
    const dim3 grid(per_xcd * 8), block(256);
    hipLaunchKernelGGL(k1_tiled, grid, block, 0, stream, hidden, lm_head, logits, M, H, Vd, mtiles, ntiles);
  }
  return hipGetLastError();
}

}  // namespace dspark
