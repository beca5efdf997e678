// Stage 1: draft base logits, logits[m, j] = sum_h hidden[m, h] * lm_head[j, h]
// (bf16 in, fp32 accumulate and out) on gfx950 MFMA (v_mfma_f32_16x16x32_bf16).
//
// Four tilings, picked by the shape (M = B * N, the number of draft positions):
//  * stream (M <= 16, H % 512 == 0, H <= 4096): bound by streaming the LM head
//    from HBM (2 * Vd * H bytes, read once).  One persistent workgroup per CU
//    walks a contiguous run of 16-row blocks of the LM head; each block's rows
//    arrive 512 k at a time (1 KB per row) through a 3-stage LDS ring filled by
//    direct global->LDS loads, so every load instruction reads 1 KB contiguous and
//    two stages stay in flight across the barriers.  The hidden rows sit in
//    registers for the whole kernel (each wave always takes the same 4 k steps of
//    a stage); the 4 waves' partial sums of a block are added in LDS, and the
//    outputs stay in LDS until the stream is done.
//  * skinny (other M <= 64): each wave owns 16*FR vocabulary rows and streams them
//    straight from global memory into MFMA B fragments; the hidden rows (A
//    fragments) come from L1/L2.  No LDS.
//  * ping-pong (M > 64, H % 64 == 0): MFMA-bound.  256 x 256 or 256 x 320 output
//    tiles, 8 waves (two per SIMD), each a 128 x 64 or 128 x 80 block, the two
//    waves of a SIMD in alternating phases over a ring of four BK = 32 stages; the
//    output leaves through LDS in whole rows.  The context-KV product runs the same
//    kernel at 256 x 256 with an epilogue that writes the normalised, rotated K and
//    the V heads to the caches in bf16.
//  * tiled (other M > 64): 128 x 128 output tiles, BK = 64, both operands staged
//    through double-buffered LDS; 4 waves, each a 64 x 64 block of 16x16 MFMA
//    fragments.  Both MFMA tilings take a grouped tile order (a few row tiles at
//    a time), XCD by XCD.
//
// Optional extra row (the confidence head's hidden-state weights): with `wx` set, the
// LM head is read as Vd + 1 rows, row Vd being wx, and output column Vd goes to
// xout[m] instead of the logits.  Every tiling handles it as one more vocabulary row.
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

// row j of the LM head extended by the extra row: j < Vd: lm_head row j; j == Vd: wx
__device__ __forceinline__ const uint16_t* head_row(const uint16_t* W, const uint16_t* wx, int j, int Vd, int H) {
  return j < Vd ? W + (size_t)j * H : wx;
}

// output column j of row m: the logits, or the extra row's output
__device__ __forceinline__ void put_out(float* C, float* xout, int m, int j, int Vd, float v) {
  if (j < Vd) C[(size_t)m * Vd + j] = v;
  else xout[m] = v;
}

// ------------------------------------------------------------------ skinny

template <int FR, int MT>
__global__ __launch_bounds__(256) void k1_skinny(const uint16_t* __restrict__ A,
                                                 const uint16_t* __restrict__ W,
                                                 float* __restrict__ C, int M, int H, int Vd,
                                                 const uint16_t* __restrict__ wx, float* __restrict__ xout) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int Vt = Vd + (wx ? 1 : 0);
  const int j0 = wave * (16 * FR);
  if (j0 >= Vt) return;  // whole wave
  const int n = lane & 15, g = lane >> 4;

  const uint16_t* wrow[FR];
  bool wok[FR];
#pragma unroll
  for (int f = 0; f < FR; ++f) {
    const int j = j0 + 16 * f + n;
    wok[f] = j < Vt;
    wrow[f] = head_row(W, wx, wok[f] ? j : 0, Vd, H);
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
      if (j >= Vt) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * t + 4 * g + i;
        if (m < M) put_out(C, xout, m, j, Vd, acc[t][f][i]);
      }
    }
}

// ------------------------------------------------------------------ stream

constexpr int SNS = 3;                        // ring stages
constexpr int SROW = 1024 + 16;               // LDS bytes per row of a stage (512 k + pad)
constexpr int SSTAGE = 16 * SROW;             // one stage: 16 rows x 512 k
constexpr int SRED = 4 * 64 * 4;              // floats of one block's partial sums (4 waves x 64 lanes x 4)
constexpr int SFIXED = SNS * SSTAGE + 2 * SRED * 4;  // ring + two partial-sum buffers (bytes)
constexpr int SOUT_MAX = 96 * 1024;           // bytes of outputs a workgroup may hold in LDS

__global__ __launch_bounds__(256) void k1_stream(const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
                                                 float* __restrict__ C, int M, int H, int Vd,
                                                 const uint16_t* __restrict__ wx, float* __restrict__ xout) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* ring = smem;
  float* red = reinterpret_cast<float*>(smem + SNS * SSTAGE);  // [2][SRED], by block parity
  float* outl = red + 2 * SRED;                                // [M][16 * blocks] this workgroup's outputs
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int spb = H / 512;  // stages per 16-row block (<= 8)

  // hidden rows: fragment of stage st, k step 4*wave+u (rows >= M are zero)
  bf16x8 af[8][4];
#pragma unroll
  for (int st = 0; st < 8; ++st)
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = st * 512 + (wave * 4 + u) * 32 + 8 * g;
      af[st][u] = (st < spb && n < M) ? load_bf16x8(A + (size_t)n * H + k) : zero_bf16x8();
    }

  // A contiguous run of LM-head rows per workgroup (the row counts differ by at most
  // one, so no workgroup streams a whole block more than another), in 16-row blocks
  // from its first row; the last block may be partial.
  const int Vt = Vd + (wx ? 1 : 0);  // rows, with the extra one
  const int r0 = (int)((long)Vt * blockIdx.x / gridDim.x);
  const int r1 = (int)((long)Vt * (blockIdx.x + 1) / gridDim.x);
  const int nb = (r1 - r0 + 15) / 16, L = 16 * nb;
  const int T = nb * spb;  // stages this workgroup consumes
  // stage t: block t / spb, k range (t % spb) * 512 .. +512; wave w loads rows
  // w, w+4, w+8, w+12 of it (one 1 KB instruction each).  Rows past this run load
  // its last row again (a cache hit, never stored), which keeps four loads per wave
  // and stage for the ring's counted waits.
  auto issue = [&](int t) {
    const int blk = t / spb, kst = t % spb;
    char* base = ring + (t % SNS) * SSTAGE;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = wave + 4 * q;
      const int j = min(r0 + blk * 16 + row, r1 - 1);
      __builtin_amdgcn_global_load_lds(head_row(W, wx, j, Vd, H) + kst * 512 + lane * 8, base + row * SROW, 16, 0, 0);
    }
  };
  // a finished block: wave w adds the four waves' partial sums of output rows
  // 4w .. 4w+3 (MFMA lane groups g = w) and keeps them in LDS
  auto finish_block = [&](int blk_local) {
    const float* rb = red + (blk_local & 1) * SRED;
    const int i = lane >> 4, m = 4 * wave + i;
    float v = rb[(16 * wave + n) * 4 + i];
#pragma unroll
    for (int w = 1; w < 4; ++w) v += rb[(w * 64 + 16 * wave + n) * 4 + i];
    if (m < M) outl[m * L + 16 * blk_local + n] = v;
  };

  for (int t = 0; t < SNS - 1 && t < T; ++t) issue(t);
  floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
  for (int t = 0; t < T; ++t) {
    // this wave's loads of stage t are done once at most (SNS-2) later stages are
    // pending (nothing else touches global memory inside the loop)
    if (t + SNS - 2 < T) asm volatile("s_waitcnt vmcnt(%0)" ::"n"((SNS - 2) * 4) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    lds_barrier();  // every wave's share of stage t is in LDS; stage t-1's buffer is free
    if (t >= 1 && (t - 1) % spb == spb - 1) finish_block((t - 1) / spb);  // its partials are visible now
    if (t + SNS - 1 < T) issue(t + SNS - 1);
    const char* buf = ring + (t % SNS) * SSTAGE;
    const int kst = t % spb;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      if (st != kst) continue;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int s = wave * 4 + u;
        const bf16x8 b =
            __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(buf + n * SROW + (s * 32 + 8 * g) * 2));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[st][u], b, acc, 0, 0, 0);
      }
    }
    if (kst == spb - 1) {  // block done: this wave's partial sums (the buffer alternates,
                           // so a block's sums never overwrite ones still being read)
      *reinterpret_cast<floatx4*>(red + ((t / spb) & 1) * SRED + (wave * 64 + lane) * 4) = acc;
      acc = floatx4{0.f, 0.f, 0.f, 0.f};
    }
  }
  if (T > 0) {
    lds_barrier();
    finish_block(nb - 1);
  }
  __syncthreads();
  // the outputs leave only after the whole stream: a contiguous run of each output
  // row (writes interleaved with the stream cost it several percent)
  for (int m = 0; m < M; ++m)
    for (int x = tid; x < r1 - r0; x += 256) put_out(C, xout, m, r0 + x, Vd, outl[m * L + x]);
}

size_t k1_stream_lds(int M, int Vd, int grid) {
  const size_t maxrows = ((size_t)Vd + grid - 1) / grid;  // the longest run of rows
  const size_t maxb = (maxrows + 15) / 16;
  return SFIXED + (size_t)M * 16 * maxb * 4;
}

int cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// ------------------------------------------------------------------ tiled

constexpr int TBM = 128, TBN = 128, TBK = 64;
constexpr int TLDS_ROW = TBK * 2 + 16;  // bytes per LDS row (16-byte pad)

// rows row0 .. row0+127 of a matrix of nrows rows: row gr < nsrc from src, row nsrc
// (when nrows > nsrc) from the extra row wx
__device__ __forceinline__ void tile_global_load(uint4 (&regs)[4], const uint16_t* __restrict__ src,
                                                 const uint16_t* __restrict__ wx, int row0, int nsrc, int nrows,
                                                 int k0, int H, int tid) {
  // 128 rows x 64 bf16 = 1024 chunks of 16 bytes; thread takes chunks tid + 256 * p
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int c = tid + 256 * p;
    const int row = c >> 3, col = (c & 7) * 8;
    const int gr = row0 + row, gk = k0 + col;
    regs[p] = (gr < nrows && gk < H) ? *reinterpret_cast<const uint4*>(head_row(src, wx, gr, nsrc, H) + gk)
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
                                                int ntiles, const uint16_t* __restrict__ wx,
                                                float* __restrict__ xout) {
  __shared__ __attribute__((aligned(16))) char lds[2][2][TBM * TLDS_ROW];  // [buf][A|W]
  // XCD-aware, grouped order: blocks are dispatched round-robin over 8 XCDs; each
  // XCD takes a contiguous run of the linear tile order, and that order walks groups
  // of kGroupM row tiles column by column, so the ~64 workgroups an XCD runs at once
  // cover about 8 row tiles x 8 column tiles and share both operands' k slices in
  // its L2 (a column-major walk shares only the LM-head rows and re-reads the whole
  // hidden matrix for every column tile).
  constexpr int kGroupM = 8;
  const int total = mtiles * ntiles;
  const int per_xcd = (total + 7) / 8;
  const int lin = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (lin >= total) return;
  const int group = lin / (kGroupM * ntiles), first_m = group * kGroupM;
  const int gm = min(mtiles - first_m, kGroupM), within = lin - group * kGroupM * ntiles;
  const int mt = first_m + within % gm, nt = within / gm;
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
  const int Vt = Vd + (wx ? 1 : 0);
  uint4 ra[4], rw[4];
  tile_global_load(ra, A, nullptr, m0, M, M, 0, H, tid);
  tile_global_load(rw, W, wx, n0, Vd, Vt, 0, H, tid);
  tile_lds_store(lds[0][0], ra, tid);
  tile_lds_store(lds[0][1], rw, tid);
  __syncthreads();

  for (int ks = 0; ks < ksteps; ++ks) {
    const int cur = ks & 1;
    const bool more = ks + 1 < ksteps;
    if (more) {
      tile_global_load(ra, A, nullptr, m0, M, M, (ks + 1) * TBK, H, tid);
      tile_global_load(rw, W, wx, n0, Vd, Vt, (ks + 1) * TBK, H, tid);
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
      if (col >= Vt) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = m0 + wm * 64 + 16 * i + 4 * g + q;
        if (row < M) put_out(C, xout, row, col, Vd, acc[i][j][q]);
      }
    }
}

// ------------------------------------------------------------------ big tiles

// Hidden rows per tile of the many-row products; the epilogue stages each wave's
// 128 x 64 fp32 block in 16 KB of the operand ring (8 waves: 128 KB).
constexpr int BBM = 256;
constexpr int BSTAGE_OUT = 8 * 16384;

__device__ __forceinline__ void dma16_g(const uint16_t* src, char* lds_base) {
  __builtin_amdgcn_global_load_lds(src, lds_base, 16, 0, 0);
}

// bf16 bits of a float, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint4 pack_bf16x8(const float (&v)[8]) {
  return make_uint4(bf16_rne(v[0]) | (bf16_rne(v[1]) << 16), bf16_rne(v[2]) | (bf16_rne(v[3]) << 16),
                    bf16_rne(v[4]) | (bf16_rne(v[5]) << 16), bf16_rne(v[6]) | (bf16_rne(v[7]) << 16));
}

__device__ __forceinline__ void add_bf16x8(float (&v)[8], const uint16_t* b) {
  const uint4 q = *reinterpret_cast<const uint4*>(b);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    v[2 * k] += bf16_to_f32(w[k] & 0xFFFF);
    v[2 * k + 1] += bf16_to_f32(w[k] >> 16);
  }
}

// The K/V product's epilogue over one half of the staged tile (every wave's rows
// 64 h .. 64 h + 63, all 256 columns: two head blocks of 128).  Value (row r of wave
// row-half wm, tile column c) sits in wave (wm | (c / 64) << 1)'s 16 KB block, row r,
// piece (c % 64) / 4 at p ^ (r & 7).  Two threads take one (row, head block): for a K
// block thread t holds the rotary pairs (i, i + 64), i in [32 t, 32 t + 32), eight at a
// time; for a V block the dims [64 t, 64 t + 64).
__device__ __forceinline__ void kv_epilogue_half(const char* smem, int h, int m0, int n0, int M, int ncols,
                                                 const KvEpilogue& ep) {
  const int tid = threadIdx.x, t = tid & 1, item = tid >> 1;
  const int j = item & 1, r = (item >> 1) & 63, wm = item >> 7;
  const int row = m0 + wm * 128 + 64 * h + r;
  const int col0 = n0 + j * 128;              // first column of the head block
  if (row >= M || col0 >= ncols) return;
  const int64_t slot = ep.slots[row];
  if (slot < 0 || slot >= ep.num_slots) return;
  const int hb = col0 / 128, nkv = ep.nkv;
  const int layer = hb / (2 * nkv), isv = (hb / nkv) & 1, head = hb % nkv;
  const size_t cbase = (((size_t)layer * ep.num_slots + slot) * nkv + head) * 128;
  auto lds8 = [&](int c, float (&v)[8]) {     // tile columns c .. c + 7 of this row, c % 8 == 0
    const int wv = wm | ((c >> 6) << 1), p = (c & 63) >> 2;
    const char* base = smem + wv * 16384 + r * 256;
    const floatx4 a = *reinterpret_cast<const floatx4*>(base + ((p ^ (r & 7)) << 4));
    const floatx4 b = *reinterpret_cast<const floatx4*>(base + (((p + 1) ^ (r & 7)) << 4));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[k] = a[k];
      v[4 + k] = b[k];
    }
  };
  if (isv) {
#pragma unroll 2
    for (int q = 0; q < 8; ++q) {
      const int d = 64 * t + 8 * q;
      float v[8];
      lds8(j * 128 + d, v);
      add_bf16x8(v, ep.kv_b + col0 + d);
      *reinterpret_cast<uint4*>(ep.vc + cbase + d) = pack_bf16x8(v);
    }
    return;
  }
  float ss = 0.0f;
#pragma unroll 2
  for (int q = 0; q < 4; ++q) {
    const int i = 32 * t + 8 * q;
    float x[8], y[8];
    lds8(j * 128 + i, x);
    lds8(j * 128 + 64 + i, y);
    add_bf16x8(x, ep.kv_b + col0 + i);
    add_bf16x8(y, ep.kv_b + col0 + 64 + i);
#pragma unroll
    for (int k = 0; k < 8; ++k) ss = fmaf(x[k], x[k], fmaf(y[k], y[k], ss));
  }
  ss += __shfl_xor(ss, 1);
  const float inv = 1.0f / sqrtf(ss / 128.0f + ep.eps);
  const uint16_t* kw = ep.knorm_w + (size_t)layer * 128;
  const float* cs = ep.rope + (size_t)row * 128;
#pragma unroll 2
  for (int q = 0; q < 4; ++q) {
    const int i = 32 * t + 8 * q;
    float x[8], y[8], wx[8] = {}, wy[8] = {};
    lds8(j * 128 + i, x);
    lds8(j * 128 + 64 + i, y);
    add_bf16x8(x, ep.kv_b + col0 + i);
    add_bf16x8(y, ep.kv_b + col0 + 64 + i);
    add_bf16x8(wx, kw + i);
    add_bf16x8(wy, kw + 64 + i);
    const float4 c0 = *reinterpret_cast<const float4*>(cs + i), c1 = *reinterpret_cast<const float4*>(cs + i + 4);
    const float4 s0 = *reinterpret_cast<const float4*>(cs + 64 + i);
    const float4 s1 = *reinterpret_cast<const float4*>(cs + 64 + i + 4);
    const float c[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
    const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
    float lo[8], hi[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float a = x[k] * inv * wx[k], b = y[k] * inv * wy[k];
      lo[k] = a * c[k] - b * sn[k];
      hi[k] = b * c[k] + a * sn[k];
    }
    *reinterpret_cast<uint4*>(ep.kc + cbase + i) = pack_bf16x8(lo);
    *reinterpret_cast<uint4*>(ep.kc + cbase + 64 + i) = pack_bf16x8(hi);
  }
}

// The plain product at many rows: 256 x 64 NB output tiles (NB = 4 or 5 LM-head
// fragments per wave), eight waves (two per SIMD), with the two waves of each SIMD in
// alternating phases.  Group X = waves 0-3, group Y = waves 4-7 (one of each per SIMD);
// wave w owns hidden rows 128 (w & 1) .. +127 and LM-head rows 16 NB (w >> 1) .. +16 NB - 1
// of the tile (8 x NB fragments).  The k dimension runs in BK = 32 stages through a
// ring of four LDS buffers:
//   phase 2t:   X reads stage t's fragments and issues the A rows of stage t + 3;
//               Y runs the MFMAs of stage t - 1;
//   phase 2t+1: X runs the MFMAs of stage t; Y reads stage t and issues the W rows of
//               stage t + 3.
// Every phase ends with a workgroup barrier, so on every SIMD one wave's MFMAs run
// while the other waits on LDS.  Stage t + 3 goes into the buffer of stage t - 1, whose
// last reader (Y, phase 2t - 1) is done before the barrier that opens phase 2t; each
// group waits for its half of stage t + 1 before the barrier that closes phase 2t + 1,
// so a stage's DMA has five or six phases to land.  LDS rows are 64 bytes (32 bf16):
// logical piece p of row r sits at slot (p + (r >> 1)) & 3.  Rotating the pieces by
// row pairs keeps a fragment read (16 rows x 4 pieces) free of bank conflicts on
// gfx950, which a rotation by groups of four rows is not (it read LDS at 58% of the
// conflict-free rate).  NB = 5 does 40 MFMAs per phase instead of 32 against the same
// barrier and moves fewer LDS and L2 bytes per flop.  The accumulation order over k is
// that of every other tiling here, so the extra row (wx) and the two tile widths
// leave the logits' bits unchanged.  Requires H % 32 == 0.
constexpr int PK = 32, PNS = 4, PWOFF = BBM * PK * 2;
__host__ __device__ constexpr int pp_stage(int NB) { return (BBM + 64 * NB) * PK * 2; }
__host__ __device__ constexpr int pp_lds(int NB) { return PNS * pp_stage(NB); }
static_assert(pp_lds(4) >= BSTAGE_OUT && pp_lds(5) >= BSTAGE_OUT, "the epilogue stages 8 x 16 KB in the ring");

// kKV (NB = 4): the context-KV product, the normalised context states (A, M x H) times
// every layer's fused K/V weights (W, Vd = L * 2 * nkv * 128 rows); a 256-column tile
// holds two whole heads, and the epilogue (kv_epilogue_half) adds the bias, normalises
// and rotates the K heads and writes both caches in bf16 (C, wx, xout unused).
template <int NB, bool kKV>
__global__ __launch_bounds__(512) void k1_pingpong(const uint16_t* __restrict__ A, const uint16_t* __restrict__ W,
                                                   float* __restrict__ C, int M, int H, int Vd, int mtiles,
                                                   int ntiles, const uint16_t* __restrict__ wx,
                                                   float* __restrict__ xout, const KvEpilogue ep) {
  static_assert(!kKV || NB == 4, "the cache-writing epilogue takes 256-column tiles");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int kGroupM = 4;
  constexpr int TN = 64 * NB;           // LM-head rows per tile
  constexpr int PSTAGE = pp_stage(NB);
  constexpr int NI = NB;                // DMA instructions per wave and stage of group Y (X: 4)
  const int total = mtiles * ntiles;
  const int per_xcd = (total + 7) / 8;
  const int lin = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (lin >= total) return;
  const int group = lin / (kGroupM * ntiles), first_m = group * kGroupM;
  const int gm = min(mtiles - first_m, kGroupM), within = lin - group * kGroupM * ntiles;
  const int mt = first_m + within % gm, nt = within / gm;
  const int m0 = mt * BBM, n0 = nt * TN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, w4 = wave & 3;
  const int wm = wave & 1, wn = wave >> 1;  // hidden-row half, LM-head-row quarter
  const int n = lane & 15, g = lane >> 4;

  // DMA: X fills the A rows, Y the W rows of a stage.  X wave w4 takes A rows
  // 64 w4 + 16 u .. +15 (u = 0..3), Y wave w4 W rows 16 NB w4 + 16 u .. +15
  // (u = 0..NB-1); lane L row 16 u + L / 4 of them, LDS slot L % 4, which holds
  // logical piece (L % 4 - L / 8) & 3 (both row bases are multiples of 8).  Each lane
  // keeps a pointer per instruction: hidden rows past the last are clamped to it, and
  // LM-head rows from Vd on are the extra row wx if there is one, else row Vd - 1
  // (outputs past the last column are never stored).
  const int rbase = grp == 0 ? 64 * w4 : 16 * NB * w4;
  const char* srcp[NI];
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    const int r = rbase + 16 * u + (lane >> 2);
    const int p = ((lane & 3) - (lane >> 3)) & 3;
    const uint16_t* row;
    if (grp == 0) row = A + (size_t)min(m0 + r, M - 1) * H;
    else row = (n0 + r < Vd) ? W + (size_t)(n0 + r) * H : (wx != nullptr ? wx : W + (size_t)(Vd - 1) * H);
    srcp[u] = reinterpret_cast<const char*>(row) + p * 16;
  }
  const int dst0 = (grp == 0 ? 0 : PWOFF) + rbase * (PK * 2);
  auto issue = [&](int t) {
    char* st = smem + (t % PNS) * PSTAGE + dst0;
#pragma unroll
    for (int u = 0; u < NI; ++u)
      if (grp == 1 || u < 4)
        dma16_g(reinterpret_cast<const uint16_t*>(srcp[u] + t * PK * 2), st + 16 * u * (PK * 2));
  };

  floatx4 acc[8][NB];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};
  // fragment reads: row 16 i + n of the wave's rows, logical piece g
  const int slot = ((g + (n >> 1)) & 3) * 16;
  const int ard = (wm * 128 + n) * (PK * 2) + slot, brd = PWOFF + (wn * 16 * NB + n) * (PK * 2) + slot;
  bf16x8 af[8], bf[NB];
  auto read = [&](int t) {
    const char* st = smem + (t % PNS) * PSTAGE;
#pragma unroll
    for (int j = 0; j < NB; ++j)
      bf[j] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(st + brd + j * 16 * (PK * 2)));
#pragma unroll
    for (int i = 0; i < 8; ++i)
      af[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(st + ard + i * 16 * (PK * 2)));
  };
  auto mfma = [&]() {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_s_setprio(0);
  };
  // wait until this wave's DMA of stage s has landed, stages up to `last` issued (n
  // instructions each, completing in order; n = 4 for X, NB for Y)
  auto wait_stage = [&](int s, int last) {
    const int after = last - s;
    if (grp == 0 || NB == 4) {
      if (after >= 2) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
      else if (after == 1) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
      static_assert(NB == 4 || NB == 5, "the waits below count five instructions per stage");
      if (after >= 2) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
      else if (after == 1) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
  };

  const int KT = H / PK;
  const int pro = min(3, KT);
  for (int t = 0; t < pro; ++t) issue(t);
  wait_stage(0, pro - 1);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  if (grp == 0) {
    for (int t = 0; t < KT; ++t) {
      read(t);                                                   // phase 2t
      __builtin_amdgcn_sched_barrier(0);
      if (t + 3 < KT) issue(t + 3);
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      mfma();                                                    // phase 2t + 1
      __builtin_amdgcn_sched_barrier(0);
      if (t + 1 < KT) wait_stage(t + 1, min(t + 3, KT - 1));
      asm volatile("s_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    asm volatile("s_barrier" ::: "memory");                      // phase 0
    __builtin_amdgcn_sched_barrier(0);
    for (int t = 0; t < KT; ++t) {
      read(t);                                                   // phase 2t + 1
      __builtin_amdgcn_sched_barrier(0);
      if (t + 3 < KT) issue(t + 3);
      if (t + 1 < KT) wait_stage(t + 1, min(t + 3, KT - 1));
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      mfma();                                                    // phase 2t + 2
      __builtin_amdgcn_sched_barrier(0);
      if (t + 1 < KT) asm volatile("s_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Every stage has been read and no DMA is in flight (X passed the last common
  // barrier after Y's last reads; Y's last MFMAs touch registers only).  Fragments
  // j = 0..3 of each wave (128 x 64) are staged in the wave's own 16 KB of the ring,
  // in two halves of 64 rows, and leave as whole 256-byte row pieces; fragment j = 4
  // (NB = 5) is stored straight from the accumulators, 64 bytes per row.  Column Vd
  // (the extra row's output) goes to xout.
  char* stage = smem + wave * 16384;
  if constexpr (kKV) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h == 1) __syncthreads();   // every (row, head) item of half 0 is done with the staging
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 16 * i + n, p = 4 * j + g;
          *reinterpret_cast<floatx4*>(stage + r * 256 + ((p ^ (r & 7)) * 16)) = acc[4 * h + i][j];
        }
      __syncthreads();
      kv_epilogue_half(smem, h, m0, n0, M, Vd, ep);
    }
    return;
  }
  const bool vec = (Vd % 4 == 0) && ((reinterpret_cast<uintptr_t>(C) & 15) == 0);
  const int cbase = n0 + wn * 16 * NB;
  const int Vt = Vd + (wx != nullptr ? 1 : 0);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * i + n, p = 4 * j + g;
        *reinterpret_cast<floatx4*>(stage + r * 256 + ((p ^ (r & 7)) * 16)) = acc[4 * h + i][j];
      }
#pragma unroll 4
    for (int t = 0; t < 16; ++t) {
      const int r = 4 * t + (lane >> 4), p = lane & 15;
      const floatx4 v = *reinterpret_cast<const floatx4*>(stage + r * 256 + ((p ^ (r & 7)) * 16));
      const int row = m0 + wm * 128 + 64 * h + r, col = cbase + 4 * p;
      if (row >= M || col >= Vt) continue;
      if (vec && col + 3 < Vd) {
        // streamed out: the logits are read back only by the next stage
        __builtin_nontemporal_store(v, reinterpret_cast<floatx4*>(C + (size_t)row * Vd + col));
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (col + q < Vt) put_out(C, xout, row, col + q, Vd, v[q]);
      }
    }
  }
  if constexpr (NB == 5) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = m0 + wm * 128 + 16 * i + n, col = cbase + 64 + 4 * g;
      if (row >= M || col >= Vt) continue;
      if (vec && col + 3 < Vd) {
        *reinterpret_cast<floatx4*>(C + (size_t)row * Vd + col) = acc[i][4];
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (col + q < Vt) put_out(C, xout, row, col + q, Vd, acc[i][4][q]);
      }
    }
  }
}

// Fragments per wave for the plain product: the one with fewer fragment-waves of tiles
// over the chip (ties: five, which does more MFMAs per barrier)
int pingpong_nb(int M, int Vd, int cus) {
  const long mt = (M + BBM - 1) / BBM;
  const long w4 = (mt * ((Vd + 255) / 256) + cus - 1) / cus * 4;
  const long w5 = (mt * ((Vd + 319) / 320) + cus - 1) / cus * 5;
  return w5 <= w4 ? 5 : 4;
}

template <int NB>
hipError_t launch_pingpong(const uint16_t* hidden, const uint16_t* lm_head, float* logits, int M, int H, int Vd,
                           const uint16_t* wx, float* xout, hipStream_t stream) {
  static bool attr_set[64] = {false};
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev >= 0 && dev < 64 && !attr_set[dev]) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k1_pingpong<NB, false>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, pp_lds(NB));
    if (e != hipSuccess) return e;
    attr_set[dev] = true;
  }
  const int Vt = Vd + (wx != nullptr ? 1 : 0);
  const int mtiles = (M + BBM - 1) / BBM, ntiles = (Vt + 64 * NB - 1) / (64 * NB);
  const int per_xcd = (mtiles * ntiles + 7) / 8;
  hipLaunchKernelGGL((k1_pingpong<NB, false>), dim3(per_xcd * 8), dim3(512), pp_lds(NB), stream, hidden, lm_head,
                     logits, M, H, Vd, mtiles, ntiles, wx, xout, KvEpilogue{});
  return hipSuccess;
}

}  // namespace

hipError_t launch_draft_logits(const uint16_t* hidden, const uint16_t* lm_head, float* logits, int M, int H,
                               int Vd, const uint16_t* wx, float* xout, hipStream_t stream) {
  if (M <= 0) return hipSuccess;
  const int Vt = Vd + (wx ? 1 : 0);  // LM-head rows including the extra one
  const int sgrid = min(cu_count(), (Vt + 15) / 16);
  // (at least half of a CU's 160 KB: one stream workgroup per CU, also when another
  // stream's kernels fill the chip at the same time; two on one CU would halve both)
  const size_t slds = std::max(k1_stream_lds(M, Vt, sgrid), (size_t)(81 * 1024));
  if (M <= 16 && H % 512 == 0 && H <= 4096 && slds <= SFIXED + SOUT_MAX) {
    static bool attr_set[64] = {false};
    int dev = 0;
    (void)hipGetDevice(&dev);
    if (dev >= 0 && dev < 64 && !attr_set[dev]) {
      const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k1_stream),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, SFIXED + SOUT_MAX);
      if (e != hipSuccess) return e;
      attr_set[dev] = true;
    }
    hipLaunchKernelGGL(k1_stream, dim3(sgrid), dim3(256), slds, stream, hidden, lm_head, logits, M, H, Vd, wx,
                       xout);
  } else if (M <= 64) {
    constexpr int FR = 2;
    const int waves = (Vt + 16 * FR - 1) / (16 * FR);
    const dim3 grid((waves + 3) / 4), block(256);
    if (M <= 16)
      hipLaunchKernelGGL((k1_skinny<FR, 1>), grid, block, 0, stream, hidden, lm_head, logits, M, H, Vd, wx, xout);
    else if (M <= 32)
      hipLaunchKernelGGL((k1_skinny<FR, 2>), grid, block, 0, stream, hidden, lm_head, logits, M, H, Vd, wx, xout);
    else
      hipLaunchKernelGGL((k1_skinny<FR, 4>), grid, block, 0, stream, hidden, lm_head, logits, M, H, Vd, wx, xout);
  } else if (H % 64 == 0) {
    const hipError_t e = pingpong_nb(M, Vt, cu_count()) == 5
                             ? launch_pingpong<5>(hidden, lm_head, logits, M, H, Vd, wx, xout, stream)
                             : launch_pingpong<4>(hidden, lm_head, logits, M, H, Vd, wx, xout, stream);
    if (e != hipSuccess) return e;
  } else {
    const int mtiles = (M + TBM - 1) / TBM, ntiles = (Vt + TBN - 1) / TBN;
    const int total = mtiles * ntiles;
    const int per_xcd = (total + 7) / 8;
    const dim3 grid(per_xcd * 8), block(256);
    hipLaunchKernelGGL(k1_tiled, grid, block, 0, stream, hidden, lm_head, logits, M, H, Vd, mtiles, ntiles, wx,
                       xout);
  }
  return hipGetLastError();
}

bool kv_product_fused(int M, int Hd, int hd) { return hd == 128 && M > 64 && Hd % 64 == 0; }

hipError_t launch_kv_product(const uint16_t* normed, const uint16_t* kv_w, int M, int Hd, int ncols,
                             const KvEpilogue& ep, hipStream_t stream) {
  static bool attr_set[64] = {false};
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev >= 0 && dev < 64 && !attr_set[dev]) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k1_pingpong<4, true>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, pp_lds(4));
    if (e != hipSuccess) return e;
    attr_set[dev] = true;
  }
  const int mtiles = (M + BBM - 1) / BBM, ntiles = (ncols + 255) / 256;
  const int per_xcd = (mtiles * ntiles + 7) / 8;
  hipLaunchKernelGGL((k1_pingpong<4, true>), dim3(per_xcd * 8), dim3(512), pp_lds(4), stream, normed, kv_w, nullptr,
                     M, Hd, ncols, mtiles, ntiles, nullptr, nullptr, ep);
  return hipGetLastError();
}

}  // namespace dspark
