// Small-batch LLVQ dequant-GEMM on matrix cores (gfx950): y[n][r] = sum_k W[r][k] x[n][k]
// for 2 <= batch <= 16 bf16 activation rows.  Included once by llvq.hip after
// llvq_tile.h.
//
// A workgroup owns groups of 16 rows.  The row group is processed in column chunks of
// at most w blocks: the tile engine decodes the 16 x w blocks into the LDS byte tile,
// then each wave runs one v_mfma_f32_16x16x32_bf16 per block column it owns:
//   A (16 x 32): the block's 24 values of the 16 rows as exact small integers in bf16,
//                the last 8 k zero;
//   B (32 x 16): the block's 24 activations of every batch row, read from global memory;
//   C (16 x 16): the block's dot products, scaled by each row's block scale and added to
//                the wave's accumulator (the scale differs per block, so every block has
//                its own product).
// After the row group the 16 waves' accumulators are summed in a fixed order.  The
// result does not depend on scheduling, and all rounding is fp32 accumulation.

#pragma once

typedef __bf16 llvq_bf16x8 __attribute__((ext_vector_type(8)));
typedef float llvq_f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGRows = 16;   // rows per group (MFMA M)

struct GArgs {
  EArgs e;        // engine layout; e.xs = byte tile, e.xsum = wave accumulators
  int w;          // blocks per column chunk
  int nchunk;     // column chunks per row group
  int ngroups;    // row groups
  int batch;
};

// 8 biased value bytes -> 8 bf16 values (byte - 12, exact)
__device__ __forceinline__ llvq_bf16x8 bytes_to_bf16x8(uint2 u) {
  float v[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) v[q] = (float)(((q < 4 ? u.x : u.y) >> (8 * (q & 3))) & 0xffu) - (float)kBias;
  const uint4 pk = make_uint4(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]),
                              pack_bf16(v[6], v[7]));
  return __builtin_bit_cast(llvq_bf16x8, pk);
}

__global__ __launch_bounds__(kEThreads) void k_gemm_mfma(KDesc d, GArgs g, const uint8_t* __restrict__ packed,
                                                          const __half* __restrict__ scales,
                                                          const uint16_t* __restrict__ x, float* __restrict__ y,
                                                          int32_t* err) {
  extern __shared__ __align__(16) uint8_t smem[];
  const ELayout& L = g.e.L;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kb = d.kb;
  const int K = d.cols;
  const bool sg = d.mode == LLVQ_MODE_SHAPEGAIN;
  const uint32_t tb = g.e.xs;
  float* red = reinterpret_cast<float*>(smem + g.e.xsum);   // [kEWaves][64][4]
  const bool xa16 = ((((uintptr_t)x) & 15u) == 0u) && ((K & 7) == 0);

  engine_prologue(smem, L, d, g.e.nbuckets, scales, tid);
  int* ctr = reinterpret_cast<int*>(smem + L.buf[0].ctr);
  int* work = reinterpret_cast<int*>(smem + L.work);
  const float* part = reinterpret_cast<const float*>(smem + L.buf[0].part);

  // lane roles in the MFMA: A row / B column = lane % 16, k group = lane / 16
  const int mr = lane & 15;
  const int kg = lane >> 4;

  for (int grp = blockIdx.x; grp < g.ngroups; grp += gridDim.x) {
    const int row0 = grp * kGRows;
    const int nrows = min(kGRows, d.rows - row0);
    llvq_f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int cc = 0; cc < g.nchunk; ++cc) {
      const int b0 = cc * g.w;
      const int w = min(g.w, kb - b0);
      const int T = nrows * w;
      if (tid == 0) { ctr[0] = 0; ctr[1] = 0; work[0] = 0; }
      __syncthreads();
      const TileMap tm = {(uint32_t)(row0 * kb + b0), (uint32_t)w, (uint32_t)kb, 1.0f / (float)w};
      if (wave * kEUnit < T) classify_unit(smem, L, L.buf[0], d, packed, tm, T, wave, lane, err, true);
      __syncthreads();
      const int nodd = ctr[0];
      const int neven = ctr[1];
      const int nco = (nodd + 63) >> 6;
      const int nch = nco + ((neven + 63) >> 6);
      for (;;) {
        int c = 0;
        if (lane == 0) c = atomicAdd(&work[0], 1);
        c = __builtin_amdgcn_readfirstlane(c);
        if (c >= nch) break;
        bytes_chunk(smem, L, L.buf[0], tb, T, c, nco, nodd, neven, lane);
      }
      __syncthreads();

      // ---- matrix-core phase: wave takes block columns wave, wave + 16, ...
      const uint32_t rowbytes = 24u * (uint32_t)w;
      for (int bl = wave; bl < w; bl += kEWaves) {
        uint2 ab = make_uint2(0x0c0c0c0cu, 0x0c0c0c0cu);   // value 0
        if (kg < 3 && mr < nrows)
          ab = *reinterpret_cast<const uint2*>(smem + tb + (uint32_t)mr * rowbytes + 24u * (uint32_t)bl + 8u * kg);
        const llvq_bf16x8 av = bytes_to_bf16x8(ab);
        uint4 xb = make_uint4(0u, 0u, 0u, 0u);
        const int col = (b0 + bl) * 24 + 8 * kg;
        if (kg < 3 && mr < g.batch) {
          const uint16_t* xr = x + (size_t)mr * (size_t)K;
          if (xa16 && col + 8 <= K) {
            xb = *reinterpret_cast<const uint4*>(xr + col);
          } else {
            uint32_t wv[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int q = 0; q < 8; ++q)
              if (col + q < K) wv[q >> 1] |= (uint32_t)xr[col + q] << (16 * (q & 1));
            xb = make_uint4(wv[0], wv[1], wv[2], wv[3]);
          }
        }
        const llvq_bf16x8 bv = __builtin_bit_cast(llvq_bf16x8, xb);
        const llvq_f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
        const llvq_f32x4 cb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, zero, 0, 0, 0);
        // D rows 4 kg + i, column mr; scale of (row, block) from the engine's slot
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 4 * kg + i;
          const float sc = r < nrows ? part[r * w + bl] : 0.0f;
          acc[i] = __builtin_fmaf(sc, cb[i], acc[i]);
        }
      }
      __syncthreads();
    }
    // ---- reduce the waves' accumulators in a fixed order
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * 64 + lane) * 4 + i] = acc[i];
    __syncthreads();
    if (tid < kGRows * 16) {
      const int r = tid >> 4;       // row in group
      const int n = tid & 15;       // batch row
      const int l = n + 16 * (r >> 2);
      const int i = r & 3;
      float s = 0.0f;
      for (int wv = 0; wv < kEWaves; ++wv) s += red[(wv * 64 + l) * 4 + i];
      if (r < nrows && n < g.batch) {
        const float rs = sg ? 1.0f : __half2float(scales[row0 + r]);
        y[(size_t)n * d.rows + row0 + r] = s * rs;
      }
    }
    __syncthreads();
  }
}
