// Small-batch LLVQ dequant-GEMM on matrix cores (gfx950): y[n][r] = sum_k W[r][k] x[n][k]
// for 2 <= batch <= 16 bf16 activation rows.  Included once by llvq.hip after
// llvq_tile.h.
//
// A workgroup owns groups of 16 rows.  The row group is processed in column chunks of
// at most w blocks: the tile engine decodes the 16 x w blocks into the LDS byte tile,
// then each wave takes the block columns it owns through the matrix cores
// (v_mfma_f32_16x16x32_bf16, D = A B + C):
//   A (16 x 32): the block's 24 activations of every batch row (k 24..31 zero), read
//                from global memory with buffer loads (lanes without data read zeros);
//   B (32 x 16): the block's 24 biased value bytes (v + 12) of the 16 rows as exact bf16
//                integers, with a second product against a constant -12 operand removing
//                the bias, so the byte -> bf16 conversion is one instruction per value;
//   D (16 x 16): the block's dot products of every (batch row, row) pair; each lane holds
//                one weight row and four batch rows, so the block scale of the row is a
//                single LDS read, applied with four fused multiply-adds into the wave's
//                accumulator (the scale differs per block, so every block has its own
//                product).
// After the row group the 16 waves' accumulators are summed in a fixed order.  The
// result does not depend on scheduling, and all rounding is fp32 accumulation.
//
// Phases of a workgroup, over its chunks q = 0, 1, ... (row groups in grid stride, column
// chunks in order):
//   decode q:      the chunk's queue entries -> byte tile;
//   products q + classification q + 1: the matrix-core work of chunk q, while the waves
//                  with a classification unit of chunk q + 1 first classify it.  The queue
//                  is free once decode q has ended; the block scales and fill counters
//                  alternate between two sets, so chunk q's scales stay readable.
// One barrier ends each phase; after the last chunk of a row group the accumulators are
// summed through the byte tile (two more barriers).

#pragma once

typedef __bf16 llvq_bf16x8 __attribute__((ext_vector_type(8)));
typedef float llvq_f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGRows = 16;   // rows per group (MFMA M)

struct GArgs {
  EArgs e;        // engine layout (one tile buffer); e.xs = byte tile and reduction buffer
  uint32_t part2; // the second block-scale array
  int rbal;       // block columns that weigh as much as one classification unit
  int w;          // blocks per column chunk
  int nchunk;     // column chunks per row group
  int ngroups;    // row groups
  int batch;
};

// 8 biased value bytes -> 8 bf16 values of the bytes themselves (0..24, exact)
__device__ __forceinline__ llvq_bf16x8 biased_to_bf16x8(uint2 u) {
  float v[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) v[q] = (float)(((q < 4 ? u.x : u.y) >> (8 * (q & 3))) & 0xffu);
  const uint4 pk = make_uint4(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]),
                              pack_bf16(v[6], v[7]));
  return __builtin_bit_cast(llvq_bf16x8, pk);
}

// Block columns [*cb, *cb + *n) of wave `wave` among w columns, when waves 0..ncls-1 also
// classify one unit each and a unit weighs as much as `rbal` columns: every wave gets the
// same total weight as far as whole columns allow (a fixed function of its arguments, so
// the accumulation order does not depend on scheduling).
__device__ __forceinline__ void column_range(int w, int ncls, int rbal, int wave, int* cb, int* n) {
  const int nfree = kEWaves - ncls;
  if (nfree > 0 && w < nfree * rbal) {   // the waves without a unit take every column
    const int a = w / nfree, r = w % nfree, i = wave - ncls;
    *cb = i < 0 ? 0 : i * a + min(i, r);
    *n = i < 0 ? 0 : a + (i < r ? 1 : 0);
    return;
  }
  const int base = w - nfree * rbal;   // columns beyond the waves' unit weights
  const int b = base / kEWaves, r = base % kEWaves;
  *cb = wave * b + min(wave, r) + rbal * max(0, wave - ncls);
  *n = b + (wave < r ? 1 : 0) + (wave >= ncls ? rbal : 0);
}

// One block column through the matrix cores: acc[i] += sc * sum_k xa[4 kg + i][k] (w[mr][k] - 12)
// for this lane's weight row mr and batch rows 4 kg + i.
__device__ __forceinline__ void mfma_column(llvq_f32x4& acc, llvq_u32x4 xa, uint2 wb, float sc,
                                            llvq_bf16x8 m12) {
  const llvq_bf16x8 av = __builtin_bit_cast(llvq_bf16x8, xa);
  const llvq_f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
  llvq_f32x4 cb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, m12, zero, 0, 0, 0);
  cb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, biased_to_bf16x8(wb), cb, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(sc, cb[i], acc[i]);
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
  float* red = reinterpret_cast<float*>(smem + tb);   // [kEWaves][64][4], between row groups
  const bool xa16 = ((((uintptr_t)x) & 15u) == 0u) && ((K & 7) == 0);
  int* work = reinterpret_cast<int*>(smem + L.work);   // [0] decode items, [2..3] counters of set 1
  // scale arrays and fill counters of even / odd chunks; the queue is shared
  const TileBuf set0 = L.buf[0];
  const TileBuf set1 = {L.work + 8u, L.buf[0].queue, g.part2};

  // chunk q of this workgroup
  struct Chunk {
    int grp, cc, b0, w, nrows, T;
  };
  auto chunk = [&](int q) {
    Chunk c;
    c.grp = blockIdx.x + (q / g.nchunk) * (int)gridDim.x;
    c.cc = q % g.nchunk;
    c.b0 = c.cc * g.w;
    c.w = min(g.w, kb - c.b0);
    c.nrows = min(kGRows, d.rows - c.grp * kGRows);
    c.T = c.nrows * c.w;
    return c;
  };
  auto tile_map = [&](const Chunk& c) {
    return TileMap{(uint32_t)(c.grp * kGRows * kb + c.b0), (uint32_t)c.w, (uint32_t)kb, 1.0f / (float)c.w};
  };
  // the grid never exceeds the group count
  const int nq = ((g.ngroups - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x) * g.nchunk;

  // classification of chunk 0: its fields are requested before the tables are staged (a
  // wave without a unit reads the chunk's last unit and ignores it; a chunk holds at most
  // 16 x 256 blocks, one unit per wave)
  {
    const Chunk c0 = chunk(0);
    const UnitFields uf0 = load_unit(d, packed, tile_map(c0), c0.T, min(wave, (c0.T - 1) / kEUnit), lane);
    engine_prologue(smem, L, d, g.e.nbuckets, scales, tid);
    if (tid == 0) {
      int* c0c = reinterpret_cast<int*>(smem + set0.ctr);
      int* c1c = reinterpret_cast<int*>(smem + set1.ctr);
      c0c[0] = 0; c0c[1] = 0; c1c[0] = 0; c1c[1] = 0; work[0] = 0;
    }
    __syncthreads();
    if (wave * kEUnit < c0.T) classify_fields(smem, L, set0, d, uf0, c0.T, wave, lane, err, true);
    __syncthreads();
  }

  // lane roles in the MFMA: A row (batch row) / B column (weight row) = lane % 16,
  // k group = lane / 16
  const int mr = lane & 15;
  const int kg = lane >> 4;
  const bool xlane = kg < 3 && mr < g.batch;
  // activations as a buffer resource: reads past the end of x return zeros
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(x), (short)0, g.batch * K * 2, 0x00020000);
  const llvq_bf16x8 m12 = __builtin_bit_cast(llvq_bf16x8, llvq_u32x4{0xc140c140u, 0xc140c140u, 0xc140c140u, 0xc140c140u});

  llvq_f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int q = 0; q < nq; ++q) {
    const Chunk c = chunk(q);
    const TileBuf cur = (q & 1) ? set1 : set0;
    const TileBuf nxt = (q & 1) ? set0 : set1;
    const int b0 = c.b0;
    const int w = c.w;

    // ---- decode of chunk q into the byte tile
    {
      const int* ctr = reinterpret_cast<const int*>(smem + cur.ctr);
      const int nodd = ctr[0];
      const int neven = ctr[1];
      const int nco = (nodd + 63) >> 6;
      const int nch = nco + ((neven + 63) >> 6);
      if (tid == 0) {   // counters of chunk q + 1 (last read by decode q - 1)
        int* cn = reinterpret_cast<int*>(smem + nxt.ctr);
        cn[0] = 0;
        cn[1] = 0;
      }
      for (;;) {
        int ci = 0;
        if (lane == 0) ci = atomicAdd(&work[0], 1);
        ci = __builtin_amdgcn_readfirstlane(ci);
        if (ci >= nch) break;
        bytes_chunk(smem, L, cur, tb, c.T, ci, nco, nodd, neven, lane);
      }
    }
    // fields of this wave's classification unit of chunk q + 1, requested as the wave runs
    // out of decode work so that they arrive during the wait for the other waves
    const bool more = q + 1 < nq;
    const Chunk cn = chunk(more ? q + 1 : q);
    UnitFields uf;
    if (more && wave * kEUnit < cn.T) uf = load_unit(d, packed, tile_map(cn), cn.T, wave, lane);
    __syncthreads();
    if (tid == 0) work[0] = 0;

    // ---- classification of chunk q + 1 (waves with a unit)
    if (more && wave * kEUnit < cn.T) classify_fields(smem, L, nxt, d, uf, cn.T, wave, lane, err, true);

    // ---- chunk q through the matrix cores: wave takes the block columns [cb, cb + ncw).
    // The lane (mr, kg) reads 8 value bytes of row mr at k = 8 kg (k 24..31 read the next
    // bytes: finite values that meet zero activations), the block scale of row mr, and 8
    // activations of batch row mr.  Rows past nrows read stale finite bytes and stale
    // scales; they only reach accumulators of rows that are never written.
    {
      int cb, ncw;
      column_range(w, more ? min(kEWaves, (cn.T + kEUnit - 1) / kEUnit) : 0, g.rbal, wave, &cb, &ncw);
      const uint32_t rowbytes = 24u * (uint32_t)w;
      const uint32_t abase = tb + (uint32_t)mr * rowbytes + 24u * (uint32_t)cb + 8u * (uint32_t)kg;
      const uint32_t pbase = cur.part + 4u * ((uint32_t)mr * (uint32_t)w + (uint32_t)cb);
      if (xa16) {
        // With K % 8 == 0 a lane's 8 activations are all inside the row or all past it,
        // except in a last block of K % 24 columns, which its wave takes separately.
        const bool tail = (K % 24 != 0) && (b0 + w == kb) && ncw > 0 && cb + ncw == w;
        const int nfast = ncw - (tail ? 1 : 0);
        const int nfull = nfast >> 2;
        const int rem = nfast & 3;
        // byte offset of this lane's activations in column j = 0; column j adds 48 j
        const uint32_t vbase =
            xlane ? 2u * ((uint32_t)mr * (uint32_t)K + (uint32_t)(b0 + cb) * 24u + 8u * (uint32_t)kg) : 0x80000000u;
        llvq_u32x4 xa[4], xb[4];
        auto xload = [&](llvq_u32x4 (&xv)[4], int s4) {
          const uint32_t vo = vbase + 192u * (uint32_t)s4;
#pragma unroll
          for (int t = 0; t < 4; ++t) xv[t] = __builtin_amdgcn_raw_buffer_load_b128(xrs, vo + 48u * t, 0, 0);
        };
        auto batch = [&](const llvq_u32x4 (&xv)[4], int s4) {
          const uint32_t ao = abase + 96u * (uint32_t)s4;
          const uint32_t po = pbase + 16u * (uint32_t)s4;
          uint2 wb[4];
          float sc[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            wb[t] = *reinterpret_cast<const uint2*>(smem + ao + 24u * t);
            sc[t] = *reinterpret_cast<const float*>(smem + po + 4u * t);
          }
#pragma unroll
          for (int t = 0; t < 4; ++t) mfma_column(acc, xv[t], wb[t], sc[t], m12);
        };
        auto partial = [&](const llvq_u32x4 (&xv)[4], int s4) {
#pragma unroll
          for (int t = 0; t < 3; ++t) {
            if (t < rem) {
              const uint2 wb = *reinterpret_cast<const uint2*>(smem + abase + 96u * (uint32_t)s4 + 24u * t);
              const float sc = *reinterpret_cast<const float*>(smem + pbase + 16u * (uint32_t)s4 + 4u * t);
              mfma_column(acc, xv[t], wb, sc, m12);
            }
          }
        };
        // batches of 4 columns, the next batch's activations requested before the current
        // batch's products (loads past the last column read unused data or zeros)
        xload(xa, 0);
        int s4 = 0;
        for (;;) {
          if (s4 >= nfull) {
            if (rem) partial(xa, s4);
            break;
          }
          xload(xb, s4 + 1);
          batch(xa, s4);
          ++s4;
          if (s4 >= nfull) {
            if (rem) partial(xb, s4);
            break;
          }
          xload(xa, s4 + 1);
          batch(xb, s4);
          ++s4;
        }
        if (tail) {
          const int j = ncw - 1;
          const bool in = xlane && 8 * kg < K % 24;
          const llvq_u32x4 xv =
              __builtin_amdgcn_raw_buffer_load_b128(xrs, in ? vbase + 48u * (uint32_t)j : 0x80000000u, 0, 0);
          const uint2 wb = *reinterpret_cast<const uint2*>(smem + abase + 24u * (uint32_t)j);
          const float sc = *reinterpret_cast<const float*>(smem + pbase + 4u * (uint32_t)j);
          mfma_column(acc, xv, wb, sc, m12);
        }
      } else {
        for (int j = 0; j < ncw; ++j) {
          const int col = (b0 + cb + j) * 24 + 8 * kg;
          uint32_t wv[4] = {0u, 0u, 0u, 0u};
          if (xlane) {
            const uint16_t* xr = x + (size_t)mr * (size_t)K;
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (col + e < K) wv[e >> 1] |= (uint32_t)xr[col + e] << (16 * (e & 1));
          }
          const uint2 wb = *reinterpret_cast<const uint2*>(smem + abase + 24u * (uint32_t)j);
          const float sc = *reinterpret_cast<const float*>(smem + pbase + 4u * (uint32_t)j);
          mfma_column(acc, llvq_u32x4{wv[0], wv[1], wv[2], wv[3]}, wb, sc, m12);
        }
      }
    }

    // ---- after the row group's last chunk: sum the waves' accumulators in a fixed order
    // (the byte tile is free once every wave's products are done)
    if (c.cc == g.nchunk - 1) {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 4; ++i) red[(wave * 64 + lane) * 4 + i] = acc[i];
      __syncthreads();
      if (tid < kGRows * 16) {
        const int r = tid >> 4;       // row in group
        const int n = tid & 15;       // batch row
        const int l = r + 16 * (n >> 2);
        const int i = n & 3;
        float s = 0.0f;
        for (int wv = 0; wv < kEWaves; ++wv) s += red[(wv * 64 + l) * 4 + i];
        if (r < c.nrows && n < g.batch) {
          const int row = c.grp * kGRows + r;
          const float rs = sg ? 1.0f : __half2float(scales[row]);
          y[(size_t)n * d.rows + row] = s * rs;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = 0.0f;
    }
    __syncthreads();
  }
}
