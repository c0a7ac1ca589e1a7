// Fused LLVQ dequant-GEMV for one activation row (batch 1), gfx950.
// Included once by llvq.hip after llvq_engine.h.
//
// The tile engine decodes each block; this consumer dots the 24 decoded values with the
// block's 24 activations straight from registers (odd blocks, position order) or from
// LDS by position (even blocks, decode order), never storing the weights.  Block results
// are scaled in their LDS slot, and the tile's rows are summed in a fixed order, so
// results do not depend on which wave decoded which block.

#pragma once

template <bool XF32>
__device__ __forceinline__ void load_x24(const uint8_t* smem, uint32_t xs, uint32_t blk, float xv[24]) {
  if (XF32) {
    const float4* p = reinterpret_cast<const float4*>(smem + xs + blk * 96u);
#pragma unroll
    for (int q = 0; q < 6; ++q) {
      const float4 v = p[q];
      xv[4 * q] = v.x; xv[4 * q + 1] = v.y; xv[4 * q + 2] = v.z; xv[4 * q + 3] = v.w;
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(smem + xs + blk * 48u);
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const uint4 v = p[q];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        xv[8 * q + 2 * h] = __uint_as_float(w[h] << 16);
        xv[8 * q + 2 * h + 1] = __uint_as_float(w[h] & 0xffff0000u);
      }
    }
  }
}

// activation at column col (LDS)
template <bool XF32>
__device__ __forceinline__ float x_at(const uint8_t* smem, uint32_t xs, uint32_t col) {
  if (XF32) return reinterpret_cast<const float*>(smem + xs)[col];
  return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(smem + xs)[col] << 16);
}

__device__ __forceinline__ uint32_t block_col(uint32_t f, float inv_kb, uint32_t kb) {
  const uint32_t rl = (uint32_t)(((float)f + 0.5f) * inv_kb);
  return f - rl * kb;
}

// One decode chunk: 64 consecutive entries of one parity queue (chunks 0..nco-1 are the
// odd queue, the rest the even queue), one block per lane.  Result: part[f] *= dot.
template <bool XF32>
__device__ __forceinline__ void gemv_chunk(uint8_t* smem, const EArgs& a, const TileBuf& tb, int T, uint32_t kb,
                                           float inv_kb, int c, int nco, int nodd, int neven, int lane) {
  const ELayout& L = a.L;
  const LlvqClassHot* cls = reinterpret_cast<const LlvqClassHot*>(smem + L.cls);
  const float* xsum = reinterpret_cast<const float*>(smem + a.xsum);
  const uint64_t* queue = reinterpret_cast<const uint64_t*>(smem + tb.queue);
  float* part = reinterpret_cast<float*>(smem + tb.part);
  if (c < nco) {
    const int e = (c << 6) + lane;
    if (e >= nodd) return;
    const uint64_t eo = queue[e];
    const uint32_t fo = entry_f(eo);
    const uint32_t bo = block_col(fo, inv_kb, kb);
    const LlvqClassHot hO = cls[entry_k(eo)];
    const BlockStart so = block_start(smem, L, entry_J(eo), hO);
    float xv[24];
    load_x24<XF32>(smem, a.xs, bo, xv);
    OddDec od;
    od.init(hO, so);
    float ao0 = 0.0f, ao1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 24; ++i) {
      const uint32_t bvo = od.step(smem, L, i);
      if (i & 1)
        ao1 = __builtin_fmaf((float)(bvo & 0xffu), xv[i], ao1);
      else
        ao0 = __builtin_fmaf((float)(bvo & 0xffu), xv[i], ao0);
    }
    part[fo] *= __builtin_fmaf(-(float)kBias, xsum[bo], ao0 + ao1);
  } else {
    const int e = ((c - nco) << 6) + lane;
    if (e >= neven) return;
    const uint64_t ee = queue[T - 1 - e];
    const uint32_t fe = entry_f(ee);
    const uint32_t be = block_col(fe, inv_kb, kb);
    const LlvqClassHot hE = cls[entry_k(ee)];
    const BlockStart se = block_start(smem, L, entry_J(ee), hE);
    EvenDec ev;
    ev.init(hE, se, L.cls + entry_k(ee) * (uint32_t)sizeof(LlvqClassHot));
    const uint32_t col0 = be * 24u;
    float ae0 = 0.0f, ae1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 24; ++i) {
      uint32_t pos;
      const uint32_t bve = ev.step(smem, L, i, pos);
      const float xp = x_at<XF32>(smem, a.xs, col0 + pos);
      if (i & 1)
        ae1 = __builtin_fmaf((float)(bve & 0xffu), xp, ae1);
      else
        ae0 = __builtin_fmaf((float)(bve & 0xffu), xp, ae0);
    }
    part[fe] *= __builtin_fmaf(-(float)kBias, xsum[be], ae0 + ae1);
  }
}

template <bool XF32>
__global__ __launch_bounds__(kEThreads) void k_gemv_b1(KDesc d, EArgs a, const uint8_t* __restrict__ packed,
                                                        const __half* __restrict__ scales, const void* __restrict__ xv,
                                                        float* __restrict__ y, int32_t* err) {
  extern __shared__ __align__(16) uint8_t smem[];
  const ELayout& L = a.L;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kb = d.kb;
  const bool sg = d.mode == LLVQ_MODE_SHAPEGAIN;

  // ---- set-up: the first tile's fields are requested before the tables and activations
  // are staged in LDS, so their memory latency overlaps the staging
  const float inv_kb0 = 1.0f / (float)kb;
  int row00 = blockIdx.x * a.rows_per_tile;
  const int T0 = min(a.rows_per_tile, d.rows - row00) * kb;
  const TileMap tm0 = {(uint32_t)(row00 * kb), (uint32_t)kb, (uint32_t)kb, inv_kb0};
  // (unconditional, so the loads stay in flight: the grid never exceeds the tile count, so
  // T0 >= 1, and a wave without a unit of tile 0 reads unit 0 and ignores it)
  const UnitFields uf0 = load_unit(d, packed, tm0, T0, min(wave, (T0 - 1) / kEUnit), lane);
  // activations: the whole 16-byte words of a 16-byte aligned bf16 row go with the table
  // copies; the rest (and the zero padding to Kb * 24 columns) follows
  const bool xa16 = !XF32 && ((((uintptr_t)xv) & 15u) == 0u);
  const int xw = xa16 ? (d.cols >> 3) : 0;
  engine_prologue(smem, L, d, a.nbuckets, scales, tid, CopySeg{reinterpret_cast<const uint4*>(xv), a.xs, xw});
  {
    const int ncol = kb * 24;
    if (xa16) {
      uint16_t* xs = reinterpret_cast<uint16_t*>(smem + a.xs);
      const uint16_t* xg = reinterpret_cast<const uint16_t*>(xv);
      for (int i = (xw << 3) + tid; i < ncol; i += kEThreads) xs[i] = i < d.cols ? xg[i] : (uint16_t)0;
    } else if (XF32) {
      float* xs = reinterpret_cast<float*>(smem + a.xs);
      const float* xg = reinterpret_cast<const float*>(xv);
      for (int i = tid; i < ncol; i += kEThreads) xs[i] = i < d.cols ? xg[i] : 0.0f;
    } else {
      // pairs of bf16 as dwords when the row is dword aligned
      uint16_t* xs = reinterpret_cast<uint16_t*>(smem + a.xs);
      const uint16_t* xg = reinterpret_cast<const uint16_t*>(xv);
      if ((((uintptr_t)xg) & 3u) == 0u) {
        const int full = d.cols >> 1;
        const uint32_t* xg2 = reinterpret_cast<const uint32_t*>(xg);
        uint32_t* xs2 = reinterpret_cast<uint32_t*>(xs);
        for (int i = tid; i < ncol / 2; i += kEThreads)
          xs2[i] = i < full ? xg2[i] : ((i == full && (d.cols & 1)) ? (uint32_t)xg[d.cols - 1] : 0u);
      } else {
        for (int i = tid; i < ncol; i += kEThreads) xs[i] = i < d.cols ? xg[i] : (uint16_t)0;
      }
    }
  }
  __syncthreads();
  {
    float* xsum = reinterpret_cast<float*>(smem + a.xsum);
    for (int b = tid; b < kb; b += kEThreads) {
      float xx[24];
      load_x24<XF32>(smem, a.xs, (uint32_t)b, xx);
      float s0 = 0.0f;
#pragma unroll
      for (int p = 0; p < 24; ++p) s0 += xx[p];
      xsum[b] = s0;
    }
  }
  int* work = reinterpret_cast<int*>(smem + L.work);
  const float inv_kb = 1.0f / (float)kb;

  // Tiles of this workgroup: blockIdx.x + lt * gridDim.x, using buffer lt & 1.  Phase lt
  // decodes tile lt and, as work runs out, classifies tile lt + 1 into the other buffer, so
  // the classification fills the tail of the decode; then the rows of tile lt are summed.
  auto tile_rows = [&](int tile, int* row0, int* nrows) {
    *row0 = tile * a.rows_per_tile;
    *nrows = min(a.rows_per_tile, d.rows - *row0);
  };
  // classify tile 0 (fields loaded above)
  if (blockIdx.x < a.ntiles) {
    if (tid == 0) {
      int* c0 = reinterpret_cast<int*>(smem + L.buf[0].ctr);
      int* c1 = reinterpret_cast<int*>(smem + L.buf[1].ctr);
      c0[0] = 0; c0[1] = 0; c1[0] = 0; c1[1] = 0; work[0] = 0; work[1] = 0;
    }
    __syncthreads();
    const int nun0 = (T0 + kEUnit - 1) / kEUnit;
    if (wave < nun0) classify_fields(smem, L, L.buf[0], d, uf0, T0, wave, lane, err);
    // units past the first kEWaves (tiles of more than kEWaves * kEUnit blocks), handed out
    // by their own counter
    for (;;) {
      int u = 0;
      if (lane == 0) u = atomicAdd(&work[1], 1);
      u = __builtin_amdgcn_readfirstlane(u) + kEWaves;
      if (u >= nun0) break;
      classify_unit(smem, L, L.buf[0], d, packed, tm0, T0, u, lane, err);
    }
    __syncthreads();
  }
  int lt = 0;
  for (int tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x, ++lt) {
    const TileBuf& cur = L.buf[lt & 1];
    const TileBuf& nxt = L.buf[(lt & 1) ^ 1];
    int row0, nrows;
    tile_rows(tile, &row0, &nrows);
    const int T = nrows * kb;
    const int* ctr = reinterpret_cast<const int*>(smem + cur.ctr);
    const int nodd = ctr[0];
    const int neven = ctr[1];
    const int nco = (nodd + 63) >> 6;
    const int nch = nco + ((neven + 63) >> 6);
    // next tile's classify units
    const int tile1 = tile + gridDim.x;
    int row1 = 0, nrows1 = 0, T1 = 0, nun1 = 0;
    if (tile1 < a.ntiles) {
      tile_rows(tile1, &row1, &nrows1);
      T1 = nrows1 * kb;
      nun1 = (T1 + kEUnit - 1) / kEUnit;
    }
    const TileMap tm1 = {(uint32_t)(row1 * kb), (uint32_t)kb, (uint32_t)kb, inv_kb};

    // ---- decode + dot of this tile (odd chunks first), then classify units of the next
    for (;;) {
      int c = 0;
      if (lane == 0) c = atomicAdd(&work[0], 1);
      c = __builtin_amdgcn_readfirstlane(c);
      if (c < nch) {
        gemv_chunk<XF32>(smem, a, cur, T, (uint32_t)kb, inv_kb, c, nco, nodd, neven, lane);
      } else if (c < nch + nun1) {
        classify_unit(smem, L, nxt, d, packed, tm1, T1, c - nch, lane, err);
      } else {
        break;
      }
    }
    __syncthreads();

    // ---- row sums of this tile (fixed order); reset this buffer's counters for tile lt + 2
    const float* part = reinterpret_cast<const float*>(smem + cur.part);
    for (int rl = wave; rl < nrows; rl += kEWaves) {
      float acc = 0.0f;
      for (int b = lane; b < kb; b += 64) acc += part[rl * kb + b];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
      if (lane == 0) {
        const int r = row0 + rl;
        const float rs = sg ? 1.0f : __half2float(scales[r]);
        y[r] = acc * rs;
      }
    }
    if (tid == 0) {
      int* cc = reinterpret_cast<int*>(smem + cur.ctr);
      cc[0] = 0;
      cc[1] = 0;
      work[0] = 0;
    }
    __syncthreads();
  }
}
