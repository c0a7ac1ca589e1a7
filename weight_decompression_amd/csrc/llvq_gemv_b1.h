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
__device__ __forceinline__ void gemv_chunk(uint8_t* smem, const EArgs& a, int T, uint32_t kb, float inv_kb, int c,
                                           int nco, int nodd, int neven, int lane) {
  const ELayout& L = a.L;
  const LlvqClassHot* cls = reinterpret_cast<const LlvqClassHot*>(smem + L.cls);
  const float* xsum = reinterpret_cast<const float*>(smem + a.xsum);
  const uint64_t* queue = reinterpret_cast<const uint64_t*>(smem + L.queue);
  float* part = reinterpret_cast<float*>(smem + L.part);
  if (c < nco) {
    const int e = (c << 6) + lane;
    if (e >= nodd) return;
    const uint64_t eo = queue[e];
    const uint32_t fo = entry_f(eo);
    const uint32_t bo = block_col(fo, inv_kb, kb);
    const LlvqClassHot hO = cls[entry_k(eo)];
    const BlockStart so = block_start(smem, L, entry_I(eo), hO);
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
    const BlockStart se = block_start(smem, L, entry_I(ee), hE);
    EvenDec ev;
    ev.init(hE, se);
    const uint32_t col0 = be * 24u;
    float ae0 = 0.0f, ae1 = 0.0f;
#pragma unroll
    for (int i = 0; i < 24; ++i) {
      uint32_t pos;
      const uint32_t bve = ev.step(smem, L, hE, i, pos);
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

  // ---- set-up: tables and activations into LDS
  engine_prologue(smem, L, d, a.nbuckets, scales, tid);
  {
    const int ncol = kb * 24;
    if (XF32) {
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
  int* ctr = reinterpret_cast<int*>(smem + L.ctr);
  const float* part = reinterpret_cast<const float*>(smem + L.part);
  const float inv_kb = 1.0f / (float)kb;

  for (int tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
    const int row0 = tile * a.rows_per_tile;
    const int nrows = min(a.rows_per_tile, d.rows - row0);
    const int T = nrows * kb;
    if (tid == 0) { ctr[0] = 0; ctr[1] = 0; ctr[2] = 0; }
    __syncthreads();

    // ---- 1. classify: wave w takes unit w (T <= kEWaves * kEUnit)
    const TileMap tm = {(uint32_t)(row0 * kb), (uint32_t)kb, (uint32_t)kb, inv_kb};
    if (wave * kEUnit < T) classify_unit(smem, L, d, packed, tm, T, wave, lane, err);
    __syncthreads();
    const int nodd = ctr[0];
    const int neven = ctr[1];
    const int nco = (nodd + 63) >> 6;
    const int nch = nco + ((neven + 63) >> 6);

    // ---- 2. decode + dot: 64-block chunks handed out dynamically (odd chunks first)
    for (;;) {
      int c = 0;
      if (lane == 0) c = atomicAdd(&ctr[2], 1);
      c = __builtin_amdgcn_readfirstlane(c);
      if (c >= nch) break;
      gemv_chunk<XF32>(smem, a, T, (uint32_t)kb, inv_kb, c, nco, nodd, neven, lane);
    }
    __syncthreads();

    // ---- 3. row sums (fixed order)
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
    __syncthreads();
  }
}
