// Byte-tile consumers of the tile engine (gfx950): decode of whole tensors to bf16
// weights or int8 lattice points.  Included once by llvq.hip after llvq_engine.h.
//
// The decode phase writes each block's 24 biased value bytes (12 + v) into an LDS tile
// laid out like the tensor ([rows][Kb * 24], row-major), odd blocks with 8-byte writes
// in position order, even blocks with byte writes at their positions.  The store phase
// then walks the tile row by row with 8 consecutive columns per lane, so the global
// writes of a wavefront are contiguous.

#pragma once

// Decode chunk c of a tile (queues of buffer qb) into the byte tile (same chunk numbering
// as the GEMV).  A block queued with class kInvalidClass gets 24 zero values.
__device__ __forceinline__ void bytes_chunk(uint8_t* smem, const ELayout& L, const TileBuf& qb, uint32_t tb, int T,
                                            int c, int nco, int nodd, int neven, int lane) {
  const LlvqClassHot* cls = reinterpret_cast<const LlvqClassHot*>(smem + L.cls);
  const uint64_t* queue = reinterpret_cast<const uint64_t*>(smem + qb.queue);
  if (c < nco) {
    const int e = (c << 6) + lane;
    if (e >= nodd) return;
    const uint64_t eo = queue[e];
    const uint32_t f = entry_f(eo);
    const LlvqClassHot h = cls[entry_k(eo)];
    const BlockStart bs = block_start(smem, L, entry_J(eo), h);
    OddDec od;
    od.init(h, bs);
    uint2* dst = reinterpret_cast<uint2*>(smem + tb + 24u * f);
    uint32_t w0 = 0u, w1 = 0u;
#pragma unroll
    for (int p = 0; p < 24; ++p) {
      const uint32_t bv = od.step(smem, L, p);
      const int q = p & 7;
      if (q == 0) w0 = bv;
      else if (q < 4) w0 |= bv << (8 * q);
      else if (q == 4) w1 = bv;
      else w1 |= bv << (8 * (q - 4));
      if (q == 7) dst[p >> 3] = make_uint2(w0, w1);
    }
  } else {
    const int e = ((c - nco) << 6) + lane;
    if (e >= neven) return;
    const uint64_t ee = queue[T - 1 - e];
    const uint32_t f = entry_f(ee);
    if (entry_k(ee) == kInvalidClass) {
      uint2* zb = reinterpret_cast<uint2*>(smem + tb + 24u * f);
      const uint2 z = make_uint2(0x0c0c0c0cu, 0x0c0c0c0cu);
      zb[0] = z;
      zb[1] = z;
      zb[2] = z;
      return;
    }
    const LlvqClassHot h = cls[entry_k(ee)];
    const BlockStart bs = block_start(smem, L, entry_J(ee), h);
    EvenDec ev;
    ev.init(h, bs, L.cls + entry_k(ee) * (uint32_t)sizeof(LlvqClassHot));
    uint8_t* dst = smem + tb + 24u * f;
#pragma unroll
    for (int i = 0; i < 24; ++i) {
      uint32_t pos;
      const uint32_t bv = ev.step(smem, L, i, pos);
      dst[pos] = (uint8_t)bv;
    }
  }
}

typedef float llvq_f2 __attribute__((ext_vector_type(2)));
typedef __bf16 llvq_bf2 __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16 pair, round to nearest even
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const llvq_f2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, llvq_bf2));
}

// 4 biased bytes -> 4 int8 values (byte - 12, two's complement), without carries
// between bytes: (u | 0x80) - 12 stays in [0x74, 0x8c] for u in [0, 24].
__device__ __forceinline__ uint32_t unbias4(uint32_t u) { return ((u | 0x80808080u) - 0x0c0c0c0cu) ^ 0x80808080u; }

// Store phase: the byte tile of rows row0 .. row0 + nrows - 1 to the output, row by row
// with 8 consecutive columns per lane (the global writes of a wavefront are contiguous).
template <int OUT>
__device__ __forceinline__ void store_tile(const uint8_t* smem, uint32_t tb, const float* part, const KDesc& d,
                                           int row0, int nrows, const __half* __restrict__ scales,
                                           void* __restrict__ out, int tid) {
  const int kb = d.kb;
  const bool sg = d.mode == LLVQ_MODE_SHAPEGAIN;
  const uint32_t rowbytes = (uint32_t)kb * 24u;
  if (OUT == LLVQ_OUT_POINTS_I8) {
    const bool a8 = (((uintptr_t)out) & 7u) == 0u;
    const uint32_t n8 = rowbytes >> 3;
    for (int rl = 0; rl < nrows; ++rl) {
      int8_t* orow = static_cast<int8_t*>(out) + (size_t)(row0 + rl) * rowbytes;
      const uint8_t* trow = smem + tb + (uint32_t)rl * rowbytes;
      for (uint32_t j = (uint32_t)tid; j < n8; j += kEThreads) {
        const uint2 u = *reinterpret_cast<const uint2*>(trow + 8u * j);
        const uint32_t lo = unbias4(u.x), hi = unbias4(u.y);
        if (a8) {
          *reinterpret_cast<uint2*>(orow + 8u * j) = make_uint2(lo, hi);
        } else {
          reinterpret_cast<uint32_t*>(orow + 8u * j)[0] = lo;
          reinterpret_cast<uint32_t*>(orow + 8u * j)[1] = hi;
        }
      }
    }
  } else {
    const int K = d.cols;
    const bool a16 = ((((uintptr_t)out) & 15u) == 0u) && ((K & 7) == 0);
    const uint32_t n8 = (uint32_t)(K + 7) >> 3;
    for (int rl = 0; rl < nrows; ++rl) {
      const int r = row0 + rl;
      uint16_t* orow = static_cast<uint16_t*>(out) + (size_t)r * (size_t)K;
      const uint8_t* trow = smem + tb + (uint32_t)rl * rowbytes;
      const float rs = sg ? 0.0f : __half2float(scales[r]);
      for (uint32_t j = (uint32_t)tid; j < n8; j += kEThreads) {
        const uint2 u = *reinterpret_cast<const uint2*>(trow + 8u * j);
        const float sc = sg ? part[rl * kb + (int)(j / 3u)] : rs;
        float v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint32_t byte = ((q < 4 ? u.x : u.y) >> (8 * (q & 3))) & 0xffu;
          v[q] = __fmul_rn((float)((int)byte - kBias), sc);
        }
        const uint4 pk = make_uint4(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]),
                                    pack_bf16(v[6], v[7]));
        const uint32_t col = 8u * j;
        if (a16) {
          *reinterpret_cast<uint4*>(orow + col) = pk;
        } else {
          const uint32_t w[4] = {pk.x, pk.y, pk.z, pk.w};
#pragma unroll
          for (int q = 0; q < 8; ++q)
            if ((int)(col + q) < K) orow[col + q] = (uint16_t)(w[q >> 1] >> (16 * (q & 1)));
        }
      }
    }
  }
}

template <int OUT>
__global__ __launch_bounds__(kEThreads) void k_decode_tile(KDesc d, EArgs a, const uint8_t* __restrict__ packed,
                                                            const __half* __restrict__ scales, void* __restrict__ out,
                                                            int32_t* err) {
  extern __shared__ __align__(16) uint8_t smem[];
  const ELayout& L = a.L;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kb = d.kb;
  const uint32_t tb = a.xs;                 // byte tile
  const float inv_kb = 1.0f / (float)kb;

  // Tiles of this workgroup: blockIdx.x + lt * gridDim.x, queues and scale slots in buffer
  // lt & 1.  Phase lt decodes tile lt into the byte tile and, as work runs out, classifies
  // tile lt + 1 into the other buffer; then the byte tile is stored.  The first tile's
  // fields are requested before the tables are staged (the grid never exceeds the tile
  // count, so T0 >= 1; a wave without a unit reads the tile's last unit and ignores it).
  const int row00 = blockIdx.x * a.rows_per_tile;
  const int T0 = min(a.rows_per_tile, d.rows - row00) * kb;
  const TileMap tm0 = {(uint32_t)(row00 * kb), (uint32_t)kb, (uint32_t)kb, inv_kb};
  const UnitFields uf0 = load_unit(d, packed, tm0, T0, min(wave, (T0 - 1) / kEUnit), lane);
  engine_prologue(smem, L, d, a.nbuckets, scales, tid);
  int* work = reinterpret_cast<int*>(smem + L.work);
  if (tid == 0) {
    int* c0 = reinterpret_cast<int*>(smem + L.buf[0].ctr);
    int* c1 = reinterpret_cast<int*>(smem + L.buf[1].ctr);
    c0[0] = 0; c0[1] = 0; c1[0] = 0; c1[1] = 0; work[0] = 0; work[1] = 0;
  }
  __syncthreads();
  {
    const int nun0 = (T0 + kEUnit - 1) / kEUnit;
    if (wave < nun0) classify_fields(smem, L, L.buf[0], d, uf0, T0, wave, lane, err, true);
    for (;;) {
      int u = 0;
      if (lane == 0) u = atomicAdd(&work[1], 1);
      u = __builtin_amdgcn_readfirstlane(u) + kEWaves;
      if (u >= nun0) break;
      classify_unit(smem, L, L.buf[0], d, packed, tm0, T0, u, lane, err, true);
    }
  }
  __syncthreads();

  int lt = 0;
  for (int tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x, ++lt) {
    const TileBuf& cur = L.buf[lt & 1];
    const TileBuf& nxt = L.buf[(lt & 1) ^ 1];
    const int row0 = tile * a.rows_per_tile;
    const int nrows = min(a.rows_per_tile, d.rows - row0);
    const int T = nrows * kb;
    const int* ctr = reinterpret_cast<const int*>(smem + cur.ctr);
    const int nodd = ctr[0];
    const int neven = ctr[1];
    const int nco = (nodd + 63) >> 6;
    const int nch = nco + ((neven + 63) >> 6);
    const int tile1 = tile + gridDim.x;
    int T1 = 0, nun1 = 0;
    if (tile1 < a.ntiles) {
      T1 = min(a.rows_per_tile, d.rows - tile1 * a.rows_per_tile) * kb;
      nun1 = (T1 + kEUnit - 1) / kEUnit;
    }
    const TileMap tm1 = {(uint32_t)(tile1 * a.rows_per_tile * kb), (uint32_t)kb, (uint32_t)kb, inv_kb};
    for (;;) {
      int c = 0;
      if (lane == 0) c = atomicAdd(&work[0], 1);
      c = __builtin_amdgcn_readfirstlane(c);
      if (c < nch) {
        bytes_chunk(smem, L, cur, tb, T, c, nco, nodd, neven, lane);
      } else if (c < nch + nun1) {
        classify_unit(smem, L, nxt, d, packed, tm1, T1, c - nch, lane, err, true);
      } else {
        break;
      }
    }
    __syncthreads();
    store_tile<OUT>(smem, tb, reinterpret_cast<const float*>(smem + cur.part), d, row0, nrows, scales, out, tid);
    if (tid == 0) {
      int* cc = reinterpret_cast<int*>(smem + cur.ctr);
      cc[0] = 0;
      cc[1] = 0;
      work[0] = 0;
    }
    __syncthreads();
  }
}
