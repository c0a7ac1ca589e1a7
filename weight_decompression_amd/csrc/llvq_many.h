// Decode of several tensors in one launch (gfx950): the tiles of all tensors form one
// list, handed to the workgroups in grid stride, with the two-buffer pipeline of
// k_decode_tile (the next tile, of whichever tensor, is classified inside the decode work
// of the current one; then the byte tile is stored).  One set of tables serves every
// tensor (they share the shell range and the field widths); shape-gain tensors each bring
// their gain table.  With many tiles per workgroup the workgroups drift out of step, so
// one workgroup's stores overlap the others' decode instead of all hitting memory at
// once, and the set-up is paid once for all tensors.  Included once by llvq.hip after
// llvq_tile.h.

#pragma once

constexpr int kManyMax = 16;

struct MTensor {
  const uint8_t* packed;
  const __half* scales;
  void* out;
  int rows, cols, kb, rows_per_tile, tile0;   // tile0: the tensor's first tile in the list
};

struct MArgs {
  EArgs e;          // layout (two tile buffers, gain tables of every tensor), nbuckets
  int n;            // tensors
  int ntiles;       // tiles of all tensors
  MTensor t[kManyMax];
};

// tile `tile` of the list: its tensor, rows and stream map
struct MTile {
  int ti, row0, nrows, T;
  TileMap tm;
};

__device__ __forceinline__ MTile many_tile(const MArgs& m, int tile) {
  MTile r;
  int ti = 0;
#pragma unroll
  for (int j = 1; j < kManyMax; ++j)
    if (j < m.n && tile >= m.t[j].tile0) ti = j;
  const MTensor& t = m.t[ti];
  r.ti = ti;
  r.row0 = (tile - t.tile0) * t.rows_per_tile;
  r.nrows = min(t.rows_per_tile, t.rows - r.row0);
  r.T = r.nrows * t.kb;
  r.tm = TileMap{(uint32_t)(r.row0 * t.kb), (uint32_t)t.kb, (uint32_t)t.kb, 1.0f / (float)t.kb};
  return r;
}

// descriptor of tensor ti (shared widths and shell range, its own shape)
__device__ __forceinline__ KDesc many_desc(const KDesc& d0, const MTensor& t) {
  KDesc d = d0;
  d.rows = t.rows;
  d.cols = t.cols;
  d.kb = t.kb;
  return d;
}

// layout with tensor ti's gain table in place of the first
__device__ __forceinline__ ELayout many_layout(const ELayout& L, const KDesc& d0, int ti) {
  ELayout l = L;
  if (d0.mode == LLVQ_MODE_SHAPEGAIN) l.gains += 4u * ((uint32_t)ti << d0.gain_bits);
  return l;
}

template <int OUT>
__global__ __launch_bounds__(kEThreads) void k_decode_many(KDesc d0, MArgs m, int32_t* err) {
  extern __shared__ __align__(16) uint8_t smem[];
  const ELayout& L = m.e.L;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const uint32_t tb = m.e.xs;

  // the first tile's fields are requested before the tables are staged (the grid never
  // exceeds the tile count; a wave without a unit reads the tile's last unit)
  const MTile t0 = many_tile(m, blockIdx.x);
  const KDesc dt0 = many_desc(d0, m.t[t0.ti]);
  const UnitFields uf0 = load_unit(dt0, m.t[t0.ti].packed, t0.tm, t0.T, min(wave, (t0.T - 1) / kEUnit), lane);
  engine_prologue(smem, L, d0, m.e.nbuckets, m.t[0].scales, tid);
  if (OUT == LLVQ_OUT_BF16 && d0.mode == LLVQ_MODE_SHAPEGAIN) {
    const int ng = 1 << d0.gain_bits;
    float* G = reinterpret_cast<float*>(smem + L.gains);
    for (int i = ng + tid; i < m.n * ng; i += kEThreads) G[i] = __half2float(m.t[i >> d0.gain_bits].scales[i & (ng - 1)]);
  }
  int* work = reinterpret_cast<int*>(smem + L.work);
  if (tid == 0) {
    int* c0 = reinterpret_cast<int*>(smem + L.buf[0].ctr);
    int* c1 = reinterpret_cast<int*>(smem + L.buf[1].ctr);
    c0[0] = 0; c0[1] = 0; c1[0] = 0; c1[1] = 0; work[0] = 0; work[1] = 0;
  }
  __syncthreads();
  {
    const ELayout l0 = many_layout(L, d0, t0.ti);
    const int nun0 = (t0.T + kEUnit - 1) / kEUnit;
    if (wave < nun0) classify_fields(smem, l0, L.buf[0], dt0, uf0, t0.T, wave, lane, err, true);
    for (;;) {
      int u = 0;
      if (lane == 0) u = atomicAdd(&work[1], 1);
      u = __builtin_amdgcn_readfirstlane(u) + kEWaves;
      if (u >= nun0) break;
      classify_unit(smem, l0, L.buf[0], dt0, m.t[t0.ti].packed, t0.tm, t0.T, u, lane, err, true);
    }
  }
  __syncthreads();

  int lt = 0;
  for (int tile = blockIdx.x; tile < m.ntiles; tile += gridDim.x, ++lt) {
    const TileBuf& cur = L.buf[lt & 1];
    const TileBuf& nxt = L.buf[(lt & 1) ^ 1];
    const MTile tc = many_tile(m, tile);
    const KDesc dc = many_desc(d0, m.t[tc.ti]);
    const int* ctr = reinterpret_cast<const int*>(smem + cur.ctr);
    const int nodd = ctr[0];
    const int neven = ctr[1];
    const int nco = (nodd + 63) >> 6;
    const int nch = nco + ((neven + 63) >> 6);
    const int tile1 = tile + gridDim.x;
    const MTile tn = many_tile(m, tile1 < m.ntiles ? tile1 : tile);
    const int nun1 = tile1 < m.ntiles ? (tn.T + kEUnit - 1) / kEUnit : 0;
    const KDesc dn = many_desc(d0, m.t[tn.ti]);
    const ELayout ln = many_layout(L, d0, tn.ti);
    for (;;) {
      int c = 0;
      if (lane == 0) c = atomicAdd(&work[0], 1);
      c = __builtin_amdgcn_readfirstlane(c);
      if (c < nch) {
        bytes_chunk(smem, L, cur, tb, tc.T, c, nco, nodd, neven, lane);
      } else if (c < nch + nun1) {
        classify_unit(smem, ln, nxt, dn, m.t[tn.ti].packed, tn.tm, tn.T, c - nch, lane, err, true);
      } else {
        break;
      }
    }
    __syncthreads();
    store_tile<OUT>(smem, tb, reinterpret_cast<const float*>(smem + cur.part), dc, tc.row0, tc.nrows,
                    m.t[tc.ti].scales, m.t[tc.ti].out, tid);
    if (tid == 0) {
      int* cc = reinterpret_cast<int*>(smem + cur.ctr);
      cc[0] = 0;
      cc[1] = 0;
      work[0] = 0;
    }
    __syncthreads();
  }
}
