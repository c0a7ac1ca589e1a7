// Decode of whole tensors to bf16 weights or int8 lattice points, streamed (gfx950).
// Included once by llvq.hip after llvq_gemv_b1.h (whose ring classification it shares)
// and llvq_tile.h.
//
// One launch serves one or several tensors (same shell range and field widths).  Their
// rows, concatenated, are cut into one contiguous range per workgroup holding the same
// number of blocks up to a row; a workgroup's range is walked in tiles of whole rows of
// one tensor (at most kETileMax blocks, the LDS slots of one tile).  Inside a tile the
// waves classify units of 64 fields into their odd / even ring queues exactly as the
// batch-1 GEMV does, and decode a full chunk of 64 blocks whenever a ring holds one; at
// the tile's end the rings' remainders are gathered and decoded by all waves.
//
// A decoded chunk goes to global memory from the wave that decoded it, without a tile-wide
// store phase: each lane leaves its block's 24 codes in a private 24-byte LDS slot (odd
// blocks in position order, even blocks by position), the wave reads them back transposed
// so that three adjacent lanes hold one block's outputs, and stores them one iteration
// later (stream_transpose).  The stores of one wave overlap the decode of the others;
// there is no byte tile, so a tile costs 4 bytes of LDS per block and the workgroup's
// whole range is a few tiles.
// The Golay codeword table is staged in LDS too: with stores in flight, a global table
// read would make each block wait for the previous chunk's stores to complete.
//
// bf16 values: the decoders give each value's selector into the block's fp8 value table
// (v exactly, E4M3); a pair converts to two fp32 with one v_cvt_scalef32_pk_f32_fp8
// (scale 1.0, exact), is multiplied by the block's scale (fp32) and rounded to a bf16
// pair (RNE), which is bf16_rne(f32(v) * f32 scale) per value.  An index past the shell
// union writes 24 zeros (+0.0 for bf16) and is counted.

#pragma once

constexpr int kManyMax = 16;                  // tensors per launch
constexpr int kStageBytes = kEThreads * 24;   // the lanes' 24-byte value slots

typedef float llvq_f32x2 __attribute__((ext_vector_type(2)));

struct STensor {
  const uint8_t* packed;
  const __half* scales;   // SHAPEGAIN: gains (staged in LDS); EUCLID: row scales
  void* out;
  int rows, cols, kb;
  uint32_t pad_;
  long long blk0;         // the tensor's first block in the concatenation
};

struct SArgs {
  ELayout L;              // tables (the Golay table too), the gain tables of every tensor, counters
  uint32_t rings;         // the waves' rings, then the shared leftover queue
  uint32_t part;          // float[tmax]: block scales of the tile
  uint32_t stage;         // uint8[kStageBytes]
  int nbuckets;
  int n;
  int tmax;               // blocks per tile at most
  long long total;        // blocks of all tensors
  STensor t[kManyMax];
};

// Where one tile's outputs go.
struct SOut {
  uint8_t* out;           // the tile's first output row (tile offsets below are 32-bit)
  const __half* rs;       // the tile's first row scale (EUCLID)
  int cols, kb;
  float inv_kb;
  bool vec;               // whole-vector stores allowed (alignment)
};

// (tensor, row) of the first row that starts at or after block p of the concatenation;
// (n, 0) past the last row start.
struct SPos {
  int t, row;
};

__device__ __forceinline__ SPos stream_snap(const SArgs& m, long long p) {
  for (int i = 0; i < m.n; ++i) {
    const long long end = m.t[i].blk0 + (long long)m.t[i].rows * m.t[i].kb;
    if (p < end) {
      const long long q = p - m.t[i].blk0;
      const int row = (int)((q + m.t[i].kb - 1) / m.t[i].kb);
      if (row < m.t[i].rows) return {i, row};
      return {i + 1, 0};          // past the tensor's last row start: the next tensor's first
    }
  }
  return {m.n, 0};
}

// Row of block f inside the tile and its first column (24-bit multiplies: rl, kb < 2^24).
__device__ __forceinline__ void stream_where(const SOut& o, uint32_t f, uint32_t& rl, uint32_t& col0) {
  rl = (uint32_t)__builtin_fmaf((float)f, o.inv_kb, 0.5f * o.inv_kb);   // (f + 1/2) / Kb, f < 2^22
  col0 = 24u * (f - __umul24(rl, (uint32_t)o.kb));
}

// 24 zero outputs (an index past the shell union)
template <int OUT>
__device__ __forceinline__ void stream_zero(const SOut& o, uint32_t f) {
  uint32_t rl, col0;
  stream_where(o, f, rl, col0);
  if (OUT == LLVQ_OUT_POINTS_I8) {
    uint8_t* dst = o.out + rl * (uint32_t)(o.kb * 24) + col0;
    for (int q = 0; q < 24; ++q) dst[q] = 0;
  } else {
    uint16_t* dst = reinterpret_cast<uint16_t*>(o.out) + rl * (uint32_t)o.cols + col0;
    for (int q = 0; q < 24; ++q)
      if ((int)col0 + q < o.cols) dst[q] = 0;
  }
}

// Stores of one decoded chunk after its transposition: lane l holds pieces p = 64 q + l
// (q = 0..2) of the chunk, piece p being values 8 (p mod 3) .. + 7 of the chunk's block
// p / 3, as 4 bf16 pairs (or 2 dwords of int8 values).  Three adjacent lanes thus write
// one block's 48 (24) contiguous bytes with one store instruction, instead of each lane
// writing its own block in three instructions: a store instruction touches about a third
// as many cache lines.
struct SPend {
  uint32_t d[3][4];
  uint32_t off[3];  // byte offset of the piece from the tile's first output row
  uint32_t m;       // bits 4q..4q+3: values of piece q to store (0: none, 8: the whole piece)
};

template <int OUT>
__device__ __forceinline__ void stream_put(const SOut& o, const SPend& P) {
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    const uint32_t m = (P.m >> (4 * q)) & 15u;
    if (m == 0u) continue;
    uint8_t* dst = o.out + P.off[q];
    if (OUT == LLVQ_OUT_POINTS_I8) {
      if (o.vec) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(P.d[q][0], P.d[q][1]);
      } else {
        reinterpret_cast<uint32_t*>(dst)[0] = P.d[q][0];   // rows are whole dwords, out 4-byte aligned
        reinterpret_cast<uint32_t*>(dst)[1] = P.d[q][1];
      }
    } else if (o.vec && m == 8u) {
      *reinterpret_cast<uint4*>(dst) = make_uint4(P.d[q][0], P.d[q][1], P.d[q][2], P.d[q][3]);
    } else {
      uint16_t* d16 = reinterpret_cast<uint16_t*>(dst);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if ((uint32_t)e < m) d16[e] = (uint16_t)(P.d[q][e >> 1] >> (16 * (e & 1)));
    }
  }
}

// two fp8 codes (bytes 0, 1 of c, or 2, 3 with HI) times sc, as a bf16 pair
template <bool HI>
__device__ __forceinline__ uint32_t fp8_pair_bf16(uint32_t c, float sc) {
  const llvq_f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c, 1.0f, HI);
  return pack_bf16(v.x * sc, v.y * sc);
}

// The transposition of a chunk whose n blocks (lanes 0 .. n-1, block index f in the tile)
// left their 24 codes in the wave's value slots (fp8 codes, or biased bytes for int8
// output; slot of lane l at wbase + 24 l): each lane reads its three pieces, converts them
// (scale of the piece's block from its LDS slot) and computes where they go.
template <int OUT>
__device__ __forceinline__ void stream_transpose(const uint8_t* smem, const float* part, const SOut& o, uint32_t wbase,
                                                 uint32_t f, int n, int lane, SPend& P) {
  // the wave's slot writes before its reads of other lanes' slots
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  P.m = 0u;
#pragma unroll
  for (int q = 0; q < 3; ++q) {
    const uint32_t p = 64u * (uint32_t)q + (uint32_t)lane;   // < 192
    const uint32_t b = (p * 43691u) >> 17;                   // p / 3
    const uint32_t r = p - 3u * b;
    const uint32_t fb = (uint32_t)__builtin_amdgcn_ds_bpermute((int)(b << 2), (int)f);
    if ((int)b < n) {
      const uint2 c = *reinterpret_cast<const uint2*>(smem + wbase + 24u * b + 8u * r);
      uint32_t rl, col0;
      stream_where(o, fb, rl, col0);
      const uint32_t col = col0 + 8u * r;
      if (OUT == LLVQ_OUT_POINTS_I8) {
        P.d[q][0] = unbias4(c.x);
        P.d[q][1] = unbias4(c.y);
        P.off[q] = rl * (uint32_t)(o.kb * 24) + col;
        P.m |= 8u << (4 * q);
      } else {
        const float sc = part[fb];
        P.d[q][0] = fp8_pair_bf16<false>(c.x, sc);
        P.d[q][1] = fp8_pair_bf16<true>(c.x, sc);
        P.d[q][2] = fp8_pair_bf16<false>(c.y, sc);
        P.d[q][3] = fp8_pair_bf16<true>(c.y, sc);
        P.off[q] = (rl * (uint32_t)o.cols + col) * 2u;
        const int left = o.cols - (int)col;
        P.m |= (uint32_t)(left >= 8 ? 8 : (left > 0 ? left : 0)) << (4 * q);
      }
    }
  }
}

// Decode one odd-coset block (queue entry e) into the lane's value slot: its 24 fp8 codes
// (or biased bytes) in position order.  Returns the block's index in the tile.
template <int OUT>
__device__ __forceinline__ uint32_t stream_odd_codes(uint8_t* smem, const ELayout& L, uint64_t e, uint8_t* slot) {
  const LlvqClassHot* cls = reinterpret_cast<const LlvqClassHot*>(smem + L.cls);
  const uint32_t f = entry_f(e);
  const LlvqClassHot h = cls[entry_k(e)];
  const BlockStart bs = block_start<true>(smem, L, entry_J(e), h);
  OddDec<> od;
  od.init(h, bs);
  uint32_t w[6];
  // four values per dword: biased bytes (the class's int8 table) or fp8 codes
  if (OUT != LLVQ_OUT_POINTS_I8) od.load_fp8(h);
  {
#pragma unroll
    for (int q = 0; q < 6; ++q) {
      const uint32_t k0 = od.slot(smem, L, 4 * q);
      const uint32_t k1 = od.slot(smem, L, 4 * q + 1);
      const uint32_t k2 = od.slot(smem, L, 4 * q + 2);
      const uint32_t k3 = od.slot(smem, L, 4 * q + 3);
      w[q] = od.quad_codes(k0, k1, k2, k3, q);
    }
  }
  uint2* s2 = reinterpret_cast<uint2*>(slot);
  s2[0] = make_uint2(w[0], w[1]);
  s2[1] = make_uint2(w[2], w[3]);
  s2[2] = make_uint2(w[4], w[5]);
  return f;
}

// The same for an even-coset block: its values come in decode order and go to the slot
// by position.
template <int OUT>
__device__ __forceinline__ uint32_t stream_even_codes(uint8_t* smem, const ELayout& L, uint64_t e, uint8_t* slot) {
  const LlvqClassHot* cls = reinterpret_cast<const LlvqClassHot*>(smem + L.cls);
  const uint32_t f = entry_f(e);
  const LlvqClassHot h = cls[entry_k(e)];
  const BlockStart bs = block_start<true>(smem, L, entry_J(e), h);
  EvenDec<> ev;
  ev.init(h, bs, L.cls + entry_k(e) * (uint32_t)sizeof(LlvqClassHot));
  if (OUT == LLVQ_OUT_POINTS_I8) {
#pragma unroll
    for (int i = 0; i < 24; ++i) {
      uint32_t pos;
      const uint32_t bv = ev.step(smem, L, i, pos);
      slot[pos] = (uint8_t)bv;
    }
  } else {
    ev.load_fp8(h);
#pragma unroll
    for (int i = 0; i < 24; ++i) {
      uint32_t pos;
      const uint32_t k = ev.slot(smem, L, i, pos);
      slot[pos] = (uint8_t)__builtin_amdgcn_perm(ev.svhi, ev.svlo, k);
    }
  }
  return f;
}

template <int OUT>
__global__ __launch_bounds__(kEThreads) void k_decode_stream(KDesc d0, SArgs m, int32_t* err) {
  extern __shared__ __align__(16) uint8_t smem[];
  const ELayout& L = m.L;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const bool sg = d0.mode == LLVQ_MODE_SHAPEGAIN;
  float* part = reinterpret_cast<float*>(smem + m.part);
  int* work = reinterpret_cast<int*>(smem + L.work);   // unit counter, leftover counts, chunk counter
  uint64_t* shq = reinterpret_cast<uint64_t*>(smem + m.rings);
  uint8_t* slot = smem + m.stage + 24u * (uint32_t)tid;
  const uint32_t wbase = m.stage + 24u * 64u * (uint32_t)wave;

  // this workgroup's rows: [first row at or after block total * w / grid, the same for w + 1)
  const SPos p0 = stream_snap(m, m.total * blockIdx.x / gridDim.x);
  const SPos p1 = stream_snap(m, m.total * (blockIdx.x + 1) / gridDim.x);

  // Tile iteration: tensor ti, rows [row0, row0 + nrows) of its segment [.., rb), cut
  // into tiles of rpt rows (equal but the last, at most tmax blocks each).  Inside the
  // range ti < n and row0 < rb always hold.
  int ti = p0.t, row0 = p0.row, rb = 0, rpt = 1;
  auto in_range = [&]() { return ti < p1.t || (ti == p1.t && row0 < p1.row); };
  auto seg_begin = [&]() {
    const int kb = m.t[ti].kb;
    rb = ti == p1.t ? p1.row : m.t[ti].rows;
    const int rmax = m.tmax / kb;                      // >= 1 (checked on the host)
    const int nt = (rb - row0 + rmax - 1) / rmax;
    rpt = (rb - row0 + nt - 1) / nt;                  // <= rmax
  };
  if (in_range()) seg_begin();

  // the first tile's fields are requested before the tables are staged
  LaneField lf = {};
  if (in_range()) {
    const int nr = min(rpt, rb - row0);
    const int T0 = nr * m.t[ti].kb;
    KDesc dt = d0;
    dt.rows = m.t[ti].rows;
    dt.cols = m.t[ti].cols;
    dt.kb = m.t[ti].kb;
    lf = load_lane_field(dt, m.t[ti].packed, (uint32_t)(row0 * dt.kb), T0, min(wave, (T0 - 1) >> 6), lane);
  }
  engine_prologue(smem, L, d0, m.nbuckets, m.t[0].scales, tid);
  if (sg && OUT == LLVQ_OUT_BF16) {
    const int ng = 1 << d0.gain_bits;
    float* G = reinterpret_cast<float*>(smem + L.gains);
    for (int i = ng + tid; i < m.n * ng; i += kEThreads) G[i] = __half2float(m.t[i >> d0.gain_bits].scales[i & (ng - 1)]);
  }
  if (tid < 4) work[tid] = 0;
  __syncthreads();

  Rings R;
  R.odd = shq + (size_t)(2 * wave) * kRing;
  R.even = R.odd + kRing;
  for (int lt = 0; in_range(); ++lt) {
    const STensor& ts = m.t[ti];
    KDesc d = d0;
    d.rows = ts.rows;
    d.cols = ts.cols;
    d.kb = ts.kb;
    ELayout Lt = L;
    if (sg) Lt.gains += 4u * ((uint32_t)ti << d0.gain_bits);
    const int nrows = min(rpt, rb - row0);
    const int T = nrows * ts.kb;
    const int nun = (T + 63) >> 6;
    const uint32_t j0 = (uint32_t)(row0 * ts.kb);
    SOut o;
    o.out = static_cast<uint8_t*>(ts.out) +
            (size_t)row0 * (OUT == LLVQ_OUT_POINTS_I8 ? (size_t)ts.kb * 24u : (size_t)ts.cols * 2u);
    o.rs = (!sg && ts.scales) ? ts.scales + row0 : nullptr;
    o.cols = ts.cols;
    o.kb = ts.kb;
    o.inv_kb = 1.0f / (float)ts.kb;
    o.vec = OUT == LLVQ_OUT_POINTS_I8 ? ((((uintptr_t)ts.out) & 7u) == 0u)
                                      : ((((uintptr_t)ts.out) & 15u) == 0u && (ts.cols & 7) == 0);
    int u = wave;
    if (lt > 0) lf = load_lane_field(d, ts.packed, j0, T, min(u, nun - 1), lane);
    R.oh = R.on = R.eh = R.en = 0u;
    // Per iteration: classify the unit whose fields arrived, store the chunks decoded in
    // the previous iteration, request the next unit's fields, then decode at most one full
    // chunk of each ring (into the value slots, transposed into registers).  Between a
    // field request and its use no vector memory operation is issued, so the wait for the
    // fields (which on gfx9 also waits for every older store) only covers stores one
    // chunk decode old.  Both rings hold fewer than 64 entries after every iteration.
    SPend po, pe;
    po.m = 0u;
    pe.m = 0u;
    int zf = -1;                         // a field past the shell union, zeroed one iteration late
    while (u < nun) {
      const bool bad = classify_lane<OUT == LLVQ_OUT_BF16>(smem, Lt, part, d, lf, T, u, lane, err, R, o.rs,
                                                           o.inv_kb);
      stream_put<OUT>(o, po);
      stream_put<OUT>(o, pe);
      if (zf >= 0) stream_zero<OUT>(o, (uint32_t)zf);
      zf = bad ? u * 64 + lane : -1;
      int u2 = 0;
      if (lane == 0) u2 = atomicAdd(&work[0], 1);
      u2 = __builtin_amdgcn_readfirstlane(u2) + kEWaves;
      const LaneField lf2 = load_lane_field(d, ts.packed, j0, T, min(u2, nun - 1), lane);
      po.m = 0u;
      pe.m = 0u;
      if (R.on >= 64u) {
        const uint32_t f = stream_odd_codes<OUT>(smem, L, R.odd[(R.oh + (uint32_t)lane) & (kRing - 1)], slot);
        stream_transpose<OUT>(smem, part, o, wbase, f, 64, lane, po);
        R.oh = (R.oh + 64u) & (kRing - 1);
        R.on -= 64u;
      }
      if (R.en >= 64u) {
        const uint32_t f = stream_even_codes<OUT>(smem, L, R.even[(R.eh + (uint32_t)lane) & (kRing - 1)], slot);
        stream_transpose<OUT>(smem, part, o, wbase, f, 64, lane, pe);
        R.eh = (R.eh + 64u) & (kRing - 1);
        R.en -= 64u;
      }
      u = u2;
      lf = lf2;
    }
    stream_put<OUT>(o, po);
    stream_put<OUT>(o, pe);
    if (zf >= 0) stream_zero<OUT>(o, (uint32_t)zf);

    // the rings' remainders into one shared queue, decoded by all waves as full chunks
    constexpr int kLeftEven = kEWaves * 64;
    int bo = 0, be = 0;
    if (lane == 0) {
      bo = atomicAdd(&work[1], (int)R.on);
      be = atomicAdd(&work[2], (int)R.en);
    }
    bo = __builtin_amdgcn_readfirstlane(bo);
    be = __builtin_amdgcn_readfirstlane(be);
    LLVQ_DCHECK(bo + (int)R.on <= kLeftEven && be + (int)R.en <= kLeftEven && R.on < 64u && R.en < 64u);
    const uint64_t lo = (uint32_t)lane < R.on ? R.odd[(R.oh + (uint32_t)lane) & (kRing - 1)] : 0ull;
    const uint64_t le = (uint32_t)lane < R.en ? R.even[(R.eh + (uint32_t)lane) & (kRing - 1)] : 0ull;
    __syncthreads();                        // every ring read; the queue may overwrite them
    if ((uint32_t)lane < R.on) shq[bo + lane] = lo;
    if ((uint32_t)lane < R.en) shq[kLeftEven + be + lane] = le;
    __syncthreads();
    const int nlo = work[1], nle = work[2];
    const int nco = (nlo + 63) >> 6;
    const int nch = nco + ((nle + 63) >> 6);
    for (;;) {
      int c = 0;
      if (lane == 0) c = atomicAdd(&work[3], 1);
      c = __builtin_amdgcn_readfirstlane(c);
      if (c >= nch) break;
      uint32_t f = 0u;
      int n;
      if (c < nco) {
        const int e = (c << 6) + lane;
        n = min(64, nlo - (c << 6));
        if (e < nlo) f = stream_odd_codes<OUT>(smem, L, shq[e], slot);
      } else {
        const int e = ((c - nco) << 6) + lane;
        n = min(64, nle - ((c - nco) << 6));
        if (e < nle) f = stream_even_codes<OUT>(smem, L, shq[kLeftEven + e], slot);
      }
      SPend pl;
      stream_transpose<OUT>(smem, part, o, wbase, f, n, lane, pl);
      stream_put<OUT>(o, pl);
    }
    __syncthreads();                        // slots and queue free for the next tile
    if (tid < 4) work[tid] = 0;
    __syncthreads();

    // next tile: the rest of this segment, else the next tensor's segment
    row0 += nrows;
    if (row0 >= rb) {
      ++ti;
      row0 = 0;
      if (in_range()) seg_begin();
    }
  }
}
