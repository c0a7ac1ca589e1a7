// Batch-1 GEMV and bulk decode of the general decoder with coset queues (gfx950).
// Included once by llvq.hip after llvq_wide.h, whose class search and unranking state it
// uses.
//
// The one-block-per-lane kernels (k_gemv_wide, k_decode_wide) let a wavefront mix both
// cosets, one- and two-part classes and the exact and fp64 regimes of the unranking; their
// single pass over the 24 positions picks, per position and per lane, the support or
// complement unranker, so every step copies both states in and out.  Here a 1024-lane
// workgroup (one per CU) takes tiles of whole rows and streams them as the 2-bit kernels
// do: each wave takes units of 64 consecutive blocks from an LDS counter, classifies them
// (shell and class search as in the one-block-per-lane kernels, latency-bound global
// reads that the other waves' decode covers), keeps each block's scale in its LDS slot
// and appends the block (J = I - class start, class, block) to its odd or even ring, and
// decodes a full chunk of 64 blocks of one coset whenever a ring holds one.  The rings'
// remainders are gathered and decoded by all waves at the end of the tile.
//   An odd block is one multiset over all 24 positions, decoded in position order; an
// even block decodes its support values (on the codeword's positions, ascending) and then
// its complement values, each part in its own loop with its own state.  The signs follow
// the same rules as wide_decode_point, in the same order.  The GEMV dots the values with
// the activations (registers for odd blocks, LDS by position for even ones), scales the
// block's slot and sums the rows in a fixed order; the decode writes the int8 values into
// an LDS tile laid out like the output and then stores the tile row by row.
//   The fp64 arithmetic-decoding step multiplies by 1/c from an LDS table instead of
// dividing by c: one more rounding per step (four of at most 24 x 2^-53), so the bound of
// kFpRem becomes 2 x 24 x 4 x 24 x 2^-53 x 2^38 = 0.14, every slot choice still exact.

#pragma once

constexpr int kWTThreads = 1024;
constexpr int kWTWaves = kWTThreads / 64;
constexpr int kWTTileMax = 16384;         // block index in 16 bits with the class index

constexpr int kWRing = 128;                              // entries per ring (never more than 127)
constexpr int kWRingEntries = 2 * kWTWaves * kWRing;     // odd and even ring of every wave

struct WTArgs {
  int rows_per_tile, ntiles;
  uint32_t xs;      // LDS: GEMV: x of all kb * 24 columns, zero padded (bf16 or fp32);
                    //      decode: the value tile, int8 [rows][kb * 24]
  uint32_t rc;      // LDS: double[32], rc[c] = 1 / c
  uint32_t qj;      // LDS: uint64[kWRingEntries]: the rings' J, then the shared leftover queue's
  uint32_t qk;      // LDS: uint32[kWRingEntries]: class | block << 16, the same way
  uint32_t part;    // LDS: float[tmax] block scale, then (GEMV) the block's result
  uint32_t ctr;     // LDS: int[4]: unit counter, leftover fills, chunk counter
  int tmax;
};

// A wave's rings: odd entries at j[0 .. kWRing), even at j[kWRing .. 2 kWRing) (and k the
// same); entry i of a ring at (head + i) mod kWRing.  Heads and counts are wave-uniform.
struct WRings {
  uint64_t* j;
  uint32_t* k;
  uint32_t oh, on, eh, en;
};

// Classify field f of the tile (f >= T: nothing) and append it to the wave's ring of its
// coset.  The block's scale goes to part[f] (SCALE: G[g] / (4 sqrt m), or the row scale
// with ROWSCALE), 0 for an index past the shell union, which is counted, not queued, and
// (ZERO) gets 24 zero values in the value tile.
template <bool SCALE, bool ROWSCALE, bool ZERO>
__device__ __forceinline__ void wt_classify(const WDesc& d, const uint8_t* __restrict__ packed,
                                            const __half* __restrict__ scales, uint64_t j0, int row0, int T, int f,
                                            int lane, float* part, uint8_t* tile, int32_t* err, WRings& R) {
  bool odd = false, even = false;
  uint64_t J = 0;
  uint32_t k = 0;
  if (f < T) {
    uint64_t lo, hi;
    uint32_t g;
    float sc = 0.0f;
    if (wide_block(d, packed, j0 + (uint64_t)f, lo, hi, g)) {
      k = (uint32_t)wide_find_class(lo, hi, d.max_shell);
      LLVQ_DCHECK(k < (uint32_t)LLVQ_WIDE_NUM_CLASSES && dev_tables::kWideClass[k].m <= d.max_shell);
      const LlvqWideClass& cr = dev_tables::kWideClass[k];
      J = lo - cr.start_lo;
      odd = cr.parity != 0;
      even = !odd;
      if (SCALE) {
        if (d.mode == LLVQ_MODE_SHAPEGAIN)
          sc = __fmul_rn(__half2float(scales[g]), dev_tables::kWideInvNorm32[cr.m]);
        else
          sc = ROWSCALE ? __half2float(scales[row0 + (int)(((float)f + 0.5f) / (float)d.kb)]) : 1.0f;
      }
    } else {
      if (err) atomicAdd(err, 1);
      if (ZERO) {
        uint2* z = reinterpret_cast<uint2*>(tile + 24u * (uint32_t)f);
        z[0] = make_uint2(0u, 0u);
        z[1] = make_uint2(0u, 0u);
        z[2] = make_uint2(0u, 0u);
      }
    }
    part[f] = sc;
  }
  const uint64_t bo = __ballot(odd), be = __ballot(even);
  const uint32_t po = __builtin_amdgcn_mbcnt_hi((uint32_t)(bo >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bo, 0u));
  const uint32_t pe = __builtin_amdgcn_mbcnt_hi((uint32_t)(be >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)be, 0u));
  const uint32_t kf = k | ((uint32_t)f << 16);
  if (odd) {
    const uint32_t i = (R.oh + R.on + po) & (kWRing - 1);
    R.j[i] = J;
    R.k[i] = kf;
  }
  if (even) {
    const uint32_t i = kWRing + ((R.eh + R.en + pe) & (kWRing - 1));
    R.j[i] = J;
    R.k[i] = kf;
  }
  R.on += (uint32_t)__popcll(bo);
  R.en += (uint32_t)__popcll(be);
  LLVQ_DCHECK(R.on < (uint32_t)kWRing && R.en < (uint32_t)kWRing);
  // other lanes of the wave read these entries and slots next
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One tile streamed through the rings; odd_fn(J, kf) / even_fn(J, kf) decode one block.
// Ends with the tile's every block decoded and the workgroup synchronised.
template <bool SCALE, bool ROWSCALE, bool ZERO, class OddF, class EvenF>
__device__ __forceinline__ void wt_stream_tile(uint8_t* smem, const WDesc& d, const WTArgs& a,
                                               const uint8_t* __restrict__ packed, const __half* __restrict__ scales,
                                               int row0, int T, float* part, uint8_t* tile, int32_t* err, int wave,
                                               int lane, OddF odd_fn, EvenF even_fn) {
  uint64_t* qj = reinterpret_cast<uint64_t*>(smem + a.qj);
  uint32_t* qk = reinterpret_cast<uint32_t*>(smem + a.qk);
  int* ctr = reinterpret_cast<int*>(smem + a.ctr);
  const uint64_t j0 = (uint64_t)row0 * (uint64_t)d.kb;
  const int nun = (T + 63) >> 6;
  WRings R;
  R.j = qj + (size_t)wave * 2 * kWRing;
  R.k = qk + (size_t)wave * 2 * kWRing;
  R.oh = R.on = R.eh = R.en = 0u;
  int u = wave;
  while (u < nun) {
    int u2 = 0;
    if (lane == 0) u2 = atomicAdd(&ctr[0], 1);
    u2 = __builtin_amdgcn_readfirstlane(u2) + kWTWaves;
    wt_classify<SCALE, ROWSCALE, ZERO>(d, packed, scales, j0, row0, T, u * 64 + lane, lane, part, tile, err, R);
    while (R.on >= 64u) {
      const uint32_t i = (R.oh + (uint32_t)lane) & (kWRing - 1);
      odd_fn(R.j[i], R.k[i]);
      R.oh = (R.oh + 64u) & (kWRing - 1);
      R.on -= 64u;
    }
    while (R.en >= 64u) {
      const uint32_t i = kWRing + ((R.eh + (uint32_t)lane) & (kWRing - 1));
      even_fn(R.j[i], R.k[i]);
      R.eh = (R.eh + 64u) & (kWRing - 1);
      R.en -= 64u;
    }
    u = u2;
  }
  // the rings' remainders (< 64 each) into one shared queue: odd from the front, even from
  // kLeftEven; then decoded by all waves as full chunks
  constexpr int kLeftEven = kWTWaves * 64;
  int bo = 0, be = 0;
  if (lane == 0) {
    bo = atomicAdd(&ctr[1], (int)R.on);
    be = atomicAdd(&ctr[2], (int)R.en);
  }
  bo = __builtin_amdgcn_readfirstlane(bo);
  be = __builtin_amdgcn_readfirstlane(be);
  LLVQ_DCHECK(bo + (int)R.on <= kLeftEven && be + (int)R.en <= kLeftEven && R.on < 64u && R.en < 64u);
  uint64_t lj = 0, ej = 0;
  uint32_t lk = 0, ek = 0;
  if ((uint32_t)lane < R.on) {
    const uint32_t i = (R.oh + (uint32_t)lane) & (kWRing - 1);
    lj = R.j[i];
    lk = R.k[i];
  }
  if ((uint32_t)lane < R.en) {
    const uint32_t i = kWRing + ((R.eh + (uint32_t)lane) & (kWRing - 1));
    ej = R.j[i];
    ek = R.k[i];
  }
  __syncthreads();                        // every ring read; the queue may overwrite them
  if ((uint32_t)lane < R.on) {
    qj[bo + lane] = lj;
    qk[bo + lane] = lk;
  }
  if ((uint32_t)lane < R.en) {
    qj[kLeftEven + be + lane] = ej;
    qk[kLeftEven + be + lane] = ek;
  }
  __syncthreads();
  const int nlo = ctr[1], nle = ctr[2];
  const int nco = (nlo + 63) >> 6;
  const int nch = nco + ((nle + 63) >> 6);
  for (;;) {
    int c = 0;
    if (lane == 0) c = atomicAdd(&ctr[3], 1);
    c = __builtin_amdgcn_readfirstlane(c);
    if (c >= nch) break;
    if (c < nco) {
      const int e = (c << 6) + lane;
      if (e < nlo) odd_fn(qj[e], qk[e]);
    } else {
      const int e = ((c - nco) << 6) + lane;
      if (e < nle) even_fn(qj[kLeftEven + e], qk[kLeftEven + e]);
    }
  }
  __syncthreads();
}

// One value of a multiset unranking in progress (fp64 arithmetic decoding below 2^kFpRem
// arrangements left, exact 64-bit steps above): returns the value and advances U.
__device__ __forceinline__ uint32_t wt_next(Unranker& U, const double* rc) {
  uint32_t kk;
  if (U.fp) {
    const double y = U.u * (double)U.n;
    const int fy = (int)y;
    const uint64_t run = U.cnts * 0x0101010101010101ull;
    const uint64_t over = (run + (uint64_t)(127 - fy) * 0x0101010101010101ull) & 0x8080808080808080ull;
    kk = 8u - (uint32_t)__popcll(over);
    const uint32_t ck = (uint32_t)(U.cnts >> (8 * kk)) & 0xffu;
    LLVQ_DCHECK(kk < 8u && ck != 0u);
    const uint32_t below = kk ? (uint32_t)(run >> (8 * (kk - 1))) & 0xffu : 0u;
    U.u = (y - (double)below) * rc[ck];
  } else {
    const uint64_t t_n = U.rank * U.n;
    uint32_t ck = (uint32_t)U.cnts & 0xffu;
    uint64_t below = 0, upto = U.rem * ck;
    kk = 0;
    while (kk < 7u && t_n >= upto) {
      ++kk;
      ck = (uint32_t)(U.cnts >> (8 * kk)) & 0xffu;
      below = upto;
      upto += U.rem * ck;
    }
    LLVQ_DCHECK(U.n >= 1u && U.n <= 24u && ck != 0u && t_n < upto);
    const uint32_t tz = (uint32_t)__builtin_ctz(U.n);
    const uint64_t iv = dev_tables::kWideOddInverse[U.n >> (tz + 1)];
    U.rank = ((t_n - below) >> tz) * iv;
    U.rem = ((U.rem * ck) >> tz) * iv;
    to_fp(U);
  }
  const uint32_t a = (uint32_t)(U.vals >> (8 * kk)) & 0xffu;
  U.cnts -= 1ull << (8 * kk);
  U.n -= 1u;
  return a;
}

__device__ __forceinline__ void wt_init(Unranker& U, uint64_t rank, uint64_t rem, uint32_t n, const uint8_t* cnt,
                                        const uint8_t* val) {
  U.rank = rank;
  U.rem = rem;
  U.n = n;
  U.cnts = bytes8(cnt);
  U.vals = bytes8(val);
  U.fp = false;
  U.u = 0.0;
  to_fp(U);
}

template <bool XBF16>
__device__ __forceinline__ float wt_x(const uint8_t* smem, uint32_t xs, uint32_t col) {
  if (XBF16) return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(smem + xs)[col] << 16);
  return reinterpret_cast<const float*>(smem + xs)[col];
}

// odd block: <v, x> over its 24 positions, x of the block column b
template <bool XBF16>
__device__ __forceinline__ float wt_odd_dot(const uint8_t* smem, const WTArgs& a, const double* rc, uint64_t J,
                                            const LlvqWideClass& cr, uint32_t b) {
  const uint32_t c = dev_tables::kGolayTable[(uint32_t)(J & 4095u)];
  Unranker T;
  wt_init(T, J >> 12, cr.P_T, 24u, cr.cc, cr.cv);
  float xr[24];
  if (XBF16) {
    const uint4* p = reinterpret_cast<const uint4*>(smem + a.xs + b * 48u);
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const uint4 u = p[q];
      const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xr[8 * q + 2 * e] = __uint_as_float(w4[e] << 16);
        xr[8 * q + 2 * e + 1] = __uint_as_float(w4[e] & 0xffff0000u);
      }
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(smem + a.xs + b * 96u);
#pragma unroll
    for (int q = 0; q < 6; ++q) {
      const float4 u = p[q];
      xr[4 * q] = u.x; xr[4 * q + 1] = u.y; xr[4 * q + 2] = u.z; xr[4 * q + 3] = u.w;
    }
  }
  float t = 0.0f;
#pragma unroll
  for (int p = 0; p < kDim; ++p) {
    const int v = (int)wt_next(T, rc);
    const bool neg = ((v & 3) == 1) != (((c >> p) & 1u) != 0u);
    t = fmaf((float)(neg ? -v : v), xr[p], t);
  }
  return t;
}

// even block: the support part (codeword positions, ascending), then the complement part
template <bool XBF16>
__device__ __forceinline__ float wt_even_dot(const uint8_t* smem, const WTArgs& a, const double* rc, uint64_t J,
                                             const LlvqWideClass& cr, uint32_t b) {
  const uint32_t w = cr.w;
  const uint32_t A = dev_tables::kWideCodewords[w];
  uint64_t r, ip;
  if (A == 1u) {
    r = 0;
    ip = J;
  } else {
    ip = div_u64(J, A, r);
  }
  const uint32_t B = cr.B;
  const uint32_t s = (uint32_t)(ip & ((1ull << B) - 1ull));
  const uint64_t R = ip >> B;
  const uint32_t c = dev_tables::kGolayTable[dev_tables::kWideGolayOffset[w] + (uint32_t)r];
  uint64_t rs, rt;
  if (cr.P_S == 1) {
    rs = 0;
    rt = R;
  } else {
    rs = div_u64(R, cr.P_T, rt);
  }
  const uint32_t col0 = b * 24u;
  float t = 0.0f;
  // support: w values, all nonzero; the last (highest position) takes the parity sign
  {
    Unranker S;
    wt_init(S, rs, cr.P_S, w, cr.sc, cr.sv);
    const uint32_t wm1 = w ? w - 1u : 0u;
    const uint32_t negq = (((uint32_t)__popc(s & ((1u << wm1) - 1u))) & 1u) ^ cr.pi;
    uint32_t bits = s, cm = c;
    for (uint32_t i = 0; i < w; ++i) {
      const uint32_t p = (uint32_t)__builtin_ctz(cm);
      cm &= cm - 1u;
      const int v = (int)wt_next(S, rc);
      uint32_t neg;
      if (i + 1u == w) {
        neg = negq;
      } else {
        neg = bits & 1u;
        bits >>= 1;
      }
      t = fmaf((float)(neg ? -v : v), wt_x<XBF16>(smem, a.xs, col0 + p), t);
    }
  }
  // complement: 24 - w values on the other positions, the free signs after the support's
  {
    Unranker T;
    wt_init(T, rt, cr.P_T, 24u - w, cr.cc, cr.cv);
    uint32_t bits = w ? s >> (w - 1u) : s;
    uint32_t cm = ~c & 0xffffffu;
    for (uint32_t i = w; i < 24u; ++i) {
      const uint32_t p = (uint32_t)__builtin_ctz(cm);
      cm &= cm - 1u;
      const int v = (int)wt_next(T, rc);
      uint32_t neg = 0u;
      if (v != 0) {
        neg = bits & 1u;
        bits >>= 1;
      }
      t = fmaf((float)(neg ? -v : v), wt_x<XBF16>(smem, a.xs, col0 + p), t);
    }
  }
  return t;
}

template <bool XBF16>
__global__ __launch_bounds__(kWTThreads) void k_gemv_wide_tile(WDesc d, WTArgs a, const uint8_t* __restrict__ packed,
                                                               const __half* __restrict__ scales,
                                                               const void* __restrict__ xv, float* __restrict__ y,
                                                               int32_t* err) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const bool sg = d.mode == LLVQ_MODE_SHAPEGAIN;
  const int kb = d.kb;
  const float inv_kb = 1.0f / (float)kb;
  double* rc = reinterpret_cast<double*>(smem + a.rc);
  float* part = reinterpret_cast<float*>(smem + a.part);
  int* ctr = reinterpret_cast<int*>(smem + a.ctr);

  // activations (zero past K) and the reciprocals
  {
    const int ncol = kb * 24;
    if (XBF16) {
      uint16_t* xs = reinterpret_cast<uint16_t*>(smem + a.xs);
      const uint16_t* xg = static_cast<const uint16_t*>(xv);
      for (int i = tid; i < ncol; i += kWTThreads) xs[i] = i < d.cols ? xg[i] : (uint16_t)0;
    } else {
      float* xs = reinterpret_cast<float*>(smem + a.xs);
      const float* xg = static_cast<const float*>(xv);
      for (int i = tid; i < ncol; i += kWTThreads) xs[i] = i < d.cols ? xg[i] : 0.0f;
    }
    if (tid < 32) rc[tid] = tid ? 1.0 / (double)tid : 0.0;
    if (tid < 4) ctr[tid] = 0;
  }
  __syncthreads();

  auto col_of = [&](uint32_t f) { return f - (uint32_t)(((float)f + 0.5f) * inv_kb) * (uint32_t)kb; };
  auto odd_fn = [&](uint64_t J, uint32_t kf) __attribute__((always_inline)) {
    const uint32_t f = kf >> 16;
    part[f] *= wt_odd_dot<XBF16>(smem, a, rc, J, dev_tables::kWideClass[kf & 0xffffu], col_of(f));
  };
  auto even_fn = [&](uint64_t J, uint32_t kf) __attribute__((always_inline)) {
    const uint32_t f = kf >> 16;
    part[f] *= wt_even_dot<XBF16>(smem, a, rc, J, dev_tables::kWideClass[kf & 0xffffu], col_of(f));
  };
  for (int tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
    const int row0 = tile * a.rows_per_tile;
    const int nrows = min(a.rows_per_tile, d.rows - row0);
    const int T = nrows * kb;
    wt_stream_tile<true, false, false>(smem, d, a, packed, scales, row0, T, part, nullptr, err, wave, lane, odd_fn,
                                       even_fn);
    // row sums in a fixed order
    for (int rl = wave; rl < nrows; rl += kWTWaves) {
      float acc = 0.0f;
      for (int bb = lane; bb < kb; bb += 64) acc += part[rl * kb + bb];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
      if (lane == 0) {
        const int r = row0 + rl;
        y[r] = sg ? acc : acc * __half2float(scales[r]);
      }
    }
    if (tid < 4) ctr[tid] = 0;
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Decode of the general decoder with coset queues: the same classification and per-part
// decoders, each block's 24 values written as int8 into an LDS tile laid out like the
// output ([rows][kb * 24]); then a store phase walks the tile row by row, 8 columns per lane
// (bf16 = RNE(fp32(v) x scale), or the int8 values), so a wavefront's stores are contiguous.
// The decode itself reads class records and the inverse table from global memory, which
// never waits on stores: they all come after the tile's last barrier.

// odd block's values in position order into the tile (3 x 8 bytes)
__device__ __forceinline__ void wt_odd_vals(uint8_t* tile, const double* rc, uint64_t J, const LlvqWideClass& cr) {
  const uint32_t c = dev_tables::kGolayTable[(uint32_t)(J & 4095u)];
  Unranker T;
  wt_init(T, J >> 12, cr.P_T, 24u, cr.cc, cr.cv);
  uint32_t w[6];
#pragma unroll
  for (int q = 0; q < 6; ++q) {
    uint32_t x = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int p = 4 * q + e;
      const int v = (int)wt_next(T, rc);
      const bool neg = ((v & 3) == 1) != (((c >> p) & 1u) != 0u);
      x |= (uint32_t)(uint8_t)(neg ? -v : v) << (8 * e);
    }
    w[q] = x;
  }
  uint2* d = reinterpret_cast<uint2*>(tile);
  d[0] = make_uint2(w[0], w[1]);
  d[1] = make_uint2(w[2], w[3]);
  d[2] = make_uint2(w[4], w[5]);
}

// even block's values by position into the tile
__device__ __forceinline__ void wt_even_vals(uint8_t* tile, const double* rc, uint64_t J, const LlvqWideClass& cr) {
  const uint32_t w = cr.w;
  const uint32_t A = dev_tables::kWideCodewords[w];
  uint64_t r, ip;
  if (A == 1u) {
    r = 0;
    ip = J;
  } else {
    ip = div_u64(J, A, r);
  }
  const uint32_t B = cr.B;
  const uint32_t s = (uint32_t)(ip & ((1ull << B) - 1ull));
  const uint64_t R = ip >> B;
  const uint32_t c = dev_tables::kGolayTable[dev_tables::kWideGolayOffset[w] + (uint32_t)r];
  uint64_t rs, rt;
  if (cr.P_S == 1) {
    rs = 0;
    rt = R;
  } else {
    rs = div_u64(R, cr.P_T, rt);
  }
  {
    Unranker S;
    wt_init(S, rs, cr.P_S, w, cr.sc, cr.sv);
    const uint32_t wm1 = w ? w - 1u : 0u;
    const uint32_t negq = (((uint32_t)__popc(s & ((1u << wm1) - 1u))) & 1u) ^ cr.pi;
    uint32_t bits = s, cm = c;
    for (uint32_t i = 0; i < w; ++i) {
      const uint32_t p = (uint32_t)__builtin_ctz(cm);
      cm &= cm - 1u;
      const int v = (int)wt_next(S, rc);
      uint32_t neg;
      if (i + 1u == w) {
        neg = negq;
      } else {
        neg = bits & 1u;
        bits >>= 1;
      }
      tile[p] = (uint8_t)(neg ? -v : v);
    }
  }
  {
    Unranker T;
    wt_init(T, rt, cr.P_T, 24u - w, cr.cc, cr.cv);
    uint32_t bits = w ? s >> (w - 1u) : s;
    uint32_t cm = ~c & 0xffffffu;
    for (uint32_t i = w; i < 24u; ++i) {
      const uint32_t p = (uint32_t)__builtin_ctz(cm);
      cm &= cm - 1u;
      const int v = (int)wt_next(T, rc);
      uint32_t neg = 0u;
      if (v != 0) {
        neg = bits & 1u;
        bits >>= 1;
      }
      tile[p] = (uint8_t)(neg ? -v : v);
    }
  }
}

// int8 byte q of u as fp32
__device__ __forceinline__ float wt_i8(uint32_t u, int q) {
  return (float)(int)__builtin_amdgcn_sbfe(u, 8 * q, 8);
}

template <int OUT>
__global__ __launch_bounds__(kWTThreads) void k_decode_wide_tile(WDesc d, WTArgs a, const uint8_t* __restrict__ packed,
                                                                 const __half* __restrict__ scales,
                                                                 void* __restrict__ out, int32_t* err, bool ovec) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kb = d.kb;
  const uint32_t rowbytes = (uint32_t)kb * 24u;
  double* rc = reinterpret_cast<double*>(smem + a.rc);
  float* part = reinterpret_cast<float*>(smem + a.part);
  int* ctr = reinterpret_cast<int*>(smem + a.ctr);
  uint8_t* tile = smem + a.xs;
  if (tid < 32) rc[tid] = tid ? 1.0 / (double)tid : 0.0;
  if (tid < 4) ctr[tid] = 0;
  __syncthreads();

  auto odd_fn = [&](uint64_t J, uint32_t kf) __attribute__((always_inline)) {
    wt_odd_vals(tile + 24u * (kf >> 16), rc, J, dev_tables::kWideClass[kf & 0xffffu]);
  };
  auto even_fn = [&](uint64_t J, uint32_t kf) __attribute__((always_inline)) {
    wt_even_vals(tile + 24u * (kf >> 16), rc, J, dev_tables::kWideClass[kf & 0xffffu]);
  };
  for (int tl = blockIdx.x; tl < a.ntiles; tl += gridDim.x) {
    const int row0 = tl * a.rows_per_tile;
    const int nrows = min(a.rows_per_tile, d.rows - row0);
    const int T = nrows * kb;
    wt_stream_tile<OUT == LLVQ_OUT_BF16, true, true>(smem, d, a, packed, scales, row0, T, part, tile, err, wave, lane,
                                                     odd_fn, even_fn);

    // store the tile row by row, 8 columns per lane
    if (OUT == LLVQ_OUT_POINTS_I8) {
      const uint32_t n8 = rowbytes >> 3;
      for (int rl = 0; rl < nrows; ++rl) {
        int8_t* orow = static_cast<int8_t*>(out) + (size_t)(row0 + rl) * rowbytes;
        const uint8_t* trow = tile + (uint32_t)rl * rowbytes;
        for (uint32_t j = (uint32_t)tid; j < n8; j += kWTThreads) {
          const uint2 u = *reinterpret_cast<const uint2*>(trow + 8u * j);
          if (ovec) {
            *reinterpret_cast<uint2*>(orow + 8u * j) = u;
          } else {
            reinterpret_cast<uint32_t*>(orow + 8u * j)[0] = u.x;   // rows are whole dwords, out 4-byte aligned
            reinterpret_cast<uint32_t*>(orow + 8u * j)[1] = u.y;
          }
        }
      }
    } else {
      const int K = d.cols;
      const uint32_t n8 = (uint32_t)(K + 7) >> 3;
      for (int rl = 0; rl < nrows; ++rl) {
        uint16_t* orow = static_cast<uint16_t*>(out) + (size_t)(row0 + rl) * (size_t)K;
        const uint8_t* trow = tile + (uint32_t)rl * rowbytes;
        for (uint32_t j = (uint32_t)tid; j < n8; j += kWTThreads) {
          const uint2 u = *reinterpret_cast<const uint2*>(trow + 8u * j);
          const float sc = part[rl * kb + (int)(j / 3u)];
          float v[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) v[q] = __fmul_rn(wt_i8(q < 4 ? u.x : u.y, q & 3), sc);
          const uint4 pk = make_uint4(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]), pack_bf16(v[4], v[5]),
                                      pack_bf16(v[6], v[7]));
          const uint32_t col = 8u * j;
          if (ovec && (int)col + 8 <= K) {
            *reinterpret_cast<uint4*>(orow + col) = pk;
          } else {
            const uint32_t wv[4] = {pk.x, pk.y, pk.z, pk.w};
#pragma unroll
            for (int q = 0; q < 8; ++q)
              if ((int)(col + q) < K) orow[col + q] = (uint16_t)(wv[q >> 1] >> (16 * (q & 1)));
          }
        }
      }
    }
    if (tid < 4) ctr[tid] = 0;
    __syncthreads();
  }
}
