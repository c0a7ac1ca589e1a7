// General decoder (gfx950): shells 2..42 of the Leech lattice and index fields up to 128
// bits, for rates other than the 2-bit configuration ("LLVQ: Leech Lattice Vector
// Quantization", papernotes.org notes, 关键设计 2: the same hierarchy shell -> class ->
// codeword / sign pattern / permutation rank at any shell radius; 3 bits per weight is a
// 72-bit field per 24-block, 68 shape bits reach shell 42).
//
// Beyond shell 10 the fixed-width shortcuts of the 2-bit kernels no longer hold (class
// sizes reach 2^60, the index past the codeword reaches 2^53, up to 8 distinct absolute
// values up to 25 per class, global indices past 2^64), so this decoder works with exact
// 64-bit integers inside a class and 128-bit compares for the global index:
//   * shell by binary search over 128-bit starts; class through a per-shell bucket table
//     (the offset inside the shell shifted to at most 1024 buckets) and a binary search
//     over the few class starts it leaves (records in global memory, read through the
//     caches: 38,649 classes, 2.8 MB);
//   * J = I - start < 2^63; r = J mod A, I' = J div A; s = I' mod 2^B, R = I' >> B;
//     even classes R = rank_S * P_T + rank_T;
//   * both multiset unrankings advance in one pass over the 24 positions: position p takes
//     the next value of the support sequence if p is on the codeword, of the complement
//     sequence otherwise (each sequence fills its positions in ascending order).  The
//     arrangements starting with value v are rem * count(v) / n, an exact quotient taken
//     as a product with the inverse of n's odd part modulo 2^64 (a 96-byte table read
//     through the caches; an LDS copy of it gave wrong quotients in workgroups that
//     shared a CU with another, a cause not found, so it stays in global memory); once
//     fewer than 2^kFpRem arrangements are left the part is finished by fp64 arithmetic
//     decoding (see kFpRem);
//   * signs as in the 2-bit kernels.
// One 24-block per lane; VALU-bound.  Included once by llvq.hip after the generated
// tables.

#pragma once

constexpr int kWideThreads = 256;
constexpr int kRankWideMaxShell = 33;   // the rank's output is 64-bit: shells 2..33 (C_33 < 2^64)

struct WDesc {
  int32_t mode, rows, cols, kb;
  int32_t max_shell, shape_bits, gain_bits, field_bits;
  uint64_t count_lo, count_hi;    // index count of shells 2..max_shell (128-bit)
};

struct U128 {
  uint64_t lo, hi;
};

__device__ __forceinline__ bool u128_le(uint64_t alo, uint64_t ahi, uint64_t blo, uint64_t bhi) {
  return ahi < bhi || (ahi == bhi && alo <= blo);
}

// field j of a little-endian bitstream of f-bit fields (f <= 128); reads only the dwords
// that hold the field's bits
__device__ __forceinline__ U128 read_field_wide(const uint8_t* __restrict__ packed, uint64_t j, int f) {
  const uint64_t bit = j * (uint64_t)f;
  const uint32_t* w = reinterpret_cast<const uint32_t*>(packed) + (bit >> 5);
  const uint32_t sh = (uint32_t)(bit & 31u);
  const uint32_t nw = (sh + (uint32_t)f + 31u) >> 5;     // 1..5 dwords
  uint32_t d[5];
#pragma unroll
  for (int k = 0; k < 5; ++k) d[k] = (uint32_t)k < nw ? w[k] : 0u;
  const uint64_t a = (uint64_t)d[0] | ((uint64_t)d[1] << 32);
  const uint64_t b = (uint64_t)d[2] | ((uint64_t)d[3] << 32);
  const uint64_t c = (uint64_t)d[4];
  U128 r;
  r.lo = sh ? ((a >> sh) | (b << (64u - sh))) : a;
  r.hi = sh ? ((b >> sh) | (c << (64u - sh))) : b;
  if (f < 64) {
    r.lo &= (1ull << f) - 1ull;
    r.hi = 0;
  } else if (f == 64) {
    r.hi = 0;
  } else if (f < 128) {
    r.hi &= (1ull << (f - 64)) - 1ull;
  }
  return r;
}

// q, r = x div d, x mod d for x < 2^63, 0 < d < 2^62: an fp64 estimate, one fp64 refinement
// of the signed remainder, then exact integer steps (the estimate is off by at most a few
// units, so the steps run at most a few times; the remainder never overflows)
__device__ __forceinline__ uint64_t div_u64(uint64_t x, uint64_t d, uint64_t& r) {
  uint64_t q = (uint64_t)((double)x / (double)d);
  int64_t rr = (int64_t)(x - q * d);
  q += (uint64_t)(int64_t)floor((double)rr / (double)d);
  rr = (int64_t)(x - q * d);
  while (rr < 0) {
    --q;
    rr += (int64_t)d;
  }
  while (rr >= (int64_t)d) {
    ++q;
    rr -= (int64_t)d;
  }
  r = (uint64_t)rr;
  return q;
}

// class holding global index I (< the index count of shells 2..M)
__device__ __forceinline__ int wide_find_class(uint64_t lo, uint64_t hi, int M) {
  // shell: the last m in 2..M with start(m) <= I
  int a = 2, b = M;
  while (a < b) {
    const int mid = (a + b + 1) >> 1;
    if (u128_le(dev_tables::kWideShellStart[mid][0], dev_tables::kWideShellStart[mid][1], lo, hi))
      a = mid;
    else
      b = mid - 1;
  }
  // bucket of the offset inside the shell (the offset is below 2^68, the shift below 64)
  const uint64_t slo = dev_tables::kWideShellStart[a][0], shi = dev_tables::kWideShellStart[a][1];
  const uint64_t jlo = lo - slo;
  const uint64_t jhi = hi - shi - (lo < slo ? 1u : 0u);
  const int sh = dev_tables::kWideBucketShift[a];
  const uint32_t bkt = (uint32_t)(sh ? ((jlo >> sh) | (jhi << (64 - sh))) : jlo);
  const uint16_t* bk = dev_tables::kWideBucket + dev_tables::kWideBucketOff[a];
  const int f0 = dev_tables::kWideShellFirst[a];
  // class: the last one between the bucket's two bounds with start <= I
  int ca = f0 + bk[bkt], cb = f0 + bk[bkt + 1];
  while (ca < cb) {
    const int mid = (ca + cb + 1) >> 1;
    const LlvqWideClass& c = dev_tables::kWideClass[mid];
    if (u128_le(c.start_lo, c.start_hi, lo, hi))
      ca = mid;
    else
      cb = mid - 1;
  }
  return ca;
}

// one multiset unranking in progress: rem = arrangements of what is left, n values left,
// counts and values of the distinct values (ascending) one per byte
struct Unranker {
  uint64_t rem, rank, cnts, vals;
  uint32_t n;
  bool fp;      // the rank is carried as u = (rank + 1/2) / rem in fp64 (rem < 2^kFpRem)
  double u;
};

// Below 2^kFpRem arrangements left, a part is finished by arithmetic decoding in fp64: u
// locates the rank inside [0, 1) in an interval of half-width 1/(2 rem); each step
// u' = (u n - C_k) / c_k scales the interval by n / c_k and adds three roundings of at most
// 24 x 2^-53.  An error made while rem_t arrangements were left is scaled by rem_t / rem at a
// later step, so against that step's half-width the at most 24 errors sum to below
// 2 x 24 x 3 x 24 x 2^-53 x 2^kFpRem = 0.11 (kFpRem = 38): every slot choice is exact.
constexpr int kFpRem = 38;

__device__ __forceinline__ void to_fp(Unranker& U) {
  if (!U.fp && U.rem < (1ull << kFpRem)) {
    U.u = ((double)U.rank + 0.5) / (double)U.rem;
    U.fp = true;
  }
}

__device__ __forceinline__ uint64_t bytes8(const uint8_t* p) {
  uint64_t v = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) v |= (uint64_t)p[k] << (8 * k);
  return v;
}

// Integer lattice point of global shape index I (valid: I < count).  Returns the shell.
__device__ __forceinline__ int wide_decode_point(uint64_t lo, uint64_t hi, int M, int v[kDim]) {
  const uint64_t* inv = dev_tables::kWideOddInverse;
  const int k = wide_find_class(lo, hi, M);
  LLVQ_DCHECK(k >= 0 && k < LLVQ_WIDE_NUM_CLASSES && dev_tables::kWideClass[k].m <= M);
  const LlvqWideClass& cr = dev_tables::kWideClass[k];
  const uint64_t J = lo - cr.start_lo;      // < 2^63: the high words cancel
  const int w = cr.w;
  const uint32_t A = cr.parity ? 4096u : dev_tables::kWideCodewords[w];
  uint64_t r, ip;
  if (A == 4096u) {
    r = J & 4095u;
    ip = J >> 12;
  } else if (A == 1u) {
    r = 0;
    ip = J;
  } else {
    ip = div_u64(J, A, r);
  }
  const uint32_t B = cr.B;
  const uint32_t s = (uint32_t)(ip & ((1ull << B) - 1ull));
  const uint64_t R = ip >> B;
  const uint32_t c = dev_tables::kGolayTable[(cr.parity ? 0u : dev_tables::kWideGolayOffset[w]) + (uint32_t)r];

  // support sequence (even classes, on the codeword) and complement sequence
  Unranker S, T;
  if (cr.P_S == 1) {
    S.rank = 0;
    T.rank = R;
  } else {
    S.rank = div_u64(R, cr.P_T, T.rank);
  }
  S.rem = cr.P_S;
  T.rem = cr.P_T;
  S.n = (uint32_t)w;
  T.n = (uint32_t)(kDim - w);
  S.cnts = bytes8(cr.sc);
  S.vals = bytes8(cr.sv);
  T.cnts = bytes8(cr.cc);
  T.vals = bytes8(cr.cv);
  S.fp = false;
  T.fp = false;
  S.u = 0.0;
  T.u = 0.0;
  to_fp(S);
  to_fp(T);

  const uint32_t sel = (cr.parity == 0 && w) ? c : 0u;
  const int q = (cr.parity == 0 && w) ? (31 - __clz((int)c)) : -1;
  const uint32_t wm1 = w ? (uint32_t)(w - 1) : 0u;
  uint32_t bitsS = s;
  uint32_t bitsT = (cr.parity == 0 && w) ? (s >> wm1) : s;
  const uint32_t negq = (cr.parity == 0 && w) ? (((uint32_t)__popc(s & ((1u << wm1) - 1u)) & 1u) ^ cr.pi) : 0u;
#pragma unroll
  for (int p = 0; p < kDim; ++p) {
    const bool inS = (sel >> p) & 1u;
    Unranker U = inS ? S : T;
    uint32_t kk;
    if (U.fp) {
      // arithmetic decoding: slot k is the number of running counts c_0 + .. + c_j at most
      // floor(u n) (one per byte, all below 25, compared at once)
      const double y = U.u * (double)U.n;
      const int fy = (int)y;
      const uint64_t run = U.cnts * 0x0101010101010101ull;
      const uint64_t over = (run + (uint64_t)(127 - fy) * 0x0101010101010101ull) & 0x8080808080808080ull;
      kk = 8u - (uint32_t)__popcll(over);
      const uint32_t ck = (uint32_t)(U.cnts >> (8 * kk)) & 0xffu;
      LLVQ_DCHECK(kk < 8u && ck != 0u);
      const uint32_t below = kk ? (uint32_t)(run >> (8 * (kk - 1))) & 0xffu : 0u;
      U.u = (y - (double)below) / (double)ck;
    } else {
      // the arrangements starting with value slot k number rem * c_k / n; the slot holding
      // rank is the first k with rank * n < rem * (c_0 + ... + c_k), compared without
      // dividing
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
      // new rank and count of arrangements: exact quotients by n
      LLVQ_DCHECK(U.n >= 1u && U.n <= 24u && ck != 0u && t_n < upto);
      const uint32_t tz = (uint32_t)__builtin_ctz(U.n);
      const uint64_t iv = inv[U.n >> (tz + 1)];
      U.rank = ((t_n - below) >> tz) * iv;
      U.rem = ((U.rem * ck) >> tz) * iv;
      to_fp(U);
    }
    const int a = (int)((U.vals >> (8 * kk)) & 0xffu);
    U.cnts -= 1ull << (8 * kk);
    U.n -= 1u;
    if (inS)
      S = U;
    else
      T = U;
    uint32_t neg;
    if (cr.parity) {
      neg = (uint32_t)(((a & 3) == 1) != (((c >> p) & 1u) != 0u));
    } else if (a == 0) {
      neg = 0u;
    } else if (p == q) {
      neg = negq;
    } else if (inS) {
      neg = bitsS & 1u;
      bitsS >>= 1;
    } else {
      neg = bitsT & 1u;
      bitsT >>= 1;
    }
    v[p] = neg ? -a : a;
  }
  return cr.m;
}

// shape index and gain of block j, and whether the index is in range
__device__ __forceinline__ bool wide_block(const WDesc& d, const uint8_t* __restrict__ packed, uint64_t j,
                                           uint64_t& lo, uint64_t& hi, uint32_t& g) {
  const U128 fv = read_field_wide(packed, j, d.field_bits);
  const int sb = d.shape_bits;
  if (sb < 64) {
    lo = fv.lo & ((1ull << sb) - 1ull);
    hi = 0;
    g = (uint32_t)((fv.lo >> sb) | (sb ? (fv.hi << (64 - sb)) : 0ull));
  } else if (sb == 64) {
    lo = fv.lo;
    hi = 0;
    g = (uint32_t)fv.hi;
  } else {
    lo = fv.lo;
    hi = fv.hi & ((1ull << (sb - 64)) - 1ull);
    g = (uint32_t)(fv.hi >> (sb - 64));
  }
  g &= (1u << d.gain_bits) - 1u;
  return !u128_le(d.count_lo, d.count_hi, lo, hi);     // I < count
}

// ovec (bf16): the output and its rows are 16-byte aligned, so a full block's 24 weights
// leave as three 16-byte stores
template <int OUT>
__global__ __launch_bounds__(kWideThreads) void k_decode_wide(WDesc d, const uint8_t* __restrict__ packed,
                                                              const __half* __restrict__ scales,
                                                              void* __restrict__ out, int32_t* err, bool ovec) {
  const uint64_t nblocks = (uint64_t)d.rows * (uint64_t)d.kb;
  for (uint64_t j = (uint64_t)blockIdx.x * kWideThreads + threadIdx.x; j < nblocks;
       j += (uint64_t)gridDim.x * kWideThreads) {
    uint64_t lo, hi;
    uint32_t g;
    int v[kDim];
    int m = 0;
    if (wide_block(d, packed, j, lo, hi, g)) {
      m = wide_decode_point(lo, hi, d.max_shell, v);
    } else {
#pragma unroll
      for (int p = 0; p < kDim; ++p) v[p] = 0;
      if (err) atomicAdd(err, 1);
    }
    const uint64_t r = j / (uint64_t)d.kb;
    const int b = (int)(j - r * (uint64_t)d.kb);
    if (OUT == LLVQ_OUT_POINTS_I8) {
      uint32_t* o = reinterpret_cast<uint32_t*>(static_cast<int8_t*>(out) + j * kDim);
#pragma unroll
      for (int q = 0; q < kDim / 4; ++q)
        o[q] = (uint32_t)(uint8_t)v[4 * q] | ((uint32_t)(uint8_t)v[4 * q + 1] << 8) |
               ((uint32_t)(uint8_t)v[4 * q + 2] << 16) | ((uint32_t)(uint8_t)v[4 * q + 3] << 24);
    } else {
      const float sc = d.mode == LLVQ_MODE_SHAPEGAIN
                           ? (m ? __fmul_rn(__half2float(scales[g]), dev_tables::kWideInvNorm32[m]) : 0.0f)
                           : __half2float(scales[r]);
      uint16_t* o = static_cast<uint16_t*>(out) + r * (uint64_t)d.cols + (uint64_t)b * kDim;
      const int lim = min(kDim, d.cols - b * kDim);
      if (ovec && lim == kDim) {
        uint32_t w[12];
#pragma unroll
        for (int q = 0; q < 12; ++q)
          w[q] = (uint32_t)f32_to_bf16_rne(__fmul_rn((float)v[2 * q], sc)) |
                 ((uint32_t)f32_to_bf16_rne(__fmul_rn((float)v[2 * q + 1], sc)) << 16);
        uint4* o4 = reinterpret_cast<uint4*>(o);
        o4[0] = make_uint4(w[0], w[1], w[2], w[3]);
        o4[1] = make_uint4(w[4], w[5], w[6], w[7]);
        o4[2] = make_uint4(w[8], w[9], w[10], w[11]);
      } else {
#pragma unroll
        for (int p = 0; p < kDim; ++p)
          if (p < lim) o[p] = f32_to_bf16_rne(__fmul_rn((float)v[p], sc));
      }
    }
  }
}

// y[bi][r] = sum over blocks of scale * (v . x[bi]); one wave per row, lanes over the
// row's blocks, fixed-order wave reduction (repeatable bit for bit).  MAXB: 1 for batch 1
// (fewer registers, more waves in flight to cover the table reads), else 16.  xvec: x is 16-byte
// aligned with 16-byte aligned rows, so a full block's activations load as 16-byte words.
template <bool XBF16, int MAXB>
__global__ __launch_bounds__(kWideThreads) void k_gemv_wide(WDesc d, const uint8_t* __restrict__ packed,
                                                            const __half* __restrict__ scales,
                                                            const void* __restrict__ xv, int batch, bool xvec,
                                                            float* __restrict__ y, int32_t* err) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int K = d.cols;
  for (int r = blockIdx.x * (kWideThreads / 64) + wave; r < d.rows; r += gridDim.x * (kWideThreads / 64)) {
    float acc[MAXB];
#pragma unroll
    for (int bi = 0; bi < MAXB; ++bi) acc[bi] = 0.0f;
    const float rs = d.mode == LLVQ_MODE_SHAPEGAIN ? 0.0f : __half2float(scales[r]);
    for (int b = lane; b < d.kb; b += 64) {
      const uint64_t j = (uint64_t)r * (uint64_t)d.kb + (uint64_t)b;
      uint64_t lo, hi;
      uint32_t g;
      int v[kDim];
      int m = 0;
      if (wide_block(d, packed, j, lo, hi, g)) {
        m = wide_decode_point(lo, hi, d.max_shell, v);
      } else {
#pragma unroll
        for (int p = 0; p < kDim; ++p) v[p] = 0;
        if (err) atomicAdd(err, 1);
      }
      const float sc = d.mode == LLVQ_MODE_SHAPEGAIN
                           ? (m ? __fmul_rn(__half2float(scales[g]), dev_tables::kWideInvNorm32[m]) : 0.0f)
                           : rs;
      const int k0 = b * kDim;
      const int lim = min(kDim, K - k0);
#pragma unroll
      for (int bi = 0; bi < MAXB; ++bi) {
        if (bi < batch) {
          float t = 0.0f;
          const size_t x0 = (size_t)bi * (size_t)K + (size_t)k0;
          if (xvec && lim == kDim) {
            // the block's 24 activations as 16-byte loads (3 for bf16, 6 for fp32)
            if (XBF16) {
              const uint4* xp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(xv) + x0);
#pragma unroll
              for (int q = 0; q < 3; ++q) {
                const uint4 u = xp[q];
                const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  t = fmaf((float)v[8 * q + 2 * e], __uint_as_float(w4[e] << 16), t);
                  t = fmaf((float)v[8 * q + 2 * e + 1], __uint_as_float(w4[e] & 0xffff0000u), t);
                }
              }
            } else {
              const float4* xp = reinterpret_cast<const float4*>(static_cast<const float*>(xv) + x0);
#pragma unroll
              for (int q = 0; q < 6; ++q) {
                const float4 u = xp[q];
                t = fmaf((float)v[4 * q], u.x, t);
                t = fmaf((float)v[4 * q + 1], u.y, t);
                t = fmaf((float)v[4 * q + 2], u.z, t);
                t = fmaf((float)v[4 * q + 3], u.w, t);
              }
            }
          } else {
#pragma unroll
            for (int p = 0; p < kDim; ++p) {
              if (p < lim) {
                const float xf = XBF16 ? bf16_to_f32(static_cast<const uint16_t*>(xv)[x0 + p])
                                       : static_cast<const float*>(xv)[x0 + p];
                t = fmaf((float)v[p], xf, t);
              }
            }
          }
          acc[bi] = fmaf(sc, t, acc[bi]);
        }
      }
    }
#pragma unroll
    for (int bi = 0; bi < MAXB; ++bi) {
      if (bi < batch) {
        float a = acc[bi];
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) a += __shfl_xor(a, o, 64);
        if (lane == 0) y[(size_t)bi * (size_t)d.rows + (size_t)r] = a;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Rank at shells 2..M (lattice point -> global index), the inverse of wide_decode_point.
// Membership as in the 2-bit rank (common parity p, sum = 4p mod 8, norm 16 m with
// 2 <= m <= M, the positions = 2 (p = 0) or = 1 (p = 1) mod 4 a Golay codeword, found from
// its information bits); the class by binary search of the point's key (coset, then the
// counts of its absolute values from the largest down) among the shell's class keys; the
// multiset ranks R_S, R_T accumulate rem * (c_0 + .. + c_{k-1}) / n per position (exact
// quotients); the free signs in decode order.  Returns false for a point that is not in
// the shell union.

// one multiset ranking in progress: rank so far, arrangements left, counts, values left
struct Ranker {
  uint64_t rank, rem, cnts;
  uint32_t n, present;     // present: bit v set for each value v of the multiset (fixed)
};

__device__ __forceinline__ bool wide_rank_point(const int (&v)[kDim], int M, uint64_t& lo, uint64_t& hi) {
  const uint64_t* inv = dev_tables::kWideOddInverse;
  const int par = v[0] & 1;
  int n2 = 0, sum = 0;
  uint32_t odd = 0, mask = 0, neg = 0, nz = 0;
  uint64_t key = (uint64_t)par << 62;
#pragma unroll
  for (int p = 0; p < kDim; ++p) {
    const int a = v[p];
    n2 += a * a;
    sum += a;
    odd |= (uint32_t)(a & 1) << p;
    mask |= (uint32_t)((a & 3) == (par ? 1 : 2)) << p;
    neg |= (uint32_t)(a < 0) << p;
    nz |= (uint32_t)(a != 0) << p;
  }
  if (odd != (par ? 0xffffffu : 0u) || (n2 & 15) || ((sum - 4 * par) & 7)) return false;
  const int m = n2 >> 4;
  if (m < 2 || m > M) return false;
  const uint32_t pos = dev_tables::kGolayInfoPos[(mask >> 11) & 0xfffu];
  if (dev_tables::kGolayTable[pos] != mask) return false;
#pragma unroll
  for (int p = 0; p < kDim; ++p) {
    const int a = v[p] < 0 ? -v[p] : v[p];
    if (a > par) key += 1ull << (5 * ((a - par) / 2 - 1));
  }
  int ca = dev_tables::kWideShellFirst[m], cb = dev_tables::kWideShellFirst[m + 1] - 1;
  while (ca < cb) {
    const int mid = (ca + cb + 1) >> 1;
    if (dev_tables::kWideKey[mid] <= key)
      ca = mid;
    else
      cb = mid - 1;
  }
  if (dev_tables::kWideKey[ca] != key) return false;
  const LlvqWideClass& cr = dev_tables::kWideClass[ca];
  const int w = cr.w;
  const bool two = cr.parity == 0 && w > 0;              // support part on the codeword
  const uint32_t sel = two ? mask : 0u;
  Ranker S, T;
  S.rank = 0;
  T.rank = 0;
  S.rem = cr.P_S;
  T.rem = cr.P_T;
  S.cnts = bytes8(cr.sc);
  T.cnts = bytes8(cr.cc);
  S.n = (uint32_t)w;
  T.n = (uint32_t)(kDim - w);
  S.present = 0;
  T.present = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (cr.sc[k]) S.present |= 1u << cr.sv[k];
    if (cr.cc[k]) T.present |= 1u << cr.cv[k];
  }
  const int q = two ? (31 - __clz((int)mask)) : -1;
  uint64_t s_sup = 0, s_comp = 0;
  uint32_t js = 0, jt = 0;
#pragma unroll
  for (int p = 0; p < kDim; ++p) {
    const bool inS = (sel >> p) & 1u;
    Ranker U = inS ? S : T;
    const uint32_t a = (uint32_t)(v[p] < 0 ? -v[p] : v[p]);
    const uint32_t k = (uint32_t)__popc(U.present & ((1u << a) - 1u));
    const uint64_t below = U.cnts & ((1ull << (8 * k)) - 1ull);   // k <= 7
    const uint32_t cum = (uint32_t)((below * 0x0101010101010101ull) >> 56);
    const uint32_t ck = (uint32_t)(U.cnts >> (8 * k)) & 0xffu;
    const uint32_t tz = (uint32_t)__builtin_ctz(U.n);
    const uint64_t iv = inv[U.n >> (tz + 1)];
    U.rank += ((U.rem * cum) >> tz) * iv;
    U.rem = ((U.rem * ck) >> tz) * iv;
    U.cnts -= 1ull << (8 * k);
    U.n -= 1u;
    if (inS)
      S = U;
    else
      T = U;
    // free signs: support positions but q, then nonzero complement positions
    const uint64_t nb = (neg >> p) & 1u;
    if (inS) {
      if (p != q) {
        s_sup |= nb << js;
        ++js;
      }
    } else if ((nz >> p) & 1u) {
      s_comp |= nb << jt;
      ++jt;
    }
  }
  const uint64_t s = cr.parity ? 0ull : (s_sup | (s_comp << js));
  const uint64_t R = S.rank * cr.P_T + T.rank;
  const uint32_t A = cr.parity ? 4096u : dev_tables::kWideCodewords[w];
  const uint64_t r = cr.parity ? pos : pos - dev_tables::kWideGolayOffset[w];
  const uint64_t J = r + (uint64_t)A * (s + (R << cr.B));
  lo = cr.start_lo + J;
  hi = cr.start_hi + (lo < J ? 1u : 0u);
  return true;
}

// one point per lane; WIDE: 128-bit indices as (lo, hi) pairs, shells 2..42; otherwise 64-bit
// indices, shells 2..33 (below 2^64).  A point outside the shell union gets all ones and is
// counted.
template <bool WIDE>
__global__ __launch_bounds__(kWideThreads) void k_rank_wide(const int8_t* __restrict__ pts, int64_t n, int M,
                                                            uint64_t* __restrict__ out, int32_t* err) {
  for (int64_t i = (int64_t)blockIdx.x * kWideThreads + threadIdx.x; i < n; i += (int64_t)gridDim.x * kWideThreads) {
    int v[kDim];
#pragma unroll
    for (int p = 0; p < kDim; ++p) v[p] = pts[i * kDim + p];
    uint64_t lo, hi;
    const bool ok = wide_rank_point(v, M, lo, hi);
    if (!ok) {
      lo = ~0ull;
      hi = ~0ull;
      if (err) atomicAdd(err, 1);
    }
    if (WIDE) {
      out[2 * i] = lo;
      out[2 * i + 1] = hi;
    } else {
      out[i] = lo;
    }
  }
}
