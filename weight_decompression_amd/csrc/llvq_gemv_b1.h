// Fused LLVQ dequant-GEMV for one activation row (batch 1), gfx950.
// Included once by llvq.hip (uses its KDesc, read_field and table namespaces).
//
// Work split: a workgroup of kB1Threads lanes owns tiles of R consecutive rows
// (T = R * Kb <= kB1TileMax blocks).  For each tile:
//   1. classify: every block's field is read, its class found (bucket table + short
//      scan) and its flat tile index appended to one of two LDS queues: odd-coset
//      classes at the front, even-coset classes at the back.  Invalid indices
//      (>= the shell-union size) contribute 0 and are counted.
//   2. decode + dot, one lane per block, queues processed in 64-block wave chunks so
//      that a wave is (almost always) single-parity:
//      - odd path: the 24 absolute values are unranked in position order with a
//        compile-time number of values left; the sign of each value follows from the
//        codeword bit and the value mod 4, folded into one byte-table lookup (v_perm);
//      - even path: support values then complement values in decode order, placed on
//        the codeword's (resp. complement's) positions through a per-lane LDS scratch
//        row; sign bits of s are consumed in decode order on nonzero positions, the
//        last support position taking the parity-fixing sign.
//      Each block's scaled dot product goes to an LDS partial slot.
//   3. row sums of the partial slots in a fixed order (deterministic), stored to y.
//
// Rank unranking (both paths): exact arithmetic decoding in fp64.  With y = u * n the
// value slot is the number of cumulative counts C_j <= floor(y) (SWAR compare of the
// three thresholds packed in one dword) and y <- (y - C_k) * (n' / c_k), n' the values
// left after the step, n'/c from an LDS table.  The decision margins (>= n/(2Q),
// Q <= 4.2e8 arrangements) exceed the accumulated rounding error by a factor > 1e5.
// The last 6 values come from a table of all 4^6 slot sequences grouped by composition
// in lexicographic order: with counts c (sum 6) and y in [0, 6), the rank inside the
// group is floor(y * Q(c) / 6).

#pragma once

constexpr int kB1Threads = 512;
constexpr int kB1Waves = kB1Threads / 64;
constexpr int kB1TileMax = 2048;
constexpr int kB1Bias = 12;         // value tables store 12 +- v (|v| <= 12)
constexpr int kTail = 6;            // values resolved by the tail table
constexpr int kSteps = 24 - kTail;  // values resolved step by step
constexpr int kFStride = 25;        // F[n][c] row length (c = 0..24)

struct B1Layout {
  // byte offsets inside the dynamic LDS segment
  uint32_t ftab;     // double F[25][25]: F[n][c] = n / c   (must stay at offset 0)
  uint32_t cls;      // LlvqClassHot[ncls]
  uint32_t gains;    // float[2^gain_bits]
  uint32_t bucket;   // uint8[nbuckets]
  uint32_t tail;     // uint16[4096]
  uint32_t tcomp;    // LlvqTailComp[343]
  uint32_t xs;       // x, kb*24 elements (fp32 or bf16), zero padded
  uint32_t xsum;     // float[kb]: sum of the 24 x values of each block column
  uint32_t queue;    // uint64[T]: I | f << 44 | class << 56
  uint32_t part;     // float[T]: block scale, then the block's scaled dot product
  uint32_t ctr;      // int[4]
  uint32_t total;
};

__host__ __device__ inline uint32_t align16(uint32_t v) { return (v + 15u) & ~15u; }

__host__ __device__ inline B1Layout b1_layout(int ncls, int ngains, int nbuckets, int kb, int tmax, bool xf32) {
  B1Layout L;
  uint32_t o = 0;
  L.ftab = o;    o = align16(o + 25u * kFStride * 8u);
  L.cls = o;     o = align16(o + (uint32_t)ncls * (uint32_t)sizeof(LlvqClassHot));
  L.gains = o;   o = align16(o + (uint32_t)ngains * 4u);
  L.bucket = o;  o = align16(o + (uint32_t)nbuckets);
  L.tail = o;    o = align16(o + 4096u * 2u);
  L.tcomp = o;   o = align16(o + 343u * (uint32_t)sizeof(LlvqTailComp));
  L.xs = o;      o = align16(o + (uint32_t)kb * 24u * (xf32 ? 4u : 2u));
  L.xsum = o;    o = align16(o + (uint32_t)kb * 4u);
  L.queue = o;   o = align16(o + (uint32_t)tmax * 8u);
  L.part = o;    o = align16(o + (uint32_t)tmax * 4u);
  L.ctr = o;     o = align16(o + 16u);
  L.total = o;
  return L;
}

struct B1Args {
  int rows_per_tile;
  int tile_blocks_max;
  int nbuckets;
  B1Layout L;
};

// Full-rate 24-bit multiply-add and bit count with accumulator (the compiler otherwise
// picks a quarter-rate 64-bit multiply-add, and does not fold the addend into v_bcnt).
__device__ __forceinline__ uint32_t mad_u24(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t d;
  asm("v_mad_u32_u24 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(b), "v"(c));
  return d;
}

__device__ __forceinline__ uint32_t bcnt_add(uint32_t a, uint32_t c) {
  uint32_t d;
  asm("v_bcnt_u32_b32 %0, %1, %2" : "=v"(d) : "v"(a), "s"(c));
  return d;
}

// Field j of the packed stream as (lo, hi) words, fields of f <= 64 bits.  48-bit fields
// (the 2-bit format) start at byte 6j: two dword loads and a funnel shift.
__device__ __forceinline__ void field_words(const uint8_t* __restrict__ packed, uint32_t j, int f,
                                            uint32_t& lo, uint32_t& hi) {
  if (f == 48) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(packed) + ((3u * j) >> 1);
    const uint32_t w0 = w[0], w1 = w[1];
    const uint32_t sh = (j & 1u) << 4;
    lo = __builtin_amdgcn_alignbit(w1, w0, sh);
    hi = (w1 >> sh) & 0xffffu;
  } else {
    const uint64_t v = read_field(packed, j, f);
    lo = (uint32_t)v;
    hi = (uint32_t)(v >> 32);
  }
}

__device__ __forceinline__ uint32_t lshl_add(uint32_t a, uint32_t s, uint32_t b) {
  uint32_t d;
  asm("v_lshl_add_u32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "i"(s), "v"(b));
  return d;
}

// SWAR value-slot choice: number of thresholds C_j <= f (j = 1..3), as 0/1 bytes.
__device__ __forceinline__ uint32_t swar_ge(uint32_t f, uint32_t nc) {
  const uint32_t t = mad_u24(f, 0x010101u, nc);
  return (t >> 7) & 0x010101u;
}

template <bool XF32>
__device__ __forceinline__ void load_x24(const uint8_t* smem, const B1Layout& L, uint32_t blk, float xv[24]) {
  if (XF32) {
    const float4* p = reinterpret_cast<const float4*>(smem + L.xs + blk * 96u);
#pragma unroll
    for (int q = 0; q < 6; ++q) {
      const float4 v = p[q];
      xv[4 * q] = v.x; xv[4 * q + 1] = v.y; xv[4 * q + 2] = v.z; xv[4 * q + 3] = v.w;
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(smem + L.xs + blk * 48u);
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

// Common per-block setup from the class record: J / A split, codeword, initial y.
struct BlockStart {
  uint32_t c;   // codeword
  uint32_t s;   // sign bits
  double y;     // y_0 = (R + 1/2) * n0 / P
};

__device__ __forceinline__ BlockStart block_start(double Id, const LlvqClassHot& h) {
  BlockStart bs;
  const double Jd = Id - h.start;
  const uint32_t q = (uint32_t)__builtin_fma(Jd, h.inv_a, 0x1p-13);    // floor(J / A), exact
  const uint32_t r = (uint32_t)__builtin_fma(-(double)q, h.a, Jd);      // J - q A, exact
  const uint32_t B = h.meta & 31u;
  bs.s = q & ((1u << B) - 1u);
  const uint32_t R = q >> B;
  bs.c = dev_tables::kGolayTable[h.toff + r];
  bs.y = __builtin_fma((double)R, h.y0s, 0.5 * h.y0s);
  return bs;
}

// Slot codes of the last 6 values (2 bits each, first of the six in the low bits), from
// the counts left (sum 6) and y in [0, 6).
__device__ __forceinline__ uint32_t tail_codes(const uint8_t* smem, const B1Layout& L, uint32_t cnt, double y) {
  const uint32_t ci = __builtin_amdgcn_udot4(cnt, 0x00310701u, 0u, false);   // c0 + 7 c1 + 49 c2
  const LlvqTailComp tc = reinterpret_cast<const LlvqTailComp*>(smem + L.tcomp)[ci];
  const uint32_t r = (uint32_t)((float)y * tc.q_over_6);
  return reinterpret_cast<const uint16_t*>(smem + L.tail)[tc.offset + r];
}

// bf16/fp32 activation at column col (LDS)
template <bool XF32>
__device__ __forceinline__ float x_at(const uint8_t* smem, const B1Layout& L, uint32_t col) {
  if (XF32) return reinterpret_cast<const float*>(smem + L.xs)[col];
  return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(smem + L.xs)[col] << 16);
}

// Odd coset: returns sum_p (12 + v_p) * x_p.
template <bool XF32>
__device__ __forceinline__ float dot_odd(const uint8_t* smem, const B1Layout& L, const LlvqClassHot& h,
                                         const BlockStart& bs, uint32_t blk) {
  const double* F = reinterpret_cast<const double*>(smem + L.ftab);
  float xv[24];
  load_x24<XF32>(smem, L, blk, xv);
  double y = bs.y;
  uint32_t nc = h.nc0, cnt = h.cnt0;
  const uint32_t notc = ~bs.c;
  float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
  for (int p = 0; p < kSteps; ++p) {
    const uint32_t f = (uint32_t)y;
    const uint32_t g = swar_ge(f, nc);
    const uint32_t kb = bcnt_add(g, 0x0c0c0c00u);
    const uint32_t ck = __builtin_amdgcn_perm(0u, cnt, kb);
    const uint32_t Ck = __builtin_amdgcn_udot4(g, cnt, 0u, false);
    const double fac = F[(23 - p) * kFStride + ck];
    y = (y - (double)Ck) * fac;
    cnt -= ((g << 8) | 1u) - g;
    nc += g ^ 0x010101u;
    const uint32_t sel = lshl_add(__builtin_amdgcn_ubfe(notc, p, 1), 2, kb);
    const uint32_t bv = __builtin_amdgcn_perm(h.sv0hi, h.sv0lo, sel);
    if (p & 1)
      acc1 = __builtin_fmaf((float)(bv & 0xffu), xv[p], acc1);
    else
      acc0 = __builtin_fmaf((float)(bv & 0xffu), xv[p], acc0);
  }
  const uint32_t codes = tail_codes(smem, L, cnt, y);
#pragma unroll
  for (int p = kSteps; p < 24; ++p) {
    const uint32_t k = __builtin_amdgcn_ubfe(codes, 2 * (p - kSteps), 2) | 0x0c0c0c00u;
    const uint32_t sel = lshl_add(__builtin_amdgcn_ubfe(notc, p, 1), 2, k);
    const uint32_t bv = __builtin_amdgcn_perm(h.sv0hi, h.sv0lo, sel);
    if (p & 1)
      acc1 = __builtin_fmaf((float)(bv & 0xffu), xv[p], acc1);
    else
      acc0 = __builtin_fmaf((float)(bv & 0xffu), xv[p], acc0);
  }
  return acc0 + acc1;
}

// Even coset: returns sum_p (12 + v_p) * x_p, values visited in decode order and their
// activations gathered from LDS by position.
template <bool XF32>
__device__ __forceinline__ float dot_even(const uint8_t* smem, const B1Layout& L, const LlvqClassHot& h,
                                          const BlockStart& bs, uint32_t blk) {
  const uint32_t w = (h.meta >> 8) & 31u;
  const uint32_t pi = (h.meta >> 16) & 1u;
  const bool two = w != 0u && w != 24u;
  const uint32_t n0 = w ? w : 24u;
  // last support step takes the sign fixing the parity of negatives on the support;
  // the support's other w-1 signs are bits 0..w-2 of s (all support values are nonzero)
  const uint32_t negq = w ? (((uint32_t)__builtin_popcount(bs.s & ((1u << (w - 1u)) - 1u)) & 1u) ^ pi) : 0u;
  double y = bs.y;
  uint32_t nc = h.nc0, cnt = h.cnt0, svlo = h.sv0lo, svhi = h.sv0hi;
  uint32_t nz = (h.meta >> 20) & 15u;
  uint32_t m = w ? bs.c : 0xffffffu;
  uint32_t s = bs.s;
  uint32_t nb = (n0 - 1u) * (kFStride * 8u);   // byte offset of F[n'][0], n' = values left after the step
  const uint32_t col0 = blk * 24u;
  uint32_t codes = 0;
  float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 24; ++i) {
    if (i == 8 || i == 12 || i == 16) {
      const bool sw = two && (w == (uint32_t)i);
      nc = sw ? h.nc1 : nc;
      cnt = sw ? h.cnt1 : cnt;
      svlo = sw ? h.sv1lo : svlo;
      svhi = sw ? h.sv1hi : svhi;
      nz = sw ? ((h.meta >> 24) & 15u) : nz;
      m = sw ? (~bs.c & 0xffffffu) : m;
    }
    uint32_t kb;
    if (i < kSteps) {
      const uint32_t f = (uint32_t)y;
      const uint32_t g = swar_ge(f, nc);
      kb = bcnt_add(g, 0x0c0c0c00u);
      const uint32_t ck = __builtin_amdgcn_perm(0u, cnt, kb);
      const uint32_t Ck = __builtin_amdgcn_udot4(g, cnt, 0u, false);
      const double fac = *reinterpret_cast<const double*>(smem + L.ftab + nb + (ck << 3));
      y = (y - (double)Ck) * fac;
      cnt -= ((g << 8) | 1u) - g;
      nc += g ^ 0x010101u;
      // the last support step (i = w - 1) hands over to the complement: n' = 24 - w
      if (i == 6 || i == 10 || i == 14)
        nb = (two && w == (uint32_t)(i + 2)) ? (24u - w) * (kFStride * 8u) : nb - kFStride * 8u;
      else
        nb -= kFStride * 8u;
      if (i == kSteps - 1) codes = tail_codes(smem, L, cnt, y);
    } else {
      kb = ((codes >> (2 * (i - kSteps))) & 3u) | 0x0c0c0c00u;
    }
    // sign: nonzero positions consume bits of s in decode order; the last support
    // step takes the parity-fixing sign and consumes no bit
    uint32_t free_ = (nz >> (kb & 31u)) & 1u;
    uint32_t neg = s & free_;
    if (i == 7 || i == 11 || i == 15 || i == 23) {
      const bool isq = w == (uint32_t)(i + 1);
      neg = isq ? negq : neg;
      free_ = isq ? 0u : free_;
    }
    s >>= free_;
    const uint32_t bv = __builtin_amdgcn_perm(svhi, svlo, kb + (neg << 2));
    const uint32_t pos = (uint32_t)__builtin_ctz(m);
    m &= m - 1u;
    const float xp = x_at<XF32>(smem, L, col0 + pos);
    if (i & 1)
      acc1 = __builtin_fmaf((float)(bv & 0xffu), xp, acc1);
    else
      acc0 = __builtin_fmaf((float)(bv & 0xffu), xp, acc0);
  }
  return acc0 + acc1;
}

// LDS copy of n 32-bit words with 16-byte vector moves (n a multiple of 4 where the
// source and destination are 16-byte aligned; the tail is copied word by word).
__device__ __forceinline__ void lds_copy_words(uint32_t* dst, const uint32_t* src, int n, int tid) {
  const int n4 = n >> 2;
  const uint4* s4 = reinterpret_cast<const uint4*>(src);
  uint4* d4 = reinterpret_cast<uint4*>(dst);
  for (int i = tid; i < n4; i += kB1Threads) d4[i] = s4[i];
  for (int i = (n4 << 2) + tid; i < n; i += kB1Threads) dst[i] = src[i];
}

template <bool XF32>
__global__ __launch_bounds__(kB1Threads) void k_gemv_b1(KDesc d, B1Args a, const uint8_t* __restrict__ packed,
                                                         const __half* __restrict__ scales, const void* __restrict__ xv,
                                                         float* __restrict__ y, int32_t* err) {
  extern __shared__ __align__(16) uint8_t smem[];
  const B1Layout& L = a.L;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int kb = d.kb;
  const int ncls = d.ncls;
  const bool sg = d.mode == LLVQ_MODE_SHAPEGAIN;

  // ---- prologue: tables and activations into LDS
  {
    double* F = reinterpret_cast<double*>(smem + L.ftab);
    for (int i = tid; i < 25 * kFStride; i += kB1Threads) {
      const int n = i / kFStride, c = i - n * kFStride;
      F[i] = c >= 1 ? (double)n / (double)c : 0.0;
    }
    lds_copy_words(reinterpret_cast<uint32_t*>(smem + L.cls), reinterpret_cast<const uint32_t*>(dev_tables::kClassHot),
                   ncls * (int)(sizeof(LlvqClassHot) / 4), tid);
    lds_copy_words(reinterpret_cast<uint32_t*>(smem + L.tail), reinterpret_cast<const uint32_t*>(dev_tables::kTail6),
                   2048, tid);
    lds_copy_words(reinterpret_cast<uint32_t*>(smem + L.tcomp),
                   reinterpret_cast<const uint32_t*>(dev_tables::kTailComp), 343 * 2, tid);
    lds_copy_words(reinterpret_cast<uint32_t*>(smem + L.bucket),
                   reinterpret_cast<const uint32_t*>(dev_tables::kBucketTable[d.max_shell]), (a.nbuckets + 3) >> 2, tid);
    float* G = reinterpret_cast<float*>(smem + L.gains);
    if (sg)
      for (int i = tid; i < (1 << d.gain_bits); i += kB1Threads) G[i] = __half2float(scales[i]);
    const int ncol = kb * 24;
    if (XF32) {
      float* xs = reinterpret_cast<float*>(smem + L.xs);
      const float* xg = reinterpret_cast<const float*>(xv);
      for (int i = tid; i < ncol; i += kB1Threads) xs[i] = i < d.cols ? xg[i] : 0.0f;
    } else {
      // pairs of bf16 as dwords when the row is dword aligned
      uint16_t* xs = reinterpret_cast<uint16_t*>(smem + L.xs);
      const uint16_t* xg = reinterpret_cast<const uint16_t*>(xv);
      if ((((uintptr_t)xg) & 3u) == 0u) {
        const int full = d.cols >> 1;
        const uint32_t* xg2 = reinterpret_cast<const uint32_t*>(xg);
        uint32_t* xs2 = reinterpret_cast<uint32_t*>(xs);
        for (int i = tid; i < ncol / 2; i += kB1Threads)
          xs2[i] = i < full ? xg2[i] : ((i == full && (d.cols & 1)) ? (uint32_t)xg[d.cols - 1] : 0u);
      } else {
        for (int i = tid; i < ncol; i += kB1Threads) xs[i] = i < d.cols ? xg[i] : (uint16_t)0;
      }
    }
  }
  __syncthreads();
  {
    float* xsum = reinterpret_cast<float*>(smem + L.xsum);
    for (int b = tid; b < kb; b += kB1Threads) {
      float xx[24];
      load_x24<XF32>(smem, L, (uint32_t)b, xx);
      float s0 = 0.0f;
#pragma unroll
      for (int p = 0; p < 24; ++p) s0 += xx[p];
      xsum[b] = s0;
    }
  }
  const LlvqClassHot* cls = reinterpret_cast<const LlvqClassHot*>(smem + L.cls);
  const float* G = reinterpret_cast<const float*>(smem + L.gains);
  const float* xsum = reinterpret_cast<const float*>(smem + L.xsum);
  const uint8_t* bk = smem + L.bucket;
  uint64_t* queue = reinterpret_cast<uint64_t*>(smem + L.queue);
  float* part = reinterpret_cast<float*>(smem + L.part);
  int* ctr = reinterpret_cast<int*>(smem + L.ctr);
  const float inv_kb = 1.0f / (float)kb;
  const int ntiles = (d.rows + a.rows_per_tile - 1) / a.rows_per_tile;
  constexpr int kCl = (kB1TileMax + kB1Threads - 1) / kB1Threads;   // classify blocks per thread

  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int row0 = tile * a.rows_per_tile;
    const int nrows = min(a.rows_per_tile, d.rows - row0);
    const int T = nrows * kb;
    if (tid == 0) { ctr[0] = 0; ctr[1] = 0; ctr[2] = 0; }
    __syncthreads();

    // ---- 1. classify: all field loads first, then the class search and queueing
    uint32_t flo[kCl], fhi[kCl];
#pragma unroll
    for (int t = 0; t < kCl; ++t) {
      const int f = t * kB1Threads + tid;
      flo[t] = 0u;
      fhi[t] = 0u;
      if (f < T) field_words(packed, (uint32_t)(row0 * kb + f), d.field_bits, flo[t], fhi[t]);
    }
#pragma unroll
    for (int t = 0; t < kCl; ++t) {
      const int f = t * kB1Threads + tid;
      if (t * kB1Threads >= T) break;
      bool valid = false, odd = false;
      uint64_t entry = 0;
      if (f < T) {
        const uint32_t ilo = flo[t] & d.shape_mask_lo;
        const uint32_t ihi = fhi[t] & d.shape_mask_hi;
        const uint64_t I = ((uint64_t)ihi << 32) | ilo;
        if (I < d.index_count) {
          valid = true;
          const double Id = __builtin_fma((double)ihi, 4294967296.0, (double)ilo);
          const uint32_t bidx = d.bshift >= 32 ? (ihi >> (d.bshift - 32)) : __builtin_amdgcn_alignbit(ihi, ilo, d.bshift);
          uint32_t k = bk[bidx];
          while ((int)k + 1 < ncls && Id >= cls[k + 1].start) ++k;
          const LlvqClassHot& h = cls[k];
          odd = ((h.meta >> 17) & 1u) != 0u;
          entry = I | ((uint64_t)f << 44) | ((uint64_t)k << 56);
          const uint32_t gsh = d.shape_bits >= 32 ? (fhi[t] >> (d.shape_bits - 32))
                                                  : __builtin_amdgcn_alignbit(fhi[t], flo[t], d.shape_bits);
          const uint32_t g = gsh & ((1u << d.gain_bits) - 1u);
          part[f] = sg ? G[g] * h.invnorm : 1.0f;
        } else {
          part[f] = 0.0f;
          if (err) atomicAdd(err, 1);
        }
      }
      const uint64_t bo = __ballot(valid && odd);
      const uint64_t be = __ballot(valid && !odd);
      int baseo = 0, basee = 0;
      if (lane == 0) {
        baseo = atomicAdd(&ctr[0], __popcll(bo));
        basee = atomicAdd(&ctr[1], __popcll(be));
      }
      baseo = __shfl(baseo, 0, 64);
      basee = __shfl(basee, 0, 64);
      const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      if (valid && odd) queue[baseo + __popcll(bo & below)] = entry;
      if (valid && !odd) queue[T - 1 - (basee + __popcll(be & below))] = entry;
    }
    __syncthreads();
    const int nodd = ctr[0];
    const int neven = ctr[1];
    const int nco = (nodd + 63) >> 6;
    const int nchunks = nco + ((neven + 63) >> 6);

    // ---- 2. decode + dot: 64-block chunks handed out dynamically (odd chunks first)
    for (;;) {
      int c = 0;
      if (lane == 0) c = atomicAdd(&ctr[2], 1);
      c = __shfl(c, 0, 64);
      if (c >= nchunks) break;
      const bool odd = c < nco;
      const int e = odd ? (c << 6) + lane : ((c - nco) << 6) + lane;
      if (e >= (odd ? nodd : neven)) continue;
      const uint64_t entry = queue[odd ? e : T - 1 - e];
      const uint32_t f = (uint32_t)(entry >> 44) & 0xfffu;
      const uint32_t k = (uint32_t)(entry >> 56);
      const uint32_t rl = (uint32_t)(((float)f + 0.5f) * inv_kb);
      const uint32_t b = f - rl * (uint32_t)kb;
      const LlvqClassHot h = cls[k];
      const BlockStart bs = block_start((double)(entry & 0xfffffffffffull), h);
      const float raw = odd ? dot_odd<XF32>(smem, L, h, bs, b) : dot_even<XF32>(smem, L, h, bs, b);
      part[f] *= __builtin_fmaf(-(float)kB1Bias, xsum[b], raw);
    }
    __syncthreads();

    // ---- 3. row sums (fixed order)
    for (int rl = tid >> 6; rl < nrows; rl += kB1Waves) {
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
