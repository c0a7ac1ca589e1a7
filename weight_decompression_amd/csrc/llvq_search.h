// Nearest-point search over the shell union 2..M (gfx950).  Included once by llvq.hip.
//
// The quantiser step before the decode path: for each 24-vector x find the point v of
// shells 2..M of the Leech lattice that maximises <x, v> / |v| (angular, shape-gain) or
// minimises |x - v|^2 (Euclidean, x in the lattice's integer units) (papernotes.org notes,
// 关键设计 1: search extended from one shell to the union of shells with an angular or a
// Euclidean objective; gist.science page, Methodik / 2. Multi-Shell Search).
//
// Exhaustive over every class of shells 2..M and every Golay codeword the class can use.
// Inside one (class, codeword) pair the best point is fixed by the rearrangement
// inequality, so the objective is a short fixed expression in prefix sums of sorted
// coordinates (both objectives are <x, v> up to a per-class constant, since |v| is
// constant on a class):
//   odd coset, codeword c:  y_i = x_i (i in c) or -x_i; the class's values b (b = a if
//     a = 1 mod 4, else -a) paired in ascending order with ascending y;
//   even coset, weight-w codeword c: ascending |x| on the support paired with the
//     ascending support values, likewise on the complement, signs following x; when the
//     support's count of negative x has the wrong parity the support entry with the
//     smallest |x| flips, costing 2 min|x| times the smallest support value.
// The sorting network and the per-class expressions are generated at build time
// (llvq_search.inc, from the class table).
//
// One 256-lane workgroup per vector.  The all-ones word is a codeword, so codewords come
// in complement pairs (c, ~c) and one sort serves both: in the odd coset y(~c) = -y(c),
// in the even coset the support of ~c is the complement of c.  Lane l takes the even
// coset's pairs l + 256 j (weight-8 words with their weight-16 complements, weight-12
// words with bit 23 clear, and the pair of weights 0 and 24), then the odd coset's pairs
// (representatives with bit 23 clear), scoring every class the pair's weights admit.
// The workgroup keeps the largest objective; exact float ties go to the smaller candidate
// number (the codeword mask, plus 2^24 in the odd coset) across lanes and to the earlier
// candidate within a lane.  Wavefront 0 then
// rebuilds the winner: the argmax class for that codeword, the coordinates by ranking
// (ties by position, as a stable sort), and writes the int8 point.  Under the angular
// objective a winner 2u in shell 8 or 12 with u a lattice point is replaced by u: the two
// tie exactly and u (shell 2 or 3) has the smaller index; within shells 2..13 these are
// the only collinear pairs (k v lies in shell k^2 m).  A vector with a non-finite
// coordinate gets the zero vector, which the rank step rejects.

#pragma once

constexpr int kSearchThreads = 256;
constexpr int kSearchNone = 0x7fffffff;

// objective maximum over the classes of one even-coset weight (classes of shells <= M)
template <bool EUCLID, int W>
__device__ __forceinline__ float search_even_max(const float (&Ss)[W + 1], const float (&Sc)[25 - W], float pen0,
                                                 float pen1, int M) {
  using namespace dev_tables;
  if constexpr (W == 0) return EUCLID ? llvq_even0_max_euclid(Ss, Sc, pen0, pen1, M) : llvq_even0_max_angular(Ss, Sc, pen0, pen1, M);
  if constexpr (W == 8) return EUCLID ? llvq_even8_max_euclid(Ss, Sc, pen0, pen1, M) : llvq_even8_max_angular(Ss, Sc, pen0, pen1, M);
  if constexpr (W == 12) return EUCLID ? llvq_even12_max_euclid(Ss, Sc, pen0, pen1, M) : llvq_even12_max_angular(Ss, Sc, pen0, pen1, M);
  if constexpr (W == 16) return EUCLID ? llvq_even16_max_euclid(Ss, Sc, pen0, pen1, M) : llvq_even16_max_angular(Ss, Sc, pen0, pen1, M);
  if constexpr (W == 24) return EUCLID ? llvq_even24_max_euclid(Ss, Sc, pen0, pen1, M) : llvq_even24_max_angular(Ss, Sc, pen0, pen1, M);
  return -__builtin_inff();
}

template <bool EUCLID, int W>
__device__ __forceinline__ int search_even_argmax(const float (&Ss)[W + 1], const float (&Sc)[25 - W], float pen0,
                                                  float pen1, int M, float* best) {
  using namespace dev_tables;
  if constexpr (W == 0) return EUCLID ? llvq_even0_argmax_euclid(Ss, Sc, pen0, pen1, M, best) : llvq_even0_argmax_angular(Ss, Sc, pen0, pen1, M, best);
  if constexpr (W == 8) return EUCLID ? llvq_even8_argmax_euclid(Ss, Sc, pen0, pen1, M, best) : llvq_even8_argmax_angular(Ss, Sc, pen0, pen1, M, best);
  if constexpr (W == 12) return EUCLID ? llvq_even12_argmax_euclid(Ss, Sc, pen0, pen1, M, best) : llvq_even12_argmax_angular(Ss, Sc, pen0, pen1, M, best);
  if constexpr (W == 16) return EUCLID ? llvq_even16_argmax_euclid(Ss, Sc, pen0, pen1, M, best) : llvq_even16_argmax_angular(Ss, Sc, pen0, pen1, M, best);
  if constexpr (W == 24) return EUCLID ? llvq_even24_argmax_euclid(Ss, Sc, pen0, pen1, M, best) : llvq_even24_argmax_angular(Ss, Sc, pen0, pen1, M, best);
  return -1;
}

// Prefix sums of one even-coset codeword: keys = |x| bits with bit 31 set off the support,
// sorted as unsigned integers, give the ascending support values then the ascending
// complement values.  pen_pi = -2 min|x| on the support when the support's negative count
// has parity != pi, else 0.
template <int W>
__device__ __forceinline__ void even_sums(const uint32_t (&ab)[24], uint32_t xneg, uint32_t c, float (&Ss)[W + 1],
                                          float (&Sc)[25 - W], float* pen0, float* pen1) {
  uint32_t k[24];
#pragma unroll
  for (int i = 0; i < 24; ++i) k[i] = ab[i] | ((~c << (31 - i)) & 0x80000000u);
  dev_tables::llvq_sort24(k);
  Ss[0] = 0.0f;
#pragma unroll
  for (int t = 0; t < W; ++t) Ss[t + 1] = Ss[t] + __uint_as_float(k[t]);
  Sc[0] = 0.0f;
#pragma unroll
  for (int t = 0; t < 24 - W; ++t) Sc[t + 1] = Sc[t] + __uint_as_float(k[W + t] & 0x7fffffffu);
  const bool odd_neg = (__builtin_popcount(c & xneg) & 1) != 0;
  const float m2 = W ? -2.0f * __uint_as_float(k[0]) : 0.0f;
  *pen0 = odd_neg ? m2 : 0.0f;
  *pen1 = odd_neg ? 0.0f : m2;
}

// prefix sums of the ascending y of one odd-coset codeword
__device__ __forceinline__ void odd_sums(const float (&xv)[24], uint32_t c, float (&S)[25]) {
  float y[24];
#pragma unroll
  for (int i = 0; i < 24; ++i) y[i] = __uint_as_float(__float_as_uint(xv[i]) ^ ((~c << (31 - i)) & 0x80000000u));
  dev_tables::llvq_sort24(y);
  S[0] = 0.0f;
#pragma unroll
  for (int t = 0; t < 24; ++t) S[t + 1] = S[t] + y[t];
}

// An even-coset complement pair: representative c of weight W and ~c of weight 24 - W
// share one sort (the support of ~c is the complement of c).  Candidates are numbered by
// their codeword mask (even coset: bit 24 clear).
template <bool EUCLID, int W>
__device__ __forceinline__ void search_even_pair(const uint32_t (&ab)[24], uint32_t xneg, uint32_t c, int M,
                                                 float* best, int* cand) {
  float Ss[W + 1], Sc[25 - W], pen0, pen1;
  even_sums<W>(ab, xneg, c, Ss, Sc, &pen0, &pen1);
  const float o = search_even_max<EUCLID, W>(Ss, Sc, pen0, pen1, M);
  if (o > *best) {
    *best = o;
    *cand = (int)c;
  }
  // ~c: negative count on its support = all negatives minus those on c's support; its
  // smallest support |x| is c's smallest complement |x| = Sc[1]
  const uint32_t cc = ~c & 0xffffffu;
  const bool odd_neg = (__builtin_popcount(cc & xneg) & 1) != 0;
  const float m2 = W < 24 ? -2.0f * Sc[1] : 0.0f;
  const float o2 = search_even_max<EUCLID, 24 - W>(Sc, Ss, odd_neg ? m2 : 0.0f, odd_neg ? 0.0f : m2, M);
  if (o2 > *best) {
    *best = o2;
    *cand = (int)cc;
  }
}

// Winner of an even-coset codeword: class, then lane i < 24 returns coordinate i.
template <bool EUCLID, int W>
__device__ __forceinline__ int even_point(const float (&xv)[24], const uint32_t (&ab)[24], uint32_t xneg, uint32_t c,
                                          int M, int lane) {
  float Ss[W + 1], Sc[25 - W], pen0, pen1, best;
  even_sums<W>(ab, xneg, c, Ss, Sc, &pen0, &pen1);
  const int k = search_even_argmax<EUCLID, W>(Ss, Sc, pen0, pen1, M, &best);
  if (k < 0) return 0;
  const dev_tables::LlvqSearchClass& sc = dev_tables::kSearchClass[k];
  int v = 0;
  bool on = false;
  int rank = 0;
  if (lane < 24) {
    on = (c >> lane) & 1u;
    uint32_t me = 0u;
#pragma unroll
    for (int j = 0; j < 24; ++j) me = j == lane ? ab[j] : me;
#pragma unroll
    for (int j = 0; j < 24; ++j) {
      const bool same_side = (((c >> j) & 1u) != 0u) == on;
      rank += (same_side && (ab[j] < me || (ab[j] == me && j < lane))) ? 1 : 0;
    }
    const int a = sc.vals[on ? rank : W + rank];
    v = ((xneg >> lane) & 1u) ? -a : a;
  }
  // parity of the support's negative entries; the wrong parity flips the smallest |x|
  const uint64_t negm = __ballot(lane < 24 && on && v < 0);
  if (W > 0 && (int)(__popcll(negm) & 1) != (int)sc.pi && lane < 24 && on && rank == 0) v = -v;
  return v;
}

// Vectors: block b of row r of a [rows][cols] fp32 matrix with kb = ceil(cols / 24)
// blocks per row (zero past the last column), vector index r kb + b; a plain [n][24]
// array is cols = 24, kb = 1.  With rscale, row r is divided by its fp16 scale first
// (the Euclidean quantiser takes the lattice's integer units).
template <bool EUCLID>
__global__ __launch_bounds__(kSearchThreads) void k_search(const float* __restrict__ x, int64_t n, int M, int cols,
                                                           int kb, const __half* __restrict__ rscale,
                                                           int8_t* __restrict__ pts) {
  __shared__ float rv[kSearchThreads / 64];
  __shared__ int rc[kSearchThreads / 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int64_t blk = blockIdx.x; blk < n; blk += gridDim.x) {
    float xv[24];
    uint32_t ab[24];
    uint32_t xneg = 0u;
    bool finite = true;
    const int64_t row = blk / kb;
    const int c0 = (int)(blk - row * kb) * 24;
    const float* xr = x + row * (int64_t)cols;
    const float rs = rscale ? __half2float(rscale[row]) : 1.0f;
#pragma unroll
    for (int i = 0; i < 24; ++i) {
      xv[i] = c0 + i < cols ? xr[c0 + i] : 0.0f;
      if (rscale) xv[i] = xv[i] / rs;
      ab[i] = __float_as_uint(xv[i]) & 0x7fffffffu;
      xneg |= (xv[i] < 0.0f ? 1u : 0u) << i;
      finite = finite && ab[i] < 0x7f800000u;
    }
    float best = -__builtin_inff();
    int cand = kSearchNone;
    if (finite) {
      // ---- even coset: 2048 complement pairs (weights 8 + 16, 12 + 12, 0 + 24)
      for (int j = 0; j < 2048 / kSearchThreads; ++j) {
        const int i = tid + kSearchThreads * j;
        if (i < 759) search_even_pair<EUCLID, 8>(ab, xneg, dev_tables::kGolayTable[1 + i], M, &best, &cand);
        else if (i < 2047) search_even_pair<EUCLID, 12>(ab, xneg, dev_tables::kSearchW12Rep[i - 759], M, &best, &cand);
        else search_even_pair<EUCLID, 0>(ab, xneg, 0u, M, &best, &cand);
      }
      // ---- odd coset: 2048 complement pairs against every odd class; y(~c) = -y(c), so
      // the prefix sums of ~c are S'[k] = S[24 - k] - S[24]
      for (int j = 0; j < 2048 / kSearchThreads; ++j) {
        const uint32_t c = dev_tables::kSearchOddRep[tid + kSearchThreads * j];
        float S[25], S2[25];
        odd_sums(xv, c, S);
#pragma unroll
        for (int k = 0; k <= 24; ++k) S2[k] = S[24 - k] - S[24];
        const float o = EUCLID ? dev_tables::llvq_odd_max_euclid(S, M) : dev_tables::llvq_odd_max_angular(S, M);
        if (o > best) {
          best = o;
          cand = (int)(c | (1u << 24));
        }
        const float o2 = EUCLID ? dev_tables::llvq_odd_max_euclid(S2, M) : dev_tables::llvq_odd_max_angular(S2, M);
        if (o2 > best) {
          best = o2;
          cand = (int)((~c & 0xffffffu) | (1u << 24));
        }
      }
    }
    // ---- largest objective of the workgroup; ties to the smaller candidate number
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ob = __shfl_xor(best, off, 64);
      const int oc = __shfl_xor(cand, off, 64);
      if (ob > best || (ob == best && oc < cand)) {
        best = ob;
        cand = oc;
      }
    }
    if (lane == 0) {
      rv[wave] = best;
      rc[wave] = cand;
    }
    __syncthreads();
    if (wave == 0) {
      float b = rv[0];
      int cd = rc[0];
#pragma unroll
      for (int w = 1; w < kSearchThreads / 64; ++w)
        if (rv[w] > b || (rv[w] == b && rc[w] < cd)) {
          b = rv[w];
          cd = rc[w];
        }
      int v = 0;
      if (cd != kSearchNone && (cd >> 24) != 0) {
        const uint32_t c = (uint32_t)cd & 0xffffffu;
        float S[25], ob;
        odd_sums(xv, c, S);
        const int k = EUCLID ? dev_tables::llvq_odd_argmax_euclid(S, M, &ob) : dev_tables::llvq_odd_argmax_angular(S, M, &ob);
        if (k >= 0 && lane < 24) {
          // rank of y_lane among the 24 y (ties by position)
          float yv[24];
#pragma unroll
          for (int i = 0; i < 24; ++i) yv[i] = __uint_as_float(__float_as_uint(xv[i]) ^ ((~c << (31 - i)) & 0x80000000u));
          float me = 0.0f;
#pragma unroll
          for (int j = 0; j < 24; ++j) me = j == lane ? yv[j] : me;
          int rank = 0;
#pragma unroll
          for (int j = 0; j < 24; ++j) rank += (yv[j] < me || (yv[j] == me && j < lane)) ? 1 : 0;
          const int bv = dev_tables::kSearchClass[k].vals[rank];
          v = ((c >> lane) & 1u) ? bv : -bv;
        }
      } else if (cd != kSearchNone) {
        const uint32_t c = (uint32_t)cd;
        switch (__builtin_popcount(c)) {
          case 0: v = even_point<EUCLID, 0>(xv, ab, xneg, c, M, lane); break;
          case 8: v = even_point<EUCLID, 8>(xv, ab, xneg, c, M, lane); break;
          case 12: v = even_point<EUCLID, 12>(xv, ab, xneg, c, M, lane); break;
          case 16: v = even_point<EUCLID, 16>(xv, ab, xneg, c, M, lane); break;
          default: v = even_point<EUCLID, 24>(xv, ab, xneg, c, M, lane); break;
        }
      }
      if (!EUCLID) {
        // The angular objective ignores |v|: a shell-8 or shell-12 point 2u with u in the
        // lattice ties exactly with u (shell 2 or 3), whose index is smaller, and u is the
        // answer (fp32 rounding need not have seen the tie).
        int n2 = lane < 24 ? v * v : 0;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) n2 += __shfl_xor(n2, off, 64);
        const uint64_t oddc = __ballot(lane < 24 && (v & 1) != 0);
        if ((n2 == 16 * 8 || n2 == 16 * 12) && oddc == 0u) {
          const int u = v / 2;
          const int p = __shfl(u, 0, 64) & 1;
          const uint64_t par = __ballot(lane < 24 && (u & 1) != p);
          int su = lane < 24 ? u : 0;
#pragma unroll
          for (int off = 32; off >= 1; off >>= 1) su += __shfl_xor(su, off, 64);
          const uint32_t mask = (uint32_t)__ballot(lane < 24 && (u & 3) == (p ? 1 : 2)) & 0xffffffu;
          const bool cw = dev_tables::kGolayTable[dev_tables::kGolayInfoPos[(mask >> 11) & 0xfffu]] == mask;
          if (par == 0u && ((su - 4 * p) & 7) == 0 && cw) v = u;
        }
      }
      if (lane < 24) pts[blk * 24 + lane] = (int8_t)v;
    }
    __syncthreads();   // rv / rc are rewritten for the next vector
  }
}

// Packed stream of the quantiser: one thread per 32-bit word of the stream, assembling the
// bits of the (at most three) fields that overlap it, so no word is written twice.  Field j
// = shape index | gain index << shape_bits; an index the rank step rejected (UINT64_MAX)
// is written as the all-ones shape field, which every decoder treats as invalid (it is >=
// the shell union's size).  Shape-gain: the gain index is the nearest entry of the fp16
// gain table to the block's norm (computed in fp64), ties to the lower index.
__device__ __forceinline__ uint64_t quant_field(const KDesc& d, const float* __restrict__ w,
                                                const __half* __restrict__ gains, const uint64_t* __restrict__ idx,
                                                uint64_t j) {
  uint64_t I = idx[j];
  if (I >= d.index_count) I = d.shape_mask;
  uint64_t F = I & d.shape_mask;
  if (d.mode == LLVQ_MODE_SHAPEGAIN) {
    const uint64_t row = j / (uint64_t)d.kb;
    const int c0 = (int)(j - row * (uint64_t)d.kb) * 24;
    const float* xr = w + row * (uint64_t)d.cols;
    double s2 = 0.0;
    for (int i = 0; i < 24 && c0 + i < d.cols; ++i) {
      const double v = (double)xr[c0 + i];
      s2 = __builtin_fma(v, v, s2);
    }
    const double nrm = __builtin_sqrt(s2);
    int g = 0;
    double best = __builtin_fabs((double)__half2float(gains[0]) - nrm);
    for (int t = 1; t < (1 << d.gain_bits); ++t) {
      const double e = __builtin_fabs((double)__half2float(gains[t]) - nrm);
      if (e < best) {
        best = e;
        g = t;
      }
    }
    F |= (uint64_t)g << d.shape_bits;
  }
  return F;
}

// FIELDS: idx holds the finished fields (llvq_pack_fields); otherwise the fields are
// built from the shape indices, the weights and the gain table (llvq_quantize).
template <bool FIELDS>
__global__ __launch_bounds__(256) void k_pack(KDesc d, const float* __restrict__ w, const __half* __restrict__ gains,
                                              const uint64_t* __restrict__ idx, uint32_t* __restrict__ out,
                                              int64_t nwords) {
  const uint64_t nfields = (uint64_t)d.rows * (uint64_t)d.kb;
  const uint64_t f = (uint64_t)d.field_bits;
  for (int64_t wd = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; wd < nwords;
       wd += (int64_t)gridDim.x * blockDim.x) {
    const uint64_t bit0 = (uint64_t)wd * 32u;
    uint32_t word = 0u;
    for (uint64_t j = bit0 / f; j < nfields && j * f < bit0 + 32u; ++j) {
      const uint64_t F = FIELDS ? idx[j] & (f == 64 ? ~0ull : ((1ull << f) - 1ull)) : quant_field(d, w, gains, idx, j);
      const int64_t off = (int64_t)(j * f) - (int64_t)bit0;   // -64 < off < 32
      word |= off >= 0 ? (uint32_t)(F << off) : (uint32_t)(F >> (-off));
    }
    out[wd] = word;
  }
}
