// Fused LLVQ dequant-GEMV for one activation row (batch 1), gfx950.
// Included once by llvq.hip after llvq_engine.h.
//
// The tile engine's decoders turn each block back into its 24 values; this consumer dots
// them with the block's 24 activations straight from registers (odd blocks, position
// order) or from LDS by position (even blocks, decode order), never storing the weights.
// Values leave the decoders as selectors into an 8-entry table of fp8 codes; two positions
// share one v_perm, one fp8 -> bf16 conversion and one v_dot2c_f32_bf16 with the bf16
// activation pair (the products are exact; the sums are fp32).  Block results are scaled in
// their LDS slot and each row is summed in a fixed order, so results do not depend on which
// wave decoded which block.
//
// Streaming classification.  A workgroup (16 waves, one per CU) owns tiles of whole rows.
// Inside a tile the waves take units of 64 consecutive fields from an LDS counter; a wave
// requests the fields of its next unit before it classifies the current one, so the
// packed stream arrives while the workgroup decodes instead of in one burst before it.
// Classification appends each block to one of the wave's two ring queues in LDS (odd or
// even coset, so a wavefront runs one of the two very different decoders without
// divergence), and the wave decodes a full chunk of 64 blocks whenever a ring holds one.
// At the end of the tile the rings' remainders (fewer than 64 per ring) are gathered into
// one shared queue between two barriers and decoded as full chunks by all waves; then the
// rows are summed (a fixed-order DPP reduction per row).  No wave ever waits on another
// except at those barriers.

#pragma once

constexpr int kRing = 128;              // entries per ring (a ring never holds more than 127)
constexpr int kRingBytes = 2 * kEWaves * kRing * 8;   // odd and even ring of every wave

typedef __bf16 llvq_bf16x2 __attribute__((ext_vector_type(2)));
typedef uint16_t llvq_u16x2 __attribute__((ext_vector_type(2)));

// Two decoded values (selectors ka, kb into the fp8 table svhi:svlo, each in byte 0 with
// 0x0c above) as a bf16 pair: one v_perm joins the selectors, one picks both fp8 codes, one
// conversion widens them exactly.
__device__ __forceinline__ llvq_bf16x2 value_pair(uint32_t svhi, uint32_t svlo, uint32_t ka, uint32_t kb) {
  const uint32_t sel = __builtin_amdgcn_perm(kb, ka, 0x0c0c0400u);     // ka.byte0, kb.byte0, 0, 0
  const uint32_t codes = __builtin_amdgcn_perm(svhi, svlo, sel);
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, false);
}

// acc + v.x a.x + v.y a.y for bf16 activations (one v_dot2c_f32_bf16) or fp32 ones
template <bool XF32>
__device__ __forceinline__ float dot_pair(float acc, llvq_bf16x2 v, uint32_t xb, float x0, float x1) {
  if (!XF32) return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(llvq_bf16x2, xb), v, acc, false);
  const uint32_t vb = __builtin_bit_cast(uint32_t, v);
  acc = __builtin_fmaf(__uint_as_float(vb << 16), x0, acc);
  return __builtin_fmaf(__uint_as_float(vb & 0xffff0000u), x1, acc);
}

// Sum of a float over the 64 lanes in a fixed order: each 16-lane row is reduced by four
// DPP rotations (8, 4, 2, 1) inside the row, then the four row totals (lanes 0, 16, 32,
// 48) are added in row order.  Uniform result.
__device__ __forceinline__ float wave_sum_fixed(float v) {
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x128, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x124, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x122, 0xf, 0xf, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x121, 0xf, 0xf, false));
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return ((r0 + r1) + r2) + r3;
}

__device__ __forceinline__ uint32_t block_col(uint32_t f, float inv_kb, uint32_t kb) {
  // (f + 1/2) / Kb in one fma: with f < 2^22 its error stays below the 1/(2 Kb) margin
  const uint32_t rl = (uint32_t)__builtin_fmaf((float)f, inv_kb, 0.5f * inv_kb);
  return f - __umul24(rl, kb);    // both below 2^24: the full-rate 24-bit multiply
}

// Decode one odd-coset block (queue entry e) and multiply its slot by the dot product.
// The block's activations are read as 16-byte words (bf16 pairs, or fp32 values).
template <bool XF32, int TAIL>
__device__ __forceinline__ void gemv_odd(uint8_t* smem, const EArgs& a, float* part, uint64_t e, uint32_t kb,
                                         float inv_kb) {
  const ELayout& L = a.L;
  const LlvqClassHot* cls = reinterpret_cast<const LlvqClassHot*>(smem + L.cls);
  const uint32_t fo = entry_f(e);
  const uint32_t bo = block_col(fo, inv_kb, kb);
  const LlvqClassHot hO = cls[entry_k(e)];
  const BlockStart so = block_start(smem, L, entry_J(e), hO);
  uint32_t xw[12];
  float xf[24];
  if (XF32) {
    const float4* p = reinterpret_cast<const float4*>(smem + a.xs + bo * 96u);
#pragma unroll
    for (int q = 0; q < 6; ++q) {
      const float4 v = p[q];
      xf[4 * q] = v.x; xf[4 * q + 1] = v.y; xf[4 * q + 2] = v.z; xf[4 * q + 3] = v.w;
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(smem + a.xs + bo * 48u);
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const uint4 v = p[q];
      xw[4 * q] = v.x; xw[4 * q + 1] = v.y; xw[4 * q + 2] = v.z; xw[4 * q + 3] = v.w;
    }
  }
  OddDec<TAIL> od;
  od.init(hO, so);
  od.load_fp8(hO);
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int q = 0; q < 6; ++q) {
    const uint32_t k0 = od.slot(smem, L, 4 * q);
    const uint32_t k1 = od.slot(smem, L, 4 * q + 1);
    const uint32_t k2 = od.slot(smem, L, 4 * q + 2);
    const uint32_t k3 = od.slot(smem, L, 4 * q + 3);
    const uint32_t codes = od.quad_codes(k0, k1, k2, k3, q);
    const llvq_bf16x2 v01 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, false);
    const llvq_bf16x2 v23 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, 1.0f, true);
    a0 = dot_pair<XF32>(a0, v01, XF32 ? 0u : xw[2 * q], XF32 ? xf[4 * q] : 0.0f, XF32 ? xf[4 * q + 1] : 0.0f);
    a1 = dot_pair<XF32>(a1, v23, XF32 ? 0u : xw[2 * q + 1], XF32 ? xf[4 * q + 2] : 0.0f,
                        XF32 ? xf[4 * q + 3] : 0.0f);
  }
  part[fo] *= a0 + a1;
}

// The same for an even-coset block; its values come in decode order, so each one's
// activation is read from LDS by position.
template <bool XF32, int TAIL>
__device__ __forceinline__ void gemv_even(uint8_t* smem, const EArgs& a, float* part, uint64_t e, uint32_t kb,
                                          float inv_kb) {
  const ELayout& L = a.L;
  const LlvqClassHot* cls = reinterpret_cast<const LlvqClassHot*>(smem + L.cls);
  const uint32_t fe = entry_f(e);
  const uint32_t be = block_col(fe, inv_kb, kb);
  const LlvqClassHot hE = cls[entry_k(e)];
  const BlockStart se = block_start<false, false>(smem, L, entry_J(e), hE);
  EvenDec<TAIL, 2> ev;
  ev.init(hE, se, L.cls + entry_k(e) * (uint32_t)sizeof(LlvqClassHot));
  ev.load_fp8(hE);
  // the block's activations; a value's position comes as its byte offset 2 p in bf16
  const uint8_t* xrow = smem + a.xs + be * (XF32 ? 96u : 48u);
  float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    uint32_t pa, pb;
    const uint32_t ka = ev.slot(smem, L, 2 * i, pa);
    const uint32_t kb2 = ev.slot(smem, L, 2 * i + 1, pb);
    const llvq_bf16x2 v = value_pair(ev.svhi, ev.svlo, ka, kb2);
    uint32_t xb = 0u;
    float x0 = 0.0f, x1 = 0.0f;
    if (XF32) {
      x0 = *reinterpret_cast<const float*>(xrow + 2u * pa);
      x1 = *reinterpret_cast<const float*>(xrow + 2u * pb);
    } else {
      // the two 16-bit loads joined into one register (one permute)
      llvq_u16x2 h2;
      h2.x = *reinterpret_cast<const uint16_t*>(xrow + pa);
      h2.y = *reinterpret_cast<const uint16_t*>(xrow + pb);
      xb = __builtin_bit_cast(uint32_t, h2);
    }
    if (i & 1)
      a1 = dot_pair<XF32>(a1, v, xb, x0, x1);
    else
      a0 = dot_pair<XF32>(a0, v, xb, x0, x1);
  }
  part[fe] *= a0 + a1;
}

// A wave's two rings: entry i of a ring sits at (head + i) mod kRing.  Heads and counts
// are the same in every lane (they change only by wave-wide ballot counts).
struct Rings {
  uint64_t* odd;
  uint64_t* even;   // always odd + kRing
  uint32_t oh, on, eh, en;
};

// One field per lane (unit u of the tile: f = 64 u + lane), loaded as three words.
struct LaneField {
  uint32_t w0, w1, w2, sh;
};

__device__ __forceinline__ LaneField load_lane_field(const KDesc& d, const uint8_t* __restrict__ packed,
                                                     uint32_t j0, int T, int u, int lane) {
  LaneField lf;
  const int f = min(u * 64 + lane, T - 1);       // past the tile: the tile's last field, unused
  // the tile's first bit in 64 bits (uniform), the lane's offset from its word in 32 bits
  // (f < 2^14 and field_bits <= 64: a 24-bit multiply)
  const uint64_t tbit = (uint64_t)j0 * (uint32_t)d.field_bits;
  const uint32_t* base = reinterpret_cast<const uint32_t*>(packed) + (tbit >> 5);
  const uint32_t bit = ((uint32_t)tbit & 31u) + __umul24((uint32_t)f, (uint32_t)d.field_bits);
  const uint32_t* p = base + (bit >> 5);
  lf.w0 = p[0];
  lf.w1 = p[1];
  lf.w2 = p[2];
  lf.sh = bit;                                   // the funnel shifts take its low 5 bits
  return lf;
}

// Classify the lane's field: class search (bucket table on the top index bits, then the
// class starts), the block's scale into its slot, and the block appended to the wave's
// odd or even ring.  An index >= the shell-union size gets slot 0 (it contributes
// nothing), is counted and is not queued; the return value says so (true for such a
// field inside the tile).  ROWSCALE (the Euclidean decode): the slot takes the scale of
// the block's row, rs[f / Kb], instead of 1.
template <bool ROWSCALE = false>
__device__ __forceinline__ bool classify_lane(uint8_t* smem, const ELayout& L, float* part, const KDesc& d,
                                              const LaneField& lf, int T, int u, int lane, int32_t* err, Rings& R,
                                              const __half* rs = nullptr, float inv_kb = 0.0f) {
  const LlvqClassHot* cls = reinterpret_cast<const LlvqClassHot*>(smem + L.cls);
  const float* G = reinterpret_cast<const float*>(smem + L.gains);
  const uint8_t* bk = smem + L.bucket;
  const int f = u * 64 + lane;
  const uint32_t flo = __builtin_amdgcn_alignbit(lf.w1, lf.w0, lf.sh);
  const uint32_t fhi = __builtin_amdgcn_alignbit(lf.w2, lf.w1, lf.sh);
  const uint32_t ilo = flo & d.shape_mask_lo;
  const uint32_t ihi = fhi & d.shape_mask_hi;
  const uint64_t I = ((uint64_t)ihi << 32) | ilo;
  const bool valid = f < T && I < d.index_count;
  const double Id = valid ? __builtin_fma((double)ihi, 4294967296.0, (double)ilo) : 0.0;
  const uint32_t bidx = d.bshift >= 32 ? (ihi >> (d.bshift - 32)) : __builtin_amdgcn_alignbit(ihi, ilo, d.bshift);
  uint32_t k = bk[valid ? bidx : 0u];
  const bool c1 = Id >= cls[k + 1].start;
  const bool c2 = Id >= cls[k + 2].start;
  k += (uint32_t)c1 + (uint32_t)c2;                 // c2 implies c1
  if (__ballot(c2)) {
    while (Id >= cls[k + 1].start) ++k;             // the sentinel records end the scan
  }
  LLVQ_DCHECK(!valid || (int)k < d.ncls);
  // (the record's byte offset by a 24-bit multiply-add, not the compiler's 32-bit multiply)
  const LlvqClassHot& h = *reinterpret_cast<const LlvqClassHot*>(
      smem + mad_u24(k, (uint32_t)sizeof(LlvqClassHot), L.cls));
  const bool odd = ((h.meta >> 17) & 1u) != 0u;
  // J = I - start as the low bits of 2^52 + J (exact: J < 2^41 < 2^52)
  const uint64_t jb = __builtin_bit_cast(uint64_t, Id + (0x1p52 - h.start));
  const uint32_t ehi = ((uint32_t)(jb >> 32) & 0x3ffu) | ((uint32_t)f << 10) | (k << 24);
  const uint64_t entry = ((uint64_t)ehi << 32) | (uint32_t)jb;
  const uint32_t gsh = d.shape_bits >= 32 ? (fhi >> (d.shape_bits - 32))
                                          : __builtin_amdgcn_alignbit(fhi, flo, d.shape_bits);
  const uint32_t g = gsh & ((1u << d.gain_bits) - 1u);
  float sc = d.mode == LLVQ_MODE_SHAPEGAIN ? G[g] * h.invnorm : 1.0f;
  if (ROWSCALE && d.mode != LLVQ_MODE_SHAPEGAIN && f < T)
    sc = __half2float(rs[(uint32_t)(((float)f + 0.5f) * inv_kb)]);
  if (f < T) part[f] = valid ? sc : 0.0f;
  if (f < T && !valid && err) atomicAdd(err, 1);
  const uint64_t bo = __ballot(valid && odd);
  const uint64_t be = __ballot(valid && !odd);
  const uint32_t po = __builtin_amdgcn_mbcnt_hi((uint32_t)(bo >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bo, 0u));
  const uint32_t pe = __builtin_amdgcn_mbcnt_hi((uint32_t)(be >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)be, 0u));
  // one store: the even ring follows the odd one (R.even == R.odd + kRing)
  const uint32_t slot = odd ? ((R.oh + R.on + po) & (kRing - 1)) : kRing + ((R.eh + R.en + pe) & (kRing - 1));
  if (valid) R.odd[slot] = entry;
  R.on += (uint32_t)__popcll(bo);
  R.en += (uint32_t)__popcll(be);
  LLVQ_DCHECK(R.on < (uint32_t)kRing && R.en < (uint32_t)kRing);
  return f < T && !valid;
}

template <bool XF32, int TAIL>
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
  float* part = reinterpret_cast<float*>(smem + L.buf[0].part);
  int* work = reinterpret_cast<int*>(smem + L.work);   // unit counter, leftover counts, chunk counter
  uint64_t* shq = reinterpret_cast<uint64_t*>(smem + a.rings);   // the rings, then the leftover queue
  const float inv_kb = 1.0f / (float)kb;

  // ---- set-up: the first unit's fields are requested before the tables and activations
  // are staged in LDS, so their memory latency overlaps the staging.  (The grid never
  // exceeds the tile count, so tile blockIdx.x exists and T0 >= 1.)
  const int row00 = blockIdx.x * a.rows_per_tile;
  const int T0 = min(a.rows_per_tile, d.rows - row00) * kb;
  LaneField lf = load_lane_field(d, packed, (uint32_t)(row00 * kb), T0, min(wave, (T0 - 1) >> 6), lane);
  // activations: the whole 16-byte words of a 16-byte aligned bf16 row go with the table
  // copies; the rest (and the zero padding to Kb * 24 columns) follows
  const bool xa16 = !XF32 && ((((uintptr_t)xv) & 15u) == 0u);
  const int xw = xa16 ? (d.cols >> 3) : 0;
  engine_prologue<TAIL>(smem, L, d, a.nbuckets, scales, tid, CopySeg{reinterpret_cast<const uint4*>(xv), a.xs, xw});
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
  if (tid < 4) work[tid] = 0;
  __syncthreads();

  Rings R;
  R.odd = shq + (size_t)(2 * wave) * kRing;
  R.even = R.odd + kRing;
  for (int tile = blockIdx.x, lt = 0; tile < a.ntiles; tile += gridDim.x, ++lt) {
    const int row0 = tile * a.rows_per_tile;
    const int nrows = min(a.rows_per_tile, d.rows - row0);
    const int T = nrows * kb;
    const int nun = (T + 63) >> 6;
    const uint32_t j0 = (uint32_t)(row0 * kb);
    // units 0..kEWaves-1 go to the waves in order, the rest through the counter
    int u = wave;
    if (lt > 0) lf = load_lane_field(d, packed, j0, T, min(u, nun - 1), lane);
    R.oh = R.on = R.eh = R.en = 0u;
    while (u < nun) {
      int u2 = 0;
      if (lane == 0) u2 = atomicAdd(&work[0], 1);
      u2 = __builtin_amdgcn_readfirstlane(u2) + kEWaves;
      const LaneField lf2 = load_lane_field(d, packed, j0, T, min(u2, nun - 1), lane);
      classify_lane(smem, L, part, d, lf, T, u, lane, err, R);
      while (R.on >= 64u) {
        gemv_odd<XF32, TAIL>(smem, a, part, R.odd[(R.oh + (uint32_t)lane) & (kRing - 1)], (uint32_t)kb, inv_kb);
        R.oh = (R.oh + 64u) & (kRing - 1);
        R.on -= 64u;
      }
      while (R.en >= 64u) {
        gemv_even<XF32, TAIL>(smem, a, part, R.even[(R.eh + (uint32_t)lane) & (kRing - 1)], (uint32_t)kb, inv_kb);
        R.eh = (R.eh + 64u) & (kRing - 1);
        R.en -= 64u;
      }
      u = u2;
      lf = lf2;
    }

    // ---- the rings' remainders into one shared queue (odd entries from the front, even
    // from position kLeftEven), then decoded by all waves as full chunks
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
    // even chunks (the longer decode) first, so that the last ones handed out are short
    const int nlo = work[1], nle = work[2];
    const int nce = (nle + 63) >> 6;
    const int nch = nce + ((nlo + 63) >> 6);
    for (;;) {
      int c = 0;
      if (lane == 0) c = atomicAdd(&work[3], 1);
      c = __builtin_amdgcn_readfirstlane(c);
      if (c >= nch) break;
      if (c < nce) {
        const int e = (c << 6) + lane;
        if (e < nle) gemv_even<XF32, TAIL>(smem, a, part, shq[kLeftEven + e], (uint32_t)kb, inv_kb);
      } else {
        const int e = ((c - nce) << 6) + lane;
        if (e < nlo) gemv_odd<XF32, TAIL>(smem, a, part, shq[e], (uint32_t)kb, inv_kb);
      }
    }
    __syncthreads();

    // ---- row sums of this tile (fixed order); counters reset for the next tile
    for (int rl = wave; rl < nrows; rl += kEWaves) {
      float acc = 0.0f;
      for (int b = lane; b < kb; b += 64) acc += part[rl * kb + b];
      const float tot = wave_sum_fixed(acc);
      if (lane == 0) {
        const int r = row0 + rl;
        const float rs = sg ? 1.0f : __half2float(scales[r]);
        y[r] = tot * rs;
      }
    }
    if (tid < 4) work[tid] = 0;
    __syncthreads();
  }
}
