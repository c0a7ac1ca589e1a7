// Tiled LLVQ block decoder shared by the fused kernels (gfx950).
// Included once by llvq.hip (uses its KDesc, read_field and table namespaces).
//
// A workgroup of kEThreads lanes (16 waves, one workgroup per CU) is persistent over
// tiles of R consecutive rows (T = R * Kb <= kETileMax blocks).  Per tile, with a
// workgroup barrier between the phases:
//   1. classify: every block's field is read, its class found (bucket table on the top
//      index bits + a short scan of the class starts) and the block appended to one of
//      two LDS queues: odd-coset classes from the front, even-coset classes from the
//      back.  The block's scale goes to an LDS slot.  Indices >= the shell-union size
//      contribute 0 and are counted.
//   2. decode: chunks of 64 consecutive entries of one queue, one block per lane, so a
//      wavefront runs one of the two (very different) decoders without divergence;
//      chunks are handed out by an LDS counter, odd chunks first.
//   3. a consumer turns the decoded values into the kernel's result (dot product,
//      stored weights, ...).
//
// Rank unranking: exact arithmetic decoding in fp64.  With y = u * n the value slot is
// the number of cumulative counts C_j <= floor(y) (SWAR compare of the three thresholds
// packed in one dword) and y <- (y - C_k) * (n' / c_k), n' the values left after the
// step, n'/c from an LDS table.  Counts are kept times 8 (a count byte is then the
// byte offset of its table entry), so the step computes (8 y - 8 C_k) * (n' / 8 c_k),
// which rounds exactly like the unscaled form.  The decision margins (>= n/(2Q),
// Q <= 4.2e8 arrangements) exceed the accumulated rounding error by a factor > 1e5.  The last 6
// values (TAIL = 6, or 7 for the batch-1 GEMV, which has the LDS to spare) come from a
// table of all 4^TAIL slot sequences grouped by composition in lexicographic order: with
// counts c (sum TAIL) and y in [0, TAIL), the rank inside the group is
// floor(y * Q(c) / TAIL).

#pragma once

constexpr int kEThreads = 1024;
constexpr int kEWaves = kEThreads / 64;
constexpr int kETileMax = 16384;    // block index inside a tile fits 14 bits
constexpr int kEUnit = 256;         // fields per classify unit (4 per lane)
constexpr int kBias = 12;           // value tables store 12 +- v (|v| <= 12)
// Tail of TAIL values resolved by one table lookup (6 or 7; 7 is the most the even-coset
// decoder allows: its part switch at value 16 must be a step).  steps: values resolved
// step by step; wdot: udot4 weights of the composition index c0 + (TAIL+1) c1 +
// (TAIL+1)^2 c2; ncomp / nseq: entries of the composition and sequence tables.
template <int TAIL>
struct TailSpec {
  static_assert(TAIL == 6 || TAIL == 7, "tail of 6 or 7 values");
  static constexpr int steps = 24 - TAIL;
  static constexpr uint32_t wdot = (uint32_t)(1 | ((TAIL + 1) << 8) | ((TAIL + 1) * (TAIL + 1) << 16));
  static constexpr int ncomp = (TAIL + 1) * (TAIL + 1) * (TAIL + 1);
  static constexpr int nseq = 1 << (2 * TAIL);
};
constexpr int kFStride = 32;        // F row length (c = 0..24, padded to 256 bytes)
constexpr uint32_t kInvalidClass = 0xffu;   // queue entry class of a block to be written as zeros
constexpr uint32_t kFRow = kFStride * 8u;   // F row in bytes

// One tile's queues and block slots.
struct TileBuf {
  uint32_t ctr;       // int[2]: odd queue fill, even queue fill
  uint32_t queue;     // uint64[tmax]: J | f << 42 | class << 56 (see entry_J)
  uint32_t part;      // float[tmax]: block scale, then the block's result
};

struct ELayout {
  // byte offsets inside the dynamic LDS segment
  uint32_t ftab;      // double F[25][32]: F[r][c] = (23 - r) / (8 c) (c = 1..24), always at offset 0
  uint32_t cls;       // LlvqClassHot[ncls + 2]: the last two are sentinels (start only, +inf)
  uint32_t gains;     // float[2^gain_bits]
  uint32_t bucket;    // uint8[nbuckets]
  uint32_t tail;      // uint16[4^TAIL]
  uint32_t tcomp;     // LlvqTailComp[(TAIL+1)^3]
  uint32_t work;      // int[4]: work-item counter of the current phase
  TileBuf buf[2];     // one or two tile buffers
  uint32_t total;     // end of the engine's part; consumer data follows
  uint32_t golay;     // uint32[4096]: a copy of the Golay codeword table, when a consumer stages one
};

__host__ __device__ inline uint32_t align16(uint32_t v) { return (v + 15u) & ~15u; }

__host__ __device__ inline uint32_t engine_layout_base(ELayout& L, int ncls, int ngains, int nbuckets, int tmax,
                                                      int nbuf = 1, int tail = 6) {
  uint32_t o = 0;
  L.ftab = o;     o = align16(o + 800u * 8u);
  L.golay = 0u;
  L.cls = o;      o = align16(o + (uint32_t)(ncls + 2) * (uint32_t)sizeof(LlvqClassHot));
  L.gains = o;    o = align16(o + (uint32_t)ngains * 4u);
  L.bucket = o;   o = align16(o + (uint32_t)nbuckets);
  L.tail = o;     o = align16(o + (2u << (2 * tail)));
  L.tcomp = o;    o = align16(o + (uint32_t)((tail + 1) * (tail + 1) * (tail + 1)) * (uint32_t)sizeof(LlvqTailComp));
  L.work = o;     o = align16(o + 16u);
  for (int b = 0; b < 2; ++b) {
    if (b < nbuf) {
      L.buf[b].ctr = o;    o = align16(o + 16u);
      L.buf[b].queue = o;  o = align16(o + (uint32_t)tmax * 8u);
      L.buf[b].part = o;   o = align16(o + (uint32_t)tmax * 4u);
    } else {
      L.buf[b] = L.buf[0];
    }
  }
  L.total = o;
  return o;
}

struct EArgs {
  int rows_per_tile;
  int ntiles;
  int nbuckets;
  ELayout L;
  uint32_t xs;     // GEMV: x, kb*24 elements (fp32 or bf16), zero padded
  uint32_t xsum;   // GEMV: float[kb], sum of the 24 x values of each block column
  uint32_t rings;  // batch-1 GEMV: the waves' ring queues, then the shared leftover queue
};

// ---------------------------------------------------------------------------
// ALU helpers.  Full-rate 24-bit multiply-add and bit count with accumulator (the
// compiler otherwise picks a quarter-rate 64-bit multiply-add, and does not fold the
// addend into v_bcnt).

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

// (a << 8) | 1: the one-hot count decrement (a - this) of a SWAR slot choice a.
__device__ __forceinline__ uint32_t shl8_or1(uint32_t a) {
  uint32_t d;
  asm("v_lshl_or_b32 %0, %1, 8, 1" : "=v"(d) : "v"(a));
  return d;
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

// popcount(a) + b, b in a vector register
__device__ __forceinline__ uint32_t bcnt_addv(uint32_t a, uint32_t b) {
  uint32_t d;
  asm("v_bcnt_u32_b32 %0, %1, %2" : "=v"(d) : "v"(a), "v"(b));
  return d;
}

// 8 at the byte of the slot chosen by the SWAR flags g: (g << 8 | 1) - g = 255 g + 1 is
// the one-hot byte of the slot, times 8 for the scaled counts.
__device__ __forceinline__ uint32_t dec8(uint32_t g) {
  uint32_t d;
  asm("v_mad_u32_u24 %0, %1, %2, 8" : "=v"(d) : "v"(g), "s"(2040u));
  return d;
}

// median of (a, b, 1): 1 if a >= 1, else b (b in {0, 1})
__device__ __forceinline__ uint32_t med3_1(uint32_t a, uint32_t b) {
  uint32_t d;
  asm("v_med3_u32 %0, %1, %2, 1" : "=v"(d) : "v"(a), "v"(b));
  return d;
}

// Entry of the F table at byte offset o.  The table sits at offset 0 of the dynamic LDS
// segment, and the engine's kernels declare no static LDS, so o is the LDS address itself
// (no base register add per step).
typedef const __attribute__((address_space(3))) double* lds_f64_ptr;
__device__ __forceinline__ double ftab_at(const uint8_t* smem, uint32_t o) {
  (void)smem;
  return *reinterpret_cast<lds_f64_ptr>((uintptr_t)o);
}

// ---------------------------------------------------------------------------
// per-block decoders

// Common per-block setup from the class record: J / A split, codeword, initial y.
struct BlockStart {
  uint32_t c;   // codeword (not loaded with WANTC = false)
  uint32_t ci;  // its index in the Golay table
  uint32_t s;   // sign bits
  double y;     // y_0 = (R + 1/2) * n0 / P
};

// LG: the codeword comes from the LDS copy of the Golay table at L.golay (the streamed
// decode, which stores to global memory while it decodes: on gfx9 the wait for a load
// counts every older vector-memory operation, stores included, so a global table read
// would wait for the chunk stores in flight).
template <bool LG = false, bool WANTC = true>
__device__ __forceinline__ BlockStart block_start(const uint8_t* smem, const ELayout& L, double Jd,
                                                  const LlvqClassHot& h) {
  BlockStart bs;
  const uint32_t q = (uint32_t)__builtin_fma(Jd, h.inv_a, 0x1p-13);    // floor(J / A), exact
  const uint32_t r = (uint32_t)__builtin_fma(-(double)q, h.a, Jd);      // J - q A, exact
  LLVQ_DCHECK((double)r < h.a);
  const uint32_t B = h.meta & 31u;
  bs.s = q & ((1u << B) - 1u);
  const uint32_t R = q >> B;
  bs.ci = h.toff + r;
  bs.c = !WANTC ? 0u
                : LG ? reinterpret_cast<const uint32_t*>(smem + L.golay)[bs.ci] : dev_tables::kGolayTable[bs.ci];
  bs.y = __builtin_fma((double)R, h.y0s, 0.5 * h.y0s);
  return bs;
}

// Slot codes of the last TAIL values (2 bits each, first of them in the low bits), from
// the counts left (times 8, sum 8 TAIL) and y in [0, TAIL).
template <int TAIL>
__device__ __forceinline__ uint32_t tail_codes(const uint8_t* smem, const ELayout& L, uint32_t cnt8, double y) {
  typedef TailSpec<TAIL> TS;
  const uint32_t ci8 = __builtin_amdgcn_udot4(cnt8, TS::wdot, 0u, false);   // 8 (c0 + b c1 + b^2 c2)
  LLVQ_DCHECK(ci8 < (uint32_t)TS::ncomp * 8u);
  const LlvqTailComp tc = *reinterpret_cast<const LlvqTailComp*>(smem + L.tcomp + ci8);
  const uint32_t r = (uint32_t)((float)y * tc.q_over_n);
  LLVQ_DCHECK(tc.offset + r < (uint32_t)TS::nseq && (float)r < tc.q_over_n * (float)TAIL);
  return reinterpret_cast<const uint16_t*>(smem + L.tail)[tc.offset + r];
}

// One arithmetic-decoding step on (y, nc, cnt8) with F row offset fo (bytes): returns the
// SWAR flags g of the chosen slot; k = popcount(g) + sel is the caller's selector.  The
// table entry's offset is v_perm(hi, cnt8, k): byte 0 is the count byte 8 c_k (selector
// byte 0 picks a byte of cnt8, or of hi = cnt8 when the +4 rides there); a selector byte 1
// of 4 adds byte 0 of hi as bits 8..15, a per-lane row offset in units of 256 bytes (the
// even decoder's rows of a two-part class's support), else 0x0c makes it zero.
struct StepOut {
  uint32_t g, k;
};

__device__ __forceinline__ StepOut decode_step(const uint8_t* smem, double& y, uint32_t& nc, uint32_t& cnt8,
                                               uint32_t sel, uint32_t fo, uint32_t hi) {
  const uint32_t f = (uint32_t)y;
  const uint32_t g = swar_ge(f, nc);
  const uint32_t k = bcnt_addv(g, sel);
  const uint32_t c8 = __builtin_amdgcn_perm(hi, cnt8, k);          // 8 c_k (+ row offset)
  const uint32_t C8 = __builtin_amdgcn_udot4(g, cnt8, 0u, false);  // 8 C_k
  LLVQ_DCHECK((c8 & 0xffu) != 0u && (c8 & 0xffu) <= 192u && fo + c8 < 25u * kFRow);   // the slot has values left
  const double fac = ftab_at(smem, fo + c8);                       // n' / (8 c_k)
  y = __builtin_fma(y, 8.0, -(double)C8) * fac;
  cnt8 -= dec8(g);
  nc += g ^ 0x010101u;
  return {g, k};
}

// Odd coset: one part of 24 values, visited in position order.  slot(p) returns the
// value's slot selector; quad_codes turns four of them into four bytes of the class's
// 8-byte value table (biased values 12 + v_p, or fp8 codes after load_fp8).  The sign of
// each value follows from the codeword bit and the value mod 4, folded into the table
// lookup: the table holds each slot's value and its negation, and the selector's +4
// (negated entry) for positions off the codeword is added per four positions.
template <int TAIL = 6>
struct OddDec {
  static constexpr int kSteps = TailSpec<TAIL>::steps;
  double y;
  uint32_t nc, cnt8, notc4, svlo, svhi, codes;

  __device__ __forceinline__ void init(const LlvqClassHot& h, const BlockStart& bs) {
    y = bs.y;
    nc = h.nc0;
    cnt8 = h.cnt0;
    notc4 = ~bs.c << 2;   // bit p + 2 = position p is off the codeword
    svlo = h.sv0lo;
    svhi = h.sv0hi;
    codes = 0u;
  }

  // load_fp8 switches to the fp8 value table.  slot(p): the value's slot selector (byte 0:
  // slot 0..3; callers use byte 0 only, the bytes above are not defined), so that four
  // positions share one v_perm (quad_codes).  The codeword's +4 (negated entry, off the
  // codeword) is not in it: sign_quad gives it for four positions at once, added to their
  // joined selector (one add per four positions rather than a shift and an and-or per
  // position).
  __device__ __forceinline__ void load_fp8(const LlvqClassHot& h) {
    svlo = h.sv0lo8;
    svhi = h.sv0hi8;
  }

  __device__ __forceinline__ uint32_t slot(const uint8_t* smem, const ELayout& L, int p) {
    if (p < kSteps) {
      const uint32_t k = decode_step(smem, y, nc, cnt8, 0x0c0c0c00u, kFRow * (uint32_t)p, cnt8).k;
      if (p == kSteps - 1) codes = tail_codes<TAIL>(smem, L, cnt8, y);
      return k;
    }
    return __builtin_amdgcn_ubfe(codes, 2 * (p - kSteps), 2);
  }

  // The fp8 codes of positions 4q .. 4q+3 in one dword: the four slot selectors (byte 0
  // of each) joined into one selector with their codeword +4s added (a byte never exceeds
  // 7, so nothing carries), then one v_perm picks all four codes.
  __device__ __forceinline__ uint32_t quad_codes(uint32_t k0, uint32_t k1, uint32_t k2, uint32_t k3, int q) const {
    const uint32_t j01 = __builtin_amdgcn_perm(k1, k0, 0x0c0c0400u);   // k0, k1, 0, 0
    const uint32_t j23 = __builtin_amdgcn_perm(k3, k2, 0x04000c0cu);   // 0, 0, k2, k3
    return __builtin_amdgcn_perm(svhi, svlo, j01 + j23 + sign_quad(q));
  }

  // The +4 of positions 4q .. 4q+3 (set off the codeword) at bits 2, 10, 18 and 26: the
  // nibble's bit e moves to bit 8 e + 2 under one multiply (its other shifted copies land
  // on bits the mask clears, and no two copies overlap, so nothing carries).
  __device__ __forceinline__ uint32_t sign_quad(int q) const {
    const uint32_t nib = __builtin_amdgcn_ubfe(notc4, 4 * q + 2, 4);
    return __umul24(nib, 0x00810204u) & 0x04040404u;
  }
};

// Even coset: support values (on the codeword's positions, ascending) then complement
// values (other positions, ascending), on one arithmetic-decoding state.  step(i)
// returns the biased value byte of the i-th decoded value in its low 8 bits (the bits
// above are not defined) and its position.  Nonzero values take the bits of s in decode
// order; the last support value's sign fixes the parity of negatives on the support, and
// init inserts it into s at bit w - 1 (the support values are all nonzero, so they take
// bits 0..w-1).  Zero can only be a part's
// slot 0, so a value takes a sign bit unless its slot is 0 and the part's slot 0 is zero.
// s is kept shifted left by 2, so the next sign bit sits at the selector's +4 bit and
// joins the selector with one and-or; a zero value that takes no bit still gets the
// current one in its selector, harmlessly, since the negated entry of a zero is zero.
// POSTAB: 0, the positions in decode order come from the codeword's bits (a find-first-set
// and a clear per value); 1 or 2, from kEvenIdx or kEvenPos (indexed by the block's
// codeword, p or 2 p per byte: one byte extract per value), and step() and slot() give p
// or 2 p (the byte offset of the position in bf16 activations).  The table is read from
// global memory at init: a kernel with global stores in flight issues init before them.
template <int TAIL = 6, int POSTAB = 0>
struct EvenDec {
  static constexpr int kSteps = TailSpec<TAIL>::steps;
  double y;
  uint32_t nc, cnt8, svlo, svhi, nz0, nz1, m, s, codes, c, hp, fo, swi;
  uint32_t pt[6];

  // hp: LDS byte offset of the class record
  __device__ __forceinline__ void init(const LlvqClassHot& h, const BlockStart& bs, uint32_t hp_) {
    const uint32_t w = (h.meta >> 8) & 31u;
    const uint32_t pi = (h.meta >> 16) & 1u;
    const bool two = w != 0u && w != 24u;
    swi = two ? w : 0u;
    s = bs.s;
    if (w) {
      const uint32_t lo = s & ((1u << (w - 1u)) - 1u);
      const uint32_t negq = ((uint32_t)__builtin_popcount(lo) & 1u) ^ pi;
      s = lo | (negq << (w - 1u)) | ((s >> (w - 1u)) << w);
    }
    s <<= 2;
    y = bs.y;
    nc = h.nc0;
    cnt8 = h.cnt0;
    svlo = h.sv0lo;
    svhi = h.sv0hi;
    nz0 = (h.meta >> 20) & 1u;
    nz1 = (h.meta >> 24) & 1u;
    if (POSTAB) {
      const uint2* t = reinterpret_cast<const uint2*>((POSTAB == 2 ? dev_tables::kEvenPos : dev_tables::kEvenIdx) +
                                                      6u * bs.ci);
      const uint2 t0 = t[0], t1 = t[1], t2 = t[2];
      pt[0] = t0.x; pt[1] = t0.y; pt[2] = t1.x; pt[3] = t1.y; pt[4] = t2.x; pt[5] = t2.y;
      c = 0u;
      m = 0u;
    } else {
      c = bs.c;
      m = w ? bs.c : 0xffffffu;
    }
    // F rows: values left after step i are w - 1 - i on the support of a two-part class
    // (row i + 24 - w), else 23 - i (row i); the last support step continues into the
    // complement (24 - w left), row i.
    fo = two ? (24u - w) * kFRow : 0u;
    hp = hp_;
    codes = 0u;
  }

  __device__ __forceinline__ uint32_t step(const uint8_t* smem, const ELayout& L, int i, uint32_t& pos) {
    if (i == 8 || i == 12 || i == 16) {
      if (swi == (uint32_t)i) {   // two-part class: the complement's tables
        const uint4 q = *reinterpret_cast<const uint4*>(smem + hp + 64u);
        nc = q.x;
        cnt8 = q.y;
        svlo = q.z;
        svhi = q.w;
        nz0 = nz1;
        if (!POSTAB) m = ~c & 0xffffffu;
      }
    }
    uint32_t kb, free_;
    if (i < kSteps) {
      // the row offset fo / 256 joins the table offset through the selector's byte 1, which
      // also leaves garbage in bits 8..15 of the returned byte (callers keep the low byte)
      const StepOut so = decode_step(smem, y, nc, cnt8, 0x0c0c0400u, kFRow * (uint32_t)i, fo >> 8);
      kb = so.k;
      free_ = med3_1(so.g, nz0);
      if (i == 6 || i == 10 || i == 14) fo = swi == (uint32_t)(i + 2) ? 0u : fo;
      if (i == kSteps - 1) codes = tail_codes<TAIL>(smem, L, cnt8, y);
    } else {
      const uint32_t code = __builtin_amdgcn_ubfe(codes, 2 * (i - kSteps), 2);
      kb = code;   // (byte 0 is the one used)
      free_ = med3_1(code, nz0);
    }
    const uint32_t sel = kb | (s & 4u);
    s >>= free_;
    if (POSTAB) {
      pos = (pt[i >> 2] >> (8 * (i & 3))) & 0xffu;
    } else {
      pos = (uint32_t)__builtin_ctz(m);
      m &= m - 1u;
    }
    return __builtin_amdgcn_perm(svhi, svlo, sel);
  }

  // The fp8 form (see OddDec::slot): fp8 tables, and the selector of the i-th decoded
  // value (byte 0: slot 0..3, + 4 when negative; callers use byte 0 only) with its
  // position.  A two-part class switches to the complement's fp8 table at an even i, so
  // the two positions of a pair always share a table.
  __device__ __forceinline__ void load_fp8(const LlvqClassHot& h) {
    svlo = h.sv0lo8;
    svhi = h.sv0hi8;
  }

  __device__ __forceinline__ uint32_t slot(const uint8_t* smem, const ELayout& L, int i, uint32_t& pos) {
    if (i == 8 || i == 12 || i == 16) {
      if (swi == (uint32_t)i) {   // two-part class: the complement's tables
        const uint2 q = *reinterpret_cast<const uint2*>(smem + hp + 64u);
        const uint2 t = *reinterpret_cast<const uint2*>(smem + hp + 88u);
        nc = q.x;
        cnt8 = q.y;
        svlo = t.x;
        svhi = t.y;
        nz0 = nz1;
        if (!POSTAB) m = ~c & 0xffffffu;
      }
    }
    uint32_t kb, free_;
    if (i < kSteps) {
      // the row offset fo / 256 joins the table offset through the selector's byte 1 (only
      // byte 0 of the returned selector is used)
      const StepOut so = decode_step(smem, y, nc, cnt8, 0x0c0c0400u, kFRow * (uint32_t)i, fo >> 8);
      kb = so.k;
      free_ = med3_1(so.g, nz0);
      if (i == 6 || i == 10 || i == 14) fo = swi == (uint32_t)(i + 2) ? 0u : fo;
      if (i == kSteps - 1) codes = tail_codes<TAIL>(smem, L, cnt8, y);
    } else {
      const uint32_t code = __builtin_amdgcn_ubfe(codes, 2 * (i - kSteps), 2);
      kb = code;   // (byte 0 is the one used)
      free_ = med3_1(code, nz0);
    }
    const uint32_t sel = kb | (s & 4u);
    s >>= free_;
    if (POSTAB) {
      pos = (pt[i >> 2] >> (8 * (i & 3))) & 0xffu;
    } else {
      pos = (uint32_t)__builtin_ctz(m);
      m &= m - 1u;
    }
    return sel;
  }
};

// ---------------------------------------------------------------------------
// workgroup set-up and classification

// A copy of n4 16-byte words from global memory into LDS (byte offset dst, 16-byte
// aligned), split so that a lane's loads (its first two words) can be issued before any
// store: copy_issue, then copy_finish.
struct CopySeg {
  const uint4* src;
  uint32_t dst;
  int n4;
};

typedef uint32_t llvq_u32x4 __attribute__((ext_vector_type(4)));

struct CopyRegs {
  llvq_u32x4 a, b;   // words tid and tid + kEThreads
};

__device__ __forceinline__ CopyRegs copy_issue(const CopySeg& c, int tid) {
  const llvq_u32x4* s = reinterpret_cast<const llvq_u32x4*>(c.src);
  CopyRegs v = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
  if (tid < c.n4) v.a = s[tid];
  if (tid + kEThreads < c.n4) v.b = s[tid + kEThreads];
  return v;
}

__device__ __forceinline__ void copy_finish(uint8_t* smem, const CopyRegs& v, const CopySeg& c, int tid) {
  llvq_u32x4* d = reinterpret_cast<llvq_u32x4*>(smem + c.dst);
  if (tid < c.n4) d[tid] = v.a;
  if (tid + kEThreads < c.n4) d[tid + kEThreads] = v.b;
  const llvq_u32x4* s = reinterpret_cast<const llvq_u32x4*>(c.src);
  for (int i = tid + 2 * kEThreads; i < c.n4; i += kEThreads) d[i] = s[i];
}

// Words n4 * 4 .. nw - 1 of a table (the part past its whole 16-byte words).
__device__ __forceinline__ void copy_word_tail(uint8_t* smem, uint32_t dst, const void* src, int nw, int tid) {
  for (int i = (nw & ~3) + tid; i < nw; i += kEThreads)
    reinterpret_cast<uint32_t*>(smem + dst)[i] = reinterpret_cast<const uint32_t*>(src)[i];
}

// Tables into LDS (the step factors F, the class records, the tail tables, the bucket
// table, the Golay table when the layout has a place for it), plus an optional extra
// segment (a consumer's activations).  All of a lane's global loads are issued before its
// first LDS store, so the workgroup waits for about one memory latency rather than one
// per copy.  The caller synchronises afterwards.
template <int TAIL = 6>
__device__ __forceinline__ void engine_prologue(uint8_t* smem, const ELayout& L, const KDesc& d, int nbuckets,
                                                const __half* __restrict__ scales, int tid,
                                                CopySeg extra = {nullptr, 0u, 0}) {
  typedef TailSpec<TAIL> TS;
  const uint16_t* tail_src = TAIL == 6 ? dev_tables::kTail6 : dev_tables::kTail7;
  const LlvqTailComp* tcomp_src = TAIL == 6 ? dev_tables::kTailComp6 : dev_tables::kTailComp7;
  const int cls_w = d.ncls * (int)(sizeof(LlvqClassHot) / 4);
  const int bk_w = (nbuckets + 3) >> 2;
  const uint8_t* bk_src = dev_tables::kBucketTable[d.max_shell];
  const CopySeg s_cls = {reinterpret_cast<const uint4*>(dev_tables::kClassHot), L.cls, cls_w >> 2};
  const CopySeg s_tail = {reinterpret_cast<const uint4*>(tail_src), L.tail, TS::nseq * 2 / 16};
  const CopySeg s_tcomp = {reinterpret_cast<const uint4*>(tcomp_src), L.tcomp, (TS::ncomp * 2) >> 2};
  const CopySeg s_bk = {reinterpret_cast<const uint4*>(bk_src), L.bucket, bk_w >> 2};
  const CopySeg s_f = {reinterpret_cast<const uint4*>(dev_tables::kFTable), L.ftab, 800 * 8 / 16};
  const CopySeg s_g = {reinterpret_cast<const uint4*>(dev_tables::kGolayTable), L.golay, L.golay ? 4096 * 4 / 16 : 0};
  const CopyRegs v_cls = copy_issue(s_cls, tid);
  const CopyRegs v_tail = copy_issue(s_tail, tid);
  const CopyRegs v_tcomp = copy_issue(s_tcomp, tid);
  const CopyRegs v_bk = copy_issue(s_bk, tid);
  const CopyRegs v_f = copy_issue(s_f, tid);
  const CopyRegs v_g = copy_issue(s_g, tid);
  const CopyRegs v_x = copy_issue(extra, tid);
  if (d.mode == LLVQ_MODE_SHAPEGAIN && scales != nullptr) {
    float* G = reinterpret_cast<float*>(smem + L.gains);
    for (int i = tid; i < (1 << d.gain_bits); i += kEThreads) G[i] = __half2float(scales[i]);
  }
  copy_finish(smem, v_cls, s_cls, tid);
  copy_finish(smem, v_tail, s_tail, tid);
  copy_finish(smem, v_tcomp, s_tcomp, tid);
  copy_finish(smem, v_bk, s_bk, tid);
  copy_finish(smem, v_f, s_f, tid);
  copy_finish(smem, v_g, s_g, tid);
  copy_finish(smem, v_x, extra, tid);
  copy_word_tail(smem, L.cls, dev_tables::kClassHot, cls_w, tid);
  if (tid < 2) reinterpret_cast<LlvqClassHot*>(smem + L.cls)[d.ncls + tid].start = __builtin_inf();
  copy_word_tail(smem, L.tcomp, tcomp_src, TS::ncomp * 2, tid);
  copy_word_tail(smem, L.bucket, bk_src, bk_w, tid);
}

// Field index in the stream of tile block f.  A tile is nr rows of w blocks starting at
// field j0 (row stride Kb fields); w == Kb makes the tile one contiguous run.
struct TileMap {
  uint32_t j0;      // stream index of the tile's first block
  uint32_t w;       // blocks per tile row
  uint32_t stride;  // stream fields per tensor row (Kb)
  float inv_w;      // 1 / w
  __device__ __forceinline__ uint32_t field(uint32_t f) const {
    if (w == stride) return j0 + f;
    const uint32_t rl = (uint32_t)(((float)f + 0.5f) * inv_w);
    return j0 + rl * stride + (f - rl * w);
  }
};

// Fields of classify unit u of a tile, 4 per lane (f = 256 u + 64 t + lane), as raw
// words: the field is bits sh.. of the 96-bit word triple (w2:w1:w0), any width up to
// 64 bits.  Bits above the field are not cleared (the consumers mask what they extract).
// The four fields' words are requested together by straight-line code and not used here,
// so the loads stay in flight until the classification needs them.  A field past the
// tile reads the tile's last field (T >= 1 for every unit handed out) and is not used.
// The reads stay inside the packed buffer's 16 bytes of slack.
struct UnitFields {
  uint32_t w0[kEUnit / 64], w1[kEUnit / 64], w2[kEUnit / 64], sh[kEUnit / 64];
};

__device__ __forceinline__ UnitFields load_unit(const KDesc& d, const uint8_t* __restrict__ packed,
                                                const TileMap& tm, int T, int u, int lane) {
  UnitFields uf;
#pragma unroll
  for (int t = 0; t < kEUnit / 64; ++t) {
    const int f = min(u * kEUnit + t * 64 + lane, T - 1);
    const uint64_t bit = (uint64_t)tm.field((uint32_t)f) * (uint32_t)d.field_bits;
    const uint32_t* p = reinterpret_cast<const uint32_t*>(packed) + (bit >> 5);
    uf.w0[t] = p[0];
    uf.w1[t] = p[1];
    uf.w2[t] = p[2];
    uf.sh[t] = (uint32_t)bit & 31u;
  }
  return uf;
}

// Classify the loaded unit: class search, block scale, queue append.  The four fields of
// a lane are searched together (independent LDS reads), the bucket's first two class
// boundaries are tested at once (a longer scan is rare; the sentinel records end it), and
// one queue reservation per parity covers the whole unit.  The common path is straight-line
// code: an invalid block (index >= the shell-union size) is classified as block 0 of class
// 0 and dropped.
// With queue_invalid set, an invalid block of the tile is appended to the even queue with
// class kInvalidClass, for consumers that write every block (its values are zero).
__device__ __forceinline__ void classify_fields(uint8_t* smem, const ELayout& L, const TileBuf& tb, const KDesc& d,
                                                const UnitFields& uf, int T, int u, int lane, int32_t* err,
                                                bool queue_invalid = false) {
  int* ctr = reinterpret_cast<int*>(smem + tb.ctr);
  uint64_t* queue = reinterpret_cast<uint64_t*>(smem + tb.queue);
  float* part = reinterpret_cast<float*>(smem + tb.part);
  const LlvqClassHot* cls = reinterpret_cast<const LlvqClassHot*>(smem + L.cls);
  const float* G = reinterpret_cast<const float*>(smem + L.gains);
  const uint8_t* bk = smem + L.bucket;
  const bool sg = d.mode == LLVQ_MODE_SHAPEGAIN;
  constexpr int kPer = kEUnit / 64;
  bool valid[kPer];
  uint32_t kk[kPer], flo[kPer], fhi[kPer];
  double Id[kPer];
#pragma unroll
  for (int t = 0; t < kPer; ++t) {
    const int f = u * kEUnit + t * 64 + lane;
    flo[t] = __builtin_amdgcn_alignbit(uf.w1[t], uf.w0[t], uf.sh[t]);
    fhi[t] = __builtin_amdgcn_alignbit(uf.w2[t], uf.w1[t], uf.sh[t]);
    const uint32_t ilo = flo[t] & d.shape_mask_lo;
    const uint32_t ihi = fhi[t] & d.shape_mask_hi;
    const uint64_t I = ((uint64_t)ihi << 32) | ilo;
    valid[t] = f < T && I < d.index_count;
    Id[t] = valid[t] ? __builtin_fma((double)ihi, 4294967296.0, (double)ilo) : 0.0;
    const uint32_t bidx = d.bshift >= 32 ? (ihi >> (d.bshift - 32)) : __builtin_amdgcn_alignbit(ihi, ilo, d.bshift);
    kk[t] = bk[valid[t] ? bidx : 0u];
  }
  bool more = false;
#pragma unroll
  for (int t = 0; t < kPer; ++t) {
    const uint32_t k = kk[t];
    const bool c1 = Id[t] >= cls[k + 1].start;
    const bool c2 = Id[t] >= cls[k + 2].start;
    kk[t] = k + (uint32_t)c1 + (uint32_t)c2;   // c2 implies c1
    more = more || c2;
  }
  if (more) {
#pragma unroll
    for (int t = 0; t < kPer; ++t)
      while (Id[t] >= cls[kk[t] + 1].start) ++kk[t];
  }
  int no = 0, ne = 0;
  uint64_t bo[kPer], be[kPer];
  uint64_t entry[kPer];
  uint32_t po[kPer], pe[kPer];
  bool bad = false;
#pragma unroll
  for (int t = 0; t < kPer; ++t) {
    const int f = u * kEUnit + t * 64 + lane;
    const uint32_t k = kk[t];
    LLVQ_DCHECK(!valid[t] || (int)k < d.ncls);
    const LlvqClassHot& h = cls[k];
    const bool odd = ((h.meta >> 17) & 1u) != 0u;
    // J = I - start as the low bits of 2^52 + J (exact: J < 2^41 < 2^52)
    const uint64_t jb = __builtin_bit_cast(uint64_t, Id[t] + (0x1p52 - h.start));
    const uint32_t ehi = ((uint32_t)(jb >> 32) & 0x3ffu) | ((uint32_t)f << 10) | ((valid[t] ? k : kInvalidClass) << 24);
    entry[t] = ((uint64_t)ehi << 32) | (uint32_t)jb;
    const bool qinv = queue_invalid && f < T && !valid[t];
    const uint32_t gsh = d.shape_bits >= 32 ? (fhi[t] >> (d.shape_bits - 32))
                                            : __builtin_amdgcn_alignbit(fhi[t], flo[t], d.shape_bits);
    const uint32_t g = gsh & ((1u << d.gain_bits) - 1u);
    const float sc = sg ? G[g] * h.invnorm : 1.0f;
    if (f < T) part[f] = valid[t] ? sc : 0.0f;
    bad = bad || (f < T && !valid[t]);
    bo[t] = __ballot(valid[t] && odd);
    be[t] = __ballot((valid[t] && !odd) || qinv);
    po[t] = __builtin_amdgcn_mbcnt_hi((uint32_t)(bo[t] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bo[t], 0u));
    pe[t] = __builtin_amdgcn_mbcnt_hi((uint32_t)(be[t] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)be[t], 0u));
    no += __popcll(bo[t]);
    ne += __popcll(be[t]);
  }
  if (bad) {
#pragma unroll
    for (int t = 0; t < kPer; ++t) {
      const int f = u * kEUnit + t * 64 + lane;
      if (f < T && !valid[t] && err) atomicAdd(err, 1);
    }
  }
  int baseo = 0, basee = 0;
  if (lane == 0) {
    baseo = atomicAdd(&ctr[0], no);
    basee = atomicAdd(&ctr[1], ne);
  }
  baseo = __builtin_amdgcn_readfirstlane(baseo);
  basee = __builtin_amdgcn_readfirstlane(basee);
#pragma unroll
  for (int t = 0; t < kPer; ++t) {
    const bool odd = (bo[t] >> lane) & 1u;
    const bool even = (be[t] >> lane) & 1u;
    LLVQ_DCHECK(!(odd || even) || baseo + (int)po[t] < T - (basee + (int)pe[t]));
    if (odd) queue[baseo + (int)po[t]] = entry[t];
    if (even) queue[T - 1 - (basee + (int)pe[t])] = entry[t];
    baseo += __popcll(bo[t]);
    basee += __popcll(be[t]);
  }
}

__device__ __forceinline__ void classify_unit(uint8_t* smem, const ELayout& L, const TileBuf& tb, const KDesc& d,
                                              const uint8_t* __restrict__ packed, const TileMap& tm, int T, int u,
                                              int lane, int32_t* err, bool queue_invalid = false) {
  const UnitFields uf = load_unit(d, packed, tm, T, u, lane);
  classify_fields(smem, L, tb, d, uf, T, u, lane, err, queue_invalid);
}

// Queue entry fields: J | f << 42 | k << 56 with J = I - start(k) the index inside the
// class (every class has fewer than 2^41 indices), f the block's index in the tile and
// k the class.  J comes back as a double by placing it in the mantissa of 2^52.
__device__ __forceinline__ uint32_t entry_f(uint64_t e) { return (uint32_t)(e >> 42) & 0x3fffu; }
__device__ __forceinline__ uint32_t entry_k(uint64_t e) { return (uint32_t)(e >> 56); }
__device__ __forceinline__ double entry_J(uint64_t e) {
  const uint32_t hi = ((uint32_t)(e >> 32) & 0x3ffu) | 0x43300000u;
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | (uint32_t)e) - 0x1p52;
}
