// Rank (lattice point -> global shape index) kernel, gfx950.  Included once by llvq.hip.
//
// The inverse of the decode hierarchy (papernotes.org notes, 方法详解 / 关键设计 2: the
// index is built from shell, class, codeword r, signs s and the lexicographic rank R as
// I = start + r + A (s + 2^B R)).  One lane per point, 24 int8 coordinates held as six
// packed dwords:
//   * membership: common parity p, sum = 4p (mod 8), norm 16 m with 2 <= m <= M, and the
//     positions = 2 (p = 0) or = 1 (p = 1) mod 4 form a Golay codeword.  The codeword is
//     found from its information bits (coordinates 11..22) and compared;
//   * class: the power sums s1, s3, s4 of |x_i| (byte dot products) identify the class
//     among all classes of both cosets; a collision-free hash maps them to a candidate
//     whose stored key is compared;
//   * R: lexicographic rank of the slot sequence (position of each |x_i| in the class's
//     ascending value list, by a byte-table lookup), accumulated in fp64 as
//     sum_i P_i C_k / n_i with P_i the arrangements left; every term and every P_i is an
//     integer below 2^35, so rounding each product to the nearest integer is exact.
//     Even classes rank the support values (codeword positions, ascending) and the
//     complement values separately, R = R_S P_T + R_T, and read the free signs in that
//     order (all support positions but the last, then the nonzero complement positions);
//   * the per-slot counts must be used up exactly, which with the key check makes the
//     absolute values the class's multiset.
// A point failing any check gets UINT64_MAX and is counted.
// The two cosets take very different rank code, so each 256-point step first moves the
// workgroup's odd points (coordinate 0 odd) to the low lanes and the others to the high
// lanes through LDS: all but one wavefront then run a single branch.

#pragma once

// 4 packed sign bits of dword bytes (bit 0 of each byte) -> 4-bit nibble
__device__ __forceinline__ uint32_t byte_bits4(uint32_t b01) { return __builtin_amdgcn_udot4(b01, 0x08040201u, 0u, false); }

template <bool ALIGNED8>
__global__ __launch_bounds__(256) void k_rank(const int8_t* __restrict__ pts, int64_t n, int max_shell,
                                              uint64_t* __restrict__ out, int32_t* err) {
  __shared__ double inv_n[25];
  __shared__ uint32_t rows[256 * 6];    // per-lane slot bytes (even classes read them by position)
  __shared__ uint32_t stage[7 * 256];   // partitioned points: dword q of slot s at q * 256 + s; q = 6: source lane
  __shared__ int wodd[4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  if (tid < 25) inv_n[tid] = tid ? 1.0 / (double)tid : 0.0;
  uint8_t* row = reinterpret_cast<uint8_t*>(rows + 6 * tid);

  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t base = (int64_t)blockIdx.x * 256; base < n; base += stride) {
    uint32_t w[6] = {0u, 0u, 0u, 0u, 0u, 0u};
    const int64_t tl = base + tid;
    if (tl < n) {
      if (ALIGNED8) {
        const uint2* p2 = reinterpret_cast<const uint2*>(pts + tl * 24);
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          const uint2 v = p2[q];
          w[2 * q] = v.x;
          w[2 * q + 1] = v.y;
        }
      } else {
        const uint8_t* pb = reinterpret_cast<const uint8_t*>(pts + tl * 24);
#pragma unroll
        for (int q = 0; q < 6; ++q)
          w[q] = (uint32_t)pb[4 * q] | ((uint32_t)pb[4 * q + 1] << 8) | ((uint32_t)pb[4 * q + 2] << 16) |
                 ((uint32_t)pb[4 * q + 3] << 24);
      }
    }
    // ---- partition: odd points to slots 0.., the rest after them
    const bool odd_pt = tl < n && (w[0] & 1u);
    const uint64_t oddm = __ballot(odd_pt);
    if (lane == 0) wodd[wv] = __popcll(oddm);
    __syncthreads();
    int obase = 0, nodd = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      obase += q < wv ? wodd[q] : 0;
      nodd += wodd[q];
    }
    const int below =
        (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(oddm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)oddm, 0u));
    const int slot = odd_pt ? obase + below : nodd + (tid - obase - below);
#pragma unroll
    for (int q = 0; q < 6; ++q) stage[q * 256 + slot] = w[q];
    stage[6 * 256 + slot] = (uint32_t)tid;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 6; ++q) w[q] = stage[q * 256 + tid];
    const int64_t t = base + (int64_t)stage[6 * 256 + tid];
    if (t < n) {
      const uint32_t p = w[0] & 1u;
      const uint32_t pb = p ? 0x01010101u : 0u;
      bool ok = true;
      int sum = 0;
      uint32_t s1 = 0, s2 = 0, s3 = 0, s4 = 0, mask = 0, negm = 0, nzm = 0;
      uint32_t sl[6];
#pragma unroll
      for (int q = 0; q < 6; ++q) {
        const uint32_t x = w[q];
        ok = ok && ((x & 0x01010101u) == pb);
        sum = __builtin_amdgcn_sdot4((int)x, 0x01010101, sum, false);
        const uint32_t sgn = (x >> 7) & 0x01010101u;
        const uint32_t a = (x ^ ((sgn << 8) - sgn)) + sgn;          // |x| per byte
        s2 = __builtin_amdgcn_udot4(a, a, s2, false);
        s1 = __builtin_amdgcn_udot4(a, 0x01010101u, s1, false);
        // squares of a <= 15 by byte tables (valid points have a <= 12)
        const uint32_t sq_lo = __builtin_amdgcn_perm(0x31241910u, 0x09040100u, a);
        const uint32_t sq_hi = __builtin_amdgcn_perm(0xe1c4a990u, 0x79645140u, a & 0x07070707u);
        const uint32_t b3 = (a >> 3) & 0x01010101u;
        const uint32_t bm = (b3 << 8) - b3;
        const uint32_t sq = (sq_hi & bm) | (sq_lo & ~bm);
        s3 = __builtin_amdgcn_udot4(a, sq, s3, false);
        s4 = __builtin_amdgcn_udot4(sq, sq, s4, false);
        mask |= byte_bits4(((x >> 1) ^ pb) & 0x01010101u) << (4 * q);
        negm |= byte_bits4(sgn) << (4 * q);
        nzm |= byte_bits4(((a + 0x7f7f7f7fu) >> 7) & 0x01010101u) << (4 * q);
        sl[q] = (a >> 1) & 0x07070707u;   // slot selectors, resolved once the class is known
      }
      const uint32_t m = s2 >> 4;
      ok = ok && ((s2 & 15u) == 0u) && m >= 2u && m <= (uint32_t)max_shell && (((sum - 4 * (int)p) & 7) == 0);
      uint64_t I = ~0ull;
      if (ok) {
        const uint32_t key = s1 | (s3 << 6) | (s4 << 17);
        const uint32_t h = ((key ^ (p << 31)) * LLVQ_RANK_HASH_MULT) >> 20;
        const int k = (int)dev_tables::kRankHash[h] - 1;
        const uint32_t pos = dev_tables::kGolayInfoPos[(mask >> 11) & 0xfffu];
        ok = k >= 0 && dev_tables::kGolayTable[pos] == mask;
        if (ok) {
          const LlvqClassRank cr = dev_tables::kClassRank[k];
          const uint32_t meta = cr.meta;
          const uint32_t r = pos - cr.toff;
          ok = cr.key == key && ((meta >> 17) & 1u) == p && ((meta >> 20) & 15u) == m && r < cr.A;
          uint32_t bad = 0;
#pragma unroll
          for (int q = 0; q < 6; ++q) {
            sl[q] = __builtin_amdgcn_perm(cr.slot_hi, cr.slot_lo, sl[q]);
            bad |= sl[q];
          }
          ok = ok && (bad & 0x80808080u) == 0u;
          double R = 0.0;
          uint32_t s = 0;
          if (ok && p) {
            // odd class: one part of 24 values in position order
            uint32_t cnt = cr.cnt_t;
            uint32_t cum = (cnt << 8) + (cnt << 16) + (cnt << 24);
            double P = cr.p_t;
#pragma unroll
            for (int i = 0; i < 24; ++i) {
              const uint32_t sh = __builtin_amdgcn_ubfe(sl[i >> 2], 8 * (i & 3), 8) << 3;
              const double tq = P * (1.0 / (double)(24 - i));
              R += __builtin_rint(tq * (double)__builtin_amdgcn_ubfe(cum, sh, 8));
              P = __builtin_rint(tq * (double)__builtin_amdgcn_ubfe(cnt, sh, 8));
              cnt -= 1u << sh;
              cum -= 0x01010100u << sh;
            }
            ok = cnt == 0u;
          } else if (ok) {
            // even class: support part then complement part, positions from the masks
#pragma unroll
            for (int q = 0; q < 6; ++q) rows[6 * tid + q] = sl[q];
            const uint32_t wt = (meta >> 8) & 31u;
            uint32_t cnt = cr.cnt_s;
            uint32_t cum = (cnt << 8) + (cnt << 16) + (cnt << 24);
            double P = cr.p_s;
            double RS = 0.0;
            uint32_t ms = mask;
            for (uint32_t j = 0; j < wt; ++j) {
              const uint32_t ps = (uint32_t)__builtin_ctz(ms);
              ms &= ms - 1u;
              const uint32_t sh = (uint32_t)row[ps] << 3;
              const double tq = P * inv_n[wt - j];
              RS += __builtin_rint(tq * (double)__builtin_amdgcn_ubfe(cum, sh, 8));
              P = __builtin_rint(tq * (double)__builtin_amdgcn_ubfe(cnt, sh, 8));
              cnt -= 1u << sh;
              cum -= 0x01010100u << sh;
              if (j + 1u < wt) s |= ((negm >> ps) & 1u) << j;
            }
            ok = cnt == 0u;
            cnt = cr.cnt_t;
            cum = (cnt << 8) + (cnt << 16) + (cnt << 24);
            P = cr.p_t;
            double RT = 0.0;
            uint32_t mt = ~mask & 0xffffffu;
            uint32_t sb = wt ? wt - 1u : 0u;
            for (uint32_t j = 0; j < 24u - wt; ++j) {
              const uint32_t ps = (uint32_t)__builtin_ctz(mt);
              mt &= mt - 1u;
              const uint32_t sh = (uint32_t)row[ps] << 3;
              const double tq = P * inv_n[24u - wt - j];
              RT += __builtin_rint(tq * (double)__builtin_amdgcn_ubfe(cum, sh, 8));
              P = __builtin_rint(tq * (double)__builtin_amdgcn_ubfe(cnt, sh, 8));
              cnt -= 1u << sh;
              cum -= 0x01010100u << sh;
              const uint32_t nzb = (nzm >> ps) & 1u;
              s |= (((negm >> ps) & 1u) & nzb) << sb;
              sb += nzb;
            }
            ok = ok && cnt == 0u;
            R = __builtin_fma(RS, cr.p_t, RT);
          }
          if (ok) {
            const uint32_t B = meta & 31u;
            I = cr.start + (uint64_t)r + (uint64_t)cr.A * ((uint64_t)s + ((uint64_t)R << B));
          }
        }
      }
      out[t] = I;
      if (!ok && err) atomicAdd(err, 1);
    }
    __syncthreads();   // stage and wodd are rewritten by the next step
  }
}
