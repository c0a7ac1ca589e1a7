// Byte-tile decode of the tile engine (gfx950), used by the matrix-core GEMM: each
// block's 24 biased value bytes (12 + v) go into an LDS tile, odd blocks with 8-byte
// writes in position order, even blocks with byte writes at their positions; plus the
// bf16 pair packing and int8 unbiasing helpers shared with the streamed decode.
// Included once by llvq.hip after llvq_engine.h.

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
    OddDec<> od;
    od.init(h, bs);
    uint2* dst = reinterpret_cast<uint2*>(smem + tb + 24u * f);
    uint32_t w[6];
#pragma unroll
    for (int q = 0; q < 6; ++q) {   // four biased bytes per dword
      const uint32_t k0 = od.slot(smem, L, 4 * q);
      const uint32_t k1 = od.slot(smem, L, 4 * q + 1);
      const uint32_t k2 = od.slot(smem, L, 4 * q + 2);
      const uint32_t k3 = od.slot(smem, L, 4 * q + 3);
      w[q] = od.quad_codes(k0, k1, k2, k3, q);
      if (q & 1) dst[q >> 1] = make_uint2(w[q - 1], w[q]);
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
    const BlockStart bs = block_start<false, false>(smem, L, entry_J(ee), h);
    EvenDec<6, 1> ev;   // positions from the table
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
