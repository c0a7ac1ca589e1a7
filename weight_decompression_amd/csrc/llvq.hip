// LLVQ decode / fused dequant-GEMV / rank kernels for gfx950, and the C ABI around them.
//
// Method: "Leech Lattice Vector Quantization for Efficient LLM Compression"
// (papernotes.org notes, 方法详解 / 关键设计 2 for the index hierarchy and its
// div/mod inverse, 关键设计 4 for the fused kernel; gist.science summary, Methodik /
// 4. Dequantisierungskernel).  Conventions are those of include/llvq.h and of the table
// generator gen_tables.cpp.
//
// Decode of one 24-block (one lane):
//   field -> shape index I (and gain index g)
//   class k with start_k <= I < start_{k+1}: bucket table on the top bits of I, then a
//     short forward scan;
//   J = I - start_k;  r = J mod A,  I' = J div A,  s = I' mod 2^B,  R = I' div 2^B;
//   codeword c = T[toff + r];
//   R is the lexicographic rank of the absolute values.  It is unranked by exact
//     arithmetic decoding: u = (R + 1/2) / P and, at each of the 24 steps with n values
//     left and counts c_j, the value index is the number of cumulative counts
//     C_j <= u*n; then u <- (u*n - C_k) / c_k.  In fp64 the decision margins
//     (>= n/(2Q) with Q <= 4.2e8 arrangements left) dwarf the rounding error, so every
//     decision is exact.  Even classes run the support values (w steps) and then the
//     complement values on the same u; this reproduces I'' = rank_S * P_T + rank_T.
//   Values are placed in position order (support values on the codeword's positions,
//     complement values on the others) and signed: odd classes by the codeword and
//     |v| mod 4; even classes from the bits of s on the nonzero positions in ascending
//     order, except the highest codeword position, whose sign fixes the parity pi.

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <stddef.h>

#include <mutex>

#include "llvq.h"
#include "llvq_tables.h"

#define LLVQ_API extern "C" __attribute__((visibility("default")))

namespace host_tables {
#define LLVQ_TABLE static const
#include "llvq_tables.inc"
#undef LLVQ_TABLE
}  // namespace host_tables

namespace dev_tables {
#define LLVQ_TABLE __device__ const
#include "llvq_tables.inc"
#undef LLVQ_TABLE
}  // namespace dev_tables

// key order of the generated sorting network (floats, or unsigned integer keys)
__device__ __forceinline__ float llvq_kmin(float a, float b) { return __builtin_fminf(a, b); }
__device__ __forceinline__ float llvq_kmax(float a, float b) { return __builtin_fmaxf(a, b); }
__device__ __forceinline__ uint32_t llvq_kmin(uint32_t a, uint32_t b) { return a < b ? a : b; }
__device__ __forceinline__ uint32_t llvq_kmax(uint32_t a, uint32_t b) { return a < b ? b : a; }

// nearest-point search: sorting network, class records and per-class objectives
namespace dev_tables {
#define LLVQ_TABLE __device__ const
#include "llvq_search.inc"
#undef LLVQ_TABLE
}  // namespace dev_tables

// general decoder: shells 2..42, fields up to 128 bits (the class records on the device only)
namespace host_tables {
#define LLVQ_TABLE static const
#include "llvq_wide.inc"
#undef LLVQ_TABLE
}  // namespace host_tables
namespace dev_tables {
#define LLVQ_TABLE __device__ const
#define LLVQ_WIDE_CLASSES
#include "llvq_wide.inc"
#undef LLVQ_WIDE_CLASSES
#undef LLVQ_TABLE
}  // namespace dev_tables

// Device checks (build flag LLVQ_DEVICE_CHECKS): invariants the kernels rely on for their
// memory accesses and for exact decoding are tested in the kernels, and every failure adds
// one to a device counter that llvq_device_checks reads.  Nothing traps; a normal build
// compiles the checks away.
#ifdef LLVQ_DEVICE_CHECKS
__device__ unsigned int g_llvq_check_failures;
#define LLVQ_DCHECK(cond)                                               \
  do {                                                                  \
    if (!(cond)) atomicAdd(&g_llvq_check_failures, 1u);                 \
  } while (0)
#else
#define LLVQ_DCHECK(cond) \
  do {                    \
  } while (0)
#endif

namespace {

constexpr int kDim = 24;

struct KDesc {
  int32_t mode, rows, cols, kb;
  int32_t max_shell, shape_bits, gain_bits, field_bits;
  uint64_t index_count;
  uint64_t shape_mask;
  uint32_t shape_mask_lo, shape_mask_hi;
  int32_t ncls, bshift;
};

// ---------------------------------------------------------------------------
// device helpers

__device__ __forceinline__ uint64_t read_field(const uint8_t* __restrict__ packed, uint64_t j, int f) {
  const uint64_t bit = j * (uint64_t)f;
  const uint32_t* w = reinterpret_cast<const uint32_t*>(packed) + (bit >> 5);
  const uint32_t sh = (uint32_t)(bit & 31u);
  uint64_t v = ((uint64_t)w[0] | ((uint64_t)w[1] << 32)) >> sh;
  if (sh + (uint32_t)f > 64u) v |= (uint64_t)w[2] << (64u - sh);
  return f == 64 ? v : (v & ((1ull << f) - 1ull));
}

__device__ __forceinline__ int find_class(uint64_t I, const KDesc& d) {
  int k = dev_tables::kBucketTable[d.max_shell][(uint32_t)(I >> d.bshift)];
  while (k + 1 < d.ncls && I >= dev_tables::kClassTable[k + 1].start) ++k;
  return k;
}

// Integer lattice point of shape index I (class k already found).
__device__ __forceinline__ void decode_point(uint64_t I, int k, int v[kDim]) {
  const LlvqClassRec& cr = dev_tables::kClassTable[k];
  const uint64_t J = I - cr.start;
  const uint32_t A = cr.A;
  uint32_t r, ip;
  if (A == 4096u) {
    r = (uint32_t)J & 4095u;
    ip = (uint32_t)(J >> 12);
  } else if (A == 1u) {
    r = 0u;
    ip = (uint32_t)J;
  } else {
    // quotient < 2^32; fp64 estimate then one exact correction on the remainder
    uint32_t q = (uint32_t)((double)J / (double)A);
    int32_t rem = (int32_t)((uint32_t)J - q * A);
    if (rem < 0) {
      q -= 1u;
      rem += (int32_t)A;
    } else if (rem >= (int32_t)A) {
      q += 1u;
      rem -= (int32_t)A;
    }
    r = (uint32_t)rem;
    ip = q;
  }
  const uint32_t B = cr.B;
  const uint32_t s = ip & ((1u << B) - 1u);
  const uint32_t R = ip >> B;
  const uint32_t c = dev_tables::kGolayTable[cr.toff + r];
  const int w = cr.w;

  double u = ((double)R + 0.5) * cr.inv_p;
  uint32_t cnt = w ? cr.cnt_s : cr.cnt_t;
  uint64_t codes = 0;
#pragma unroll
  for (int i = 0; i < kDim; ++i) {
    if (i == w) cnt = cr.cnt_t;
    const int left = (i < w) ? (w - i) : (kDim - i);
    const double y = u * (double)left;
    const int c0 = cnt & 0xff, c1 = (cnt >> 8) & 0xff, c2 = (cnt >> 16) & 0xff, c3 = (int)(cnt >> 24);
    const int t1 = c0, t2 = t1 + c1, t3 = t2 + c2;
    const int kk = (y >= (double)t1) + (y >= (double)t2) + (y >= (double)t3);
    const int ck = kk == 0 ? c0 : kk == 1 ? c1 : kk == 2 ? c2 : c3;
    const int Ck = kk == 0 ? 0 : kk == 1 ? t1 : kk == 2 ? t2 : t3;
    u = (y - (double)Ck) / (double)ck;
    cnt -= 1u << (8 * kk);
    codes |= (uint64_t)kk << (2 * i);
  }

  // signs of even classes: bits 0..w-2 of s go to the support positions below q (the
  // highest support position) in ascending order, the following bits to the nonzero
  // complement positions in ascending order; q fixes the parity of support negatives
  const uint32_t sel = w ? c : 0u;
  uint64_t sS = codes;
  uint64_t sT = codes >> (2 * w);
  const int q = w ? (31 - __clz((int)c)) : -1;
  const uint32_t wm1 = w ? (uint32_t)(w - 1) : 0u;
  uint32_t bitsS = s;
  uint32_t bitsT = wm1 ? (s >> wm1) : s;
  const uint32_t negq = w ? (((uint32_t)__popc(s & ((1u << wm1) - 1u)) & 1u) ^ cr.pi) : 0u;
#pragma unroll
  for (int p = 0; p < kDim; ++p) {
    const bool inS = (sel >> p) & 1u;
    const uint32_t code = (uint32_t)(inS ? sS : sT) & 3u;
    if (inS)
      sS >>= 2;
    else
      sT >>= 2;
    const uint32_t vals = inS ? cr.vals_s : cr.vals_t;
    const int a = (int)((vals >> (8 * code)) & 0xffu);
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
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

#include "llvq_engine.h"
#include "llvq_gemv_b1.h"
#include "llvq_tile.h"
#include "llvq_gemm.h"
#include "llvq_stream.h"
#include "llvq_wide.h"
#include "llvq_wide_tile.h"

// ---------------------------------------------------------------------------
// kernels

__global__ __launch_bounds__(256) void k_decode_points(KDesc d, const uint8_t* __restrict__ packed,
                                                        int8_t* __restrict__ out, int32_t* err) {
  const uint64_t nblocks = (uint64_t)d.rows * (uint64_t)d.kb;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < nblocks; j += stride) {
    const uint64_t I = read_field(packed, j, d.field_bits) & d.shape_mask;
    int v[kDim];
    if (I < d.index_count) {
      decode_point(I, find_class(I, d), v);
    } else {
#pragma unroll
      for (int p = 0; p < kDim; ++p) v[p] = 0;
      if (err) atomicAdd(err, 1);
    }
    uint32_t* o = reinterpret_cast<uint32_t*>(out + j * kDim);
#pragma unroll
    for (int qd = 0; qd < kDim / 4; ++qd) {
      o[qd] = ((uint32_t)(v[4 * qd] & 0xff)) | ((uint32_t)(v[4 * qd + 1] & 0xff) << 8) |
              ((uint32_t)(v[4 * qd + 2] & 0xff) << 16) | ((uint32_t)(v[4 * qd + 3] & 0xff) << 24);
    }
  }
}

__global__ __launch_bounds__(256) void k_decode_bf16(KDesc d, const uint8_t* __restrict__ packed,
                                                      const __half* __restrict__ scales,
                                                      uint16_t* __restrict__ out, int32_t* err) {
  const uint64_t nblocks = (uint64_t)d.rows * (uint64_t)d.kb;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < nblocks; j += stride) {
    const uint64_t fld = read_field(packed, j, d.field_bits);
    const uint64_t I = fld & d.shape_mask;
    const uint32_t row = (uint32_t)(j / (uint64_t)d.kb);
    const uint32_t blk = (uint32_t)(j - (uint64_t)row * d.kb);
    int v[kDim];
    float scale = 0.0f;
    if (I < d.index_count) {
      const int k = find_class(I, d);
      decode_point(I, k, v);
      if (d.mode == LLVQ_MODE_SHAPEGAIN) {
        const uint32_t g = (uint32_t)(fld >> d.shape_bits);
        scale = __fmul_rn(__half2float(scales[g]), dev_tables::kInvNorm32[dev_tables::kClassTable[k].m]);
      } else {
        scale = __half2float(scales[row]);
      }
    } else {
#pragma unroll
      for (int p = 0; p < kDim; ++p) v[p] = 0;
      if (err) atomicAdd(err, 1);
    }
    uint16_t* o = out + (uint64_t)row * d.cols + (uint64_t)blk * kDim;
    const int lim = d.cols - (int)blk * kDim;
#pragma unroll
    for (int p = 0; p < kDim; ++p)
      if (p < lim) o[p] = f32_to_bf16_rne(__fmul_rn((float)v[p], scale));
  }
}

template <int BATCH, bool XBF16>
__global__ __launch_bounds__(256) void k_gemv(KDesc d, const uint8_t* __restrict__ packed,
                                               const __half* __restrict__ scales, const void* __restrict__ xv,
                                               float* __restrict__ y, int32_t* err) {
  const int lane = threadIdx.x & 63;
  const int wave = (int)((blockIdx.x * blockDim.x + threadIdx.x) >> 6);
  const int nwaves = (int)((gridDim.x * blockDim.x) >> 6);
  const float* xf = reinterpret_cast<const float*>(xv);
  const uint16_t* xb = reinterpret_cast<const uint16_t*>(xv);
  for (int r = wave; r < d.rows; r += nwaves) {
    float acc[BATCH];
#pragma unroll
    for (int bb = 0; bb < BATCH; ++bb) acc[bb] = 0.0f;
    for (int blk = lane; blk < d.kb; blk += 64) {
      const uint64_t j = (uint64_t)r * d.kb + blk;
      const uint64_t fld = read_field(packed, j, d.field_bits);
      const uint64_t I = fld & d.shape_mask;
      if (I >= d.index_count) {
        if (err) atomicAdd(err, 1);
        continue;
      }
      const int k = find_class(I, d);
      int v[kDim];
      decode_point(I, k, v);
      float scale = 1.0f;
      if (d.mode == LLVQ_MODE_SHAPEGAIN) {
        const uint32_t g = (uint32_t)(fld >> d.shape_bits);
        scale = __half2float(scales[g]) * dev_tables::kInvNorm32[dev_tables::kClassTable[k].m];
      }
      const int col0 = blk * kDim;
      const int lim = d.cols - col0;
#pragma unroll
      for (int bb = 0; bb < BATCH; ++bb) {
        float dot = 0.0f;
#pragma unroll
        for (int p = 0; p < kDim; ++p) {
          if (p < lim) {
            const uint64_t xi = (uint64_t)bb * d.cols + col0 + p;
            const float xval = XBF16 ? bf16_to_f32(xb[xi]) : xf[xi];
            dot = fmaf((float)v[p], xval, dot);
          }
        }
        acc[bb] = fmaf(scale, dot, acc[bb]);
      }
    }
#pragma unroll
    for (int bb = 0; bb < BATCH; ++bb) {
      float t = acc[bb];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) t += __shfl_xor(t, off, 64);
      acc[bb] = t;
    }
    if (lane == 0) {
      const float rs = d.mode == LLVQ_MODE_SHAPEGAIN ? 1.0f : __half2float(scales[r]);
#pragma unroll
      for (int bb = 0; bb < BATCH; ++bb) y[(uint64_t)bb * d.rows + r] = acc[bb] * rs;
    }
  }
}

#include "llvq_rank.h"
#include "llvq_search.h"
#include "llvq_gptq.h"

// ---------------------------------------------------------------------------
// host side

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int make_kdesc(const llvq_desc* d, KDesc* k) {
  if (!d) return LLVQ_EINVAL;
  if (d->mode != LLVQ_MODE_EUCLID && d->mode != LLVQ_MODE_SHAPEGAIN) return LLVQ_EINVAL;
  if (d->rows <= 0 || d->cols <= 0) return LLVQ_EINVAL;
  if (d->max_shell < 2 || d->max_shell > LLVQ_MAX_SHELL) return LLVQ_EINVAL;
  if (d->shape_bits < 1 || d->shape_bits > 60) return LLVQ_EINVAL;
  if (d->mode == LLVQ_MODE_EUCLID && d->gain_bits != 0) return LLVQ_EINVAL;
  if (d->mode == LLVQ_MODE_SHAPEGAIN && (d->gain_bits < 1 || d->gain_bits > 8)) return LLVQ_EINVAL;
  if (d->shape_bits + d->gain_bits > 64) return LLVQ_EINVAL;
  const uint64_t count = host_tables::kIndexCount[d->max_shell];
  if (d->shape_bits < 64 && count > (1ull << d->shape_bits)) return LLVQ_EINVAL;
  k->mode = d->mode;
  k->rows = d->rows;
  k->cols = d->cols;
  k->kb = (d->cols + kDim - 1) / kDim;
  k->max_shell = d->max_shell;
  k->shape_bits = d->shape_bits;
  k->gain_bits = d->gain_bits;
  k->field_bits = d->shape_bits + d->gain_bits;
  k->index_count = count;
  k->shape_mask = (1ull << d->shape_bits) - 1ull;
  k->shape_mask_lo = (uint32_t)k->shape_mask;
  k->shape_mask_hi = (uint32_t)(k->shape_mask >> 32);
  k->ncls = host_tables::kNumClassesUpTo[d->max_shell];
  k->bshift = host_tables::kBucketShift[d->max_shell];
  return LLVQ_OK;
}

// Descriptors beyond the 2-bit kernels' range: shells past 10 or fields past 64 bits.
bool wide_needed(const llvq_desc* d) {
  return d->max_shell > LLVQ_MAX_SHELL || d->shape_bits > 60 || d->shape_bits + d->gain_bits > 64;
}

int make_wdesc(const llvq_desc* d, WDesc* w) {
  if (!d) return LLVQ_EINVAL;
  if (d->mode != LLVQ_MODE_EUCLID && d->mode != LLVQ_MODE_SHAPEGAIN) return LLVQ_EINVAL;
  if (d->rows <= 0 || d->cols <= 0) return LLVQ_EINVAL;
  if (d->max_shell < 2 || d->max_shell > LLVQ_WIDE_MAX_SHELL) return LLVQ_EINVAL;
  if (d->shape_bits < 1 || d->shape_bits > 120) return LLVQ_EINVAL;
  if (d->mode == LLVQ_MODE_EUCLID && d->gain_bits != 0) return LLVQ_EINVAL;
  if (d->mode == LLVQ_MODE_SHAPEGAIN && (d->gain_bits < 1 || d->gain_bits > 8)) return LLVQ_EINVAL;
  const uint64_t clo = host_tables::kWideShellStart[d->max_shell + 1][0];
  const uint64_t chi = host_tables::kWideShellStart[d->max_shell + 1][1];
  // index count <= 2^shape_bits
  if (d->shape_bits < 64) {
    if (chi != 0 || clo > (1ull << d->shape_bits)) return LLVQ_EINVAL;
  } else if (d->shape_bits < 128) {
    const int hb = d->shape_bits - 64;
    if (chi > (1ull << hb) || (chi == (1ull << hb) && clo != 0)) return LLVQ_EINVAL;
  }
  w->mode = d->mode;
  w->rows = d->rows;
  w->cols = d->cols;
  w->kb = (d->cols + kDim - 1) / kDim;
  w->max_shell = d->max_shell;
  w->shape_bits = d->shape_bits;
  w->gain_bits = d->gain_bits;
  w->field_bits = d->shape_bits + d->gain_bits;
  w->count_lo = clo;
  w->count_hi = chi;
  return LLVQ_OK;
}

// make_kdesc for the calls that only run the 2-bit kernels: a descriptor that only the
// general decoder takes is LLVQ_EUNSUPPORTED there
int make_kdesc_narrow(const llvq_desc* d, KDesc* k) {
  const int st = make_kdesc(d, k);
  if (st == LLVQ_EINVAL && d && wide_needed(d)) {
    WDesc w;
    if (make_wdesc(d, &w) == LLVQ_OK) return LLVQ_EUNSUPPORTED;
  }
  return st;
}

int64_t packed_bytes_of(const KDesc& k) {
  const uint64_t nbits = (uint64_t)k.rows * (uint64_t)k.kb * (uint64_t)k.field_bits;
  uint64_t nbytes = (nbits + 7) / 8;
  nbytes = (nbytes + 15) / 16 * 16;
  return (int64_t)(nbytes + 16);
}

unsigned grid_for(uint64_t work_items, unsigned block) {
  uint64_t g = (work_items + block - 1) / block;
  if (g < 1) g = 1;
  if (g > 65536) g = 65536;
  return (unsigned)g;
}

int launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? LLVQ_OK : LLVQ_EHIP;
}

}  // namespace

LLVQ_API int llvq_index_count(int32_t max_shell, uint64_t* out) {
  if (!out || max_shell < 2 || max_shell > LLVQ_MAX_SHELL) return LLVQ_EINVAL;
  *out = host_tables::kIndexCount[max_shell];
  return LLVQ_OK;
}

LLVQ_API int llvq_index_count_wide(int32_t max_shell, uint64_t* lo, uint64_t* hi) {
  if (!lo || !hi || max_shell < 2 || max_shell > LLVQ_WIDE_MAX_SHELL) return LLVQ_EINVAL;
  *lo = host_tables::kWideShellStart[max_shell + 1][0];
  *hi = host_tables::kWideShellStart[max_shell + 1][1];
  return LLVQ_OK;
}

LLVQ_API int64_t llvq_packed_bytes(const llvq_desc* d) {
  if (d && wide_needed(d)) {
    WDesc w;
    const int st = make_wdesc(d, &w);
    if (st != LLVQ_OK) return st;
    KDesc k = {};
    k.rows = w.rows;
    k.kb = w.kb;
    k.field_bits = w.field_bits;
    return packed_bytes_of(k);
  }
  KDesc k;
  const int st = make_kdesc(d, &k);
  if (st != LLVQ_OK) return st;
  return packed_bytes_of(k);
}

LLVQ_API const char* llvq_error_string(int code) {
  switch (code) {
    case LLVQ_OK: return "ok";
    case LLVQ_EINVAL: return "invalid argument";
    case LLVQ_EUNSUPPORTED: return "unsupported request";
    case LLVQ_EHIP: return "HIP launch error";
    case LLVQ_ETOOLARGE: return "request larger than the library's fixed workspace (llvq_quantize_noalloc)";
    default: return "unknown error code";
  }
}

static_assert(sizeof(LlvqClassHot) == 96, "hot class record: six 16-byte rows");
static_assert(offsetof(LlvqClassHot, nc1) == 64 && offsetof(LlvqClassHot, sv1lo8) == 88,
              "the even decoder reads part 1 at these offsets");

namespace {
// Per-device launch limits of the one-workgroup-per-CU kernels: the workgroups of a grid
// (one per CU) and the LDS of one workgroup (at most 160 KB, the gfx950 figure the tiles are
// sized for).  Queried once per device and kept.
struct DevLimits {
  uint32_t lds;
  int grid;
};
constexpr int kMaxLimitDevices = 64;
std::mutex g_limits_mu;
DevLimits g_limits[kMaxLimitDevices];

DevLimits device_limits(hipStream_t stream) {
  DevLimits l = {160u * 1024u, 256};
  int dev = -1;
  // (a failed query leaves its error pending, so the call's launch status reports it; a
  // caller's pending error is not cleared here either)
  if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= kMaxLimitDevices) return l;
  std::lock_guard<std::mutex> lock(g_limits_mu);
  if (g_limits[dev].grid == 0) {
    int cus = 0, lds = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0) l.grid = cus;
    if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess && lds > 0 &&
        (uint32_t)lds < l.lds)
      l.lds = (uint32_t)lds;
    g_limits[dev] = l;
  }
  return g_limits[dev];
}

// Rows per tile for the engine kernels: among the R with R * Kb <= tmax, the one that
// minimises the work of the busiest workgroup, counting each tile as its blocks plus a
// fixed overhead of kTileOverhead blocks (a tile's first classify unit and its last,
// partly filled chunks leave waves idle).  Ties go to larger tiles.
constexpr long kTileOverhead = 1024;

int pick_rows_per_tile(int rows, int kb, int tmax, int gmax, int* ntiles_out, int* grid_out) {
  int rmax = tmax / kb;
  if (rmax > rows) rmax = rows;
  if (rmax < 1) return 0;
  int best_r = 0;
  long best_cost = -1;
  for (int r = rmax; r >= 1; --r) {
    const long nt = (rows + r - 1) / r;
    const long g = nt < gmax ? nt : gmax;
    const long cost = ((nt + g - 1) / g) * ((long)r * kb + kTileOverhead);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best_r = r;
    }
  }
  const int nt = (rows + best_r - 1) / best_r;
  *ntiles_out = nt;
  *grid_out = nt < gmax ? nt : gmax;
  return best_r;
}

// Batch-1 fused GEMV (llvq_gemv_b1.h) with a TAIL-value tail table.  Returns
// LLVQ_EUNSUPPORTED when the shape does not fit its tiling.
template <int TAIL>
int launch_gemv_b1_tail(const KDesc& k, const void* packed, const void* scales, const void* x, int32_t x_dtype,
                        float* y, int32_t* err, hipStream_t s) {
  const DevLimits lim = device_limits(s);
  const uint32_t lds = lim.lds;
  const int gmax = lim.grid;
  if ((uint64_t)k.rows * (uint64_t)k.kb >= (1ull << 30)) return LLVQ_EUNSUPPORTED;   // 32-bit field index
  const bool xf32 = x_dtype == LLVQ_X_F32;
  const int nbuckets = (int)(((host_tables::kIndexCount[k.max_shell] - 1) >> k.bshift) + 1);
  // LDS: fixed tables, the waves' rings, 4 bytes per block of the tile (its slot), x
  ELayout L;
  const uint32_t xbytes = align16((uint32_t)k.kb * 24u * (xf32 ? 4u : 2u));
  const uint32_t base = engine_layout_base(L, k.ncls, 1 << k.gain_bits, nbuckets, 0, 1, TAIL);
  const uint32_t fixed = base + (uint32_t)kRingBytes + xbytes + 16u;
  if (fixed + 4u * (uint32_t)k.kb > lds) return LLVQ_EUNSUPPORTED;
  int tmax = (int)((lds - fixed) / 4u);
  if (tmax > kETileMax) tmax = kETileMax;
  EArgs a = {};
  int grid = 0;
  // every workgroup's rows as one tile when they fit, else the cost-model tiling
  const int r1 = (k.rows + gmax - 1) / gmax;
  if ((long)r1 * k.kb <= tmax) {
    a.rows_per_tile = r1;
    a.ntiles = (k.rows + r1 - 1) / r1;
    grid = a.ntiles;
  } else {
    int nt = 0, g = 0;
    const int r = pick_rows_per_tile(k.rows, k.kb, tmax, gmax, &nt, &g);
    if (r == 0) return LLVQ_EUNSUPPORTED;
    a.rows_per_tile = r;
    a.ntiles = nt;
    grid = g;
  }
  a.nbuckets = nbuckets;
  engine_layout_base(a.L, k.ncls, 1 << k.gain_bits, nbuckets, 0, 1, TAIL);
  a.rings = align16(a.L.total);
  a.L.buf[0].part = a.rings + (uint32_t)kRingBytes;
  a.xs = align16(a.L.buf[0].part + 4u * (uint32_t)(a.rows_per_tile * k.kb));
  const uint32_t total = a.xs + align16((uint32_t)k.kb * 24u * (xf32 ? 4u : 2u));
  if (total > lds) return LLVQ_EUNSUPPORTED;
  if (xf32)
    hipLaunchKernelGGL((k_gemv_b1<true, TAIL>), dim3(grid), dim3(kEThreads), total, s, k, a,
                       static_cast<const uint8_t*>(packed), static_cast<const __half*>(scales), x, y, err);
  else
    hipLaunchKernelGGL((k_gemv_b1<false, TAIL>), dim3(grid), dim3(kEThreads), total, s, k, a,
                       static_cast<const uint8_t*>(packed), static_cast<const __half*>(scales), x, y, err);
  return launch_status();
}

// Batch-1 fused GEMV: the 7-value tail (one arithmetic-decoding step less per block) when
// its 25 KB of extra tables fit beside the activations, else the 6-value tail.
// LLVQ_EUNSUPPORTED when neither fits (the generic kernel then runs).
int launch_gemv_b1(const KDesc& k, const void* packed, const void* scales, const void* x, int32_t x_dtype,
                   float* y, int32_t* err, hipStream_t s) {
  const int st = launch_gemv_b1_tail<7>(k, packed, scales, x, x_dtype, y, err, s);
  if (st != LLVQ_EUNSUPPORTED) return st;
  return launch_gemv_b1_tail<6>(k, packed, scales, x, x_dtype, y, err, s);
}

// Streamed decode of one or several tensors (llvq_stream.h): LDS holds the tables (with
// the Golay table), the waves' rings, the lanes' 24-byte value slots and 4 bytes per
// block of a tile.
// LLVQ_EUNSUPPORTED when a row does not fit a tile (the caller then falls back).
int launch_decode_stream(const KDesc* k, int n, const void* const* packed, const void* const* scales,
                         int32_t out_kind, void* const* outs, int32_t* err, hipStream_t s) {
  const DevLimits lim = device_limits(s);
  const uint32_t lds = lim.lds;
  const int gmax = lim.grid;
  const KDesc& k0 = k[0];
  const int nbuckets = (int)(((host_tables::kIndexCount[k0.max_shell] - 1) >> k0.bshift) + 1);
  const int ng = (k0.mode == LLVQ_MODE_SHAPEGAIN ? 1 << k0.gain_bits : 1) * n;
  SArgs m = {};
  const uint32_t base = engine_layout_base(m.L, k0.ncls, ng, nbuckets, 0, 1);
  m.L.golay = align16(base);
  m.rings = m.L.golay + 4096u * 4u;
  m.part = m.rings + (uint32_t)kRingBytes;
  const uint32_t fixed = m.part + (uint32_t)kStageBytes + 32u;
  if (fixed >= lds) return LLVQ_EUNSUPPORTED;
  int tmax = (int)((lds - fixed) / 4u) & ~15;
  if (tmax > kETileMax) tmax = kETileMax;
  m.tmax = tmax;
  m.stage = align16(m.part + 4u * (uint32_t)tmax);
  const uint32_t total = m.stage + (uint32_t)kStageBytes;
  if (total > lds) return LLVQ_EUNSUPPORTED;
  m.nbuckets = nbuckets;
  m.n = n;
  long long blocks = 0;
  for (int i = 0; i < n; ++i) {
    if (k[i].kb > tmax || (uint64_t)k[i].rows * (uint64_t)k[i].kb >= (1ull << 30)) return LLVQ_EUNSUPPORTED;
    STensor& t = m.t[i];
    t.packed = static_cast<const uint8_t*>(packed[i]);
    t.scales = scales ? static_cast<const __half*>(scales[i]) : nullptr;
    t.out = outs[i];
    t.rows = k[i].rows;
    t.cols = k[i].cols;
    t.kb = k[i].kb;
    t.blk0 = blocks;
    blocks += (long long)k[i].rows * k[i].kb;
  }
  m.total = blocks;
  // at least ~2K blocks per workgroup, at most one workgroup per CU
  long long g = (blocks + 2047) / 2048;
  if (g > gmax) g = gmax;
  if (g < 1) g = 1;
  if (out_kind == LLVQ_OUT_POINTS_I8)
    hipLaunchKernelGGL((k_decode_stream<LLVQ_OUT_POINTS_I8>), dim3((unsigned)g), dim3(kEThreads), total, s, k0, m,
                       err);
  else
    hipLaunchKernelGGL((k_decode_stream<LLVQ_OUT_BF16>), dim3((unsigned)g), dim3(kEThreads), total, s, k0, m, err);
  return launch_status();
}

// Small-batch GEMM on matrix cores (llvq_gemm.h), bf16 activations, batch 2..16.
// LLVQ_EUNSUPPORTED when the shape does not fit (the VALU kernel then runs).
int launch_gemm_mfma(const KDesc& k, const void* packed, const void* scales, const void* x, int batch, float* y,
                     int32_t* err, hipStream_t s) {
  const DevLimits lim = device_limits(s);
  const uint32_t lds = lim.lds;
  const int gmax = lim.grid;
  if ((uint64_t)k.rows * (uint64_t)k.kb >= (1ull << 30)) return LLVQ_EUNSUPPORTED;
  // the activations are addressed with 32-bit buffer offsets (bit 31 marks "no data")
  if ((uint64_t)batch * (uint64_t)k.cols * 2u + 8192u >= (1ull << 31)) return LLVQ_EUNSUPPORTED;
  const int nbuckets = (int)(((host_tables::kIndexCount[k.max_shell] - 1) >> k.bshift) + 1);
  ELayout L;
  const uint32_t base = engine_layout_base(L, k.ncls, 1 << k.gain_bits, nbuckets, 0);
  const uint32_t red = (uint32_t)kEWaves * 64u * 4u * 4u;   // reduction buffer, over the byte tile
  // per block: queue entry 8 B + two block scales 8 B + 24 value bytes; at least one
  // block column; slack for the alignment of the three arrays
  if (base + 64u + 40u * kGRows > lds) return LLVQ_EUNSUPPORTED;
  int tmax = (int)((lds - base - 64u) / 40u);
  if (tmax > kETileMax) tmax = kETileMax;
  // chunks of at most kEWaves units of kEUnit blocks: one classification unit per wave
  const int wmax = min(tmax / kGRows, kEWaves * kEUnit / kGRows);
  GArgs g = {};
  g.nchunk = (k.kb + wmax - 1) / wmax;
  g.w = (k.kb + g.nchunk - 1) / g.nchunk;
  g.ngroups = (k.rows + kGRows - 1) / kGRows;
  g.batch = batch;
  g.rbal = 24;   // measured on 28672 x 8192, batch 2..16 (a unit classifies 256 blocks)
  g.e.rows_per_tile = kGRows;
  g.e.ntiles = g.ngroups;
  g.e.nbuckets = nbuckets;
  const uint32_t T = (uint32_t)(kGRows * g.w);
  engine_layout_base(g.e.L, k.ncls, 1 << k.gain_bits, nbuckets, (int)T);
  g.part2 = g.e.L.total;
  g.e.xs = g.part2 + align16(4u * T);
  g.e.xsum = g.e.xs;
  // (16 bytes past the tile: the k 24..31 lanes of the last block read 8 bytes beyond it)
  const uint32_t tile = align16(24u * T) + 16u;
  const uint32_t total = g.e.xs + (tile > red ? tile : red);
  if (total > lds) return LLVQ_EUNSUPPORTED;
  const int grid = g.ngroups < gmax ? g.ngroups : gmax;
  hipLaunchKernelGGL(k_gemm_mfma, dim3(grid), dim3(kEThreads), total, s, k, g, static_cast<const uint8_t*>(packed),
                     static_cast<const __half*>(scales), static_cast<const uint16_t*>(x), y, err);
  return launch_status();
}

template <int BATCH>
int launch_gemv(const KDesc& k, const void* packed, const void* scales, const void* x, int32_t x_dtype, float* y,
                int32_t* err, hipStream_t s) {
  const unsigned block = 256;
  const unsigned waves_per_block = block / 64;
  unsigned grid = (unsigned)((k.rows + waves_per_block - 1) / waves_per_block);
  if (grid > 8192) grid = 8192;
  if (x_dtype == LLVQ_X_BF16)
    hipLaunchKernelGGL((k_gemv<BATCH, true>), dim3(grid), dim3(block), 0, s, k, static_cast<const uint8_t*>(packed),
                       static_cast<const __half*>(scales), x, y, err);
  else
    hipLaunchKernelGGL((k_gemv<BATCH, false>), dim3(grid), dim3(block), 0, s, k, static_cast<const uint8_t*>(packed),
                       static_cast<const __half*>(scales), x, y, err);
  return launch_status();
}
}  // namespace

namespace {
// General decoder (llvq_wide.h): one 24-block per lane.
int launch_decode_wide_tile(const WDesc& w, const void* packed, const void* scales, int32_t out_kind, void* out,
                            int32_t* err, bool ovec, hipStream_t s);

int decode_wide(const llvq_desc* d, const void* packed, const void* scales, int32_t out_kind, void* out,
                int32_t* err_count, void* stream) {
  WDesc w;
  const int st = make_wdesc(d, &w);
  if (st != LLVQ_OK) return st;
  if (!packed || !out || !aligned(packed, 16)) return LLVQ_EINVAL;
  if (err_count && !aligned(err_count, 4)) return LLVQ_EINVAL;
  if (out_kind == LLVQ_OUT_POINTS_I8) {
    if (!aligned(out, 4)) return LLVQ_EINVAL;
  } else if (out_kind == LLVQ_OUT_BF16) {
    if (!scales || !aligned(out, 2) || !aligned(scales, 2)) return LLVQ_EINVAL;
  } else {
    return LLVQ_EINVAL;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const uint64_t nblocks = (uint64_t)w.rows * (uint64_t)w.kb;
  const unsigned grid = grid_for(nblocks, kWideThreads);
  const bool ovec = aligned(out, 16) && (w.cols % 8) == 0;
  const int st1 = launch_decode_wide_tile(w, packed, out_kind == LLVQ_OUT_BF16 ? scales : nullptr, out_kind, out,
                                          err_count, out_kind == LLVQ_OUT_POINTS_I8 ? aligned(out, 8) : ovec, s);
  if (st1 != LLVQ_EUNSUPPORTED) return st1;
  if (out_kind == LLVQ_OUT_POINTS_I8)
    hipLaunchKernelGGL((k_decode_wide<LLVQ_OUT_POINTS_I8>), dim3(grid), dim3(kWideThreads), 0, s, w,
                       static_cast<const uint8_t*>(packed), nullptr, out, err_count, false);
  else
    hipLaunchKernelGGL((k_decode_wide<LLVQ_OUT_BF16>), dim3(grid), dim3(kWideThreads), 0, s, w,
                       static_cast<const uint8_t*>(packed), static_cast<const __half*>(scales), out, err_count,
                       ovec);
  return launch_status();
}

// Batch-1 GEMV of the general decoder with coset queues (llvq_wide_tile.h): LDS holds x
// of all columns, the reciprocals, the waves' rings (12 bytes an entry) and 4 bytes per
// block of a tile.  LLVQ_EUNSUPPORTED when x or a row does not fit (the
// one-block-per-lane kernel then runs).
int launch_gemv_wide_tile(const WDesc& w, const void* packed, const void* scales, const void* x, int32_t x_dtype,
                          float* y, int32_t* err, hipStream_t s) {
  const DevLimits lim = device_limits(s);
  const uint32_t lds = lim.lds;
  const int gmax = lim.grid;
  if ((uint64_t)w.rows * (uint64_t)w.kb >= (1ull << 31)) return LLVQ_EUNSUPPORTED;
  const bool xbf16 = x_dtype == LLVQ_X_BF16;
  WTArgs a = {};
  a.xs = 0;
  a.rc = align16((uint32_t)w.kb * 24u * (xbf16 ? 2u : 4u));
  a.ctr = a.rc + 32u * 8u;
  a.qj = align16(a.ctr + 16u);
  a.qk = a.qj + 8u * (uint32_t)kWRingEntries;
  a.part = align16(a.qk + 4u * (uint32_t)kWRingEntries);
  const uint32_t fixed = a.part + 64u;
  if (fixed >= lds) return LLVQ_EUNSUPPORTED;
  int tmax = (int)((lds - a.part) / 4u) & ~15;
  if (tmax > kWTTileMax) tmax = kWTTileMax;
  if (w.kb > tmax) return LLVQ_EUNSUPPORTED;
  a.tmax = tmax;
  int grid = 0;
  const int r1 = (w.rows + gmax - 1) / gmax;
  if ((long)r1 * w.kb <= tmax) {
    a.rows_per_tile = r1;
    a.ntiles = (w.rows + r1 - 1) / r1;
    grid = a.ntiles;
  } else {
    int nt = 0, g = 0;
    const int r = pick_rows_per_tile(w.rows, w.kb, tmax, gmax, &nt, &g);
    if (r == 0) return LLVQ_EUNSUPPORTED;
    a.rows_per_tile = r;
    a.ntiles = nt;
    grid = g;
  }
  const uint32_t T = (uint32_t)(a.rows_per_tile * w.kb);
  const uint32_t total = a.part + 4u * T;
  if (total > lds) return LLVQ_EUNSUPPORTED;
  const uint8_t* pk = static_cast<const uint8_t*>(packed);
  const __half* sc = static_cast<const __half*>(scales);
  if (xbf16)
    hipLaunchKernelGGL((k_gemv_wide_tile<true>), dim3(grid), dim3(kWTThreads), total, s, w, a, pk, sc, x, y, err);
  else
    hipLaunchKernelGGL((k_gemv_wide_tile<false>), dim3(grid), dim3(kWTThreads), total, s, w, a, pk, sc, x, y, err);
  return launch_status();
}

// Decode of the general decoder with coset queues (llvq_wide_tile.h): LDS holds the
// reciprocals, the waves' rings and 28 bytes per block of a tile (scale, 24 value bytes).
// LLVQ_EUNSUPPORTED when a row does not fit (the one-block-per-lane kernel then runs).
int launch_decode_wide_tile(const WDesc& w, const void* packed, const void* scales, int32_t out_kind, void* out,
                            int32_t* err, bool ovec, hipStream_t s) {
  const DevLimits lim = device_limits(s);
  const uint32_t lds = lim.lds;
  const int gmax = lim.grid;
  if ((uint64_t)w.rows * (uint64_t)w.kb >= (1ull << 31)) return LLVQ_EUNSUPPORTED;
  WTArgs a = {};
  a.rc = 0;
  a.ctr = 32u * 8u;
  a.qj = align16(a.ctr + 16u);
  a.qk = a.qj + 8u * (uint32_t)kWRingEntries;
  a.part = align16(a.qk + 4u * (uint32_t)kWRingEntries);
  const uint32_t fixed = a.part + 64u;
  if (fixed >= lds) return LLVQ_EUNSUPPORTED;
  int tmax = (int)((lds - a.part - 16u) / 28u) & ~15;
  if (tmax > kWTTileMax) tmax = kWTTileMax;
  if (w.kb > tmax) return LLVQ_EUNSUPPORTED;
  a.tmax = tmax;
  int grid = 0;
  const int r1 = (w.rows + gmax - 1) / gmax;
  if ((long)r1 * w.kb <= tmax) {
    a.rows_per_tile = r1;
    a.ntiles = (w.rows + r1 - 1) / r1;
    grid = a.ntiles;
  } else {
    int nt = 0, g = 0;
    const int r = pick_rows_per_tile(w.rows, w.kb, tmax, gmax, &nt, &g);
    if (r == 0) return LLVQ_EUNSUPPORTED;
    a.rows_per_tile = r;
    a.ntiles = nt;
    grid = g;
  }
  const uint32_t T = (uint32_t)(a.rows_per_tile * w.kb);
  a.xs = align16(a.part + 4u * T);        // the value tile, 24 bytes per block
  const uint32_t total = a.xs + 24u * T;
  if (total > lds) return LLVQ_EUNSUPPORTED;
  const uint8_t* pk = static_cast<const uint8_t*>(packed);
  const __half* sc = static_cast<const __half*>(scales);
  if (out_kind == LLVQ_OUT_POINTS_I8)
    hipLaunchKernelGGL((k_decode_wide_tile<LLVQ_OUT_POINTS_I8>), dim3(grid), dim3(kWTThreads), total, s, w, a, pk,
                       sc, out, err, ovec);
  else
    hipLaunchKernelGGL((k_decode_wide_tile<LLVQ_OUT_BF16>), dim3(grid), dim3(kWTThreads), total, s, w, a, pk, sc,
                       out, err, ovec);
  return launch_status();
}

int gemv_wide(const llvq_desc* d, const void* packed, const void* scales, const void* x, int32_t x_dtype,
              int32_t batch, float* y, int32_t* err_count, void* stream) {
  WDesc w;
  const int st = make_wdesc(d, &w);
  if (st != LLVQ_OK) return st;
  if (!packed || !scales || !x || !y) return LLVQ_EINVAL;
  if (!aligned(packed, 16) || !aligned(scales, 2) || !aligned(y, 4)) return LLVQ_EINVAL;
  if (err_count && !aligned(err_count, 4)) return LLVQ_EINVAL;
  if (x_dtype == LLVQ_X_F32) {
    if (!aligned(x, 4)) return LLVQ_EINVAL;
  } else if (x_dtype == LLVQ_X_BF16) {
    if (!aligned(x, 2)) return LLVQ_EINVAL;
  } else {
    return LLVQ_EINVAL;
  }
  if (batch < 1 || batch > LLVQ_MAX_BATCH) return LLVQ_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (batch == 1) {
    const int st1 = launch_gemv_wide_tile(w, packed, scales, x, x_dtype, y, err_count, s);
    if (st1 != LLVQ_EUNSUPPORTED) return st1;
  }
  const unsigned grid = grid_for((uint64_t)w.rows, kWideThreads / 64);
  const int xbytes = x_dtype == LLVQ_X_BF16 ? 2 : 4;
  const bool xvec = aligned(x, 16) && ((uint64_t)w.cols * (uint64_t)xbytes) % 16u == 0;
  const uint8_t* pk = static_cast<const uint8_t*>(packed);
  const __half* sc = static_cast<const __half*>(scales);
  const dim3 g(grid), t(kWideThreads);
  if (x_dtype == LLVQ_X_BF16) {
    if (batch == 1)
      hipLaunchKernelGGL((k_gemv_wide<true, 1>), g, t, 0, s, w, pk, sc, x, batch, xvec, y, err_count);
    else
      hipLaunchKernelGGL((k_gemv_wide<true, LLVQ_MAX_BATCH>), g, t, 0, s, w, pk, sc, x, batch, xvec, y, err_count);
  } else {
    if (batch == 1)
      hipLaunchKernelGGL((k_gemv_wide<false, 1>), g, t, 0, s, w, pk, sc, x, batch, xvec, y, err_count);
    else
      hipLaunchKernelGGL((k_gemv_wide<false, LLVQ_MAX_BATCH>), g, t, 0, s, w, pk, sc, x, batch, xvec, y, err_count);
  }
  return launch_status();
}
}  // namespace

LLVQ_API int llvq_decode(const llvq_desc* d, const void* packed, const void* scales, int32_t out_kind,
                         void* out, int32_t* err_count, void* stream) {
  if (d && wide_needed(d)) return decode_wide(d, packed, scales, out_kind, out, err_count, stream);
  KDesc k;
  int st = make_kdesc(d, &k);
  if (st != LLVQ_OK) return st;
  if (!packed || !out || !aligned(packed, 16)) return LLVQ_EINVAL;
  if (err_count && !aligned(err_count, 4)) return LLVQ_EINVAL;
  if (out_kind == LLVQ_OUT_POINTS_I8) {
    if (!aligned(out, 4)) return LLVQ_EINVAL;
  } else if (out_kind == LLVQ_OUT_BF16) {
    if (!scales || !aligned(out, 2) || !aligned(scales, 2)) return LLVQ_EINVAL;
  } else {
    return LLVQ_EINVAL;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const void* pk[1] = {packed};
  const void* sc[1] = {out_kind == LLVQ_OUT_BF16 ? scales : nullptr};
  void* oo[1] = {out};
  const int st1 = launch_decode_stream(&k, 1, pk, out_kind == LLVQ_OUT_BF16 ? sc : nullptr, out_kind, oo,
                                       err_count, s);
  if (st1 != LLVQ_EUNSUPPORTED) return st1;
  const uint64_t nblocks = (uint64_t)k.rows * (uint64_t)k.kb;
  const unsigned block = 256;
  if (out_kind == LLVQ_OUT_POINTS_I8) {
    hipLaunchKernelGGL(k_decode_points, dim3(grid_for(nblocks, block)), dim3(block), 0, s, k,
                       static_cast<const uint8_t*>(packed), static_cast<int8_t*>(out), err_count);
    return launch_status();
  }
  hipLaunchKernelGGL(k_decode_bf16, dim3(grid_for(nblocks, block)), dim3(block), 0, s, k,
                     static_cast<const uint8_t*>(packed), static_cast<const __half*>(scales),
                     static_cast<uint16_t*>(out), err_count);
  return launch_status();
}

LLVQ_API int llvq_decode_many(const llvq_desc* descs, int32_t n, const void* const* packed,
                              const void* const* scales, int32_t out_kind, void* const* outs, int32_t* err_count,
                              void* stream) {
  if (!descs || !packed || !outs || n < 1 || n > kManyMax) return LLVQ_EINVAL;
  if (out_kind != LLVQ_OUT_POINTS_I8 && out_kind != LLVQ_OUT_BF16) return LLVQ_EINVAL;
  if (out_kind == LLVQ_OUT_BF16 && !scales) return LLVQ_EINVAL;
  if (err_count && !aligned(err_count, 4)) return LLVQ_EINVAL;
  bool wide = false;
  for (int i = 0; i < n; ++i) wide = wide || wide_needed(&descs[i]);
  if (wide) {
    // the general decoder: one call per tensor, after every descriptor and pointer is checked
    for (int i = 0; i < n; ++i) {
      WDesc w;
      KDesc k1;
      const int st = wide_needed(&descs[i]) ? make_wdesc(&descs[i], &w) : make_kdesc(&descs[i], &k1);
      if (st != LLVQ_OK) return st;
      if (!packed[i] || !outs[i] || !aligned(packed[i], 16)) return LLVQ_EINVAL;
      if (out_kind == LLVQ_OUT_POINTS_I8 && !aligned(outs[i], 4)) return LLVQ_EINVAL;
      if (out_kind == LLVQ_OUT_BF16 && (!scales[i] || !aligned(outs[i], 2) || !aligned(scales[i], 2)))
        return LLVQ_EINVAL;
    }
    for (int i = 0; i < n; ++i) {
      const int st1 = llvq_decode(&descs[i], packed[i], scales ? scales[i] : nullptr, out_kind, outs[i], err_count,
                                  stream);
      if (st1 != LLVQ_OK) return st1;
    }
    return LLVQ_OK;
  }
  KDesc k[kManyMax];
  for (int i = 0; i < n; ++i) {
    const int st = make_kdesc(&descs[i], &k[i]);
    if (st != LLVQ_OK) return st;
    if (k[i].mode != k[0].mode || k[i].max_shell != k[0].max_shell || k[i].shape_bits != k[0].shape_bits ||
        k[i].gain_bits != k[0].gain_bits)
      return LLVQ_EINVAL;
    if (!packed[i] || !outs[i] || !aligned(packed[i], 16)) return LLVQ_EINVAL;
    if (out_kind == LLVQ_OUT_POINTS_I8 && !aligned(outs[i], 4)) return LLVQ_EINVAL;
    if (out_kind == LLVQ_OUT_BF16 && (!scales[i] || !aligned(outs[i], 2) || !aligned(scales[i], 2))) return LLVQ_EINVAL;
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int st = launch_decode_stream(k, n, packed, out_kind == LLVQ_OUT_BF16 ? scales : nullptr, out_kind, outs,
                                      err_count, s);
  if (st != LLVQ_EUNSUPPORTED) return st;
  for (int i = 0; i < n; ++i) {
    const int st1 = llvq_decode(&descs[i], packed[i], scales ? scales[i] : nullptr, out_kind, outs[i], err_count,
                                stream);
    if (st1 != LLVQ_OK) return st1;
  }
  return LLVQ_OK;
}

LLVQ_API int llvq_gemv(const llvq_desc* d, const void* packed, const void* scales, const void* x, int32_t x_dtype,
                       int32_t batch, float* y, int32_t* err_count, void* stream) {
  if (d && wide_needed(d)) return gemv_wide(d, packed, scales, x, x_dtype, batch, y, err_count, stream);
  KDesc k;
  int st = make_kdesc(d, &k);
  if (st != LLVQ_OK) return st;
  if (!packed || !scales || !x || !y) return LLVQ_EINVAL;
  if (!aligned(packed, 16) || !aligned(scales, 2) || !aligned(y, 4)) return LLVQ_EINVAL;
  if (err_count && !aligned(err_count, 4)) return LLVQ_EINVAL;
  if (x_dtype == LLVQ_X_F32) {
    if (!aligned(x, 4)) return LLVQ_EINVAL;
  } else if (x_dtype == LLVQ_X_BF16) {
    if (!aligned(x, 2)) return LLVQ_EINVAL;
  } else {
    return LLVQ_EINVAL;
  }
  if (batch < 1 || batch > LLVQ_MAX_BATCH) return LLVQ_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (batch == 1) {
    const int st1 = launch_gemv_b1(k, packed, scales, x, x_dtype, y, err_count, s);
    if (st1 != LLVQ_EUNSUPPORTED) return st1;
  } else if (x_dtype == LLVQ_X_BF16) {
    const int st2 = launch_gemm_mfma(k, packed, scales, x, batch, y, err_count, s);
    if (st2 != LLVQ_EUNSUPPORTED) return st2;
  }
  switch (batch) {
#define LLVQ_GEMV_CASE(B) \
  case B:                 \
    return launch_gemv<B>(k, packed, scales, x, x_dtype, y, err_count, s);
    LLVQ_GEMV_CASE(1) LLVQ_GEMV_CASE(2) LLVQ_GEMV_CASE(3) LLVQ_GEMV_CASE(4)
    LLVQ_GEMV_CASE(5) LLVQ_GEMV_CASE(6) LLVQ_GEMV_CASE(7) LLVQ_GEMV_CASE(8)
    LLVQ_GEMV_CASE(9) LLVQ_GEMV_CASE(10) LLVQ_GEMV_CASE(11) LLVQ_GEMV_CASE(12)
    LLVQ_GEMV_CASE(13) LLVQ_GEMV_CASE(14) LLVQ_GEMV_CASE(15) LLVQ_GEMV_CASE(16)
#undef LLVQ_GEMV_CASE
    default:
      return LLVQ_EINVAL;
  }
}

LLVQ_API int llvq_search(const float* x, int64_t n, int32_t max_shell, int32_t objective, int8_t* points,
                         uint64_t* indices, int32_t* err_count, void* stream) {
  if (max_shell < 2 || max_shell > LLVQ_SEARCH_MAX_SHELL || n < 0) return LLVQ_EINVAL;
  if (objective != LLVQ_SEARCH_ANGULAR && objective != LLVQ_SEARCH_EUCLID) return LLVQ_EINVAL;
  if (n == 0) return LLVQ_OK;
  if (!x || !points || !indices || !aligned(x, 4) || !aligned(indices, 8)) return LLVQ_EINVAL;
  if (err_count && !aligned(err_count, 4)) return LLVQ_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const unsigned grid = n < 8192 ? (unsigned)n : 8192u;
  if (objective == LLVQ_SEARCH_EUCLID)
    hipLaunchKernelGGL((k_search<true>), dim3(grid), dim3(kSearchThreads), 0, s, x, n, max_shell, 24, 1,
                       (const __half*)nullptr, points);
  else
    hipLaunchKernelGGL((k_search<false>), dim3(grid), dim3(kSearchThreads), 0, s, x, n, max_shell, 24, 1,
                       (const __half*)nullptr, points);
  const int st = launch_status();
  if (st != LLVQ_OK) return st;
  return llvq_encode_ref(points, n, max_shell, indices, err_count, stream);
}

namespace {
uint64_t quantize_points_bytes(const KDesc& k) { return ((uint64_t)k.rows * (uint64_t)k.kb * 24u + 7u) / 8u * 8u; }

// descriptor of the quantiser: shells 2..LLVQ_SEARCH_MAX_SHELL, fields of at most 64 bits
// (past shell 10 only the fields the search, rank and pack steps read are set)
int make_kdesc_quant(const llvq_desc* d, KDesc* k) {
  if (d && d->max_shell > LLVQ_MAX_SHELL && d->max_shell <= LLVQ_SEARCH_MAX_SHELL && d->shape_bits <= 60 &&
      d->shape_bits + d->gain_bits <= 64) {
    WDesc w;
    const int st = make_wdesc(d, &w);
    if (st != LLVQ_OK) return st;
    *k = KDesc{};
    k->mode = w.mode;
    k->rows = w.rows;
    k->cols = w.cols;
    k->kb = w.kb;
    k->max_shell = w.max_shell;
    k->shape_bits = w.shape_bits;
    k->gain_bits = w.gain_bits;
    k->field_bits = w.field_bits;
    k->index_count = w.count_lo;
    k->shape_mask = (1ull << w.shape_bits) - 1ull;
    k->shape_mask_lo = (uint32_t)k->shape_mask;
    k->shape_mask_hi = (uint32_t)(k->shape_mask >> 32);
    return LLVQ_OK;
  }
  return make_kdesc_narrow(d, k);
}
}  // namespace

LLVQ_API int64_t llvq_quantize_workspace_bytes(const llvq_desc* d) {
  KDesc k;
  const int st = make_kdesc_quant(d, &k);
  if (st != LLVQ_OK) return st;
  return (int64_t)(quantize_points_bytes(k) + (uint64_t)k.rows * (uint64_t)k.kb * 8u);
}

namespace {
// The quantiser's steps on a workspace of llvq_quantize_workspace_bytes: k_search writes
// the chosen points, the rank writes their indices, k_pack the fields.  Every byte of the
// workspace that a later step reads is written by an earlier step of the same call.
int quantize_into(const KDesc& k, const float* w, const void* scales, void* packed, void* workspace,
                  int32_t* err_count, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t n = (int64_t)k.rows * (int64_t)k.kb;
  int8_t* pts = static_cast<int8_t*>(workspace);
  uint64_t* idx = reinterpret_cast<uint64_t*>(static_cast<uint8_t*>(workspace) + quantize_points_bytes(k));
  const unsigned grid = n < 8192 ? (unsigned)n : 8192u;
  if (k.mode == LLVQ_MODE_EUCLID)
    hipLaunchKernelGGL((k_search<true>), dim3(grid), dim3(kSearchThreads), 0, s, w, n, k.max_shell, k.cols, k.kb,
                       static_cast<const __half*>(scales), pts);
  else
    hipLaunchKernelGGL((k_search<false>), dim3(grid), dim3(kSearchThreads), 0, s, w, n, k.max_shell, k.cols, k.kb,
                       (const __half*)nullptr, pts);
  int st1 = launch_status();
  if (st1 != LLVQ_OK) return st1;
  st1 = llvq_encode_ref(pts, n, k.max_shell, idx, err_count, stream);
  if (st1 != LLVQ_OK) return st1;
  const int64_t nwords = packed_bytes_of(k) / 4;
  hipLaunchKernelGGL((k_pack<false>), dim3(grid_for((uint64_t)nwords, 256)), dim3(256), 0, s, k, w,
                     k.mode == LLVQ_MODE_SHAPEGAIN ? static_cast<const __half*>(scales) : (const __half*)nullptr, idx,
                     static_cast<uint32_t*>(packed), nwords);
  return launch_status();
}

int check_quantize_args(const KDesc& k, const float* w, const void* scales, const void* packed, int32_t* err_count) {
  (void)k;
  if (!w || !scales || !packed) return LLVQ_EINVAL;
  if (!aligned(w, 4) || !aligned(scales, 2) || !aligned(packed, 16)) return LLVQ_EINVAL;
  if (err_count && !aligned(err_count, 4)) return LLVQ_EINVAL;
  return LLVQ_OK;
}

// Workspace of llvq_quantize_noalloc, owned by the library: the points and indices of at
// most kNoAllocBlocks blocks (24 + 8 bytes each, 64 MiB).  Each GPU holds its own copy
// from the library's load until the process ends.  In host code the array's name is not
// a device address: kernels get the address hipGetSymbolAddress returns for the device.
constexpr uint64_t kNoAllocBlocks = 1ull << 21;
constexpr uint64_t kNoAllocBytes = kNoAllocBlocks * 32u;
static __device__ __align__(256) uint8_t scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device that `stream` belongs to, looked up once per
// device with that device current.
int scratch_address(hipStream_t stream, void** out) {
  int dev = -1, cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return LLVQ_EHIP;
  if (hipStreamGetDevice(stream, &dev) != hipSuccess) return LLVQ_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return LLVQ_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return LLVQ_EHIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) return LLVQ_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LLVQ_OK;
}
}  // namespace

LLVQ_API int llvq_quantize(const llvq_desc* d, const float* w, const void* scales, void* packed, void* workspace,
                           int32_t* err_count, void* stream) {
  KDesc k;
  const int st = make_kdesc_quant(d, &k);
  if (st != LLVQ_OK) return st;
  const int st2 = check_quantize_args(k, w, scales, packed, err_count);
  if (st2 != LLVQ_OK) return st2;
  if (!workspace || !aligned(workspace, 8)) return LLVQ_EINVAL;
  return quantize_into(k, w, scales, packed, workspace, err_count, stream);
}

LLVQ_API int llvq_quantize_noalloc(const llvq_desc* d, const float* w, const void* scales, void* packed,
                                   int32_t* err_count, void* stream) {
  KDesc k;
  const int st = make_kdesc_quant(d, &k);
  if (st != LLVQ_OK) return st;
  const int st2 = check_quantize_args(k, w, scales, packed, err_count);
  if (st2 != LLVQ_OK) return st2;
  if ((uint64_t)k.rows * (uint64_t)k.kb > kNoAllocBlocks) return LLVQ_ETOOLARGE;
  void* ws = nullptr;
  const int st3 = scratch_address(reinterpret_cast<hipStream_t>(stream), &ws);
  if (st3 != LLVQ_OK) return st3;
  return quantize_into(k, w, scales, packed, ws, err_count, stream);
}

LLVQ_API int64_t llvq_quantize_noalloc_max_blocks(void) { return (int64_t)kNoAllocBlocks; }

LLVQ_API int llvq_pack_fields(const llvq_desc* d, const uint64_t* fields, void* packed, void* stream) {
  KDesc k;
  const int st = make_kdesc_narrow(d, &k);
  if (st != LLVQ_OK) return st;
  if (!fields || !packed || !aligned(fields, 8) || !aligned(packed, 16)) return LLVQ_EINVAL;
  const int64_t nwords = packed_bytes_of(k) / 4;
  hipLaunchKernelGGL((k_pack<true>), dim3(grid_for((uint64_t)nwords, 256)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), k, (const float*)nullptr, (const __half*)nullptr, fields,
                     static_cast<uint32_t*>(packed), nwords);
  return launch_status();
}

LLVQ_API int llvq_encode_ref(const int8_t* points, int64_t n, int32_t max_shell, uint64_t* indices,
                             int32_t* err_count, void* stream) {
  if (max_shell < 2 || max_shell > kRankWideMaxShell || n < 0) return LLVQ_EINVAL;
  if (n == 0) return LLVQ_OK;
  if (!points || !indices || !aligned(indices, 8)) return LLVQ_EINVAL;
  if (err_count && !aligned(err_count, 4)) return LLVQ_EINVAL;
  const unsigned block = 256;
  if (max_shell > LLVQ_MAX_SHELL) {
    // the general rank (shells past 10)
    hipLaunchKernelGGL(k_rank_wide<false>, dim3(grid_for((uint64_t)n, kWideThreads)), dim3(kWideThreads), 0,
                       reinterpret_cast<hipStream_t>(stream), points, n, max_shell, indices, err_count);
    return launch_status();
  }
  if (aligned(points, 8))
    hipLaunchKernelGGL((k_rank<true>), dim3(grid_for((uint64_t)n, block)), dim3(block), 0,
                       reinterpret_cast<hipStream_t>(stream), points, n, max_shell, indices, err_count);
  else
    hipLaunchKernelGGL((k_rank<false>), dim3(grid_for((uint64_t)n, block)), dim3(block), 0,
                       reinterpret_cast<hipStream_t>(stream), points, n, max_shell, indices, err_count);
  return launch_status();
}

LLVQ_API int llvq_encode_wide(const int8_t* points, int64_t n, int32_t max_shell, uint64_t* indices,
                              int32_t* err_count, void* stream) {
  if (max_shell < 2 || max_shell > LLVQ_WIDE_MAX_SHELL || n < 0) return LLVQ_EINVAL;
  if (n == 0) return LLVQ_OK;
  if (!points || !indices || !aligned(indices, 8)) return LLVQ_EINVAL;
  if (err_count && !aligned(err_count, 4)) return LLVQ_EINVAL;
  hipLaunchKernelGGL(k_rank_wide<true>, dim3(grid_for((uint64_t)n, kWideThreads)), dim3(kWideThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), points, n, max_shell, indices, err_count);
  return launch_status();
}

// ---------------------------------------------------------------------------
// spherical GPTQ (llvq_gptq.h)

namespace {
int64_t gptq_kp(int32_t cols) { return 24ll * ((cols + 23) / 24); }
}  // namespace

LLVQ_API int64_t llvq_gptq_workspace_bytes(int32_t cols) {
  if (cols <= 0 || cols > (1 << 20)) return LLVQ_EINVAL;
  const int64_t kp = gptq_kp(cols), kb = kp / 24;
  return kp * kp * 8 + kb * 576 * 8 + 256;
}

LLVQ_API int llvq_gptq_factor(int32_t cols, const double* H, double damp, double* U, void* workspace,
                              int32_t* err_count, void* stream) {
  if (cols <= 0 || cols > (1 << 20) || !H || !U || !workspace || !(damp >= 0.0) || !(damp < 1e300)) return LLVQ_EINVAL;
  if (!aligned(H, 8) || !aligned(U, 8) || !aligned(workspace, 8)) return LLVQ_EINVAL;
  if (err_count && !aligned(err_count, 4)) return LLVQ_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int Kp = (int)gptq_kp(cols), Kb = Kp / 24;
  double* A = static_cast<double*>(workspace);
  double* Linv = A + (size_t)Kp * (size_t)Kp;
  double* mean = Linv + (size_t)Kb * 576;
  const unsigned gfull = grid_for((uint64_t)Kp * (uint64_t)Kp, 256);
  hipLaunchKernelGGL(k_gptq_diag_mean, dim3(1), dim3(256), 0, s, H, cols, mean);
  hipLaunchKernelGGL(k_gptq_reverse_damp, dim3(gfull), dim3(256), 0, s, H, cols, Kp, mean, damp, A);
  for (int jb = 0; jb < Kb; ++jb) {
    const int j0 = 24 * jb;
    hipLaunchKernelGGL(k_gptq_potrf_diag, dim3(1), dim3(64), 0, s, A, Kp, j0, Linv + (size_t)jb * 576, err_count);
    const int rest = Kp - j0 - 24;
    if (rest > 0) {
      hipLaunchKernelGGL(k_gptq_panel, dim3((rest + 255) / 256), dim3(256), 0, s, A, Kp, j0,
                         Linv + (size_t)jb * 576);
      const int nt = (rest + kGTile - 1) / kGTile;
      hipLaunchKernelGGL(k_gptq_syrk, dim3(nt, nt), dim3(256), 0, s, A, Kp, j0);
    }
  }
  hipLaunchKernelGGL(k_gptq_inv_diag, dim3(gfull), dim3(256), 0, s, Kp, Linv, U);
  for (int kb = 0; kb + 1 < Kb; ++kb) {
    hipLaunchKernelGGL(k_gptq_inv_update, dim3(Kb - 1 - kb, kb + 1), dim3(576), 0, s, A, Kp, kb, U);
    hipLaunchKernelGGL(k_gptq_inv_solve, dim3(kb + 1), dim3(576), 0, s, Kp, kb + 1, Linv, U);
  }
  hipLaunchKernelGGL(k_gptq_reverse, dim3(gfull), dim3(256), 0, s, Kp, U);
  return launch_status();
}

LLVQ_API int llvq_gptq_begin(int32_t rows, int32_t cols, const float* W, double* Wq, float* x0, void* stream) {
  if (rows <= 0 || cols <= 0 || cols > (1 << 20) || !W || !Wq || !x0) return LLVQ_EINVAL;
  if (!aligned(W, 4) || !aligned(Wq, 8) || !aligned(x0, 4)) return LLVQ_EINVAL;
  const int Kp = (int)gptq_kp(cols);
  hipLaunchKernelGGL(k_gptq_begin, dim3(grid_for((uint64_t)rows * (uint64_t)Kp, 256)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), W, rows, cols, Kp, Wq, x0);
  return launch_status();
}

LLVQ_API int llvq_gptq_column(const llvq_desc* d, int32_t block, int32_t variant, const void* gains, double* Wq,
                              const double* U, const int8_t* points, const uint64_t* indices, uint64_t* fields,
                              double* ework, float* x_next, void* stream) {
  KDesc k;
  const int st = make_kdesc_quant(d, &k);
  if (st != LLVQ_OK) return st;
  if (k.mode != LLVQ_MODE_SHAPEGAIN) return LLVQ_EINVAL;
  if (variant < 0 || variant > 2 || block < 0 || block >= k.kb) return LLVQ_EINVAL;
  const bool last = block == k.kb - 1;
  if (!gains || !Wq || !U || !points || !indices || !fields || (!last && !x_next) || (variant != 2 && !ework))
    return LLVQ_EINVAL;
  if (!aligned(gains, 2) || !aligned(Wq, 8) || !aligned(U, 8) || !aligned(indices, 8) || !aligned(fields, 8) ||
      (ework && !aligned(ework, 8)) || (x_next && !aligned(x_next, 4)))
    return LLVQ_EINVAL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  GptqCol g;
  g.rows = k.rows;
  g.Kp = 24 * k.kb;
  g.kb = k.kb;
  g.block = block;
  g.variant = variant;
  g.gain_bits = k.gain_bits;
  g.shape_bits = k.shape_bits;
  g.last = last ? 1 : 0;
  hipLaunchKernelGGL(k_gptq_residual, dim3((k.rows + 255) / 256), dim3(256), 0, s, g, Wq, U,
                     static_cast<const __half*>(gains), points, indices, fields, ework);
  if (!last) {
    if (variant != 2) {
      const int f0 = (block + 1) * 24;
      hipLaunchKernelGGL(k_gptq_update, dim3((g.Kp - f0 + 255) / 256, (k.rows + 31) / 32), dim3(256), 0, s, g, Wq, U,
                         ework, x_next);
    } else {
      hipLaunchKernelGGL(k_gptq_next, dim3(grid_for((uint64_t)k.rows * 24u, 256)), dim3(256), 0, s, g, Wq, x_next);
    }
  }
  return launch_status();
}

LLVQ_API int llvq_device_checks(uint32_t* failures, int32_t reset) {
#ifdef LLVQ_DEVICE_CHECKS
  if (!failures) return LLVQ_EINVAL;
  if (hipMemcpyFromSymbol(failures, HIP_SYMBOL(g_llvq_check_failures), sizeof(uint32_t)) != hipSuccess)
    return LLVQ_EHIP;
  if (reset) {
    const uint32_t zero = 0;
    if (hipMemcpyToSymbol(HIP_SYMBOL(g_llvq_check_failures), &zero, sizeof(uint32_t)) != hipSuccess) return LLVQ_EHIP;
  }
  return LLVQ_OK;
#else
  (void)failures;
  (void)reset;
  return LLVQ_EUNSUPPORTED;
#endif
}
