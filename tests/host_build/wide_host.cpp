// Host build of the general decoder's device functions (weight_decompression_amd/csrc/
// llvq_wide.h, included unchanged) for sanitizer runs on the CPU: the tests compile it with
// g++ -fsanitize=address,undefined, so every table read (the class records, bucket tables,
// shell starts and the odd-part inverse table) is bounds-checked and every shift and
// integer conversion of the exact 64-bit / 128-bit arithmetic is checked for undefined
// behaviour, while the decoded points and ranks are compared with the oracle.
//
// The few HIP names the header uses outside the decode and rank functions (kernel
// qualifiers, thread indices, fp16 / bf16 helpers, atomics) get host stand-ins below; the
// kernels themselves are templates that are never instantiated here.
//
// stdin, one request per line:
//   D M lo hi           decode global index lo | hi << 64 at shells 2..M -> "m v0 .. v23"
//   R M v0 .. v23       rank the point at shells 2..M -> "lo hi" (or "none")

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <cmath>

#define __device__
#define __host__
#define __forceinline__ inline
#define __global__ static inline
#define __launch_bounds__(x)
// the in-kernel invariant checks of the device-checks build: fatal here
#define LLVQ_DCHECK(cond)                                           \
  do {                                                              \
    if (!(cond)) {                                                  \
      fprintf(stderr, "invariant failed: %s (line %d)\n", #cond, __LINE__); \
      abort();                                                      \
    }                                                               \
  } while (0)

struct HostDim3 {
  unsigned x, y, z;
};
static HostDim3 threadIdx, blockIdx, blockDim, gridDim;
struct __half {
  uint16_t bits;
};
static inline float __half2float(__half) { abort(); }
static inline int __clz(int x) { return x ? __builtin_clz((unsigned)x) : 32; }
static inline int __popc(unsigned x) { return __builtin_popcount(x); }
static inline int __popcll(unsigned long long x) { return __builtin_popcountll(x); }
static inline float __uint_as_float(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}
static inline float __fmul_rn(float a, float b) { return a * b; }
static inline int atomicAdd(int32_t* p, int v) { abort(); (void)p; return v; }
static inline float __shfl_xor(float v, int, int) { abort(); return v; }
struct uint4 {
  uint32_t x, y, z, w;
};
struct float4 {
  float x, y, z, w;
};
static inline uint4 make_uint4(uint32_t a, uint32_t b, uint32_t c, uint32_t d) { return uint4{a, b, c, d}; }
static inline uint16_t f32_to_bf16_rne(float) { abort(); }
static inline float bf16_to_f32(uint16_t) { abort(); }
using std::floor;
using std::min;

#include "llvq.h"
#include "llvq_tables.h"

namespace dev_tables {
#define LLVQ_TABLE static const
#include "llvq_tables.inc"
#define LLVQ_WIDE_CLASSES
#include "llvq_wide.inc"
#undef LLVQ_WIDE_CLASSES
#undef LLVQ_TABLE
}  // namespace dev_tables

constexpr int kDim = 24;

#include "llvq_wide.h"

int main() {
  char op[4];
  int M;
  while (scanf("%3s %d", op, &M) == 2) {
    if (op[0] == 'D') {
      unsigned long long lo, hi;
      if (scanf("%llu %llu", &lo, &hi) != 2) return 2;
      int v[kDim];
      const int m = wide_decode_point(lo, hi, M, v);
      printf("%d", m);
      for (int p = 0; p < kDim; ++p) printf(" %d", v[p]);
      printf("\n");
    } else if (op[0] == 'R') {
      int v[kDim];
      for (int p = 0; p < kDim; ++p)
        if (scanf("%d", &v[p]) != 1) return 2;
      uint64_t lo = 0, hi = 0;
      if (wide_rank_point(v, M, lo, hi))
        printf("%llu %llu\n", (unsigned long long)lo, (unsigned long long)hi);
      else
        printf("none\n");
    } else {
      return 2;
    }
  }
  return 0;
}
