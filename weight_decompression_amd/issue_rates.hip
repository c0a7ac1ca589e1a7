// VALU issue-rate microbenchmarks for gfx950: one kernel per instruction, 16 independent
// dependency chains per lane, each chain step a single inline-asm ALU instruction (no
// memory access inside the timed loop).  The rate of an instruction is
// (launched lanes x ITERS x CH) / 64 / seconds / 256 CUs / clock: wave-instructions issued
// per CU per clock.  Used to check the VALU peak assumed for the decode kernels against the
// instruction mix those kernels actually execute.

#include <hip/hip_runtime.h>
#include <stdint.h>

#define ITERS 512
#define CH 16

#define K32(NAME, ASM)                                                                              \
  __global__ __launch_bounds__(256) void NAME(uint32_t* out, uint32_t seed) {                      \
    uint32_t a[CH];                                                                                 \
    const uint32_t b = seed, c = seed * 3u;                                                         \
    for (int j = 0; j < CH; ++j) a[j] = threadIdx.x * 7u + j + seed;                                \
    for (int it = 0; it < ITERS; ++it) {                                                            \
      _Pragma("unroll") for (int j = 0; j < CH; ++j) asm volatile(ASM : "+v"(a[j]) : "v"(b), "v"(c)); \
    }                                                                                               \
    uint32_t s = 0;                                                                                 \
    for (int j = 0; j < CH; ++j) s ^= a[j];                                                         \
    out[blockIdx.x * 256 + threadIdx.x] = s;                                                        \
  }

#define K64(NAME, ASM)                                                                              \
  __global__ __launch_bounds__(256) void NAME(uint32_t* out, uint32_t seed) {                      \
    double a[CH];                                                                                   \
    const double b = 1.0 + 1e-9 * seed, c = 1e-7;                                                   \
    for (int j = 0; j < CH; ++j) a[j] = threadIdx.x * 0.5 + j;                                      \
    for (int it = 0; it < ITERS; ++it) {                                                            \
      _Pragma("unroll") for (int j = 0; j < CH; ++j) asm volatile(ASM : "+v"(a[j]) : "v"(b), "v"(c)); \
    }                                                                                               \
    double s = 0;                                                                                   \
    for (int j = 0; j < CH; ++j) s += a[j];                                                         \
    out[blockIdx.x * 256 + threadIdx.x] = (uint32_t)s;                                              \
  }

// The instruction list: name (as the assembler prints it, without _e32/_e64) and its kernel.
K32(k_add_u32, "v_add_u32 %0, %0, %1")
K32(k_sub_u32, "v_sub_u32 %0, %0, %1")
K32(k_and_b32, "v_and_b32 %0, %0, %1")
K32(k_or_b32, "v_or_b32 %0, %0, %1")
K32(k_xor_b32, "v_xor_b32 %0, %0, %1")
K32(k_not_b32, "v_not_b32 %0, %0")
K32(k_mov_b32, "v_mov_b32 %0, %1")
K32(k_lshrrev_b32, "v_lshrrev_b32 %0, %1, %0")
K32(k_lshlrev_b32, "v_lshlrev_b32 %0, %1, %0")
// lane-select with a 64-bit mask in a scalar register pair (the form the kernels use)
__global__ __launch_bounds__(256) void k_cndmask_b32(uint32_t* out, uint32_t seed) {
  uint32_t a[CH];
  const uint32_t b = seed;
  const uint64_t m = __ballot((threadIdx.x & 1u) != 0u);
  for (int j = 0; j < CH; ++j) a[j] = threadIdx.x * 7u + j + seed;
  for (int it = 0; it < ITERS; ++it) {
#pragma unroll
    for (int j = 0; j < CH; ++j) asm volatile("v_cndmask_b32_e64 %0, %0, %1, %2" : "+v"(a[j]) : "v"(b), "s"(m));
  }
  uint32_t s = 0;
  for (int j = 0; j < CH; ++j) s ^= a[j];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}
K32(k_mul_f32, "v_mul_f32 %0, %0, %1")
K32(k_add_f32, "v_add_f32 %0, %0, %1")
K32(k_fmac_f32, "v_fmac_f32 %0, %1, %2")
K32(k_fma_f32, "v_fma_f32 %0, %0, %1, %2")
K32(k_cvt_f32_u32, "v_cvt_f32_u32 %0, %0")
K32(k_cvt_f32_ubyte0, "v_cvt_f32_ubyte0 %0, %0")
K32(k_xad_u32, "v_xad_u32 %0, %0, %1, %2")
K32(k_ffbl_b32, "v_ffbl_b32 %0, %0")
K32(k_bfi_b32, "v_bfi_b32 %0, %0, %1, %2")
K32(k_bfe_u32, "v_bfe_u32 %0, %0, %1, 4")
K32(k_alignbit_b32, "v_alignbit_b32 %0, %0, %1, %2")
K32(k_lshl_or_b32, "v_lshl_or_b32 %0, %0, 3, %1")
K32(k_lshl_add_u32, "v_lshl_add_u32 %0, %0, 3, %1")
K32(k_add3_u32, "v_add3_u32 %0, %0, %1, %2")
K32(k_and_or_b32, "v_and_or_b32 %0, %0, %1, %2")
K32(k_or3_b32, "v_or3_b32 %0, %0, %1, %2")
K32(k_mad_u32_u24, "v_mad_u32_u24 %0, %0, %1, %2")
K32(k_mul_lo_u32, "v_mul_lo_u32 %0, %0, %1")
K32(k_perm_b32, "v_perm_b32 %0, %0, %1, %2")
K32(k_dot4_u32_u8, "v_dot4_u32_u8 %0, %0, %1, %2")
K32(k_bcnt_u32_b32, "v_bcnt_u32_b32 %0, %0, %1")
K32(k_med3_u32, "v_med3_u32 %0, %0, %1, %2")
K32(k_min_f32, "v_min_f32 %0, %0, %1")
K32(k_max_f32, "v_max_f32 %0, %0, %1")
K32(k_min_u32, "v_min_u32 %0, %0, %1")
K32(k_max_u32, "v_max_u32 %0, %0, %1")
K32(k_max3_f32, "v_max3_f32 %0, %0, %1, %2")
K64(k_fma_f64, "v_fma_f64 %0, %0, %1, %2")
K64(k_mul_f64, "v_mul_f64 %0, %0, %1")
K64(k_add_f64, "v_add_f64 %0, %0, %1")

// conversions between fp64 and u32 (the arithmetic decoder's per-step pair)
__global__ __launch_bounds__(256) void k_cvt_u32_f64(uint32_t* out, uint32_t seed) {
  uint32_t a[CH];
  const double b = 3.5 + seed;
  for (int j = 0; j < CH; ++j) a[j] = threadIdx.x * 7u + j + seed;
  for (int it = 0; it < ITERS; ++it) {
#pragma unroll
    for (int j = 0; j < CH; ++j) asm volatile("v_cvt_u32_f64 %0, %1" : "+v"(a[j]) : "v"(b));
  }
  uint32_t s = 0;
  for (int j = 0; j < CH; ++j) s ^= a[j];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}
__global__ __launch_bounds__(256) void k_cvt_f64_u32(uint32_t* out, uint32_t seed) {
  double a[CH];
  const uint32_t b = seed + 5u;
  for (int j = 0; j < CH; ++j) a[j] = threadIdx.x * 0.5 + j;
  for (int it = 0; it < ITERS; ++it) {
#pragma unroll
    for (int j = 0; j < CH; ++j) asm volatile("v_cvt_f64_u32 %0, %1" : "+v"(a[j]) : "v"(b));
  }
  double s = 0;
  for (int j = 0; j < CH; ++j) s += a[j];
  out[blockIdx.x * 256 + threadIdx.x] = (uint32_t)s;
}
// bf16 pair dot product accumulating in fp32, and the fp8 pair -> bf16 pair conversion
K32(k_dot2c_f32_bf16, "v_dot2c_f32_bf16 %0, %1, %2")
K32(k_cvt_scalef32_pk_bf16_fp8, "v_cvt_scalef32_pk_bf16_fp8 %0, %0, %1")
K32(k_bitop3_b32, "v_bitop3_b32 %0, %0, %1, %2 bitop3:0xc")
K32(k_mbcnt_lo_u32_b32, "v_mbcnt_lo_u32_b32 %0, %1, %0")
__global__ __launch_bounds__(256) void k_cmp_ne_u32(uint32_t* out, uint32_t seed) {
  uint32_t a[CH];
  const uint32_t b = seed;
  for (int j = 0; j < CH; ++j) a[j] = threadIdx.x * 7u + j + seed;
  for (int it = 0; it < ITERS; ++it) {
#pragma unroll
    for (int j = 0; j < CH; ++j) asm volatile("v_cmp_ne_u32_e32 vcc, %0, %1" : : "v"(a[j]), "v"(b) : "vcc");
  }
  uint32_t s = 0;
  for (int j = 0; j < CH; ++j) s ^= a[j];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

// 64-bit integer chains (the exact index arithmetic of the general decoder and the ranker)
#define KU64(NAME, ASM, ...)                                                                        \
  __global__ __launch_bounds__(256) void NAME(uint32_t* out, uint32_t seed) {                      \
    uint64_t a[CH];                                                                                 \
    const uint64_t b = seed * 0x9e3779b97f4a7c15ull;                                                \
    const uint32_t c = seed & 7u;                                                                   \
    for (int j = 0; j < CH; ++j) a[j] = threadIdx.x * 7ull + j + seed;                              \
    for (int it = 0; it < ITERS; ++it) {                                                            \
      _Pragma("unroll") for (int j = 0; j < CH; ++j) asm volatile(ASM : "+v"(a[j]) : "v"(b), "v"(c) __VA_ARGS__); \
    }                                                                                               \
    uint64_t s = 0;                                                                                 \
    for (int j = 0; j < CH; ++j) s ^= a[j];                                                         \
    out[blockIdx.x * 256 + threadIdx.x] = (uint32_t)(s ^ (s >> 32));                                \
  }
KU64(k_mad_u64_u32, "v_mad_u64_u32 %0, vcc, %2, %2, %0", : "vcc")
KU64(k_lshl_add_u64, "v_lshl_add_u64 %0, %0, 2, %1")
KU64(k_mov_b64, "v_mov_b64 %0, %1")
KU64(k_lshrrev_b64, "v_lshrrev_b64 %0, %2, %0")
// 32-bit chains with a carry or condition output in vcc
#define K32V(NAME, ASM)                                                                             \
  __global__ __launch_bounds__(256) void NAME(uint32_t* out, uint32_t seed) {                      \
    uint32_t a[CH];                                                                                 \
    const uint32_t b = seed, c = seed * 3u;                                                         \
    for (int j = 0; j < CH; ++j) a[j] = threadIdx.x * 7u + j + seed;                                \
    for (int it = 0; it < ITERS; ++it) {                                                            \
      _Pragma("unroll") for (int j = 0; j < CH; ++j) asm volatile(ASM : "+v"(a[j]) : "v"(b), "v"(c) : "vcc"); \
    }                                                                                               \
    uint32_t s = 0;                                                                                 \
    for (int j = 0; j < CH; ++j) s ^= a[j];                                                         \
    out[blockIdx.x * 256 + threadIdx.x] = s;                                                        \
  }
K32V(k_add_co_u32, "v_add_co_u32 %0, vcc, %0, %1")
K32(k_cvt_pk_bf16_f32, "v_cvt_pk_bf16_f32 %0, %0, %1")
// fp64 chains with a condition in vcc, and the fp64 division steps
#define K64V(NAME, ASM)                                                                             \
  __global__ __launch_bounds__(256) void NAME(uint32_t* out, uint32_t seed) {                      \
    double a[CH];                                                                                   \
    const double b = 1.0 + 1e-9 * seed, c = 1e-7;                                                  \
    for (int j = 0; j < CH; ++j) a[j] = threadIdx.x * 0.5 + j + 1.0;                                \
    for (int it = 0; it < ITERS; ++it) {                                                            \
      _Pragma("unroll") for (int j = 0; j < CH; ++j) asm volatile(ASM : "+v"(a[j]) : "v"(b), "v"(c) : "vcc"); \
    }                                                                                               \
    double s = 0;                                                                                   \
    for (int j = 0; j < CH; ++j) s += a[j];                                                         \
    out[blockIdx.x * 256 + threadIdx.x] = (uint32_t)s;                                              \
  }
K64(k_fmac_f64, "v_fmac_f64 %0, %1, %2")
K64V(k_cmp_ge_f64, "v_cmp_ge_f64_e32 vcc, %0, %1")
K64V(k_div_scale_f64, "v_div_scale_f64 %0, vcc, %0, %1, %0")
K64V(k_div_fmas_f64, "v_div_fmas_f64 %0, %0, %1, %2")
K64(k_div_fixup_f64, "v_div_fixup_f64 %0, %0, %1, %2")
K64(k_rcp_f64, "v_rcp_f64 %0, %0")
__global__ __launch_bounds__(256) void k_ldexp_f64(uint32_t* out, uint32_t seed) {
  double a[CH];
  const int32_t e = (int32_t)(seed & 1u);
  for (int j = 0; j < CH; ++j) a[j] = threadIdx.x * 0.5 + j + 1.0;
  for (int it = 0; it < ITERS; ++it) {
#pragma unroll
    for (int j = 0; j < CH; ++j) asm volatile("v_ldexp_f64 %0, %0, %1" : "+v"(a[j]) : "v"(e));
  }
  double s = 0;
  for (int j = 0; j < CH; ++j) s += a[j];
  out[blockIdx.x * 256 + threadIdx.x] = (uint32_t)s;
}
K64(k_rndne_f64, "v_rndne_f64 %0, %0")
K32(k_rcp_f32, "v_rcp_f32 %0, %0")
K32V(k_div_scale_f32, "v_div_scale_f32 %0, vcc, %0, %1, %0")
// cross-lane moves between VGPRs and SGPRs (wave-uniform values)
__global__ __launch_bounds__(256) void k_readlane_b32(uint32_t* out, uint32_t seed) {
  uint32_t a[CH], t[CH];
  for (int j = 0; j < CH; ++j) a[j] = threadIdx.x * 7u + j + seed;
  for (int j = 0; j < CH; ++j) t[j] = 0;
  for (int it = 0; it < ITERS; ++it) {
#pragma unroll
    for (int j = 0; j < CH; ++j) asm volatile("v_readlane_b32 %0, %1, 5" : "=s"(t[j]) : "v"(a[j]));
  }
  uint32_t s = 0;
  for (int j = 0; j < CH; ++j) s ^= a[j] ^ t[j];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}
__global__ __launch_bounds__(256) void k_readfirstlane_b32(uint32_t* out, uint32_t seed) {
  uint32_t a[CH], t[CH];
  for (int j = 0; j < CH; ++j) a[j] = threadIdx.x * 7u + j + seed;
  for (int j = 0; j < CH; ++j) t[j] = 0;
  for (int it = 0; it < ITERS; ++it) {
#pragma unroll
    for (int j = 0; j < CH; ++j) asm volatile("v_readfirstlane_b32 %0, %1" : "=s"(t[j]) : "v"(a[j]));
  }
  uint32_t s = 0;
  for (int j = 0; j < CH; ++j) s ^= a[j] ^ t[j];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}
__global__ __launch_bounds__(256) void k_writelane_b32(uint32_t* out, uint32_t seed) {
  uint32_t a[CH];
  for (int j = 0; j < CH; ++j) a[j] = threadIdx.x * 7u + j + seed;
  for (int it = 0; it < ITERS; ++it) {
#pragma unroll
    for (int j = 0; j < CH; ++j) asm volatile("v_writelane_b32 %0, %1, 5" : "+v"(a[j]) : "s"(seed));
  }
  uint32_t s = 0;
  for (int j = 0; j < CH; ++j) s ^= a[j];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

typedef void (*kfn)(uint32_t*, uint32_t);
static const kfn kKernels[] = {
    k_add_u32,     k_sub_u32,      k_and_b32,        k_or_b32,       k_xor_b32,      k_not_b32,      k_mov_b32,
    k_lshrrev_b32, k_lshlrev_b32,  k_cndmask_b32,    k_mul_f32,      k_add_f32,      k_fmac_f32,     k_fma_f32,
    k_cvt_f32_u32, k_cvt_f32_ubyte0, k_xad_u32,      k_ffbl_b32,     k_bfi_b32,      k_bfe_u32,      k_alignbit_b32,
    k_lshl_or_b32, k_lshl_add_u32, k_add3_u32,       k_and_or_b32,   k_or3_b32,      k_mad_u32_u24,  k_mul_lo_u32,
    k_perm_b32,    k_dot4_u32_u8,  k_bcnt_u32_b32,   k_med3_u32,     k_min_f32,      k_max_f32,      k_min_u32,
    k_max_u32,     k_max3_f32,     k_fma_f64,        k_mul_f64,      k_add_f64,      k_cvt_u32_f64,  k_cvt_f64_u32,
    k_dot2c_f32_bf16, k_cvt_scalef32_pk_bf16_fp8, k_bitop3_b32, k_mbcnt_lo_u32_b32, k_cmp_ne_u32,
    k_mad_u64_u32, k_lshl_add_u64, k_mov_b64, k_lshrrev_b64, k_add_co_u32, k_cvt_pk_bf16_f32, k_fmac_f64,
    k_cmp_ge_f64, k_div_scale_f64, k_div_fmas_f64, k_div_fixup_f64, k_rcp_f64, k_ldexp_f64, k_readlane_b32,
    k_readfirstlane_b32, k_writelane_b32, k_rndne_f64, k_rcp_f32, k_div_scale_f32};

extern "C" __attribute__((visibility("default"))) int ir_count() { return (int)(sizeof(kKernels) / sizeof(kKernels[0])); }

// Instructions per chain step and per-launch geometry, for the caller's rate arithmetic.
extern "C" __attribute__((visibility("default"))) int ir_iters() { return ITERS * CH; }

// Launch kernel `which` on `blocks` workgroups of 256 lanes writing out[blocks * 256]
// (device memory owned by the caller) on the null stream.  0 on success.
extern "C" __attribute__((visibility("default"))) int ir_run(int which, void* out, uint32_t seed, int blocks) {
  if (which < 0 || which >= ir_count() || blocks <= 0 || !out) return -1;
  hipLaunchKernelGGL(kKernels[which], dim3(blocks), dim3(256), 0, 0, static_cast<uint32_t*>(out), seed);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
