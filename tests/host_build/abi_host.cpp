// Host checks of the C ABI's argument validation, built with the library's sources under
// AddressSanitizer and UndefinedBehaviorSanitizer on the host side (no GPU needed: every call
// here is refused before any launch).  Prints "ok <checks>" and exits 0, or names the first
// failed check and exits 1.

#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "llvq.h"

static int g_checks = 0;
#define CHECK(cond)                                                  \
  do {                                                               \
    ++g_checks;                                                      \
    if (!(cond)) {                                                   \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      return 1;                                                      \
    }                                                                \
  } while (0)

int main() {
  uint64_t n = 0, hi = 0;
  CHECK(llvq_index_count(1, &n) == LLVQ_EINVAL);
  CHECK(llvq_index_count(11, &n) == LLVQ_EINVAL);
  CHECK(llvq_index_count(10, nullptr) == LLVQ_EINVAL);
  CHECK(llvq_index_count(10, &n) == LLVQ_OK && n == 13503934538640ull);
  CHECK(llvq_index_count(3, &n) == LLVQ_OK && n == 16969680ull);
  CHECK(llvq_index_count_wide(43, &n, &hi) == LLVQ_EINVAL);
  CHECK(llvq_index_count_wide(42, &n, &hi) == LLVQ_OK && hi > 0);

  llvq_desc good = {LLVQ_MODE_SHAPEGAIN, 4096, 11008, 10, 44, 4};
  const int64_t pb = llvq_packed_bytes(&good);
  CHECK(pb == (int64_t)((4096ll * 459 * 6 + 15) / 16 * 16 + 16));
  llvq_desc bad[] = {
      {7, 16, 240, 10, 44, 4},                      // mode
      {LLVQ_MODE_SHAPEGAIN, 0, 240, 10, 44, 4},     // rows
      {LLVQ_MODE_SHAPEGAIN, 16, -1, 10, 44, 4},     // cols
      {LLVQ_MODE_SHAPEGAIN, 16, 240, 1, 44, 4},     // shell range
      {LLVQ_MODE_SHAPEGAIN, 16, 240, 10, 40, 4},    // too few shape bits for shells 2..10
      {LLVQ_MODE_EUCLID, 16, 240, 3, 25, 2},        // gain bits in Euclidean mode
      {LLVQ_MODE_SHAPEGAIN, 16, 240, 10, 44, 0},    // no gain bits in shape-gain mode
      {LLVQ_MODE_SHAPEGAIN, 16, 240, 10, 44, 9},    // gain table too large
  };
  for (const llvq_desc& d : bad) CHECK(llvq_packed_bytes(&d) < 0);
  CHECK(llvq_packed_bytes(nullptr) < 0);

  alignas(16) static uint8_t buf[4096];
  void* p = buf;
  void* mis = buf + 1;
  for (const llvq_desc& d : bad) {
    CHECK(llvq_decode(&d, p, p, LLVQ_OUT_BF16, p, nullptr, nullptr) == LLVQ_EINVAL);
    CHECK(llvq_gemv(&d, p, p, p, LLVQ_X_BF16, 1, (float*)p, nullptr, nullptr) == LLVQ_EINVAL);
  }
  llvq_desc small = {LLVQ_MODE_SHAPEGAIN, 16, 240, 10, 44, 4};
  CHECK(llvq_decode(nullptr, p, p, LLVQ_OUT_BF16, p, nullptr, nullptr) == LLVQ_EINVAL);
  CHECK(llvq_decode(&small, nullptr, p, LLVQ_OUT_BF16, p, nullptr, nullptr) == LLVQ_EINVAL);
  CHECK(llvq_decode(&small, mis, p, LLVQ_OUT_BF16, p, nullptr, nullptr) == LLVQ_EINVAL);
  CHECK(llvq_decode(&small, p, nullptr, LLVQ_OUT_BF16, p, nullptr, nullptr) == LLVQ_EINVAL);
  CHECK(llvq_decode(&small, p, p, 5, p, nullptr, nullptr) == LLVQ_EINVAL);
  CHECK(llvq_decode(&small, p, p, LLVQ_OUT_POINTS_I8, mis, nullptr, nullptr) == LLVQ_EINVAL);
  CHECK(llvq_decode(&small, p, p, LLVQ_OUT_BF16, p, (int32_t*)mis, nullptr) == LLVQ_EINVAL);
  CHECK(llvq_gemv(&small, p, p, p, LLVQ_X_BF16, 0, (float*)p, nullptr, nullptr) == LLVQ_EINVAL);
  CHECK(llvq_gemv(&small, p, p, p, LLVQ_X_BF16, 17, (float*)p, nullptr, nullptr) == LLVQ_EINVAL);
  CHECK(llvq_gemv(&small, p, p, p, 3, 1, (float*)p, nullptr, nullptr) == LLVQ_EINVAL);
  CHECK(llvq_gemv(&small, p, p, mis, LLVQ_X_F32, 1, (float*)p, nullptr, nullptr) == LLVQ_EINVAL);
  CHECK(llvq_gemv(&small, p, p, p, LLVQ_X_BF16, 1, (float*)mis, nullptr, nullptr) == LLVQ_EINVAL);
  CHECK(llvq_gemv(&small, p, p, p, LLVQ_X_BF16, 1, nullptr, nullptr, nullptr) == LLVQ_EINVAL);

  const llvq_desc many[2] = {small, small};
  const void* pp[2] = {p, p};
  void* oo[2] = {p, p};
  CHECK(llvq_decode_many(many, 0, pp, pp, LLVQ_OUT_BF16, oo, nullptr, nullptr) == LLVQ_EINVAL);
  CHECK(llvq_decode_many(many, 17, pp, pp, LLVQ_OUT_BF16, oo, nullptr, nullptr) == LLVQ_EINVAL);
  CHECK(llvq_decode_many(many, 2, pp, nullptr, LLVQ_OUT_BF16, oo, nullptr, nullptr) == LLVQ_EINVAL);
  CHECK(llvq_decode_many(nullptr, 2, pp, pp, LLVQ_OUT_BF16, oo, nullptr, nullptr) == LLVQ_EINVAL);

  CHECK(llvq_encode_ref((const int8_t*)p, 10, 1, (uint64_t*)p, nullptr, nullptr) == LLVQ_EINVAL);
  CHECK(llvq_encode_ref((const int8_t*)p, -1, 10, (uint64_t*)p, nullptr, nullptr) == LLVQ_EINVAL);
  CHECK(llvq_encode_ref((const int8_t*)p, 10, 10, (uint64_t*)mis, nullptr, nullptr) == LLVQ_EINVAL);
  CHECK(llvq_encode_wide((const int8_t*)p, 10, 43, (uint64_t*)p, nullptr, nullptr) == LLVQ_EINVAL);
  CHECK(llvq_search((const float*)p, 10, 14, LLVQ_SEARCH_ANGULAR, (int8_t*)p, (uint64_t*)p, nullptr, nullptr) ==
        LLVQ_EINVAL);
  CHECK(llvq_search((const float*)p, 10, 10, 7, (int8_t*)p, (uint64_t*)p, nullptr, nullptr) == LLVQ_EINVAL);
  CHECK(llvq_search((const float*)mis, 10, 10, LLVQ_SEARCH_ANGULAR, (int8_t*)p, (uint64_t*)p, nullptr, nullptr) ==
        LLVQ_EINVAL);

  CHECK(llvq_quantize_workspace_bytes(&bad[0]) < 0);
  CHECK(llvq_quantize_workspace_bytes(&small) == (int64_t)((16 * 10 * 24 + 7) / 8 * 8 + 16 * 10 * 8));
  CHECK(llvq_quantize(&small, nullptr, p, p, p, nullptr, nullptr) == LLVQ_EINVAL);
  CHECK(llvq_quantize(&small, (const float*)p, p, p, mis, nullptr, nullptr) == LLVQ_EINVAL);
  llvq_desc huge = {LLVQ_MODE_SHAPEGAIN, 16385, 3072, 10, 44, 4};
  CHECK(llvq_quantize_noalloc(&huge, (const float*)p, p, p, nullptr, nullptr) == LLVQ_ETOOLARGE);
  CHECK(llvq_quantize_noalloc_max_blocks() == (1 << 21));
  CHECK(llvq_pack_fields(&small, nullptr, p, nullptr) == LLVQ_EINVAL);

  CHECK(llvq_gptq_workspace_bytes(0) == LLVQ_EINVAL);
  CHECK(llvq_gptq_workspace_bytes(240) == 240ll * 240 * 8 + 10 * 576 * 8 + 256);
  CHECK(llvq_gptq_factor(240, nullptr, 0.01, (double*)p, p, nullptr, nullptr) == LLVQ_EINVAL);
  CHECK(llvq_gptq_factor(240, (const double*)p, -0.5, (double*)p, p, nullptr, nullptr) == LLVQ_EINVAL);
  CHECK(llvq_gptq_begin(0, 240, (const float*)p, (double*)p, (float*)p, nullptr) == LLVQ_EINVAL);
  CHECK(llvq_gptq_column(&small, 10, 0, p, (double*)p, (const double*)p, (const int8_t*)p, (const uint64_t*)p,
                         (uint64_t*)p, (double*)p, (float*)p, nullptr) == LLVQ_EINVAL);
  CHECK(llvq_gptq_column(&small, 0, 3, p, (double*)p, (const double*)p, (const int8_t*)p, (const uint64_t*)p,
                         (uint64_t*)p, (double*)p, (float*)p, nullptr) == LLVQ_EINVAL);

  uint32_t f = 0;
  CHECK(llvq_device_checks(&f, 0) == LLVQ_EUNSUPPORTED);
  for (int c = 0; c >= -5; --c) CHECK(llvq_error_string(c) != nullptr && strlen(llvq_error_string(c)) > 0);
  printf("ok %d\n", g_checks);
  return 0;
}
