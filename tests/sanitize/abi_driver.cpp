// Host sanitizer driver for the C ABI's host side (test infrastructure).
//
// Linked with csrc/api.hip compiled with AddressSanitizer and
// UndefinedBehaviorSanitizer on its host code (tests/test_sanitizers.py). It
// drives every entry point's validation with NULL pointers, misaligned
// addresses, negative, zero and extreme sizes (where products of int32
// arguments overflow if not widened) and unknown widths, plus the host
// helpers. No call here passes validation with work to do, so no kernel is
// ever launched: the launch functions below are stand-ins that report a
// failure if they are reached.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include <hip/hip_runtime.h>

#include "../../include/kvq.h"
#include "../../kv_cache_quantization_row_amd/csrc/kernels.h"

static int reached = 0;
namespace kvq {
hipError_t launch_sym_quant(const SymQuantArgs &, int, int, hipStream_t) { ++reached; return hipErrorNotSupported; }
hipError_t launch_sym_dequant(const SymDequantArgs &, int, int, hipStream_t) { ++reached; return hipErrorNotSupported; }
hipError_t launch_kivi(const KiviArgs &, hipStream_t) { ++reached; return hipErrorNotSupported; }
hipError_t launch_kivi_unpack(KiviUnpackArgs, hipStream_t) { ++reached; return hipErrorNotSupported; }
hipError_t launch_nuq(const NuqArgs &, int, int, bool, hipStream_t) { ++reached; return hipErrorNotSupported; }
hipError_t launch_attn_decode(AttnArgs, hipStream_t) { ++reached; return hipErrorNotSupported; }
}  // namespace kvq

static int failures = 0;
#define EXPECT(call, status)                                                                       \
  do {                                                                                             \
    const int rc_ = (call);                                                                        \
    if (rc_ != (status)) {                                                                         \
      std::fprintf(stderr, "line %d: %s gave %d, expected %d (%s)\n", __LINE__, #call, rc_, (int)(status), \
                   kvq_last_error());                                                              \
      ++failures;                                                                                  \
    }                                                                                              \
    (void)std::strlen(kvq_last_error());                                                           \
  } while (0)

int main() {
  uint8_t *F = reinterpret_cast<uint8_t *>((uintptr_t)1 << 20);  // aligned, never dereferenced
  uint16_t *F16 = reinterpret_cast<uint16_t *>(F);
  float *Ff = reinterpret_cast<float *>(F);
  int32_t *Fi = reinterpret_cast<int32_t *>(F);
  int64_t *Fl = reinterpret_cast<int64_t *>(F);
  const int32_t big = INT32_MAX;

  // host helpers
  int32_t bits = 0;
  for (const char *m : {"q8", "q6", "q4", "8", "6", "4", "6bit", "int6", "uint6"}) EXPECT(kvq_parse_mode(m, &bits), KVQ_OK);
  for (const char *m : {"q6_k", "q6_0", "", "Q6", "q5", "q66", "int6 "}) EXPECT(kvq_parse_mode(m, &bits), KVQ_ERR_MODE);
  EXPECT(kvq_parse_mode(nullptr, &bits), KVQ_ERR_NULL);
  EXPECT(kvq_parse_mode("q8", nullptr), KVQ_ERR_NULL);
  for (int b : {-1, 0, 3, 5, 7, 8, 9, 16, big}) (void)kvq_sym_qmax(b);
  for (int D : {-big, -1, 0, 1, 2, 4, 6, 256, big})
    for (int b : {4, 6, 8, 5}) (void)kvq_packed_dim(D, b);
  (void)kvq_sym_cache_bytes(INT64_MAX / 4, big, big, big, 6);
  (void)kvq_sym_cache_bytes(-1, 16, 4, 256, 6);
  (void)kvq_sym_cache_bytes(262144, 16, 4, 256, 16);
  for (int64_t off : {(int64_t)0, (int64_t)1, (int64_t)200, INT64_MAX, (int64_t)-5})
    for (int r : {0, 128, big, -1})
      for (int g : {1, 32, big, 0, -3}) (void)kvq_kivi_boundary(off, r, g);
  (void)kvq_attn_workspace_bytes(big, big, big, big);
  (void)kvq_attn_workspace_bytes(-1, 4, 256, 100);
  for (int S : {1, 4096, big})
    for (int D : {32, 128, 256, 96})
      for (double f : {0.0, 0.01, 0.999, 1.0, -0.5}) {
        (void)kvq_nuq_outlier_bound(big, S, D, 0, 4, f, 1, 0);
        (void)kvq_nuq_outlier_bound(32, S, D, 7, big, f, 0, 1);
        (void)kvq_nuq_workspace_bytes(big, S, D, 3, 0, 4, f, 1);
        (void)kvq_nuq_workspace_bytes(65535, S, D, 4, 0, big, f, 0);
      }

  // symmetric
  kvq_paged_layout lay = {16, 1024, 16, 4, 256, 6};
  kvq_paged_layout bad = lay;
  EXPECT(kvq_quant_sym(nullptr, F16, F16, 0, 1, 16, Fi, F, F16, F, F16, nullptr), KVQ_ERR_NULL);
  bad.bits = 5;
  EXPECT(kvq_quant_sym(&bad, F16, F16, 0, 1, 16, Fi, F, F16, F, F16, nullptr), KVQ_ERR_BITS);
  bad = lay; bad.head_dim = 250;
  EXPECT(kvq_quant_sym(&bad, F16, F16, 0, 1, 16, Fi, F, F16, F, F16, nullptr), KVQ_ERR_SHAPE);
  bad = lay; bad.num_pages = big; bad.page_size = big;
  EXPECT(kvq_quant_sym(&bad, F16, F16, 0, 1, 16, Fi, F, F16, F, F16, nullptr), KVQ_ERR_SHAPE);
  EXPECT(kvq_quant_sym(&lay, F16, F16, big, big, 16, Fi, F, F16, F, F16, nullptr), KVQ_ERR_SHAPE);
  EXPECT(kvq_quant_sym(&lay, F16, F16, 0, 1, big, Fi, F, F16, F, F16, nullptr), KVQ_ERR_SHAPE);
  EXPECT(kvq_quant_sym(&lay, F16, F16, 0, 1, -1, Fi, F, F16, F, F16, nullptr), KVQ_ERR_SHAPE);
  EXPECT(kvq_quant_sym(&lay, F16 + 1, F16, 0, 1, 16, Fi, F, F16, F, F16, nullptr), KVQ_ERR_ALIGN);
  EXPECT(kvq_quant_sym(&lay, F16, nullptr, 0, 1, 16, Fi, F, F16, F, F16, nullptr), KVQ_ERR_NULL);
  EXPECT(kvq_quant_sym(&lay, F16, F16, 0, 0, 16, Fi, F, F16, F, F16, nullptr), KVQ_OK);
  EXPECT(kvq_dequant_sym(&lay, F, F16, F, F16, 0, 1, Fi, big, Fi, big, big, F16, F16, nullptr), KVQ_ERR_SHAPE);
  EXPECT(kvq_dequant_sym(&lay, F, F16, F, F16, 0, 1, Fi, -1, Fi, 4, 64, F16, F16, nullptr), KVQ_ERR_SHAPE);
  EXPECT(kvq_dequant_sym(&lay, F, F16, F, F16, 0, 1, nullptr, 4, Fi, 4, 64, F16, F16, nullptr), KVQ_ERR_NULL);
  EXPECT(kvq_dequant_sym(&lay, F, F16, F, F16, 0, 1, Fi, 4, Fi, 0, 64, F16, F16, nullptr), KVQ_OK);
  EXPECT(kvq_attn_decode_sym(&lay, F, F16, F, F16, 0, F16, big, Fi, 4, Fi, 4, 64, 0.1f, F16, F, 1 << 20, nullptr),
         KVQ_ERR_SHAPE);
  EXPECT(kvq_attn_decode_sym(&lay, F, F16, F, F16, 0, F16, 16, Fi, 4, Fi, big, big, 0.1f, F16, F, 16, nullptr),
         KVQ_ERR_SHAPE);
  EXPECT(kvq_attn_decode_sym(&lay, F, F16, F, F16, 0, F16, 16, Fi, 4, Fi, 16, big, 0.1f, F16, F, 16, nullptr),
         KVQ_ERR_CAPACITY);
  EXPECT(kvq_attn_decode_sym(&lay, F, F16, F, F16, 99, F16, 16, Fi, 4, Fi, 4, 64, 0.1f, F16, F, 1 << 20, nullptr),
         KVQ_ERR_SHAPE);

  // KIVI
  EXPECT(kvq_kivi_quant_dequant(F16, F16, big, big, big, big, 0, 8, 2, 32, 1e-8f, nullptr, nullptr, nullptr, nullptr,
                                nullptr, nullptr, nullptr),
         KVQ_ERR_SHAPE);
  EXPECT(kvq_kivi_quant_dequant(F16, F16, 2, 2, 64, 64, 0, 65, 2, 32, 1e-8f, nullptr, nullptr, nullptr, nullptr,
                                nullptr, nullptr, nullptr),
         KVQ_ERR_SHAPE);
  EXPECT(kvq_kivi_quant_dequant(F16, F16, 2, 2, 64, 64, 0, 32, 3, 32, 1e-8f, nullptr, nullptr, nullptr, nullptr,
                                nullptr, nullptr, nullptr),
         KVQ_ERR_BITS);
  EXPECT(kvq_kivi_quant_dequant(F16, F16, 2, 2, 64, 64, 0, 32, 2, 32, -1.0f, nullptr, nullptr, nullptr, nullptr,
                                nullptr, nullptr, nullptr),
         KVQ_ERR_ARG);
  EXPECT(kvq_kivi_quant_dequant(F16, F16, 0, 2, 64, 64, 0, 32, 2, 32, 1e-8f, nullptr, nullptr, nullptr, nullptr,
                                nullptr, nullptr, nullptr),
         KVQ_OK);
  EXPECT(kvq_kivi_pack(F16, F16, big, big, big, 64, 0, big, 2, 32, 1e-8f, F, F16, F16, F, F16, F16, big, 0, nullptr),
         KVQ_ERR_SHAPE);
  EXPECT(kvq_kivi_pack(F16, F16, 2, 2, 64, 64, 32, 64, 2, 32, 1e-8f, F, F16, F16, F, F16, F16, big, big, nullptr),
         KVQ_ERR_SHAPE);
  EXPECT(kvq_kivi_pack(F16, F16, 0, 2, 64, 64, 32, 64, 2, 32, 1e-8f, F, F16, F16, F, F16, F16, 32, 32, nullptr),
         KVQ_OK);
  EXPECT(kvq_kivi_unpack(F, F16, F16, F, F16, F16, 2, 2, 64, 64, 0, 64, 4, 32, F16, F16, big, big, nullptr),
         KVQ_ERR_SHAPE);
  EXPECT(kvq_kivi_unpack(F, F16, F16, F, F16, F16, big, big, big, 64, 0, 8, 4, 32, F16, F16, 8, 0, nullptr),
         KVQ_ERR_SHAPE);

  // NUQ
  EXPECT(kvq_nuq_fit_quant(F16, F16, big, big, 128, 0, 3, 0.01, 8, 4, 1, Ff, F16, Ff, F, F, Fi, F16, Fi, F16,
                           INT64_MAX, Fl, nullptr, nullptr, F, INT64_MAX, nullptr),
         KVQ_ERR_SHAPE);
  EXPECT(kvq_nuq_fit_quant(F16, F16, 32, 64, 128, 0, 3, 1.0, 8, 4, 1, Ff, F16, Ff, F, F, Fi, F16, Fi, F16,
                           INT64_MAX, Fl, nullptr, nullptr, F, INT64_MAX, nullptr),
         KVQ_ERR_ARG);
  EXPECT(kvq_nuq_fit_quant(F16, F16, 32, 64, 128, 0, 3, 0.01, 8, 4, 1, Ff, F16, Ff, F, F, Fi, F16, Fi, F16, 0, Fl,
                           nullptr, nullptr, F, INT64_MAX, nullptr),
         KVQ_ERR_CAPACITY);
  EXPECT(kvq_nuq_fit_quant(F16, F16, 32, 64, 128, big, 3, 0.01, big, big, 0, Ff, F16, Ff, F, F, Fi, F16, Fi, F16,
                           INT64_MAX, Fl, nullptr, nullptr, F, INT64_MAX, nullptr),
         KVQ_ERR_ARG);
  EXPECT(kvq_nuq_fit_quant_noalloc(F16, F16, 64, 2000, 128, 5, 3, 0.5, 8, 4, 0, Ff, F16, Ff, F, F, Fi, F16, Fi,
                                   F16, INT64_MAX, Fl, nullptr, nullptr, nullptr),
         KVQ_ERR_CAPACITY);
  EXPECT(kvq_nuq_fit_quant_noalloc(F16, F16, 2, 64, 96, 0, 3, 0.01, 8, 4, 1, Ff, F16, Ff, F, F, Fi, F16, Fi, F16,
                                   INT64_MAX, Fl, nullptr, nullptr, nullptr),
         KVQ_ERR_SHAPE);
  EXPECT(kvq_nuq_fit_quant_noalloc(nullptr, F16, 2, 64, 128, 0, 3, 0.01, 8, 4, 1, Ff, F16, Ff, F, F, Fi, F16, Fi,
                                   F16, INT64_MAX, Fl, nullptr, nullptr, nullptr),
         KVQ_ERR_NULL);

  if (reached) {
    std::fprintf(stderr, "%d calls reached a kernel launch\n", reached);
    ++failures;
  }
  if (failures) return 1;
  std::printf("abi driver ok\n");
  return 0;
}
