// Host-side exercise of the C ABI (include/mapl.h) for a build of the
// library's host code with AddressSanitizer and UndefinedBehaviorSanitizer:
// every entry point is called with invalid arguments (each must return its
// documented status before touching memory), with extreme sizes (the size
// arithmetic must not overflow), and with valid shapes (which stop at the
// device set-up when there is no device).  No pointer passed here is ever
// dereferenced on the host.  Exit status 0 means every expectation held.
#include <cstdint>
#include <cstdio>
#include <limits>

#include "mapl.h"

static int failures = 0;

static void expect(int got, int want, const char* what) {
  if (got != want) {
    std::fprintf(stderr, "FAIL %s: got %d want %d\n", what, got, want);
    ++failures;
  }
}

static void expect_in(int got, int a, int b, const char* what) {
  if (got != a && got != b) {
    std::fprintf(stderr, "FAIL %s: got %d want %d or %d\n", what, got, a, b);
    ++failures;
  }
}

int main() {
  void* F = reinterpret_cast<void*>(uintptr_t(0x100000));  // never dereferenced
  int32_t* Fi = static_cast<int32_t*>(F);
  float* Ff = static_cast<float*>(F);
  uint8_t* Fu = static_cast<uint8_t*>(F);
  const int64_t big = std::numeric_limits<int64_t>::max();
  const int64_t small = std::numeric_limits<int64_t>::min();

  for (int s = 0; s >= -8; --s) (void)mapl_status_string(s);
  (void)mapl_version();
  (void)mapl_init();

  // sizes: extreme arguments must give 0 (invalid) without overflowing
  const int64_t xs[] = {0, 1, 32, 128, 1024, big, small, -1};
  for (int64_t a : xs)
    for (int64_t b : xs) {
      (void)mapl_pack_bytes(a, b, b, MAPL_BF16);
      (void)mapl_bwd_workspace_bytes(a, b, 1024, 128, 128, MAPL_BF16);
      (void)mapl_bwd_workspace_bytes(8, 2048, a, b, 128, MAPL_F32);
      (void)mapl_anchor_grad_workspace_bytes(a, b, 128, 32000);
      (void)spel_workspace_bytes(a, b);
    }

  // codec: invalid arguments
  const size_t pkb = mapl_pack_bytes(1024, 128, 128, MAPL_BF16);
  expect(mapl_compress(nullptr, Fi, F, F, F, F, 8, 2048, 1024, 128, 128, 32000, MAPL_BF16, F, pkb, 1, nullptr),
         MAPL_ERR_NULL, "compress X null");
  expect(mapl_compress(F, Fi, F, F, F, F, big, big, 1024, 128, 128, 32000, MAPL_BF16, F, pkb, 1, nullptr),
         MAPL_ERR_SHAPE, "compress B*T overflow");
  expect(mapl_compress(F, Fi, F, F, F, F, 8, 2048, big, 128, 128, 32000, MAPL_BF16, F, pkb, 1, nullptr),
         MAPL_ERR_SHAPE, "compress huge d");
  expect(mapl_compress(F, Fi, F, F, F, F, 8, 2048, 1024, 128, 128, 32000, MAPL_BF16, F, 0, 1, nullptr),
         MAPL_ERR_WORKSPACE, "compress small pack");
  expect(mapl_reconstruct(F, Fi, F, F, F, F, 8, 2048, 1024, 96, 96, 32000, MAPL_BF16, F, pkb, 1, nullptr),
         MAPL_ERR_SHAPE, "reconstruct r = 96 (bf16 takes powers of two)");
  expect(mapl_reconstruct_bwd(F, F, F, F, Ff, 2, 8, 2048, 1024, 128, MAPL_BF16, F, pkb, 1, F, 1, nullptr),
         MAPL_ERR_ARG, "reconstruct_bwd accumulate = 2");
  expect(mapl_compress_bwd(F, F, Fi, F, F, F, F, Ff, 0, 8, 2048, 1024, 128, 128, 32000, MAPL_BF16, F, pkb, 1, F, 0,
                           nullptr),
         MAPL_ERR_WORKSPACE, "compress_bwd small workspace");
  expect(mapl_anchor_grad(F, Fi, F, Ff, std::numeric_limits<float>::quiet_NaN(), 0, 8, 2048, 1024, 128, 128, 32000,
                          MAPL_BF16, F, pkb, 1, F, 1 << 30, nullptr),
         MAPL_ERR_ARG, "anchor_grad alpha NaN");
  expect(mapl_check_tids(Fi, big, 10, Fi, nullptr), MAPL_ERR_SHAPE, "check_tids huge N");

  // valid shapes: with no device they stop at the device set-up
  const size_t bws = mapl_bwd_workspace_bytes(8, 2048, 1024, 128, 128, MAPL_BF16);
  expect_in(mapl_compress(F, Fi, F, F, F, F, 8, 2048, 1024, 128, 128, 32000, MAPL_BF16, F, pkb, 1, nullptr),
            MAPL_ERR_HIP, MAPL_OK, "compress valid");
  expect_in(mapl_compress_bwd(F, F, Fi, F, F, F, F, Ff, 1, 8, 2048, 1024, 128, 128, 32000, MAPL_BF16, F, pkb, 1, F,
                              bws, nullptr),
            MAPL_ERR_HIP, MAPL_OK, "compress_bwd valid");

  // rvq
  expect(rvq_encode(F, MAPL_BF16, Ff, 0, Fu, 16384, 256, 8, 0, 2, nullptr), MAPL_ERR_SHAPE, "rvq K = 0");
  expect(rvq_encode(F, MAPL_BF16, Ff, big - 3, Fu, 16384, 256, 8, 256, 2, nullptr), MAPL_ERR_ARG,
         "rvq huge round stride");
  expect(rvq_encode(F, MAPL_BF16, Ff, 0, Fu, big, 256, 8, 256, 2, nullptr), MAPL_ERR_SHAPE, "rvq huge N");
  expect(rvq_decode(Fu, Ff, 0, F, MAPL_F32, 16384, 256, 8, 256, 65, nullptr), MAPL_ERR_SHAPE, "rvq R = 65");
  expect(rvq_stream_apply(Ff, Fi, Ff, -1, 256, 8, 256, 1, nullptr), MAPL_ERR_SHAPE, "stream n < 0");
  expect(rvq_stream_decode(Ff, 0, 1, Fi, Ff, -1, Fu, F, MAPL_F32, 16384, 256, 8, 256, 2, nullptr), MAPL_ERR_SHAPE,
         "stream+decode n < 0");
  expect(rvq_stream_decode(Ff, big - 3, 1, Fi, Ff, 8, Fu, F, MAPL_F32, 16384, 256, 8, 256, 2, nullptr), MAPL_ERR_ARG,
         "stream+decode huge round stride");
  expect_in(rvq_stream_decode(Ff, 0, 1, Fi, Ff, 8, Fu, F, MAPL_BF16, 16384, 256, 8, 256, 2, nullptr), MAPL_ERR_HIP,
            MAPL_OK, "stream+decode valid");
  expect_in(rvq_encode(F, MAPL_BF16, Ff, 0, Fu, 16384, 256, 128, 17, 2, nullptr), MAPL_ERR_HIP, MAPL_OK,
            "rvq valid K = 17");

  // spel
  const size_t sws = spel_workspace_bytes(1024, 128);
  expect(spel_step(Ff, Ff, Ff, 1e-3f, 0.9f, 8, nullptr, nullptr, big, 128, F, sws, nullptr), MAPL_ERR_SHAPE,
         "spel huge d");
  expect(spel_step_static(Ff, Ff, Ff, 1e-3f, 0.9f, 8, nullptr, nullptr, 4096, 256, nullptr), MAPL_ERR_WORKSPACE,
         "spel_step_static beyond its scratch");
  expect(spel_step_polar_express(Ff, Ff, Ff, 1e-3f, 0.9f, 5, 7, 0.f, nullptr, nullptr, 1024, 128, F, sws, nullptr),
         MAPL_ERR_ARG, "polar express ell = 0");
  double coef[96], err[32];
  expect(spel_polar_express_coefficients(1e-3, 32, coef, err), MAPL_OK, "polar express schedule");
  expect_in(spel_step(Ff, Ff, Ff, 1e-3f, 0.9f, 8, nullptr, nullptr, 1024, 128, F, sws, nullptr), MAPL_ERR_HIP,
            MAPL_OK, "spel valid");

  if (failures) std::fprintf(stderr, "%d failure(s)\n", failures);
  else std::printf("abi driver: all expectations held\n");
  return failures ? 1 : 0;
}
