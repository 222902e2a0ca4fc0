// Host-side argument checks of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code (tests/test_host_sanitizers.py).
// No GPU is needed: every call here is rejected by its argument checks (or is
// a size query), so nothing reaches a kernel launch. The sanitizers catch an
// out-of-bounds host access, an integer overflow or any other undefined
// behaviour on these paths; the expected status codes are checked too.
#include <stdint.h>
#include <stdio.h>

#include "specverify.h"

static int g_failures = 0;
static int g_checks = 0;

#define CHECK(cond)                                                  \
  do {                                                               \
    ++g_checks;                                                      \
    if (!(cond)) {                                                   \
      ++g_failures;                                                  \
      fprintf(stderr, "check failed, line %d: %s\n", __LINE__, #cond); \
    }                                                                \
  } while (0)

// A pointer that is never dereferenced on the paths exercised here, 256-byte aligned.
static void* const FAKE = reinterpret_cast<void*>(static_cast<uintptr_t>(1) << 20);
#define FI reinterpret_cast<int32_t*>(FAKE)
#define FF reinterpret_cast<float*>(FAKE)

static const int32_t kSizes[] = {INT32_MIN, -1, 0, 1, 2, 7, 8, 63, 64, 1023, 1024, 1025, 65535, 1 << 20, INT32_MAX};
static const int kDtypes[] = {-1, 0, 1, 2, 99};

static sv_status chain(const void* t, const void* d, int dt, const int32_t* x, const float* u, int32_t B, int32_t K,
                       int32_t V, int32_t* acc, int32_t* out, void* ws, size_t wsb) {
  return sv_verify_chain(t, d, static_cast<sv_dtype>(dt), x, nullptr, u, B, K, V, acc, out, nullptr, nullptr, nullptr,
                         nullptr, nullptr, ws, wsb, nullptr);
}

int main() {
  // status strings, in and out of range
  for (int c = -5; c <= 10; ++c) CHECK(sv_status_string(static_cast<sv_status>(c)) != nullptr);

  // every size query over extreme sizes: no overflow, 0 for what is invalid
  for (int32_t a : kSizes)
    for (int32_t b : kSizes)
      for (int32_t v : kSizes)
        for (int dt : kDtypes) {
          const sv_dtype d = static_cast<sv_dtype>(dt);
          const size_t w1 = sv_chain_workspace_bytes(a, b, v, d);
          const size_t w2 = sv_tree_workspace_bytes(a, b, v, d);
          const size_t w3 = sv_tree_sampling_workspace_bytes(a, b, v, d);
          const int32_t l1 = sv_chain_launches(a, b, v, d, 1, 0);
          const int32_t l2 = sv_chain_form(a, b, v, d, 0, 1);
          if (a < 0 || b < 0 || v < 1 || (dt != 0 && dt != 1)) CHECK(w1 == 0 && w2 == 0 && w3 == 0);
          CHECK(l1 >= 0 && l1 <= 2 && l2 >= 0 && l2 <= 3);
          if (dt == 1) {
            (void)sv_lm_head_chain_workspace_bytes(a, b, v, a);
            (void)sv_sample_workspace_bytes(a, v, d);
          }
        }

  // chain verification: each required pointer, sizes, dtype, alignment, workspace
  CHECK(chain(nullptr, FAKE, 1, FI, FF, 4, 2, 128, FI, FI, FAKE, 1 << 20) == SV_ERR_INVALID_ARGUMENT);
  CHECK(chain(FAKE, nullptr, 1, FI, FF, 4, 2, 128, FI, FI, FAKE, 1 << 20) == SV_ERR_INVALID_ARGUMENT);
  CHECK(chain(FAKE, FAKE, 1, nullptr, FF, 4, 2, 128, FI, FI, FAKE, 1 << 20) == SV_ERR_INVALID_ARGUMENT);
  CHECK(chain(FAKE, FAKE, 1, FI, nullptr, 4, 2, 128, FI, FI, FAKE, 1 << 20) == SV_ERR_INVALID_ARGUMENT);
  CHECK(chain(FAKE, FAKE, 1, FI, FF, 4, 2, 128, FI, nullptr, FAKE, 1 << 20) == SV_ERR_INVALID_ARGUMENT);
  CHECK(chain(FAKE, FAKE, 1, FI, FF, 4, 64, 128, FI, FI, FAKE, 1 << 20) == SV_ERR_INVALID_ARGUMENT);
  CHECK(chain(FAKE, FAKE, 1, FI, FF, 4, 2, 0, FI, FI, FAKE, 1 << 20) == SV_ERR_INVALID_ARGUMENT);
  CHECK(chain(FAKE, FAKE, 1, FI, FF, -1, 2, 128, FI, FI, FAKE, 1 << 20) == SV_ERR_INVALID_ARGUMENT);
  CHECK(chain(FAKE, FAKE, 7, FI, FF, 4, 2, 128, FI, FI, FAKE, 1 << 20) == SV_ERR_INVALID_ARGUMENT);
  CHECK(chain(static_cast<char*>(FAKE) + 1, FAKE, 1, FI, FF, 4, 2, 128, FI, FI, FAKE, 1 << 20) ==
        SV_ERR_INVALID_ARGUMENT);
  CHECK(chain(FAKE, FAKE, 1, FI, FF, 4, 2, 128, FI, FI, nullptr, 1 << 20) == SV_ERR_WORKSPACE);
  CHECK(chain(FAKE, FAKE, 1, FI, FF, 4, 2, 128, FI, FI, FAKE, 16) == SV_ERR_WORKSPACE);
  CHECK(chain(nullptr, nullptr, 1, nullptr, nullptr, 0, 2, 128, nullptr, nullptr, nullptr, 0) == SV_OK);
  for (int32_t b : kSizes)
    for (int32_t v : kSizes) {
      // sizes that pass the checks are stopped by the too-small workspace (16 bytes)
      const sv_status st = chain(FAKE, FAKE, 1, FI, FF, b, 3, v, FI, FI, FAKE, 16);
      CHECK(st == SV_OK || st == SV_ERR_INVALID_ARGUMENT || st == SV_ERR_UNSUPPORTED || st == SV_ERR_WORKSPACE);
    }

  // the no-allocation chain call: oversize and bad sizes rejected before any device call
  CHECK(sv_verify_chain_noalloc(nullptr, nullptr, SV_DTYPE_BF16, nullptr, nullptr, nullptr, 256, 63, 256000, FI,
                                nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == SV_ERR_UNSUPPORTED);
  CHECK(sv_verify_chain_noalloc(nullptr, nullptr, SV_DTYPE_BF16, nullptr, nullptr, nullptr, 4, 64, 100, FI, nullptr,
                                nullptr, nullptr, nullptr, nullptr, nullptr, nullptr) == SV_ERR_INVALID_ARGUMENT);

  // greedy tree, mask, sampling tree, draft-side sampling
  CHECK(sv_verify_tree_greedy(FAKE, SV_DTYPE_BF16, nullptr, FI, 4, 8, 100, FI, FI, FI, nullptr, FAKE, 1 << 20,
                              nullptr) == SV_ERR_INVALID_ARGUMENT);
  CHECK(sv_verify_tree_greedy(FAKE, SV_DTYPE_BF16, FI, FI, 4, 1025, 100, FI, FI, FI, nullptr, FAKE, 1 << 20,
                              nullptr) == SV_ERR_INVALID_ARGUMENT);
  CHECK(sv_verify_tree_greedy(FAKE, SV_DTYPE_BF16, FI, FI, 4, 8, 100, FI, FI, FI, nullptr, FAKE, 8, nullptr) ==
        SV_ERR_WORKSPACE);
  CHECK(sv_build_tree_mask(nullptr, 4, reinterpret_cast<uint8_t*>(FAKE), nullptr, nullptr) == SV_ERR_INVALID_ARGUMENT);
  CHECK(sv_build_tree_mask(FI, 0, reinterpret_cast<uint8_t*>(FAKE), nullptr, nullptr) == SV_ERR_INVALID_ARGUMENT);
  CHECK(sv_build_tree_mask(FI, 1025, reinterpret_cast<uint8_t*>(FAKE), nullptr, nullptr) == SV_ERR_INVALID_ARGUMENT);
  for (int32_t n : kSizes)
    for (int32_t v : kSizes) {
      const sv_status st = sv_verify_tree_sampling(FAKE, FAKE, SV_DTYPE_BF16, FI, FI, nullptr, FF, 4, n, v, FI, FI, FI,
                                                   nullptr, FAKE, 16, nullptr);
      CHECK(st != SV_OK && st != SV_ERR_HIP);
      const sv_status s2 = sv_sample_rows(FAKE, SV_DTYPE_BF16, nullptr, FF, n, v, FI, nullptr, nullptr, FAKE, 16,
                                          nullptr);
      CHECK(s2 != SV_ERR_HIP);
    }
  CHECK(sv_sample_rows(nullptr, SV_DTYPE_BF16, nullptr, FF, 4, 100, FI, nullptr, nullptr, FAKE, 1 << 20, nullptr) ==
        SV_ERR_INVALID_ARGUMENT);

  // LM-head calls: sizes, pointers, workspace
  CHECK(sv_lm_head_logits(FAKE, FAKE, 4, 63, 128, FAKE, nullptr) == SV_ERR_INVALID_ARGUMENT);   // H % 64
  CHECK(sv_lm_head_logits(FAKE, FAKE, 4, 64, 12, FAKE, nullptr) == SV_ERR_INVALID_ARGUMENT);    // V % 8
  CHECK(sv_lm_head_logits(FAKE, FAKE, -1, 64, 128, FAKE, nullptr) == SV_ERR_INVALID_ARGUMENT);
  CHECK(sv_lm_head_logits(nullptr, FAKE, 4, 64, 128, FAKE, nullptr) == SV_ERR_INVALID_ARGUMENT);
  CHECK(sv_lm_head_logits(FAKE, FAKE, 0, 64, 128, FAKE, nullptr) == SV_OK);
  for (int32_t m : kSizes)
    for (int32_t h : kSizes) {
      const sv_status st = sv_lm_head_logits(FAKE, FAKE, m, h, INT32_MAX, FAKE, nullptr);
      CHECK(st == SV_ERR_INVALID_ARGUMENT || st == SV_ERR_UNSUPPORTED || st == SV_OK);
      const sv_status s2 = sv_verify_chain_lm_head(FAKE, FAKE, h, FAKE, FAKE, FI, nullptr, FF, m, 3, 1024, FI, FI,
                                                   nullptr, nullptr, nullptr, nullptr, FAKE, 16, nullptr);
      CHECK(s2 != SV_ERR_HIP && (s2 != SV_OK || m == 0));  // B = 0: nothing to do
    }

  // the profiling hook: one event without the other is rejected, arming and disarming touch nothing
  CHECK(sv_time_next_stream_pass(reinterpret_cast<hipEvent_t>(FAKE), nullptr) == SV_ERR_INVALID_ARGUMENT);
  CHECK(sv_time_next_stream_pass(reinterpret_cast<hipEvent_t>(FAKE), reinterpret_cast<hipEvent_t>(FAKE)) == SV_OK);
  CHECK(chain(nullptr, FAKE, 1, FI, FF, 4, 2, 128, FI, FI, FAKE, 1 << 20) == SV_ERR_INVALID_ARGUMENT);  // disarms
  CHECK(sv_time_next_stream_pass(nullptr, nullptr) == SV_OK);

  printf("%d checks, %d failed\n", g_checks, g_failures);
  return g_failures == 0 ? 0 : 1;
}
