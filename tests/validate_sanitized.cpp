// Host-only driver for the argument validation of libswiglu (validate.hpp),
// built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_validate_sanitized.py.  It calls every validator over a grid of
// sizes that includes the extremes of int64 (negative, zero, the layout
// limits, 2^31 and beyond) and over null, aligned and misaligned pointers, so
// any signed overflow, shift or out-of-bounds access in the validation
// arithmetic is reported by the sanitizers (which abort the run).  It also
// checks a table of expected status codes, one per error path.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include <limits>
#include <vector>

#include "validate.hpp"

namespace {

int failures = 0;

void expect(int got, int want, const char* what, int line) {
  if (got != want) {
    fprintf(stderr, "line %d: %s: got %d, want %d\n", line, what, got, want);
    ++failures;
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

const void* const A = reinterpret_cast<const void*>(uintptr_t(0x10000));    // 256-aligned, never dereferenced
const void* const MIS = reinterpret_cast<const void*>(uintptr_t(0x10008));  // 8-aligned only
void* const WA = const_cast<void*>(A);
const float* const FA = static_cast<const float*>(A);

int in_range(int st) { return st >= SWIGLU_OK && st <= SWIGLU_ERR_SCRATCH; }

void table() {
  using namespace swg;
  const int64_t lim = kMaxLd;
  // forward
  EXPECT(validate_fwd(SWIGLU_BF16, 4, 64, 8, A, A, A, A), SWIGLU_OK);
  EXPECT(validate_fwd(7, 4, 64, 8, A, A, A, A), SWIGLU_ERR_DTYPE);
  EXPECT(validate_fwd(SWIGLU_BF16, -1, 64, 8, A, A, A, A), SWIGLU_ERR_SHAPE);
  EXPECT(validate_fwd(SWIGLU_BF16, 4, 64, 12, A, A, A, A), SWIGLU_ERR_SHAPE);
  EXPECT(validate_fwd(SWIGLU_F32, 4, 64, 6, A, A, A, A), SWIGLU_ERR_SHAPE);
  EXPECT(validate_fwd(SWIGLU_F32, 4, 64, lim + 4, A, A, A, A), SWIGLU_ERR_UNSUPPORTED);
  EXPECT(validate_fwd(SWIGLU_BF16, 4, 64, lim, A, A, A, A), SWIGLU_OK);
  EXPECT(validate_fwd(SWIGLU_BF16, 4, 64, 8, A, A, A, nullptr), SWIGLU_ERR_NULL);
  EXPECT(validate_fwd(SWIGLU_BF16, 4, 64, 8, MIS, A, A, A), SWIGLU_ERR_ALIGN);
  EXPECT(validate_fwd(SWIGLU_BF16, 0, 64, 8, nullptr, nullptr, nullptr, nullptr), SWIGLU_OK);
  EXPECT(validate_fwd(SWIGLU_BF16, int64_t(1) << 31, 64, 8, A, A, A, A), SWIGLU_ERR_SHAPE);
  // backward
  const BwdLayout L = bwd_layout(SWIGLU_BF16, 4, 64, 8);
  EXPECT(validate_bwd(SWIGLU_BF16, 4, 64, 8, A, A, A, A, WA, WA, WA, A, L.total), SWIGLU_OK);
  EXPECT(validate_bwd(SWIGLU_BF16, 4, 64, 8, A, A, A, A, WA, WA, WA, A, L.total - 1), SWIGLU_ERR_WORKSPACE);
  EXPECT(validate_bwd(SWIGLU_BF16, 4, 64, 8, A, A, A, A, WA, WA, WA, nullptr, 0), SWIGLU_ERR_WORKSPACE);
  EXPECT(validate_bwd(SWIGLU_BF16, 4, 64, 8, A, A, A, A, WA, WA, WA, MIS, L.total), SWIGLU_ERR_ALIGN);
  EXPECT(validate_bwd(SWIGLU_BF16, 4, 64, 8, A, A, A, nullptr, WA, WA, WA, A, L.total), SWIGLU_ERR_NULL);
  EXPECT(validate_bwd(SWIGLU_F32, lim + 8, 4, 8, A, A, A, A, WA, WA, WA, A, ~size_t(0)), SWIGLU_ERR_UNSUPPORTED);
  EXPECT(validate_bwd(SWIGLU_F32, 4, lim / 2 + 8, 8, A, A, A, A, WA, WA, WA, A, ~size_t(0)), SWIGLU_ERR_UNSUPPORTED);
  EXPECT(validate_bwd(SWIGLU_BF16, 4, 64, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0),
         SWIGLU_OK);
  EXPECT((int)(bwd_workspace_total(SWIGLU_BF16, (int64_t(1) << 31) - 1, (int64_t(1) << 31) - 1, 8) == 0), 1);
  EXPECT((int)(bwd_workspace_total(SWIGLU_BF16, 4, 64, 12) == 0), 1);
  EXPECT((int)(bwd_workspace_total(SWIGLU_BF16, 4, 64, 8) == L.total), 1);
  // decode
  EXPECT(validate_gemv(9, 64, 8, A, A, A, A), SWIGLU_ERR_SHAPE);
  EXPECT(validate_gemv(8, 64, 12, A, A, A, A), SWIGLU_ERR_SHAPE);
  EXPECT(validate_gemv(2, 64, 8, A, A, A, nullptr), SWIGLU_ERR_NULL);
  EXPECT(validate_gemv(2, 64, 8, A, A, A, MIS), SWIGLU_ERR_ALIGN);
  EXPECT(validate_gemv(8, 64, 4096, A, A, A, A), SWIGLU_OK);
  // FP8-output forward
  EXPECT(validate_fwd_fp8(4, 48, 8, A, A, A, A, A, nullptr), SWIGLU_ERR_SHAPE);
  EXPECT(validate_fwd_fp8(4, 64, 8, A, A, A, A, nullptr, nullptr), SWIGLU_ERR_NULL);
  EXPECT(validate_fwd_fp8(4, 64, 8, A, A, A, A, A, MIS), SWIGLU_ERR_ALIGN);
  EXPECT(validate_fwd_fp8(4, 64, lim + 8, A, A, A, A, A, nullptr), SWIGLU_ERR_UNSUPPORTED);
  // elementwise
  EXPECT(validate_act_fwd(SWIGLU_F32, 4, 12, FA, FA, INFINITY, A, nullptr), SWIGLU_ERR_SHAPE);
  EXPECT(validate_act_fwd(SWIGLU_F32, 4, 16, FA, FA, NAN, A, nullptr), SWIGLU_ERR_ARG);
  EXPECT(validate_act_fwd(SWIGLU_F32, 4, 16, FA, FA, -1.0f, A, nullptr), SWIGLU_ERR_ARG);
  EXPECT(validate_act_fwd(SWIGLU_F32, 4, 16, FA, FA, 7.0f, A, MIS), SWIGLU_OK);          // count: 8-byte aligned
  EXPECT(validate_act_fwd(SWIGLU_F32, int64_t(1) << 30, int64_t(1) << 20, FA, FA, 7.0f, A, nullptr), SWIGLU_ERR_SHAPE);
  EXPECT(validate_act_quant(4, 48, FA, FA, 7.0f, A, A, nullptr, nullptr), SWIGLU_ERR_SHAPE);
  EXPECT(validate_act_quant(4, 64, FA, FA, 7.0f, A, nullptr, nullptr, nullptr), SWIGLU_ERR_NULL);
  EXPECT(validate_act_quant(4, 64, FA, FA, 7.0f, A, A, nullptr, MIS), SWIGLU_ERR_ALIGN);
  EXPECT(validate_act_quant(0, 64, nullptr, nullptr, 7.0f, nullptr, nullptr, nullptr, nullptr), SWIGLU_OK);
  EXPECT(validate_act_bwd(SWIGLU_BF16, 4, 12, A, A, A, nullptr, 7.0f, WA, WA, nullptr), SWIGLU_ERR_SHAPE);
  EXPECT(validate_act_bwd(SWIGLU_F32, 4, 12, A, A, A, nullptr, 0.0f, WA, WA, nullptr), SWIGLU_ERR_ARG);
  EXPECT(validate_act_bwd(SWIGLU_F32, 4, 12, A, A, A, nullptr, 7.0f, nullptr, WA, nullptr), SWIGLU_ERR_NULL);
  EXPECT(validate_act_bwd(SWIGLU_F32, 4, 12, A, A, A, reinterpret_cast<const float*>(uintptr_t(0x10002)), 7.0f, WA,
                          WA, nullptr), SWIGLU_ERR_ALIGN);
}

// Every validator over the whole grid: only the absence of sanitizer reports
// and a status in range are required here.
void grid() {
  using namespace swg;
  const int64_t big = std::numeric_limits<int64_t>::max();
  const std::vector<int64_t> dims = {std::numeric_limits<int64_t>::min(), -(int64_t(1) << 40), -1, 0, 1, 4, 8, 31, 32,
                                     4096, kMaxLd - 8, kMaxLd, kMaxLd + 8, (int64_t(1) << 31) - 1, int64_t(1) << 31,
                                     int64_t(1) << 40, big};
  const std::vector<const void*> ptrs = {nullptr, A, MIS};
  const std::vector<float> limits = {-1.0f, 0.0f, 0.5f, 7.0f, INFINITY, NAN};
  long calls = 0;
  for (int dt : {-1, (int)SWIGLU_F32, (int)SWIGLU_BF16, 2})
    for (int64_t M : dims)
      for (int64_t N : dims)
        for (int64_t K : dims) {
          for (const void* p : ptrs) {
            int st = validate_fwd(dt, M, N, K, p, A, A, A);
            st |= !in_range(validate_fwd(dt, M, N, K, A, A, A, p)) << 8;
            if (!in_range(st & 0xFF) || (st >> 8)) { fprintf(stderr, "fwd status out of range\n"); ++failures; }
            for (size_t ws : {size_t(0), size_t(1) << 20, ~size_t(0)}) {
              const int b = validate_bwd(dt, M, N, K, A, A, A, A, WA, WA, WA, p, ws);
              if (!in_range(b)) { fprintf(stderr, "bwd status out of range\n"); ++failures; }
            }
            if (dt == SWIGLU_BF16) {
              if (!in_range(validate_fwd_fp8(M, N, K, A, A, A, WA, p, nullptr))) ++failures;
              if (M >= -1 && M <= 9 && !in_range(validate_gemv(M, N, K, A, A, A, p))) ++failures;
            }
            calls += 4;
          }
          // The workspace size is 0 for every shape the backward rejects,
          // and for the others its regions are ordered (no size wrapped).
          const size_t total = bwd_workspace_total(dt, M, N, K);
          if (bwd_shape_status(dt, M, N, K) != SWIGLU_OK) {
            if (total != 0) { fprintf(stderr, "workspace size for a rejected shape\n"); ++failures; }
          } else {
            const BwdLayout L = bwd_layout(dt, M, N, K);
            if (L.total != total || L.total < L.off_wt || L.off_wt < L.off_xt || L.off_xt < L.off_dt ||
                L.off_dt < L.off_d) {
              fprintf(stderr, "workspace layout not ordered\n");
              ++failures;
            }
          }
        }
  for (int dt : {-1, (int)SWIGLU_F32, (int)SWIGLU_BF16})
    for (int64_t R : dims)
      for (int64_t C : dims)
        for (float lim : limits)
          for (const void* p : ptrs) {
            const float* fp = static_cast<const float*>(p);
            if (!in_range(validate_act_fwd(dt, R, C, FA, fp, lim, A, p))) ++failures;
            if (!in_range(validate_act_quant(R, C, fp, FA, lim, A, p, p, p))) ++failures;
            if (!in_range(validate_act_bwd(dt, R, C, p, A, A, fp, lim, WA, WA, reinterpret_cast<float*>(WA))))
              ++failures;
            calls += 3;
          }
  printf("grid: %ld validator calls\n", calls);
}

}  // namespace

int main() {
  table();
  grid();
  if (failures) {
    fprintf(stderr, "%d failures\n", failures);
    return 1;
  }
  printf("validate: ok\n");
  return 0;
}
