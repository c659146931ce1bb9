// The C ABI's argument contract (include/ecc.h), exercised on the CPU against
// the stubs in hip_stubs.cpp: every entry point rejects what the header says
// it rejects, with the status it names and a message, and hands the launcher
// exactly the shape, sizes, strides and workspace layout of the call.  Built
// with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitized.py.  Device pointers are fake addresses: the host
// code must never dereference them.  Host arrays (shapes) are heap-allocated
// with their exact length, so a read past their end is reported.

#include <math.h>
#include <stdio.h>
#include <string.h>

#include <memory>

#include "ecc.h"
#include "ecc_internal.hpp"

namespace stub {
extern ecc::HardArgs hard;
extern ecc::SoftArgs soft;
extern ecc::GradArgs grad;
extern ecc::HeightArgs height;
extern int hard_calls, soft_calls, grad_calls, height_calls, height_bwd_calls, static_calls;
extern hipError_t next_error;
extern void* const kStaticWs;
}  // namespace stub

static int failures = 0;

#define CHECK(cond)                                                          \
  do {                                                                       \
    if (!(cond)) {                                                           \
      fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);        \
      ++failures;                                                            \
    }                                                                        \
  } while (0)

// status of `expr` is `want`; a failure comes with a non-empty message
#define STATUS(expr, want)                                                                         \
  do {                                                                                             \
    const int s_ = (expr);                                                                         \
    if (s_ != (want)) {                                                                            \
      fprintf(stderr, "FAIL %s:%d: %s -> %d, want %d (%s)\n", __FILE__, __LINE__, #expr, s_, (want), \
              ecc_last_error());                                                                   \
      ++failures;                                                                                  \
    } else if ((want) != ECC_OK && ecc_last_error()[0] == 0) {                                     \
      fprintf(stderr, "FAIL %s:%d: %s gave no message\n", __FILE__, __LINE__, #expr);              \
      ++failures;                                                                                  \
    }                                                                                              \
  } while (0)

namespace {

const void* const G = reinterpret_cast<const void*>(0x1000);
const float* const GF = reinterpret_cast<const float*>(0x1000);
const float* const T = reinterpret_cast<const float*>(0x2000);
int64_t* const O = reinterpret_cast<int64_t*>(0x3000);
float* const OF = reinterpret_cast<float*>(0x3000);
void* const WS = reinterpret_cast<void*>(0x4000);
const float* const GO = reinterpret_cast<const float*>(0x6000);
const size_t BIG = (size_t)1 << 40;

// a host shape array of exactly n entries
std::unique_ptr<int64_t[]> shape(std::initializer_list<int64_t> v) {
  std::unique_ptr<int64_t[]> s(new int64_t[v.size()]);
  size_t i = 0;
  for (int64_t x : v) s[i++] = x;
  return s;
}

void hard() {
  const size_t need = ecc::workspace_bytes(300);
  STATUS(ecc_hard_2d(nullptr, ECC_F32, 4, 5, T, 300, O, WS, need, nullptr), ECC_E_NULL);
  STATUS(ecc_hard_2d(G, ECC_F32, 4, 5, nullptr, 300, O, WS, need, nullptr), ECC_E_NULL);
  STATUS(ecc_hard_2d(G, ECC_F32, 4, 5, T, 300, nullptr, WS, need, nullptr), ECC_E_NULL);
  STATUS(ecc_hard_2d(G, 2, 4, 5, T, 300, O, WS, need, nullptr), ECC_E_DTYPE);
  STATUS(ecc_hard_2d(G, -1, 4, 5, T, 300, O, WS, need, nullptr), ECC_E_DTYPE);
  STATUS(ecc_hard_2d(G, ECC_F32, 0, 5, T, 300, O, WS, need, nullptr), ECC_E_SHAPE);
  STATUS(ecc_hard_2d(G, ECC_F32, 4, -5, T, 300, O, WS, need, nullptr), ECC_E_SHAPE);
  // products that overflow 64 bits are caught before they are formed
  STATUS(ecc_hard_3d(G, ECC_F32, (int64_t)1 << 40, (int64_t)1 << 40, (int64_t)1 << 40, T, 300, O, WS, need,
                     nullptr),
         ECC_E_SHAPE);
  STATUS(ecc_hard_3d(G, ECC_F32, INT64_MAX, INT64_MAX, INT64_MAX, T, 300, O, WS, need, nullptr), ECC_E_SHAPE);
  STATUS(ecc_hard_3d(G, ECC_F32, 1, (int64_t)1 << 20, ((int64_t)1 << 20) + 1, T, 300, O, WS, need, nullptr),
         ECC_E_SHAPE);
  STATUS(ecc_hard_2d(G, ECC_F32, 4, 5, T, 0, O, WS, need, nullptr), ECC_E_NTHRESH);
  STATUS(ecc_hard_2d(G, ECC_F32, 4, 5, T, ECC_MAX_THRESHOLDS + 1, O, WS, BIG, nullptr), ECC_E_NTHRESH);
  STATUS(ecc_hard_2d(G, ECC_F32, 4, 5, T, 300, O, nullptr, need, nullptr), ECC_E_WORKSPACE);
  STATUS(ecc_hard_2d(G, ECC_F32, 4, 5, T, 300, O, WS, need - 1, nullptr), ECC_E_WORKSPACE);
  CHECK(stub::hard_calls == 0);

  STATUS(ecc_hard_2d(G, ECC_U8, 4, 5, T, 300, O, WS, need, nullptr), ECC_OK);
  CHECK(stub::hard_calls == 1);
  CHECK(stub::hard.grid == G && stub::hard.dtype == ECC_U8 && stub::hard.tau == T && stub::hard.out == O);
  CHECK(stub::hard.nz == 1 && stub::hard.ny == 4 && stub::hard.nx == 5 && stub::hard.H == 300);
  CHECK(stub::hard.ws == WS && stub::hard.batch == 1 && stub::hard.acc_copies == ecc::kAccCopies);
  STATUS(ecc_hard_3d(G, ECC_F32, 3, 4, 5, T, 1, O, WS, ecc::workspace_bytes(1), nullptr), ECC_OK);
  CHECK(stub::hard.nz == 3 && stub::hard.ny == 4 && stub::hard.nx == 5 && stub::hard.H == 1);
  // the largest grid the ABI takes, 2^40 voxels
  STATUS(ecc_hard_3d(G, ECC_F32, 1 << 14, 1 << 13, 1 << 13, T, 8, O, WS, ecc::workspace_bytes(8), nullptr),
         ECC_OK);
  STATUS(ecc_hard_3d(G, ECC_F32, (1 << 14) + 1, 1 << 13, 1 << 13, T, 8, O, WS, BIG, nullptr), ECC_E_SHAPE);

  // a launch error surfaces as ECC_E_HIP with the runtime's text
  stub::next_error = hipErrorLaunchFailure;
  STATUS(ecc_hard_2d(G, ECC_F32, 4, 5, T, 300, O, WS, need, nullptr), ECC_E_HIP);
  CHECK(strstr(ecc_last_error(), "stubbed HIP error") != nullptr);
  // ... and the next good call clears the message
  STATUS(ecc_hard_2d(G, ECC_F32, 4, 5, T, 300, O, WS, need, nullptr), ECC_OK);
  CHECK(ecc_last_error()[0] == 0);
}

void hard_static() {
  const int before = stub::hard_calls;
  STATUS(ecc_hard_3d_static(G, ECC_F32, 2, 3, 4, T, ECC_MAX_THRESHOLDS + 1, O, nullptr), ECC_E_NTHRESH);
  CHECK(strstr(ecc_last_error(), "8193") != nullptr);
  STATUS(ecc_hard_3d_static(nullptr, ECC_F32, 2, 3, 4, T, 4, O, nullptr), ECC_E_NULL);
  CHECK(stub::static_calls == 0 && stub::hard_calls == before);
  STATUS(ecc_hard_3d_static(G, ECC_F32, 2, 3, 4, T, ECC_MAX_THRESHOLDS, O, nullptr), ECC_OK);
  CHECK(stub::static_calls == 1 && stub::hard.ws == stub::kStaticWs && stub::hard.H == ECC_MAX_THRESHOLDS);
  CHECK(ecc::workspace_bytes(ECC_MAX_THRESHOLDS) <= ecc::kStaticWorkspaceBytes);
}

void hard_batched() {
  const int64_t B = 5;
  const size_t need = ecc_workspace_bytes_batched(ECC_OP_HARD, B, 64);
  CHECK(need == (size_t)B * ecc::batch_ws_stride(64, B));
  STATUS(ecc_hard_3d_batched(G, ECC_F32, 0, 2, 3, 4, T, 0, 64, O, WS, need, nullptr), ECC_E_SHAPE);
  STATUS(ecc_hard_3d_batched(G, ECC_F32, B, 2, 3, 4, T, -1, 64, O, WS, need, nullptr), ECC_E_SHAPE);
  STATUS(ecc_hard_3d_batched(G, ECC_F32, (int64_t)1 << 38, 2, 3, 4, T, 0, 64, O, WS, BIG, nullptr), ECC_E_SHAPE);
  STATUS(ecc_hard_3d_batched(G, ECC_F32, INT64_MAX, 1, 1, 1, T, 0, 64, O, WS, BIG, nullptr), ECC_E_SHAPE);
  STATUS(ecc_hard_3d_batched(G, ECC_F32, B, 2, 3, 4, T, 0, 64, O, WS, need - 1, nullptr), ECC_E_WORKSPACE);
  STATUS(ecc_hard_3d_batched(G, ECC_F32, B, 2, 3, 4, T, 0, 64, O, nullptr, need, nullptr), ECC_E_WORKSPACE);
  STATUS(ecc_hard_3d_batched(G, ECC_F32, B, 2, 3, 4, T, 64, 64, O, WS, need, nullptr), ECC_OK);
  CHECK(stub::hard.batch == B && stub::hard.tau_stride == 64 && stub::hard.nz == 2);
  CHECK(stub::hard.ws_stride == ecc::batch_ws_stride(64, B) && stub::hard.acc_copies == ecc::batch_copies(B));
  STATUS(ecc_hard_2d_batched(G, ECC_U8, B, 3, 4, T, 0, 64, O, WS, need, nullptr), ECC_OK);
  CHECK(stub::hard.nz == 1 && stub::hard.ny == 3 && stub::hard.nx == 4 && stub::hard.tau_stride == 0);
}

void soft() {
  const size_t need = ecc::workspace_bytes(100);
  auto s3 = shape({3, 4, 5});
  auto s2 = shape({6, 7});
  STATUS(ecc_soft_fwd(GF, 3, nullptr, T, 100, 10.0f, OF, WS, need, nullptr), ECC_E_NULL);
  STATUS(ecc_soft_fwd(nullptr, 3, s3.get(), T, 100, 10.0f, OF, WS, need, nullptr), ECC_E_NULL);
  STATUS(ecc_soft_fwd(GF, 3, s3.get(), T, 100, 10.0f, nullptr, WS, need, nullptr), ECC_E_NULL);
  STATUS(ecc_soft_fwd(GF, 1, s3.get(), T, 100, 10.0f, OF, WS, need, nullptr), ECC_E_SHAPE);
  STATUS(ecc_soft_fwd(GF, 4, s3.get(), T, 100, 10.0f, OF, WS, need, nullptr), ECC_E_SHAPE);
  auto bad = shape({3, 0, 5});
  STATUS(ecc_soft_fwd(GF, 3, bad.get(), T, 100, 10.0f, OF, WS, need, nullptr), ECC_E_SHAPE);
  auto huge = shape({INT64_MAX, INT64_MAX, 2});
  STATUS(ecc_soft_fwd(GF, 3, huge.get(), T, 100, 10.0f, OF, WS, need, nullptr), ECC_E_SHAPE);
  for (float lam : {0.0f, -1.0f, INFINITY, -INFINITY, NAN})
    STATUS(ecc_soft_fwd(GF, 3, s3.get(), T, 100, lam, OF, WS, need, nullptr), ECC_E_LAMBDA);
  STATUS(ecc_soft_fwd(GF, 3, s3.get(), T, 0, 10.0f, OF, WS, need, nullptr), ECC_E_NTHRESH);
  STATUS(ecc_soft_fwd(GF, 3, s3.get(), T, 100, 10.0f, OF, WS, need - 8, nullptr), ECC_E_WORKSPACE);
  CHECK(stub::soft_calls == 0);

  STATUS(ecc_soft_fwd(GF, 3, s3.get(), T, 100, 10.0f, OF, WS, need, nullptr), ECC_OK);
  CHECK(stub::soft.nz == 3 && stub::soft.ny == 4 && stub::soft.nx == 5 && stub::soft.grad_out == nullptr);
  CHECK(stub::soft.H == 100 && stub::soft.lambda == 10.0f && stub::soft.out == OF && stub::soft.sum_batch == 0);
  STATUS(ecc_soft_fwd(GF, 2, s2.get(), T, 100, 0.5f, OF, WS, need, nullptr), ECC_OK);
  CHECK(stub::soft.nz == 1 && stub::soft.ny == 6 && stub::soft.nx == 7);

  STATUS(ecc_soft_bwd_tau(GF, 3, s3.get(), T, 100, 10.0f, nullptr, OF, WS, need, nullptr), ECC_E_NULL);
  STATUS(ecc_soft_bwd_tau(GF, 3, s3.get(), T, 100, 10.0f, GO, OF, WS, need, nullptr), ECC_OK);
  CHECK(stub::soft.grad_out == GO);

  STATUS(ecc_soft_bwd_grid(GF, 3, s3.get(), T, 100, 10.0f, nullptr, OF, nullptr), ECC_E_NULL);
  STATUS(ecc_soft_bwd_grid(GF, 3, s3.get(), T, 100, NAN, GO, OF, nullptr), ECC_E_LAMBDA);
  STATUS(ecc_soft_bwd_grid(GF, 2, s2.get(), T, 100, 10.0f, GO, OF, nullptr), ECC_OK);
  CHECK(stub::grad_calls == 1 && stub::grad.nz == 1 && stub::grad.ny == 6 && stub::grad.nx == 7);
  CHECK(stub::grad.batch == 1 && stub::grad.grad_out == GO && stub::grad.out == OF);
}

void soft_batched() {
  const int64_t B = 70;
  auto s3 = shape({3, 4, 5});
  const size_t need = ecc_workspace_bytes_batched(ECC_OP_SOFT_BWD, B, 100);
  STATUS(ecc_soft_fwd_batched(GF, 3, s3.get(), 0, T, 0, 100, 1.0f, OF, WS, need, nullptr), ECC_E_SHAPE);
  STATUS(ecc_soft_fwd_batched(GF, 3, s3.get(), B, T, -3, 100, 1.0f, OF, WS, need, nullptr), ECC_E_SHAPE);
  STATUS(ecc_soft_fwd_batched(GF, 3, s3.get(), B, T, 0, 100, 1.0f, OF, WS, need - 1, nullptr), ECC_E_WORKSPACE);
  STATUS(ecc_soft_fwd_batched(GF, 3, s3.get(), B, T, 100, 100, 1.0f, OF, WS, need, nullptr), ECC_OK);
  CHECK(stub::soft.batch == B && stub::soft.tau_stride == 100 && stub::soft.ws_stride == ecc::batch_ws_stride(100, B));
  STATUS(ecc_soft_bwd_tau_batched(GF, 3, s3.get(), B, T, 0, 100, 1.0f, nullptr, OF, WS, need, nullptr), ECC_E_NULL);
  STATUS(ecc_soft_bwd_tau_batched(GF, 3, s3.get(), B, T, 0, 100, 1.0f, GO, OF, WS, need, nullptr), ECC_OK);
  CHECK(stub::soft.sum_batch == 0 && stub::soft.grad_out == GO);

  STATUS(ecc_soft_bwd_tau_shared(GF, 3, s3.get(), B, T, 100, 1.0f, nullptr, OF, WS, need, nullptr), ECC_E_NULL);
  STATUS(ecc_soft_bwd_tau_shared(GF, 3, s3.get(), 0, T, 100, 1.0f, GO, OF, WS, need, nullptr), ECC_E_SHAPE);
  STATUS(ecc_soft_bwd_tau_shared(GF, 3, s3.get(), B, T, 100, 1.0f, GO, OF, WS, need - 1, nullptr), ECC_E_WORKSPACE);
  STATUS(ecc_soft_bwd_tau_shared(GF, 3, s3.get(), B, T, 100, 1.0f, GO, OF, WS, need, nullptr), ECC_OK);
  CHECK(stub::soft.sum_batch == B && stub::soft.batch == B && stub::soft.tau_stride == 0);
  CHECK(stub::soft.ws == WS && stub::soft.ws_stride == ecc::batch_ws_stride(100, B));
  // every grid's slice holds its H float64 partial sums
  CHECK(ecc::batch_ws_stride(100, B) >= ecc::kWsHeader + 100 * sizeof(double));
  CHECK(ecc::batch_ws_stride(8192, 1 << 20) >= ecc::kWsHeader + 8192 * sizeof(double));

  STATUS(ecc_soft_bwd_grid_batched(GF, 3, s3.get(), B, T, 7, 100, 1.0f, GO, OF, nullptr), ECC_OK);
  CHECK(stub::grad.batch == B && stub::grad.tau_stride == 7);
}

void heights() {
  auto s3 = shape({3, 4, 5});
  const float* U = reinterpret_cast<const float*>(0x7000);
  const float* A = reinterpret_cast<const float*>(0x8000);
  STATUS(ecc_height(GF, 3, s3.get(), U, A, 0, OF, nullptr), ECC_E_NDIRS);
  STATUS(ecc_height(GF, 3, s3.get(), U, A, ECC_MAX_DIRECTIONS + 1, OF, nullptr), ECC_E_NDIRS);
  STATUS(ecc_height(GF, 3, s3.get(), nullptr, A, 2, OF, nullptr), ECC_E_NULL);
  auto wide = shape({1, 1, ECC_MAX_AXIS + 1});
  STATUS(ecc_height(GF, 3, wide.get(), U, A, 2, OF, nullptr), ECC_E_SHAPE);
  auto many = shape({1 << 14, 1 << 14, 1 << 12});
  STATUS(ecc_height(GF, 3, many.get(), U, A, 2, OF, nullptr), ECC_E_SHAPE);
  STATUS(ecc_height(GF, 3, s3.get(), U, A, 2, OF, nullptr), ECC_OK);
  CHECK(stub::height_calls == 1 && stub::height.nd == 3 && stub::height.nz == 3 && stub::height.D == 2);
  const size_t hw = ecc_height_workspace_bytes(3, 2);
  CHECK(hw == ecc::height_workspace_bytes(3, 2) && hw > 0);
  CHECK(ecc_height_workspace_bytes(4, 2) == 0 && ecc_height_workspace_bytes(3, 0) == 0);
  float* GD = reinterpret_cast<float*>(0x9000);
  float* GA = reinterpret_cast<float*>(0xa000);
  STATUS(ecc_height_bwd(GF, 3, s3.get(), U, A, 2, OF, GD, nullptr, WS, hw, nullptr), ECC_E_NULL);
  STATUS(ecc_height_bwd(GF, 3, s3.get(), U, A, 2, OF, GD, GA, nullptr, hw, nullptr), ECC_E_WORKSPACE);
  STATUS(ecc_height_bwd(GF, 3, s3.get(), U, A, 2, OF, GD, GA, WS, hw - 1, nullptr), ECC_E_WORKSPACE);
  STATUS(ecc_height_bwd(GF, 3, s3.get(), U, A, 2, OF, nullptr, nullptr, nullptr, 0, nullptr), ECC_OK);
  STATUS(ecc_height_bwd(GF, 3, s3.get(), U, A, 2, nullptr, GD, GA, WS, hw, nullptr), ECC_OK);
  CHECK(stub::height_bwd_calls == 2 && stub::height.grad_grid == nullptr && stub::height.grad_dirs == GD);
}

void sizes_and_strings() {
  CHECK(ecc_workspace_bytes(3, 3, nullptr, 10) == 0);
  CHECK(ecc_workspace_bytes(ECC_OP_HARD, 3, nullptr, 0) == 0);
  CHECK(ecc_workspace_bytes(ECC_OP_HARD, 3, nullptr, ECC_MAX_THRESHOLDS + 1) == 0);
  CHECK(ecc_workspace_bytes(ECC_OP_SOFT_BWD, 2, nullptr, 300) == ecc::workspace_bytes(300));
  CHECK(ecc_workspace_bytes_batched(ECC_OP_HARD, 0, 10) == 0);
  CHECK(ecc_workspace_bytes_batched(ECC_OP_HARD, -5, 10) == 0);
  CHECK(ecc_workspace_bytes_batched(ECC_OP_HARD, INT64_MAX, 10) == 0);
  CHECK(ecc_workspace_bytes_batched(-1, 3, 10) == 0);
  for (int st = ECC_OK; st <= ECC_E_NDIRS; ++st) {
    const char* s = ecc_status_string(st);
    CHECK(s != nullptr && s[0] != 0 && strcmp(s, "unknown status") != 0);
  }
  CHECK(strcmp(ecc_status_string(99), "unknown status") == 0);
  CHECK(strcmp(ecc_status_string(-1), "unknown status") == 0);
  CHECK(ecc_version() != nullptr && ecc_version()[0] != 0);
}

}  // namespace

int main() {
  hard();
  hard_static();
  hard_batched();
  soft();
  soft_batched();
  heights();
  sizes_and_strings();
  if (failures) {
    fprintf(stderr, "%d contract check(s) failed\n", failures);
    return 1;
  }
  printf("abi contract: all checks passed\n");
  return 0;
}
