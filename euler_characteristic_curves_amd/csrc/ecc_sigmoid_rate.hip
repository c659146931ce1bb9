// Sigmoid-rate ceiling of the soft sweep, for the benchmark only (built into
// its own small library, libecc_sigmoid_rate.so; the ECC library does not use it).
//
// The soft curve sums sign * sigma(lambda (tau_k - v)) over (term, threshold)
// pairs ("Scalable GPU-Accelerated Euler Characteristic Curves", Method: the
// sigmoid relaxation of the indicator and its analytic backward).  The sweep
// evaluates each pair with the factored exponent t = F E (F per term, E per
// threshold): forward sigma = 1 / (1 + t) accumulated in float64, backward
// w sigma (1 - sigma) = (w F) (E sigma) sigma.  This kernel runs exactly that
// per-pair arithmetic with every operand in registers (no term loads, no LDS,
// no reduction), so its rate is the ceiling the sweep's pair loop can reach on
// this GPU: pairs / second = workgroups * 256 * iters * 8 / time.

#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kThreads = 256;
constexpr int kSlots = 8;  // thresholds per lane, as in the sweep

template <bool BWD>
__global__ __launch_bounds__(kThreads) void sigmoid_rate_kernel(double* out, int iters) {
  const int t = (int)(blockIdx.x * kThreads + threadIdx.x);
  float e[kSlots];
  double acc[kSlots];
#pragma unroll
  for (int r = 0; r < kSlots; ++r) {
    e[r] = 1.0f + 1e-3f * (float)(t & 7) + 1e-4f * (float)r;
    acc[r] = 0.0;
  }
  float a = 0.5f + 1e-7f * (float)(t & 1023);
  const double w = (t & 1) ? 1.0 : -1.0;
  for (int i = 0; i < iters; ++i) {
    // one term per iteration: its weight products once, then one pair per slot
    const double wf = w * (double)a;
#pragma unroll
    for (int r = 0; r < kSlots; ++r) {
      const float d = fmaf(a, e[r], 1.0f);
      const float rr = __builtin_amdgcn_rcpf(d);
      if constexpr (!BWD) {
        acc[r] = fma(w, (double)rr, acc[r]);
      } else {
        const float q = (e[r] * rr) * rr;
        acc[r] = fma(wf, (double)q, acc[r]);
      }
    }
    a = a * 0.9999f;  // the next term's factor
  }
  double s = 0.0;
#pragma unroll
  for (int r = 0; r < kSlots; ++r) s += acc[r];
  out[t] = s;
}

}  // namespace

// Runs `blocks` workgroups of 256 threads, each thread `iters` x 8 pairs;
// out holds blocks * 256 doubles (device memory, written, never read here).
// Returns the HIP error code of the launch (0 on success).
extern "C" int ecc_sigmoid_rate(int bwd, int blocks, int iters, double* out, void* stream) {
  if (blocks < 1 || iters < 1 || out == nullptr) return (int)hipErrorInvalidValue;
  auto s = reinterpret_cast<hipStream_t>(stream);
  if (bwd)
    hipLaunchKernelGGL(sigmoid_rate_kernel<true>, dim3((unsigned)blocks), dim3(kThreads), 0, s, out, iters);
  else
    hipLaunchKernelGGL(sigmoid_rate_kernel<false>, dim3((unsigned)blocks), dim3(kThreads), 0, s, out, iters);
  return (int)hipGetLastError();
}
