// Measurement aid: the sustained bf16 rate of the matrix cores on this device,
// the second reference (besides the published dense peak) against which the
// affinity kernel's MFMA rate is read.  Every wave runs rounds of four
// independent 32x32x16 bf16 MFMAs, accumulator k taking operand pair k from
// the caller's buffer; with random operands the power draw, and so the clock,
// is that of real data.  Nothing of the method is computed here.
#include "hna_internal.h"

namespace hna {
namespace {

__global__ __launch_bounds__(256) void mfma_rate_kernel(const uint4* __restrict__ seed, int iters,
                                                        float* __restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint4 a[4][1], b[4][1];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    a[k][0] = seed[gid * 8 + 2 * k];
    b[k][0] = seed[gid * 8 + 2 * k + 1];
  }
  f32x16 acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) acc[k] = f32x16{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 4; ++k) mma(acc[k], a[k], b[k]);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[k][e];
  out[gid] = s;
}

}  // namespace

hipError_t launch_mfma_rate(const void* seed, int n_wg, int iters, float* out, hipStream_t st) {
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(n_wg), dim3(256), 0, st, static_cast<const uint4*>(seed),
                     iters, out);
  return hipGetLastError();
}

}  // namespace hna
