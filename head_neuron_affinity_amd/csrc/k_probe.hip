// Measurement aid: the sustained bf16 rate of the matrix cores on this device,
// the second reference (besides the published dense peak) against which the
// affinity kernel's MFMA rate is read.  Every wave runs rounds of four
// independent 32x32x16 (or 16x16x32) bf16 MFMAs, accumulator k taking operand
// pair k from the caller's buffer; with random operands the power draw, and
// so the clock, is that of real data.  Nothing of the method is computed
// here.
#include "hna_internal.h"

namespace hna {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

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

// The same with 16x16x32 bf16 MFMAs: half the FLOP per instruction, so eight
// independent accumulators (operand pair k % 4) keep the FLOP per round equal
// to the 32x32x16 form and give the pipeline enough independent work.
__global__ __launch_bounds__(256) void mfma_rate16_kernel(const uint4* __restrict__ seed, int iters,
                                                          float* __restrict__ out) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  uint4 a[4], b[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    a[k] = seed[gid * 8 + 2 * k];
    b[k] = seed[gid * 8 + 2 * k + 1];
  }
  f32x4 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[k & 3]),
                                                       __builtin_bit_cast(bf16x8, b[k & 3]), acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e) s += acc[k][e];
  out[gid] = s;
}

}  // namespace

hipError_t launch_mfma_rate(const void* seed, int n_wg, int iters, int shape, float* out,
                            hipStream_t st) {
  if (shape == 1)
    hipLaunchKernelGGL(mfma_rate16_kernel, dim3(n_wg), dim3(256), 0, st,
                       static_cast<const uint4*>(seed), iters, out);
  else
    hipLaunchKernelGGL(mfma_rate_kernel, dim3(n_wg), dim3(256), 0, st, static_cast<const uint4*>(seed),
                       iters, out);
  return hipGetLastError();
}

}  // namespace hna
