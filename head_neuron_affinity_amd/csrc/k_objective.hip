// The layout objective of "Affinity-Aware Sharding for Delayed Tensor
// Parallelism", section 3, paragraph "Objective", eq. (6): every score matrix
// normalised to unit mass, and J = the sum over the N up-edge and N-1
// down-edge matrices of their co-located fractions (the mass on entries whose
// KV-group device equals the neuron device; the down edge of layer i uses the
// head devices of layer i+1).
//   unit_mass_kernel    out = S / sum(S) per matrix
//   colocation_kernel   one workgroup per matrix: total and co-located mass
//   objective_sum       J = fractions summed in matrix order
// Sums run in fp64 in a fixed order (per-thread strided sums, a fixed
// butterfly in each wave, then the waves in order), so results are
// reproducible bit for bit.  Device ids are only
// compared, never used as indices.
#include "hna_internal.h"

namespace hna {
namespace {

constexpr int kOThreads = 1024;

// fixed-order sum of one double per thread over the workgroup: each wave sums
// its lanes by a fixed butterfly, then the per-wave sums are added in wave
// order.  Returns the total in every thread.
__device__ inline double block_sum(double v, double* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  double t = 0.0;
  for (int i = 0; i < kOThreads / 64; ++i) t += red[i];
  __syncthreads();
  return t;
}

__global__ __launch_bounds__(kOThreads) void unit_mass_kernel(const float* S, int64_t count,
                                                              float* out) {
  __shared__ double red[kOThreads / 64];
  const int64_t base = (int64_t)blockIdx.x * count;
  double s = 0.0;
  for (int64_t e = threadIdx.x; e < count; e += kOThreads) s += (double)S[base + e];
  const double tot = block_sum(s, red);
  // every read above precedes every write below (out may alias S)
  for (int64_t e = threadIdx.x; e < count; e += kOThreads)
    out[base + e] = tot != 0.0 ? (float)((double)S[base + e] / tot) : 0.f;
}

struct Mat {
  const float* S;
  const int32_t* dr;  // row devices
  const int32_t* dc;  // column devices
  int rows, cols;
};

// matrix m < N: up edge of layer m, [G][I] with row devices heads[m] and
// column devices neurons[m]; matrix N + i: down edge of layer i, [I][G] with
// row devices neurons[i] and column devices heads[i + 1]
__device__ inline Mat matrix_of(int m, const float* S_up, const float* S_down,
                                const int32_t* heads, const int32_t* neurons, int N, int G,
                                int I) {
  if (m < N)
    return {S_up + (int64_t)m * G * I, heads + (int64_t)m * G, neurons + (int64_t)m * I, G, I};
  const int i = m - N;
  return {S_down + (int64_t)i * I * G, neurons + (int64_t)i * I, heads + (int64_t)(i + 1) * G, I,
          G};
}

// One workgroup per matrix.  VEC: four consecutive entries per thread and
// iteration (cols % 4 == 0, so they share a row and 16-byte alignment).
template <bool VEC>
__global__ __launch_bounds__(kOThreads) void colocation_kernel(const float* __restrict__ S_up,
                                                               const float* __restrict__ S_down,
                                                               const int32_t* __restrict__ heads,
                                                               const int32_t* __restrict__ neurons,
                                                               int N, int G, int I,
                                                               double* frac_up, double* frac_down) {
  __shared__ double red[kOThreads / 64];
  const int m = blockIdx.x;
  const Mat M = matrix_of(m, S_up, S_down, heads, neurons, N, G, I);
  const int64_t n = (int64_t)M.rows * M.cols;
  constexpr int W = VEC ? 4 : 1;
  // (r, c) of flat index e, advanced by kOThreads * W entries per iteration
  const int step = kOThreads * W;
  const int step_r = step / M.cols, step_c = step % M.cols;
  int r = (int)(threadIdx.x * W) / M.cols, c = (int)(threadIdx.x * W) % M.cols;
  double tot = 0.0, col = 0.0;
  for (int64_t e = threadIdx.x * W; e < n; e += step) {
    if constexpr (VEC) {
      const float4 v = *reinterpret_cast<const float4*>(M.S + e);
      const int4 d = *reinterpret_cast<const int4*>(M.dc + c);
      const int dr = M.dr[r];
      const double x = v.x, y = v.y, z = v.z, w = v.w;
      tot += ((x + y) + z) + w;
      col += (d.x == dr ? x : 0.0) + (d.y == dr ? y : 0.0) + (d.z == dr ? z : 0.0) +
             (d.w == dr ? w : 0.0);
    } else {
      const double v = (double)M.S[e];
      tot += v;
      if (M.dr[r] == M.dc[c]) col += v;
    }
    r += step_r;
    c += step_c;
    if (c >= M.cols) {
      c -= M.cols;
      ++r;
    }
  }
  tot = block_sum(tot, red);
  col = block_sum(col, red);
  if (threadIdx.x == 0) {
    const double f = tot != 0.0 ? col / tot : 0.0;
    if (m < N) frac_up[m] = f;
    else frac_down[m - N] = f;
  }
}

// J = frac_up[0..N) then frac_down[0..N-1) added one by one in that order;
// the loads are spread over one wave and staged in LDS.
constexpr int kMaxJTerms = 4096;
__global__ __launch_bounds__(64) void objective_sum_kernel(const double* frac_up,
                                                           const double* frac_down, int N,
                                                           double* J) {
  __shared__ double f[kMaxJTerms];
  const int n = 2 * N - 1;
  for (int i = threadIdx.x; i < n; i += 64) f[i] = i < N ? frac_up[i] : frac_down[i - N];
  __syncthreads();
  if (threadIdx.x != 0) return;
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += f[i];
  *J = s;
}

}  // namespace

hipError_t launch_unit_mass(const float* S, int64_t count, int n_mat, float* out, hipStream_t st) {
  if (count == 0 || n_mat == 0) return hipSuccess;
  hipLaunchKernelGGL(unit_mass_kernel, dim3(n_mat), dim3(kOThreads), 0, st, S, count, out);
  return hipGetLastError();
}

int max_objective_layers() { return (kMaxJTerms + 1) / 2; }

hipError_t launch_layout_objective(const float* S_up, const float* S_down, const int32_t* heads,
                                   const int32_t* neurons, int N, int G, int I, double* frac_up,
                                   double* frac_down, double* J, hipStream_t st) {
  // the vector path needs 16-byte aligned rows of both edges
  const bool vec = G % 4 == 0 && I % 4 == 0;
  if (vec)
    hipLaunchKernelGGL(colocation_kernel<true>, dim3(2 * N - 1), dim3(kOThreads), 0, st, S_up,
                       S_down, heads, neurons, N, G, I, frac_up, frac_down);
  else
    hipLaunchKernelGGL(colocation_kernel<false>, dim3(2 * N - 1), dim3(kOThreads), 0, st, S_up,
                       S_down, heads, neurons, N, G, I, frac_up, frac_down);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(objective_sum_kernel, dim3(1), dim3(64), 0, st, frac_up, frac_down, N, J);
  return hipGetLastError();
}

}  // namespace hna
