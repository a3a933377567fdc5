// Small bandwidth-bound kernels around the two matrix-core passes:
//   * ||w^d_k||^2, the squared norms of W_down's columns (section 3,
//     "Affinity scores": the FO score's write-size factor);
//   * the down edge's group sum n[g', k] over the q/k/v row segments of each
//     next-layer KV group, and S_down[k, g'] = c_k n[g', k].
#include "hna_internal.h"

namespace hna {
namespace {

// out[k] = sum_r W[r][k]^2 for a row-major [rows, cols] matrix.
// Scalar form (any column count): 64 columns per block, 4 row lanes; the 4
// lane sums are added in fixed order.
template <int BF16>
__global__ __launch_bounds__(256) void col_sqnorm_kernel(const void* __restrict__ Wv, int rows,
                                                         int cols, float* __restrict__ out) {
  __shared__ float part[4][64];
  const int cx = threadIdx.x & 63, ry = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + cx;
  float s = 0.f;
  if (c < cols) {
    for (int r = ry; r < rows; r += 4) {
      float v;
      if (BF16)
        v = bf16_bits_to_f32(static_cast<const uint16_t*>(Wv)[(int64_t)r * cols + c]);
      else
        v = static_cast<const float*>(Wv)[(int64_t)r * cols + c];
      s = fmaf(v, v, s);
    }
  }
  part[ry][cx] = s;
  __syncthreads();
  if (ry == 0 && c < cols) out[c] = (part[0][cx] + part[1][cx]) + (part[2][cx] + part[3][cx]);
}

// Vector form (16-byte aligned rows): a block covers 4 groups of EPC columns
// (one 16-byte load each) x 64 row lanes, several rows in flight per thread;
// the 64 lane sums of a column are added in a fixed tree order.
template <int BF16>
__global__ __launch_bounds__(256) void col_sqnorm16_kernel(const void* __restrict__ Wv, int rows,
                                                           int cols, float* __restrict__ out) {
  constexpr int EPC = BF16 ? 8 : 4;
  __shared__ float part[64][4 * EPC + 1];
  const int cg = threadIdx.x & 3, rl = threadIdx.x >> 2;
  const int c0 = (blockIdx.x * 4 + cg) * EPC;
  float acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
  if (c0 < cols) {
    const char* base = static_cast<const char*>(Wv) + (int64_t)c0 * (BF16 ? 2 : 4);
    const int64_t pitch = (int64_t)cols * (BF16 ? 2 : 4);
#pragma unroll 4
    for (int r = rl; r < rows; r += 64) {
      const uint4 v = *reinterpret_cast<const uint4*>(base + r * pitch);
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (BF16) {
          const float lo = bf16_bits_to_f32(w[q] & 0xffffu), hi = bf16_bits_to_f32(w[q] >> 16);
          acc[2 * q] = fmaf(lo, lo, acc[2 * q]);
          acc[2 * q + 1] = fmaf(hi, hi, acc[2 * q + 1]);
        } else {
          const float f = __uint_as_float(w[q]);
          acc[q] = fmaf(f, f, acc[q]);
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < EPC; ++e) part[rl][cg * EPC + e] = acc[e];
  __syncthreads();
  for (int half = 32; half >= 1; half >>= 1) {
    for (int x = threadIdx.x; x < half * 4 * EPC; x += 256) {
      const int r = x / (4 * EPC), c = x - r * (4 * EPC);
      part[r][c] += part[r + half][c];
    }
    __syncthreads();
  }
  if (threadIdx.x < 4 * EPC) {
    const int c = blockIdx.x * 4 * EPC + threadIdx.x;
    if (c < cols) out[c] = part[0][threadIdx.x];
  }
}

struct SegList {
  int16_t seg[3 * kMaxHeads];      // segment ids, grouped by next-layer KV group
  int16_t start[kMaxHeads + 1];    // group g' owns seg[start[g'] .. start[g'+1])
};

// n[g][k] = sum of seg_part[s][k] over the segments of group g, in list order.
__global__ __launch_bounds__(256) void down_group_sum_kernel(const float* __restrict__ seg_part,
                                                             const SegList sl, int G, int I,
                                                             float* __restrict__ n) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)G * I) return;
  const int g = (int)(idx / I), k = (int)(idx - (int64_t)g * I);
  float s = 0.f;
  for (int i = sl.start[g]; i < sl.start[g + 1]; ++i) s += seg_part[(int64_t)sl.seg[i] * I + k];
  n[idx] = s;
}

__global__ __launch_bounds__(256) void down_combine_kernel(const float* __restrict__ c,
                                                           const float* __restrict__ n, int I,
                                                           int G, float* __restrict__ S_down) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)G * I) return;
  const int k = (int)(idx / G), g = (int)(idx - (int64_t)k * G);
  S_down[idx] = c[k] * n[(int64_t)g * I + k];
}

}  // namespace

hipError_t launch_col_sqnorm(const void* W, int rows, int cols, int dtype, float* out,
                             hipStream_t st) {
  if (cols == 0) return hipSuccess;
  const int epc = dtype == 1 ? 8 : 4;
  if (cols % epc == 0 && (reinterpret_cast<uintptr_t>(W) & 15) == 0) {
    const dim3 grid((cols + 4 * epc - 1) / (4 * epc));
    if (dtype == 1) hipLaunchKernelGGL(col_sqnorm16_kernel<1>, grid, dim3(256), 0, st, W, rows, cols, out);
    else hipLaunchKernelGGL(col_sqnorm16_kernel<0>, grid, dim3(256), 0, st, W, rows, cols, out);
    return hipGetLastError();
  }
  const dim3 grid((cols + 63) / 64);
  if (dtype == 1) hipLaunchKernelGGL(col_sqnorm_kernel<1>, grid, dim3(256), 0, st, W, rows, cols, out);
  else hipLaunchKernelGGL(col_sqnorm_kernel<0>, grid, dim3(256), 0, st, W, rows, cols, out);
  return hipGetLastError();
}

hipError_t launch_down_group_sum(const float* seg_part, const int16_t* seg_list,
                                 const int16_t* group_start, int G_next, int I, float* n,
                                 hipStream_t st) {
  SegList sl{};
  const int nseg = group_start[G_next];
  for (int i = 0; i < nseg; ++i) sl.seg[i] = seg_list[i];
  for (int g = 0; g <= G_next; ++g) sl.start[g] = group_start[g];
  const int64_t total = (int64_t)G_next * I;
  hipLaunchKernelGGL(down_group_sum_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st,
                     seg_part, sl, G_next, I, n);
  return hipGetLastError();
}

hipError_t launch_down_combine(const float* c, const float* n, int I, int G_next, float* S_down,
                               hipStream_t st) {
  const int64_t total = (int64_t)G_next * I;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(down_combine_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st,
                     c, n, I, G_next, S_down);
  return hipGetLastError();
}

}  // namespace hna
