// Exact leave-one-out score of the pre-activations, from section 3 ("Affinity
// scores") of "Affinity-Aware Sharding for Delayed Tensor Parallelism": the
// pre-activation change when head h's write o_h = W_o^(h) a_h is removed from
// the residual x and the norm's rms is recomputed,
//   S_loo[g, k] = sum_{h in g} E_t[(g_k - g_k^(-h))^2 + (u_k - u_k^(-h))^2].
// With r = rms(x) and r_h = rms(x - o_h), the change splits exactly into
//   g_k - g_k^(-h) = alpha_th g_k + beta_th P_thk,   P_thk = a_th . m^g_hk,
//   alpha_th = 1 - r / r_h,  beta_th = 1 / r_h,
// (m_hk the folded weights; u likewise), so that per head and neuron
//   sum_t (...)^2 = T1 + 2 T2 + T3,
//   T1 = sum_t alpha^2 (g^2 + u^2)                      (t1_kernel)
//   T2 = m^g_hk . Y^g_h[:, k] + m^u_hk . Y^u_h[:, k],  Y_h = sum_t alpha beta a_th g_t^T
//        (two plain GEMMs over the tokens, by rocBLAS, on a scaled by alpha beta)
//   T3 = m^T C_h m,  C_h = sum_t beta_th^2 a_th a_th^T   (the Gram and quadratic-
//        form kernels of the ADD score, weighted per token and head)
// r_h^2 = (|x|^2 - 2 x . o_h + |o_h|^2) / hidden needs two moments per (token,
// head) (head_moments_kernel, in k_gemm.hip) and |x|^2 (x_sqnorm_kernel).  All
// three terms are non-cancelling in practice (T3 dominates; T2 is a fraction of
// it), so rounding a * alpha beta to bf16 for the GEMMs costs far less than the
// bf16 tolerance.
#include <rocblas/rocblas.h>

#include <cmath>
#include <mutex>

#include "hna_internal.h"

namespace hna {
namespace {

constexpr int kXRows = 4;  // rows of x per 256-thread block (one wave each)

__global__ __launch_bounds__(256) void x_sqnorm_kernel(const float* __restrict__ x, int64_t T,
                                                       int D, float* __restrict__ xx) {
  const int l = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kXRows + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = x + t * D;
  float s = 0.f;
  if ((D & 3) == 0) {
    for (int n = 4 * l; n < D; n += 256) {
      const float4 v = *reinterpret_cast<const float4*>(row + n);
      s = fmaf(v.x, v.x, s);
      s = fmaf(v.y, v.y, s);
      s = fmaf(v.z, v.z, s);
      s = fmaf(v.w, v.w, s);
    }
  } else {
    for (int n = l; n < D; n += 64) s = fmaf(row[n], row[n], s);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (l == 0) xx[t] = s;
}

// alpha, beta per (token, head); a token whose residual vanishes without the
// head (r_h = 0) gets 0, 0 and contributes nothing
__global__ __launch_bounds__(256) void loo_coef_kernel(const float* __restrict__ part,
                                                       const float* __restrict__ xx, int64_t T,
                                                       int H, int n_nt, int D,
                                                       float2* __restrict__ coef) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= T * H) return;
  const int64_t t = i / H;
  const int h = (int)(i - t * H);
  double xo = 0.0, oo = 0.0;
  for (int nt = 0; nt < n_nt; ++nt) {
    const float* pp = part + ((int64_t)(nt * H + h) * 2) * T + t;
    xo += (double)pp[0];
    oo += (double)pp[T];
  }
  const double x2 = (double)xx[t];
  const double den = x2 - 2.0 * xo + oo;
  float2 c = make_float2(0.f, 0.f);
  if (den > 0.0 && x2 > 0.0) {
    c.x = (float)(1.0 - sqrt(x2 / den));
    c.y = (float)sqrt((double)D / den);
  }
  coef[t * H + h] = c;
}

__device__ inline float load_elem(const __bf16* p, int64_t i) {
  return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
}
__device__ inline float load_elem(const float* p, int64_t i) { return p[i]; }

// As[t][h*d + j] = alpha_th beta_th a[t][h][j] (rounded to the input dtype)
template <typename E>
__global__ __launch_bounds__(256) void scale_a_kernel(const E* __restrict__ a,
                                                      const float2* __restrict__ coef, int64_t T,
                                                      int H, int d, E* __restrict__ As) {
  const int64_t n = T * H * d;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t th = i / d;
    const float2 c = coef[th];
    const float v = load_elem(a, i) * (c.x * c.y);
    if constexpr (sizeof(E) == 2) reinterpret_cast<uint16_t*>(As)[i] = (uint16_t)f32_to_bf16_bits(v);
    else As[i] = v;
  }
}

// T1 partial sums: t1[tc][h][k] = sum over token chunk tc of alpha_th^2 (g_tk^2 + u_tk^2);
// heads in blocks of 16, the chunk's alphas staged in LDS 256 tokens at a time
constexpr int kT1Chunk = 2048, kT1Stage = 256, kT1Heads = 16;
template <typename E>
__global__ __launch_bounds__(256) void t1_kernel(const E* __restrict__ g, const E* __restrict__ u,
                                                 const float2* __restrict__ coef, int64_t T,
                                                 int H, int I, float* __restrict__ t1) {
  __shared__ float al2[kT1Stage][kT1Heads];
  const int k = blockIdx.x * 256 + threadIdx.x;
  const int tc = blockIdx.y;
  const int64_t t0 = (int64_t)tc * kT1Chunk, t1e = min(T, t0 + kT1Chunk);
  for (int h0 = 0; h0 < H; h0 += kT1Heads) {
    const int nh = min(kT1Heads, H - h0);
    float acc[kT1Heads];
#pragma unroll
    for (int i = 0; i < kT1Heads; ++i) acc[i] = 0.f;
    for (int64_t ts = t0; ts < t1e; ts += kT1Stage) {
      __syncthreads();
      for (int e = threadIdx.x; e < kT1Stage * kT1Heads; e += 256) {
        const int tt = e / kT1Heads, hh = e - tt * kT1Heads;
        const int64_t t = ts + tt;
        float a2 = 0.f;
        if (t < t1e && hh < nh) {
          const float al = coef[t * H + h0 + hh].x;
          a2 = al * al;
        }
        al2[tt][hh] = a2;
      }
      __syncthreads();
      if (k < I) {
        const int n = (int)min((int64_t)kT1Stage, t1e - ts);
        for (int tt = 0; tt < n; ++tt) {
          const int64_t t = ts + tt;
          const float gv = load_elem(g, t * I + k), uv = load_elem(u, t * I + k);
          const float q = fmaf(gv, gv, uv * uv);
#pragma unroll
          for (int i = 0; i < kT1Heads; ++i) acc[i] = fmaf(al2[tt][i], q, acc[i]);
        }
      }
    }
    if (k < I)
      for (int i = 0; i < nh; ++i) t1[((int64_t)tc * H + h0 + i) * I + k] = acc[i];
  }
}

// S_loo[g][k] = scale * (sum_{h in g} (T1 + 2 T2) + T3[g][k]), float64, heads in
// group order and every inner sum in a fixed order
template <typename E>
__global__ __launch_bounds__(256) void loo_combine_kernel(const LooCombineParams p) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)p.G * p.I) return;
  const int grp = (int)(idx / p.I), k = (int)(idx - (int64_t)grp * p.I);
  const E* M = static_cast<const E*>(p.M);
  const int HD = p.H * p.d;
  double s = 0.0;
  for (int q = p.group_start[grp]; q < p.group_start[grp + 1]; ++q) {
    const int h = p.head_order[q];
    double t1 = 0.0;
    for (int tc = 0; tc < p.n_tc; ++tc) t1 += (double)p.t1[((int64_t)tc * p.H + h) * p.I + k];
    double t2 = 0.0;
    for (int gu = 0; gu < (p.Y ? 2 : 0); ++gu) {
      const float* Y = p.Y + (int64_t)gu * HD * p.I + (int64_t)k * HD + (int64_t)h * p.d;
      for (int j = 0; j < p.d; ++j)
        t2 += (double)load_elem(M, folded_index(h, j, k, gu, p.KB, p.S)) * (double)Y[j];
    }
    s += t1 + 2.0 * t2;
  }
  if (p.t3) s += (double)p.t3[(int64_t)grp * p.I32 + k];
  p.S_loo[idx] = (float)(s * (double)p.scale);
}

}  // namespace

hipError_t launch_x_sqnorm(const float* x, int64_t T, int D, float* xx, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int64_t blocks = (T + kXRows - 1) / kXRows;
  hipLaunchKernelGGL(x_sqnorm_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, T, D, xx);
  return hipGetLastError();
}

hipError_t launch_loo_coef(const float* part, const float* xx, int64_t T, int H, int n_nt, int D,
                           float2* coef, hipStream_t st) {
  const int64_t n = T * H;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(loo_coef_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part,
                     xx, T, H, n_nt, D, coef);
  return hipGetLastError();
}

hipError_t launch_scale_a(const void* a, const float2* coef, int64_t T, int H, int d, void* As,
                          int dtype, hipStream_t st) {
  const int64_t n = T * H * d;
  if (n == 0) return hipSuccess;
  const int64_t nb = (n + 255) / 256;
  const unsigned blocks = (unsigned)(nb < 65536 ? nb : 65536);
  if (dtype == 1)
    hipLaunchKernelGGL(scale_a_kernel<__bf16>, dim3(blocks), dim3(256), 0, st,
                       static_cast<const __bf16*>(a), coef, T, H, d, static_cast<__bf16*>(As));
  else
    hipLaunchKernelGGL(scale_a_kernel<float>, dim3(blocks), dim3(256), 0, st,
                       static_cast<const float*>(a), coef, T, H, d, static_cast<float*>(As));
  return hipGetLastError();
}

int t1_chunks(int64_t T) { return (int)((T + kT1Chunk - 1) / kT1Chunk); }

hipError_t launch_t1(const void* g, const void* u, const float2* coef, int64_t T, int H, int I,
                     float* t1, int dtype, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const dim3 grid((I + 255) / 256, t1_chunks(T));
  if (dtype == 1)
    hipLaunchKernelGGL(t1_kernel<__bf16>, grid, dim3(256), 0, st, static_cast<const __bf16*>(g),
                       static_cast<const __bf16*>(u), coef, T, H, I, t1);
  else
    hipLaunchKernelGGL(t1_kernel<float>, grid, dim3(256), 0, st, static_cast<const float*>(g),
                       static_cast<const float*>(u), coef, T, H, I, t1);
  return hipGetLastError();
}

hipError_t launch_loo_combine(const LooCombineParams& p, int dtype, hipStream_t st) {
  const int64_t n = (int64_t)p.G * p.I;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (dtype == 1) hipLaunchKernelGGL(loo_combine_kernel<__bf16>, grid, dim3(256), 0, st, p);
  else hipLaunchKernelGGL(loo_combine_kernel<float>, grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

// ---- the two token GEMMs, Y^g = As^T g and Y^u = As^T u, by rocBLAS
namespace {
std::mutex g_blas_mu;
rocblas_handle g_blas[64] = {};
}  // namespace

int loo_gemms(const void* As, const void* g, const void* u, float* Y, int64_t T, int HD, int I,
              int dtype, void* blas_ws, size_t blas_ws_bytes, hipStream_t st) {
  if (T == 0) return 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  std::lock_guard<std::mutex> lock(g_blas_mu);
  if (!g_blas[dev]) {
    rocblas_status cs = rocblas_create_handle(&g_blas[dev]);
    if (cs != rocblas_status_success) {
      g_blas[dev] = nullptr;
      return (int)cs;
    }
  }
  rocblas_handle hb = g_blas[dev];
  rocblas_status bs = rocblas_set_stream(hb, st);
  if (bs == rocblas_status_success) bs = rocblas_set_workspace(hb, blas_ws, blas_ws_bytes);
  const rocblas_datatype in_t = dtype == 1 ? rocblas_datatype_bf16_r : rocblas_datatype_f32_r;
  const float one = 1.0f, zero = 0.0f;
  // column-major: As is HD x T (lda HD), g and u are I x T (ldb I), Y is HD x I
  for (int gu = 0; gu < 2 && bs == rocblas_status_success; ++gu) {
    float* Yg = Y + (int64_t)gu * HD * I;
    bs = rocblas_gemm_ex(hb, rocblas_operation_none, rocblas_operation_transpose, HD, I, (int)T,
                         &one, As, in_t, HD, gu ? u : g, in_t, I, &zero, Yg,
                         rocblas_datatype_f32_r, HD, Yg, rocblas_datatype_f32_r, HD,
                         rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
  }
  return (int)bs;
}

}  // namespace hna
