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
// r_h^2 = (|x|^2 - 2 x . o_h + |o_h|^2) / hidden needs |x|^2 (x_prep_kernel)
// and two moments per (token, head): x . o_h = (x W_o)_h . a_h and
// |o_h|^2 = a_h . (Q_h a_h) with Q_h = W_o^(h)T W_o^(h), from three more plain
// GEMMs (x W_o, the Q_h, Q_h a_h; rocBLAS) and the dots in loo_coef_kernel.  All
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

// |x_t|^2 (one wave per row, fixed order) and, when xl is given, x rounded to
// bf16 for the x W_o GEMM
__global__ __launch_bounds__(256) void x_prep_kernel(const float* __restrict__ x, int64_t T, int D,
                                                     float* __restrict__ xx,
                                                     uint16_t* __restrict__ xl) {
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
      if (xl) *reinterpret_cast<uint2*>(xl + t * D + n) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
    }
  } else {
    for (int n = l; n < D; n += 64) {
      s = fmaf(row[n], row[n], s);
      if (xl) xl[t * D + n] = (uint16_t)f32_to_bf16_bits(row[n]);
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (l == 0) xx[t] = s;
}

__device__ inline void load8(const __bf16* p, float (&v)[8]) {
  const uint4 q = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = __uint_as_float(w[e] << 16);
    v[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
  }
}
__device__ inline void load8(const float* p, float (&v)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// alpha, beta per (token, head) from |x|^2, x . o_h = Z[t, h] . a_th and
// |o_h|^2 = U[t, h] . a_th (Z = x W_o, U_th = Q_h a_th, all [T][H][d]); 16
// lanes per (token, head), 8 features per lane and step, a fixed butterfly.  A
// token whose residual vanishes without the head (r_h = 0) gets 0, 0 and
// contributes nothing.
template <typename E>
__global__ __launch_bounds__(256) void loo_coef_kernel(const E* __restrict__ a,
                                                       const E* __restrict__ Z,
                                                       const E* __restrict__ U,
                                                       const float* __restrict__ xx, int64_t T,
                                                       int H, int d, int D,
                                                       float2* __restrict__ coef) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
  const int sub = threadIdx.x & 15;
  const bool ok = i < T * H;
  float xo = 0.f, oo = 0.f;
  if (ok) {
    const int64_t base = i * d;
    for (int j = 8 * sub; j < d; j += 128) {
      float av[8], zv[8], uv[8];
      load8(a + base + j, av);
      load8(Z + base + j, zv);
      load8(U + base + j, uv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        xo = fmaf(zv[e], av[e], xo);
        oo = fmaf(uv[e], av[e], oo);
      }
    }
  }
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) {
    xo += __shfl_xor(xo, o);
    oo += __shfl_xor(oo, o);
  }
  if (!ok || sub != 0) return;
  const int64_t t = i / H;
  const double x2 = (double)xx[t];
  const double den = x2 - 2.0 * (double)xo + (double)oo;
  float2 c = make_float2(0.f, 0.f);
  if (den > 0.0 && x2 > 0.0) {
    c.x = (float)(1.0 - sqrt(x2 / den));
    c.y = (float)sqrt((double)D / den);
  }
  coef[i] = c;
}

__device__ inline float load_elem(const __bf16* p, int64_t i) {
  return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
}
__device__ inline float load_elem(const float* p, int64_t i) { return p[i]; }

// As[t][h*d + j] = alpha_th beta_th a[t][h][j] (rounded to the input dtype), 8
// elements per thread (d is a multiple of 16)
template <typename E>
__global__ __launch_bounds__(256) void scale_a_kernel(const E* __restrict__ a,
                                                      const float2* __restrict__ coef, int64_t T,
                                                      int H, int d, E* __restrict__ As) {
  const int64_t n8 = T * H * d / 8;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    const int64_t th = (i * 8) / d;
    const float2 c = coef[th];
    const float w = c.x * c.y;
    float v[8];
    load8(a + i * 8, v);
    if constexpr (sizeof(E) == 2) {
      *reinterpret_cast<uint4*>(As + i * 8) =
          make_uint4(pack_bf16x2(v[0] * w, v[1] * w), pack_bf16x2(v[2] * w, v[3] * w),
                     pack_bf16x2(v[4] * w, v[5] * w), pack_bf16x2(v[6] * w, v[7] * w));
    } else {
      reinterpret_cast<float4*>(As + i * 8)[0] = make_float4(v[0] * w, v[1] * w, v[2] * w, v[3] * w);
      reinterpret_cast<float4*>(As + i * 8)[1] = make_float4(v[4] * w, v[5] * w, v[6] * w, v[7] * w);
    }
  }
}

// T1 partial sums: t1[tc][h][k] = sum over token chunk tc of alpha_th^2 (g_tk^2 + u_tk^2);
// heads in blocks of 16, the chunk's squared alphas staged in LDS 256 tokens at
// a time; V consecutive neurons per thread (V = 4 needs I % 4 == 0), eight
// tokens' loads in flight
constexpr int kT1Chunk = 512, kT1Stage = 256, kT1Heads = 16;

__device__ inline void load_v(const __bf16* p, float (&v)[4]) {
  const uint2 q = *reinterpret_cast<const uint2*>(p);
  v[0] = __uint_as_float(q.x << 16); v[1] = __uint_as_float(q.x & 0xffff0000u);
  v[2] = __uint_as_float(q.y << 16); v[3] = __uint_as_float(q.y & 0xffff0000u);
}
__device__ inline void load_v(const float* p, float (&v)[4]) {
  const float4 q = *reinterpret_cast<const float4*>(p);
  v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}
__device__ inline void load_v(const __bf16* p, float (&v)[1]) { v[0] = load_elem(p, 0); }
__device__ inline void load_v(const float* p, float (&v)[1]) { v[0] = p[0]; }

template <typename E, int V>
__global__ __launch_bounds__(256) void t1_kernel(const E* __restrict__ g, const E* __restrict__ u,
                                                 const float2* __restrict__ coef, int64_t T,
                                                 int H, int I, float* __restrict__ t1) {
  __shared__ __attribute__((aligned(16))) float al2[kT1Stage][kT1Heads];
  const int k0 = (blockIdx.x * 256 + threadIdx.x) * V;
  const int tc = blockIdx.y;
  const int64_t t0 = (int64_t)tc * kT1Chunk, t1e = min(T, t0 + kT1Chunk);
  for (int h0 = 0; h0 < H; h0 += kT1Heads) {
    const int nh = min(kT1Heads, H - h0);
    float acc[V][kT1Heads];
#pragma unroll
    for (int c = 0; c < V; ++c)
#pragma unroll
      for (int i = 0; i < kT1Heads; ++i) acc[c][i] = 0.f;
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
      if (k0 < I) {
        const int n = (int)min((int64_t)kT1Stage, t1e - ts);
        for (int tt0 = 0; tt0 < n; tt0 += 8) {
          float q[8][V];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int64_t t = ts + (tt0 + e < n ? tt0 + e : 0);   // past n: row ts, weight 0
            float gv[V], uv[V];
            load_v(g + t * I + k0, gv);
            load_v(u + t * I + k0, uv);
#pragma unroll
            for (int c = 0; c < V; ++c) q[e][c] = tt0 + e < n ? fmaf(gv[c], gv[c], uv[c] * uv[c]) : 0.f;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
#pragma unroll
            for (int i4 = 0; i4 < kT1Heads / 4; ++i4) {
              const float4 w = *reinterpret_cast<const float4*>(&al2[tt0 + e][4 * i4]);
#pragma unroll
              for (int c = 0; c < V; ++c) {
                acc[c][4 * i4] = fmaf(w.x, q[e][c], acc[c][4 * i4]);
                acc[c][4 * i4 + 1] = fmaf(w.y, q[e][c], acc[c][4 * i4 + 1]);
                acc[c][4 * i4 + 2] = fmaf(w.z, q[e][c], acc[c][4 * i4 + 2]);
                acc[c][4 * i4 + 3] = fmaf(w.w, q[e][c], acc[c][4 * i4 + 3]);
              }
            }
          }
        }
      }
    }
    if (k0 < I) {
#pragma unroll
      for (int i = 0; i < kT1Heads; ++i)   // compile-time indices keep acc in registers
        if (i < nh)
#pragma unroll
          for (int c = 0; c < V; ++c) t1[((int64_t)tc * H + h0 + i) * I + k0 + c] = acc[c][i];
    }
  }
}

// t1r[h][k] = sum over the token chunks, in order, of t1[tc][h][k] (float64)
__global__ __launch_bounds__(256) void t1_reduce_kernel(const float* __restrict__ t1, int n_tc,
                                                        int64_t HI, double* __restrict__ t1r) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= HI) return;
  double s = 0.0;
  for (int tc = 0; tc < n_tc; ++tc) s += (double)t1[(int64_t)tc * HI + i];
  t1r[i] = s;
}

// S_loo[g][k] = scale * (sum_{h in g} (T1 + 2 T2) + T3[g][k]).  One wave per
// (32-neuron block, KV group): lane l holds neuron 32 kb + (l & 31) and the
// d-half l >> 5 of every 16-wide step, which is one 16-byte piece of the fold
// layout and 8 consecutive floats of Y; the halves are added by one exchange.
// Heads in group order, every sum in a fixed order, float64 across heads.
template <typename E>
__global__ __launch_bounds__(64) void loo_combine_kernel(const LooCombineParams p) {
  const int kb = blockIdx.x, grp = blockIdx.y, l = threadIdx.x, half = l >> 5;
  const int k = kb * 32 + (l & 31);
  const E* M = static_cast<const E*>(p.M);
  const int HD = p.H * p.d;
  const bool kin = k < p.I;
  double s = 0.0;
  for (int q = p.group_start[grp]; q < p.group_start[grp + 1]; ++q) {
    const int h = p.head_order[q];
    float t2 = 0.f;
    if (p.Y) {
      for (int gu = 0; gu < 2; ++gu) {
        const float* Y = p.Y + (int64_t)gu * HD * p.I + (int64_t)(kin ? k : 0) * HD + (int64_t)h * p.d;
        for (int st = 0; st < p.S; ++st) {
          const int j0 = 16 * st + 8 * half;
          float mv[8], yv[8];
          load8(M + folded_index(h, j0, k, gu, p.KB, p.S), mv);
          load8(Y + j0, yv);
#pragma unroll
          for (int e = 0; e < 8; ++e) t2 = fmaf(mv[e], yv[e], t2);
        }
      }
    }
    t2 += __shfl_xor(t2, 32);
    const double t1 = (kin && p.t1r) ? p.t1r[(int64_t)h * p.I + k] : 0.0;
    s += t1 + 2.0 * (double)t2;
  }
  if (p.t3 && kin) s += (double)p.t3[(int64_t)grp * p.I32 + k];
  if (half == 0 && kin) p.S_loo[(int64_t)grp * p.I + k] = (float)(s * (double)p.scale);
}

}  // namespace

hipError_t launch_x_prep(const float* x, int64_t T, int D, float* xx, void* xl, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int64_t blocks = (T + kXRows - 1) / kXRows;
  hipLaunchKernelGGL(x_prep_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, T, D, xx,
                     static_cast<uint16_t*>(xl));
  return hipGetLastError();
}

hipError_t launch_loo_coef(const void* a, const void* Z, const void* U, const float* xx, int64_t T,
                           int H, int d, int D, float2* coef, int dtype, hipStream_t st) {
  const int64_t n = T * H * 16;
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (dtype == 1)
    hipLaunchKernelGGL(loo_coef_kernel<__bf16>, grid, dim3(256), 0, st,
                       static_cast<const __bf16*>(a), static_cast<const __bf16*>(Z),
                       static_cast<const __bf16*>(U), xx, T, H, d, D, coef);
  else
    hipLaunchKernelGGL(loo_coef_kernel<float>, grid, dim3(256), 0, st,
                       static_cast<const float*>(a), static_cast<const float*>(Z),
                       static_cast<const float*>(U), xx, T, H, d, D, coef);
  return hipGetLastError();
}

hipError_t launch_scale_a(const void* a, const float2* coef, int64_t T, int H, int d, void* As,
                          int dtype, hipStream_t st) {
  const int64_t n = T * H * d / 8;
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
  const bool vec = I % 4 == 0;
  const int per = vec ? 4 : 1;
  const dim3 grid((I / per + 255) / 256 + ((I % per) ? 1 : 0), t1_chunks(T));
  if (dtype == 1) {
    const auto* gb = static_cast<const __bf16*>(g);
    const auto* ub = static_cast<const __bf16*>(u);
    if (vec) hipLaunchKernelGGL((t1_kernel<__bf16, 4>), grid, dim3(256), 0, st, gb, ub, coef, T, H, I, t1);
    else hipLaunchKernelGGL((t1_kernel<__bf16, 1>), grid, dim3(256), 0, st, gb, ub, coef, T, H, I, t1);
  } else {
    const auto* gf = static_cast<const float*>(g);
    const auto* uf = static_cast<const float*>(u);
    if (vec) hipLaunchKernelGGL((t1_kernel<float, 4>), grid, dim3(256), 0, st, gf, uf, coef, T, H, I, t1);
    else hipLaunchKernelGGL((t1_kernel<float, 1>), grid, dim3(256), 0, st, gf, uf, coef, T, H, I, t1);
  }
  return hipGetLastError();
}

hipError_t launch_t1_reduce(const float* t1, int n_tc, int64_t HI, double* t1r, hipStream_t st) {
  if (HI == 0) return hipSuccess;
  hipLaunchKernelGGL(t1_reduce_kernel, dim3((unsigned)((HI + 255) / 256)), dim3(256), 0, st, t1,
                     n_tc, HI, t1r);
  return hipGetLastError();
}

hipError_t launch_loo_combine(const LooCombineParams& p, int dtype, hipStream_t st) {
  const dim3 grid((unsigned)p.KB, (unsigned)p.G);
  if (dtype == 1) hipLaunchKernelGGL(loo_combine_kernel<__bf16>, grid, dim3(64), 0, st, p);
  else hipLaunchKernelGGL(loo_combine_kernel<float>, grid, dim3(64), 0, st, p);
  return hipGetLastError();
}

// ---- plain GEMMs by rocBLAS (column-major, fp32 accumulation); one handle per
// device, created at the first call, used under a lock so that concurrent
// callers do not share its stream and workspace settings
namespace {
std::mutex g_blas_mu;
rocblas_handle g_blas[64] = {};
rocblas_datatype blas_type(int t) { return t == 1 ? rocblas_datatype_bf16_r : rocblas_datatype_f32_r; }
}  // namespace

int blas_gemm(hipStream_t st, void* ws, size_t ws_bytes, bool ta, bool tb, int m, int n, int k,
              const void* A, int at, int lda, int64_t sa, const void* B, int bt, int ldb,
              int64_t sb, void* C, int ct, int ldc, int64_t sc, int batch) {
  if (m == 0 || n == 0 || batch == 0) return 0;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  std::lock_guard<std::mutex> lock(g_blas_mu);
  if (!g_blas[dev]) {
    const rocblas_status cs = rocblas_create_handle(&g_blas[dev]);
    if (cs != rocblas_status_success) {
      g_blas[dev] = nullptr;
      return (int)cs;
    }
  }
  rocblas_handle hb = g_blas[dev];
  rocblas_status bs = rocblas_set_stream(hb, st);
  if (bs == rocblas_status_success) bs = rocblas_set_workspace(hb, ws, ws_bytes);
  const float one = 1.0f, zero = 0.0f;
  if (bs == rocblas_status_success)
    bs = rocblas_gemm_strided_batched_ex(
        hb, ta ? rocblas_operation_transpose : rocblas_operation_none,
        tb ? rocblas_operation_transpose : rocblas_operation_none, m, n, k, &one, A,
        blas_type(at), lda, sa, B, blas_type(bt), ldb, sb, &zero, C, blas_type(ct), ldc, sc, C,
        blas_type(ct), ldc, sc, batch, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
  return (int)bs;
}

}  // namespace hna
