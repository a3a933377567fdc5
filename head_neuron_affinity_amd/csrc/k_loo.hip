// Exact leave-one-out score of the pre-activations, from section 3 ("Affinity
// scores") of "Affinity-Aware Sharding for Delayed Tensor Parallelism": the
// pre-activation change when head h's write o_h = W_o^(h) a_h is removed from
// the residual x and the norm's rms is recomputed,
//   S_loo[g, k] = sum_{h in g} E_t[(g_k - g_k^(-h))^2 + (u_k - u_k^(-h))^2].
// With r = rms(x) and r_h = rms(x - o_h), the change splits exactly into
//   g_k - g_k^(-h) = alpha_th g_k + beta_th (a_h . m_hk),
//   alpha_th = 1 - r / r_h,  beta_th = 1 / r_h,
// where a_h . m_hk = (gamma * o_h) . w^g_k comes from the folded weights M and
// r_h^2 = (|x|^2 - 2 x . o_h + |o_h|^2) / hidden needs only two moments per
// (token, head) (head_moments_kernel, in k_gemm.hip).  Kernels here:
//   x_sqnorm_kernel   |x_t|^2 (both ratios use the same x, so alpha vanishes
//                     exactly when the head's removal leaves the rms alone)
//   loo_coef_kernel   the moments summed over column tiles in order -> alpha, beta
//   loo_kernel        a_h . M_h on the matrix cores per token tile and head, with
//                     the epilogue (alpha g + beta Pg)^2 + (alpha u + beta Pu)^2
//                     summed over the group's heads into per-chunk partials
//   finalize_loo      fixed-order float64 sum of the partials
#include <cmath>

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

template <typename T> struct LTraits;
template <> struct LTraits<__bf16> {
  static constexpr int kBytes = 2, kChunksPerStep = 2, kQuads = 1;
};
template <> struct LTraits<float> {
  static constexpr int kBytes = 4, kChunksPerStep = 4, kQuads = 2;
};

__device__ inline float load_elem(const __bf16* p, int64_t i) {
  return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
}
__device__ inline float load_elem(const float* p, int64_t i) { return p[i]; }

constexpr int pow2_slots(int cpr) { return cpr <= 8 ? 8 : (cpr <= 16 ? 16 : 32); }

// Work decomposition as in the first-order pass: a workgroup owns 128 neurons
// (4 waves x 32) and a chunk of up to 8 consecutive token tiles of 128 tokens;
// per tile each lane keeps g and u of its 64 (t, k) pairs in registers, the
// tile's (alpha, beta) table [128][H] sits in LDS, and for every head (in KV
// group order) a_h . M_h runs on the matrix cores from an LDS-staged a tile.
template <typename E, int S>
__global__ __launch_bounds__(256) void loo_kernel(const LooParams p) {
  using Tr = LTraits<E>;
  constexpr int Q = Tr::kQuads;
  constexpr int CPS = Tr::kChunksPerStep;
  constexpr int CPR = S * CPS;              // 16-byte chunks per row of a_h
  constexpr int SLOTS = pow2_slots(CPR);
  constexpr int ROWB = SLOTS * 16;
  constexpr int BUFB = kTileTokens * ROWB;
  constexpr int CPT = CPR / 2;              // chunks staged per thread per tile

  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  unsigned char* abuf = lds;                                       // [2][128][ROWB]
  float2* cbuf = reinterpret_cast<float2*>(lds + 2 * BUFB);        // [2][128][H]
  float* accl = reinterpret_cast<float*>(cbuf + 2 * kTileTokens * p.H);  // [G][256]

  // workgroup -> (neuron tile, token chunk); consecutive ids alternate XCDs
  const int id = blockIdx.x;
  const int xcd = id & 7, wi = id >> 3;
  const int st = xcd + 8 * (wi >> 5), mem = wi & 31;
  if (st >= p.n_st) return;
  const int kt = (st % p.n_ktg) * kSuperKt + (mem & 3);
  const int chunk = (st / p.n_ktg) * kSuperChunks + (mem >> 2);
  if (kt >= p.n_kt || chunk >= p.n_chunks) return;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int H = p.H, G = p.G, I = p.I, d = p.d;
  const int64_t NT = p.T;
  const int KB = p.I32 >> 5;
  const int nb = kt * 4 + w;
  const int nbc = nb < KB ? nb : KB - 1;     // clamped so that M reads stay in bounds
  const int k = nb * 32 + (l & 31);
  const bool kvalid = nb < KB && k < I;
  const E* a = static_cast<const E*>(p.a);
  const E* gp = static_cast<const E*>(p.g);
  const E* up = static_cast<const E*>(p.u);
  const E* M = static_cast<const E*>(p.M);

  for (int x = tid; x < G * 256; x += 256) accl[x] = 0.f;

  const int tt0 = chunk * kTilesPerChunk;
  const int ntile = min(kTilesPerChunk, p.n_tt - tt0);
  const int nsteps = ntile * H;

  uint4 stage[CPT];
  auto load_stage = [&](int step) {
    const int ti = step / H;
    const int h = p.head_order[step - ti * H];
    const int64_t t0 = (int64_t)(tt0 + ti) * kTileTokens;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int q = tid + 256 * c;
      const int row = q / CPR, col = q - (q / CPR) * CPR;
      const int64_t t = t0 + row;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (t < NT) v = *reinterpret_cast<const uint4*>(a + ((t * H + h) * d) + col * (16 / Tr::kBytes));
      stage[c] = v;
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int q = tid + 256 * c;
      const int row = q / CPR, col = q - (q / CPR) * CPR;
      const int off = row * ROWB + ((col ^ (row & (SLOTS - 1))) << 4);
      *reinterpret_cast<uint4*>(abuf + buf * BUFB + off) = stage[c];
    }
  };
  // the tile's (alpha, beta) rows; tokens past the end get zeros
  auto stage_coef = [&](int ti, int buf) {
    const int64_t t0 = (int64_t)(tt0 + ti) * kTileTokens;
    const int64_t valid = (NT - t0 < kTileTokens ? NT - t0 : kTileTokens) * H;
    float2* dst = cbuf + buf * kTileTokens * H;
    for (int e = tid; e < kTileTokens * H; e += 256)
      dst[e] = e < valid ? p.coef[t0 * H + e] : make_float2(0.f, 0.f);
  };

  load_stage(0);
  stage_coef(0, 0);
  store_stage(0);
  __syncthreads();

  f32x16 accG[4], accU[4];
  float gv[4][16], uv[4][16];
  float run[4] = {0.f, 0.f, 0.f, 0.f};
  const int64_t slab = (int64_t)64 * 8;            // elements per (h, kb, gu, s)
  const E* Mw = M + (int64_t)nbc * 2 * S * slab + l * 8;

  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    const int ti = step / H, hi = step - ti * H;
    const int h = p.head_order[hi];
    const int grp = p.head_group[hi];
    const bool has_next = step + 1 < nsteps;
    if (has_next) load_stage(step + 1);

    if (hi == 0) {
      // the tile's pre-activations, shared by all heads
      const int64_t tbase = (int64_t)(tt0 + ti) * kTileTokens;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = tb * 32 + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
          const int64_t t = tbase + row;
          const bool ok = kvalid && t < NT;
          gv[tb][v] = ok ? load_elem(gp, t * I + k) : 0.f;
          uv[tb][v] = ok ? load_elem(up, t * I + k) : 0.f;
        }
      }
    }
    if (hi == H - 1 && ti + 1 < ntile) stage_coef(ti + 1, (ti + 1) & 1);

    // a_h (128 x d) . M_h (d x [32 gate | 32 up]) on the matrix cores
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      accG[tb] = f32x16{};
      accU[tb] = f32x16{};
    }
    const unsigned char* ab = abuf + buf * BUFB;
    const E* Mh = Mw + (int64_t)h * KB * 2 * S * slab;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      uint4 bg[Q], bu[Q];
#pragma unroll
      for (int qq = 0; qq < Q; ++qq) {
        bg[qq] = *reinterpret_cast<const uint4*>(Mh + s * slab + qq * (16 / Tr::kBytes));
        bu[qq] = *reinterpret_cast<const uint4*>(Mh + (S + s) * slab + qq * (16 / Tr::kBytes));
      }
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        const int row = tb * 32 + (l & 31);
        uint4 af[Q];
#pragma unroll
        for (int qq = 0; qq < Q; ++qq) {
          const int col = s * CPS + (l >> 5) * Q + qq;
          af[qq] = *reinterpret_cast<const uint4*>(ab + row * ROWB + ((col ^ (row & (SLOTS - 1))) << 4));
        }
        mma(accG[tb], af, bg);
        mma(accU[tb], af, bu);
      }
    }

    // epilogue: the exact pre-activation changes and their squares
    const float2* cb = cbuf + (ti & 1) * kTileTokens * H + h;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = tb * 32 + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
        const float2 c = cb[row * H];
        const float dg = fmaf(c.x, gv[tb][v], c.y * accG[tb][v]);
        const float du = fmaf(c.x, uv[tb][v], c.y * accU[tb][v]);
        run[tb] = fmaf(dg, dg, fmaf(du, du, run[tb]));
      }
    }
    if (hi == H - 1 || p.head_group[hi + 1] != grp) {
      accl[grp * 256 + tid] += (run[0] + run[1]) + (run[2] + run[3]);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) run[tb] = 0.f;
    }
    if (has_next) store_stage(buf ^ 1);
    __syncthreads();
  }

  // lanes l and l+32 hold the same neuron: combine and write the partial sums
  if (l < 32 && nb < KB) {
    const int kk = nb * 32 + l;
    float* out = p.part + (int64_t)chunk * G * p.I32;
    for (int gg = 0; gg < G; ++gg)
      out[(int64_t)gg * p.I32 + kk] = accl[gg * 256 + tid] + accl[gg * 256 + tid + 32];
  }
}

// S_loo[g, k] = scale * sum over chunks (in order, float64) of the partials
__global__ __launch_bounds__(256) void finalize_loo_kernel(const float* __restrict__ part,
                                                           int n_chunks, int G, int I, int I32,
                                                           float scale, float* S_loo) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)G * I) return;
  const int g = (int)(idx / I), k = (int)(idx - (int64_t)g * I);
  double s = 0.0;
  for (int c = 0; c < n_chunks; ++c) s += part[((int64_t)c * G + g) * I32 + k];
  S_loo[idx] = (float)(s * (double)scale);
}

template <typename E, int S>
hipError_t launch_loo_typed(const LooParams& p, size_t lds, int grid, hipStream_t st) {
  auto fn = loo_kernel<E, S>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(256), lds, st, p);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_loo_steps(const LooParams& p, size_t lds, int grid, hipStream_t st) {
  switch (p.d / 16) {
    case 1: return launch_loo_typed<E, 1>(p, lds, grid, st);
    case 2: return launch_loo_typed<E, 2>(p, lds, grid, st);
    case 3: return launch_loo_typed<E, 3>(p, lds, grid, st);
    case 4: return launch_loo_typed<E, 4>(p, lds, grid, st);
    case 5: return launch_loo_typed<E, 5>(p, lds, grid, st);
    case 6: return launch_loo_typed<E, 6>(p, lds, grid, st);
    case 7: return launch_loo_typed<E, 7>(p, lds, grid, st);
    case 8: return launch_loo_typed<E, 8>(p, lds, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t loo_lds_bytes(int H, int G, int d, int dtype) {
  const int cpr = (d / 16) * (dtype == 1 ? 2 : 4);
  const int slots = pow2_slots(cpr);
  return (size_t)2 * kTileTokens * slots * 16 + (size_t)2 * kTileTokens * H * sizeof(float2) +
         (size_t)G * 256 * sizeof(float);
}

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

hipError_t launch_loo(const LooParams& p, size_t lds, int grid, int dtype, hipStream_t st) {
  if (grid == 0) return hipSuccess;
  return dtype == 1 ? launch_loo_steps<__bf16>(p, lds, grid, st)
                    : launch_loo_steps<float>(p, lds, grid, st);
}

hipError_t launch_finalize_loo(const float* part, int n_chunks, int G, int I, int I32,
                               float scale, float* S_loo, hipStream_t st) {
  const int64_t n = (int64_t)G * I;
  hipLaunchKernelGGL(finalize_loo_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     part, n_chunks, G, I, I32, scale, S_loo);
  return hipGetLastError();
}

}  // namespace hna
