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
//   T1 = sum_t alpha^2 (g^2 + u^2)      (t1_kernel, fp32 matrix cores)
//   T2 = m^g_hk . Y^g_h[:, k] + m^u_hk . Y^u_h[:, k],  Y_h = sum_t alpha beta a_th g_t^T.
//        g_t = W_g (gamma * x_t) / r_t exactly (g is the pre-activation of x), so
//        Y^g_h = R_h diag(gamma) W_g^T with R_h = sum_t (alpha beta / r_t) a_th x_t^T:
//        one token GEMM of width hidden shared by gate and up, then two small
//        weight GEMMs, instead of two token GEMMs of width I
//   T3 = m^T C_h m,  C_h = sum_t beta_th^2 a_th a_th^T   (the Gram and quadratic-
//        form kernels of the ADD score, weighted per token and head)
// r_h^2 = (|x|^2 - 2 x . o_h + |o_h|^2) / hidden needs |x|^2 (x_prep_kernel)
// and two moments per (token, head): x . o_h = (x W_o)_h . a_h and
// |o_h|^2 = a_h . (Q_h a_h) with Q_h = W_o^(h)T W_o^(h), from three more plain
// GEMMs (x W_o, the Q_h, Q_h a_h) and the dots in loo_coef_kernel.  Every GEMM
// runs on this library's own MFMA kernels (k_mm.hip for bf16, k_gemm.hip for
// fp32), which take both operands k-contiguous: the token product R reads
// transposed copies of x and of the scaled a, padded to a multiple of 8
// tokens with zeros.  All
// three terms are non-cancelling in practice (T3 dominates; T2 is a fraction of
// it), so rounding a * alpha beta / r and R_h diag(gamma) to bf16 for the GEMMs
// costs far less than the bf16 tolerance.
#include <cmath>

#include "hna_internal.h"

namespace hna {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// One pass over x: |x_t|^2, x rounded to bf16 (when xl is given: the x W_o
// GEMM's operand) and x transposed, xT [D][Tp] in the GEMM dtype (the token
// GEMM's operand; tokens T .. Tp - 1 are zeros).  A workgroup takes 64 tokens
// and walks their rows in 64-feature tiles through LDS; thread (rr, cc) holds
// columns 4 cc .. 4 cc + 3 of rows rr, rr + 16, rr + 32, rr + 48 and their
// partial squares, which a fixed butterfly over the row's 16 threads adds at
// the end.  D is a multiple of 8.
constexpr int kXT = 64;

template <typename E>
__global__ __launch_bounds__(256) void x_prep_kernel(const float* __restrict__ x, int64_t T, int D,
                                                     int64_t Tp, float* __restrict__ xx,
                                                     uint16_t* __restrict__ xl,
                                                     E* __restrict__ xT) {
  __shared__ float tile[kXT][kXT + 1];
  const int tid = threadIdx.x, cc = tid & 15, rr = tid >> 4;
  const int64_t t0 = (int64_t)blockIdx.x * kXT;
  float sq[4] = {0.f, 0.f, 0.f, 0.f};
  constexpr int EPC = 16 / sizeof(E);   // elements per 16-byte store of xT
  constexpr int CPF = kXT / EPC;        // stores per feature row of the tile
  for (int f0 = 0; f0 < D; f0 += kXT) {
    const int f = f0 + 4 * cc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rr + 16 * i;
      const int64_t t = t0 + r;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t < T && f < D) {
        v = *reinterpret_cast<const float4*>(x + t * D + f);
        if (xl)
          *reinterpret_cast<uint2*>(xl + t * D + f) =
              make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
      }
      sq[i] = fmaf(v.x, v.x, sq[i]);
      sq[i] = fmaf(v.y, v.y, sq[i]);
      sq[i] = fmaf(v.z, v.z, sq[i]);
      sq[i] = fmaf(v.w, v.w, sq[i]);
      tile[r][4 * cc] = v.x;
      tile[r][4 * cc + 1] = v.y;
      tile[r][4 * cc + 2] = v.z;
      tile[r][4 * cc + 3] = v.w;
    }
    __syncthreads();
    for (int q = tid; q < kXT * CPF; q += 256) {
      const int fr = q / CPF, tc = (q % CPF) * EPC;
      const int fg = f0 + fr;
      const int64_t tt = t0 + tc;
      if (fg < D && tt < Tp) {   // Tp and tt are multiples of EPC
        E* o = xT + (int64_t)fg * Tp + tt;
        if constexpr (sizeof(E) == 2) {
          *reinterpret_cast<uint4*>(o) = make_uint4(
              pack_bf16x2(tile[tc][fr], tile[tc + 1][fr]), pack_bf16x2(tile[tc + 2][fr], tile[tc + 3][fr]),
              pack_bf16x2(tile[tc + 4][fr], tile[tc + 5][fr]), pack_bf16x2(tile[tc + 6][fr], tile[tc + 7][fr]));
        } else {
          *reinterpret_cast<float4*>(o) =
              make_float4(tile[tc][fr], tile[tc + 1][fr], tile[tc + 2][fr], tile[tc + 3][fr]);
        }
      }
    }
    __syncthreads();
  }
  // the 16 threads of row set rr are 16 consecutive lanes of one wave
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) sq[i] += __shfl_xor(sq[i], o);
  if (cc == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t t = t0 + rr + 16 * i;
      if (t < T) xx[t] = sq[i];
    }
  }
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

// 1 / r_t = sqrt(hidden / |x_t|^2) (0 for a zero residual, whose coefficients are 0)
__device__ inline float inv_rms(float x2, int D) {
  return x2 > 0.f ? (float)sqrt((double)D / (double)x2) : 0.f;
}

// As[t][h*d + j] = (alpha_th beta_th / r_t) a[t][h][j] (rounded to the input
// dtype), 8 elements per thread (d is a multiple of 16)
template <typename E>
__global__ __launch_bounds__(256) void scale_a_kernel(const E* __restrict__ a,
                                                      const float2* __restrict__ coef,
                                                      const float* __restrict__ xx, int64_t T,
                                                      int H, int d, int D, E* __restrict__ As) {
  const int64_t n8 = T * H * d / 8;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    const int64_t th = (i * 8) / d;
    const float2 c = coef[th];
    const float w = c.x * c.y * inv_rms(xx[th / H], D);
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

// bf16 element e of 8 packed in a uint4
__device__ inline float bf16_at(const uint4& v, int e) {
  const uint32_t w = e < 2 ? v.x : e < 4 ? v.y : e < 6 ? v.z : v.w;
  return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
}

// bf16 inputs with d = 32 ND: the moments, alpha and beta, and the scaled
// head outputs in one pass over a and Z, with |o_h|^2 = a . (Q_h a) on the
// matrix cores.  One workgroup per (token range, head) stages Q_h in LDS (Q_h
// is symmetric, so its column-major GEMM output reads as row-major); each
// wave takes 16 tokens at a time and forms V^T = Q_h a^T with 16x16x32 MFMAs:
// lane l holds, as the B operand, features 32 ks + 8 (l / 16) .. + 7 of token
// l % 16, and row m of MFMA tile mt stands for Q_h row
// 32 (mt / 2) + 8 (m / 4) + 4 (mt % 2) + m % 4, which puts every entry of V
// that a lane receives on a feature whose a value the lane already holds.
// x . o_h = Z . a is dotted over the same features; two exchanges across the
// wave's quarters complete both sums.
// (alpha beta / r) a, rounded to bf16, is written transposed: ZAT[h d + j][t]
// for t < Tp (zeros for the padding tokens T .. Tp - 1).  The workgroup's four
// waves take four adjacent 16-token tiles; their values are staged through
// LDS, feature-major, so that each ZAT row receives its 64 tokens as one
// 128-byte run of 16-byte stores.
constexpr int kCoefBlocksPerHead = 128;

// XO: x . o_h comes as d / 64 fp32 partial planes xo[q][h][t] (summed here in
// plane order) instead of from Z.
template <int ND, bool XO>
__global__ __launch_bounds__(256) void loo_coef_mfma_kernel(const __bf16* __restrict__ a,
                                                            const __bf16* __restrict__ Z,
                                                            const float* __restrict__ xo_part,
                                                            __bf16* __restrict__ ZAT,
                                                            const __bf16* __restrict__ Q,
                                                            const float* __restrict__ xx,
                                                            int64_t T, int64_t Tp, int H, int D,
                                                            float2* __restrict__ coef) {
  constexpr int d = 32 * ND, QS = d + 8;  // LDS row stride, elements
  constexpr int ZS = 64 + 8;              // staged ZAT row: 64 tokens + pad
  __shared__ __attribute__((aligned(16))) uint16_t qs[d * QS];
  // the workgroup's 64 tokens of (alpha beta / r) a, feature-major, so that
  // ZAT rows go out as 128-byte runs
  __shared__ __attribute__((aligned(16))) uint16_t zst[d * ZS];
  const int h = blockIdx.y;
  const uint16_t* qh = reinterpret_cast<const uint16_t*>(Q) + (int64_t)h * d * d;
  for (int i = threadIdx.x; i < d * d / 8; i += 256) {
    const int r = (i * 8) / d, c = i * 8 - r * d;
    *reinterpret_cast<uint4*>(qs + r * QS + c) = *reinterpret_cast<const uint4*>(qh + i * 8);
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, qq = lane >> 4, tl = lane & 15;
  const uint16_t* ap = reinterpret_cast<const uint16_t*>(a);
  const uint16_t* zp = reinterpret_cast<const uint16_t*>(Z);
  uint16_t* ztp = reinterpret_cast<uint16_t*>(ZAT) + (int64_t)h * d * Tp;
  const int64_t n_tiles = (T + 15) / 16;
  const int64_t step = (int64_t)gridDim.x * 4;
  // blocks of 64 tokens, the 4 waves' tiles side by side; the trip count is
  // the workgroup's, so every wave reaches every barrier (a tile past the
  // last reads and stages zeros, and nothing of it is stored)
  const int64_t n_blk = (n_tiles + 3) / 4;
  const int wave = threadIdx.x >> 6;
  int64_t tile = (int64_t)blockIdx.x * 4 + wave;
  uint4 ar[ND], zr[XO ? 1 : ND];
  float xr = 0.f;   // XO: this token's x . o_h (lanes of quarter 0; 0 elsewhere)
  auto fetch = [&](int64_t tt) {
    const int64_t t = tt * 16 + tl;
    const bool ok = tt < n_tiles && t < T;
    const int64_t base = ((ok ? t : 0) * H + h) * d + 8 * qq;
#pragma unroll
    for (int ks = 0; ks < ND; ++ks) {
      ar[ks] = ok ? *reinterpret_cast<const uint4*>(ap + base + 32 * ks) : make_uint4(0, 0, 0, 0);
      if constexpr (!XO)
        zr[ks] = ok ? *reinterpret_cast<const uint4*>(zp + base + 32 * ks) : make_uint4(0, 0, 0, 0);
    }
    if constexpr (XO) {
      xr = 0.f;
      if (ok && qq == 0)
        for (int q = 0; q < d / 64; ++q) xr += xo_part[((int64_t)q * H + h) * T + t];
    }
  };
  fetch(tile);
  for (int64_t blk = blockIdx.x; blk < n_blk; blk += gridDim.x, tile += step) {
    uint4 a_cur[ND], z_cur[XO ? 1 : ND];
    const float x_cur = xr;
#pragma unroll
    for (int ks = 0; ks < ND; ++ks) {
      a_cur[ks] = ar[ks];
      if constexpr (!XO) z_cur[ks] = zr[ks];
    }
    fetch(tile + step);  // the next tile loads under this one's work (zeros past the last)
    const int64_t t = tile * 16 + tl;
    const bool ok = t < T;
    // re-read the Q_h fragments from LDS on every tile rather than holding all
    // of them in registers across the loop (an opaque offset stops the hoist)
    int qoff = (8 * (tl >> 2) + (tl & 3)) * QS + 8 * qq;
    asm volatile("" : "+v"(qoff));
    float oo = 0.f, xo = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2 * ND; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const int rbase = 32 * (mt >> 1) + 4 * (mt & 1);
#pragma unroll
      for (int ks = 0; ks < ND; ++ks) {
        const uint4 qa = *reinterpret_cast<const uint4*>(qs + qoff + rbase * QS + 32 * ks);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qa),
                                                      __builtin_bit_cast(bf16x8, a_cur[ks]), acc, 0, 0, 0);
      }
      // entry r is row 4 qq + r: element 4 (mt % 2) + r of chunk mt / 2
#pragma unroll
      for (int r = 0; r < 4; ++r) oo = fmaf(acc[r], bf16_at(a_cur[mt >> 1], 4 * (mt & 1) + r), oo);
    }
    if constexpr (XO) {
      xo = x_cur;
    } else {
#pragma unroll
      for (int ks = 0; ks < ND; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) xo = fmaf(bf16_at(z_cur[ks], e), bf16_at(a_cur[ks], e), xo);
    }
    xo += __shfl_xor(xo, 16);
    oo += __shfl_xor(oo, 16);
    xo += __shfl_xor(xo, 32);
    oo += __shfl_xor(oo, 32);
    float w = 0.f;
    if (ok) {
      const double x2 = (double)xx[t];
      const double den = x2 - 2.0 * (double)xo + (double)oo;
      float2 c = make_float2(0.f, 0.f);
      if (den > 0.0 && x2 > 0.0) {
        c.x = (float)(1.0 - sqrt(x2 / den));
        c.y = (float)sqrt((double)D / den);
      }
      if (qq == 0) coef[t * H + h] = c;
      w = c.x * c.y * inv_rms((float)x2, D);
    }
    // feature 32 ks + 8 qq + e of token t into column 16 wave + tl
#pragma unroll
    for (int ks = 0; ks < ND; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        zst[(32 * ks + 8 * qq + e) * ZS + 16 * wave + tl] =
            (uint16_t)f32_to_bf16_bits(bf16_at(a_cur[ks], e) * w);
    __syncthreads();
    // row f's 64 tokens as eight 16-byte pieces (tokens past Tp not stored)
    const int64_t t_blk = blk * 64;
#pragma unroll
    for (int k = 0; k < d / 32; ++k) {
      const int c = threadIdx.x + 256 * k, f = c >> 3, q = c & 7;
      const uint4 v = *reinterpret_cast<const uint4*>(zst + f * ZS + 8 * q);
      if (t_blk + 8 * q < Tp) *reinterpret_cast<uint4*>(ztp + (int64_t)f * Tp + t_blk + 8 * q) = v;
    }
    __syncthreads();
  }
}

// Rs = (sum of the token-chunk parts of R) diag(gamma) in the input dtype: each
// part is row-major [HD][hidden] fp32 (column c, the hidden index, is scaled by
// gamma[c]); the parts are added in order; 4 entries per thread
template <typename E>
__global__ __launch_bounds__(256) void scale_cols_kernel(const float* __restrict__ R, int parts,
                                                         const float* __restrict__ gamma, int D,
                                                         int64_t n, E* __restrict__ Rs) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;   // n and D are multiples of 8
  float4 v = *reinterpret_cast<const float4*>(R + i);
  for (int q = 1; q < parts; ++q) {
    const float4 w = *reinterpret_cast<const float4*>(R + (int64_t)q * n + i);
    v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
  }
  const int c = (int)(i % D);
  v.x *= gamma[c];
  v.y *= gamma[c + 1];
  v.z *= gamma[c + 2];
  v.w *= gamma[c + 3];
  if constexpr (sizeof(E) == 2) {
    *reinterpret_cast<uint2*>(Rs + i) = make_uint2(pack_bf16x2(v.x, v.y), pack_bf16x2(v.z, v.w));
  } else {
    *reinterpret_cast<float4*>(Rs + i) = v;
  }
}

// T1 partial sums: t1[tc][h][k] = sum over token chunk tc of alpha_th^2 (g_tk^2 + u_tk^2),
// a [heads x tokens] x [tokens x neurons] product, on the fp32 matrix cores
// (16x16x4: 16 heads x 16 neuron columns, 4 tokens per step).  One wave per
// 128 neurons and chunk: lane l takes token l/16 of each step of 4 and the 8
// consecutive neurons 8 (l % 16) .. +7 (one 16-byte load of g and of u for
// bf16), so that MFMA e of a step sees column n as neuron 8 n + e; its A
// operand is alpha^2 of (token l/16, head l % 16).  Token and neuron tails and
// heads past H enter as zeros; heads in blocks of 16.  VEC (I % 8 == 0) loads
// the 8 neurons at once, else one at a time.
constexpr int kT1Chunk = 512, kT1Cols = 128, kT1Steps = 2;

// 8 consecutive g or u elements of one row as raw words (bf16 pairs when VEC,
// else fp32 bit patterns), zeros where ok is false or past the row's end
template <typename E, bool VEC>
constexpr int raw_words() { return (VEC && sizeof(E) == 2) ? 4 : 8; }

template <typename E, bool VEC>
__device__ inline void load_raw(const E* __restrict__ p, int64_t row, int c0, int I, bool ok,
                                uint32_t (&r)[raw_words<E, VEC>()]) {
  if constexpr (VEC && sizeof(E) == 2) {
    const uint4 q = ok ? *reinterpret_cast<const uint4*>(p + row * I + c0) : make_uint4(0, 0, 0, 0);
    r[0] = q.x; r[1] = q.y; r[2] = q.z; r[3] = q.w;
  } else if constexpr (VEC) {
    const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
    const float4 a = ok ? reinterpret_cast<const float4*>(p + row * I + c0)[0] : z;
    const float4 b = ok ? reinterpret_cast<const float4*>(p + row * I + c0)[1] : z;
    r[0] = __float_as_uint(a.x); r[1] = __float_as_uint(a.y); r[2] = __float_as_uint(a.z);
    r[3] = __float_as_uint(a.w); r[4] = __float_as_uint(b.x); r[5] = __float_as_uint(b.y);
    r[6] = __float_as_uint(b.z); r[7] = __float_as_uint(b.w);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      r[e] = __float_as_uint((ok && c0 + e < I) ? load_elem(p, row * I + c0 + e) : 0.f);
  }
}

template <typename E, bool VEC>
__device__ inline float raw_at(const uint32_t (&r)[raw_words<E, VEC>()], int e) {
  if constexpr (VEC && sizeof(E) == 2)
    return __uint_as_float((e & 1) ? (r[e >> 1] & 0xffff0000u) : (r[e >> 1] << 16));
  else
    return __uint_as_float(r[e]);
}

template <typename E, bool VEC>
__global__ __launch_bounds__(256) void t1_kernel(const E* __restrict__ g, const E* __restrict__ u,
                                                 const float2* __restrict__ coef, int64_t T,
                                                 int H, int I, float* __restrict__ t1) {
  constexpr int NW = raw_words<E, VEC>();
  const int lane = threadIdx.x & 63;
  // grid: x = token chunk (no 65,535 limit on long inputs), y = groups of 4 neuron tiles
  const int tile = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (tile * kT1Cols >= I) return;  // whole wave
  const int c0 = tile * kT1Cols + 8 * (lane & 15);
  const int kq = lane >> 4;
  const bool col_ok = c0 < I;
  const int64_t t0 = (int64_t)blockIdx.x * kT1Chunk, te = min(T, t0 + kT1Chunk);
  for (int h0 = 0; h0 < H; h0 += 16) {
    const int ha = h0 + (lane & 15);  // head of this lane's A element
    f32x4 acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    // the next group of 4 kT1Steps tokens is fetched before this group's MFMAs
    uint32_t rg[kT1Steps][NW], ru[kT1Steps][NW];
    float al[kT1Steps];
    auto fetch = [&](int64_t t) {
#pragma unroll
      for (int s = 0; s < kT1Steps; ++s) {
        const int64_t tt = t + 4 * s + kq;
        const bool ok = tt < te;
        const int64_t row = ok ? tt : t0;  // rows past the chunk read row t0 and weigh 0
        load_raw<E, VEC>(g, row, c0, I, col_ok, rg[s]);
        load_raw<E, VEC>(u, row, c0, I, col_ok, ru[s]);
        al[s] = (ok && ha < H) ? coef[row * H + ha].x : 0.f;
      }
    };
    fetch(t0);
    for (int64_t t = t0; t < te; t += 4 * kT1Steps) {
      float w[kT1Steps][8], a2[kT1Steps];
#pragma unroll
      for (int s = 0; s < kT1Steps; ++s) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float gv = raw_at<E, VEC>(rg[s], e), uv = raw_at<E, VEC>(ru[s], e);
          w[s][e] = fmaf(gv, gv, uv * uv);
        }
        a2[s] = al[s] * al[s];
      }
      if (t + 4 * kT1Steps < te) fetch(t + 4 * kT1Steps);
#pragma unroll
      for (int s = 0; s < kT1Steps; ++s)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          acc[e] = __builtin_amdgcn_mfma_f32_16x16x4f32(a2[s], w[s][e], acc[e], 0, 0, 0);
    }
    // lane l holds rows 4 (l / 16) + r (heads) of column l % 16 (neurons c0 + e)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = h0 + 4 * kq + r;
      if (h >= H) continue;
      float* dst = t1 + ((int64_t)blockIdx.x * H + h) * I + c0;
      if (VEC) {
        if (col_ok) {
          reinterpret_cast<float4*>(dst)[0] = make_float4(acc[0][r], acc[1][r], acc[2][r], acc[3][r]);
          reinterpret_cast<float4*>(dst)[1] = make_float4(acc[4][r], acc[5][r], acc[6][r], acc[7][r]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (c0 + e < I) dst[e] = acc[e][r];
      }
    }
  }
}

// t1r[h][k] = sum over the token chunks of t1[tc][h][k] (float64): four threads
// per output each sum a quarter of the chunks in order, then the quarters are
// added in order
__global__ __launch_bounds__(256) void t1_reduce_kernel(const float* __restrict__ t1, int n_tc,
                                                        int64_t HI, double* __restrict__ t1r) {
  __shared__ double part[4][64];
  const int o = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int64_t i = (int64_t)blockIdx.x * 64 + o;
  const int per = (n_tc + 3) / 4;
  const int b = q * per, e = min(n_tc, b + per);
  double s = 0.0;
  if (i < HI) {
#pragma unroll 8
    for (int tc = b; tc < e; ++tc) s += (double)t1[(int64_t)tc * HI + i];
  }
  part[q][o] = s;
  __syncthreads();
  if (q == 0 && i < HI) t1r[i] = ((part[0][o] + part[1][o]) + part[2][o]) + part[3][o];
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

hipError_t launch_x_prep(const float* x, int64_t T, int D, int64_t Tp, float* xx, void* xl,
                         void* xT, int dtype, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const dim3 grid((unsigned)((Tp + kXT - 1) / kXT));
  if (dtype == 1)
    hipLaunchKernelGGL(x_prep_kernel<__bf16>, grid, dim3(256), 0, st, x, T, D, Tp, xx,
                       static_cast<uint16_t*>(xl), static_cast<__bf16*>(xT));
  else
    hipLaunchKernelGGL(x_prep_kernel<float>, grid, dim3(256), 0, st, x, T, D, Tp, xx,
                       static_cast<uint16_t*>(xl), static_cast<float*>(xT));
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

hipError_t launch_scale_a(const void* a, const float2* coef, const float* xx, int64_t T, int H,
                          int d, int D, void* As, int dtype, hipStream_t st) {
  const int64_t n = T * H * d / 8;
  if (n == 0) return hipSuccess;
  const int64_t nb = (n + 255) / 256;
  const unsigned blocks = (unsigned)(nb < 65536 ? nb : 65536);
  if (dtype == 1)
    hipLaunchKernelGGL(scale_a_kernel<__bf16>, dim3(blocks), dim3(256), 0, st,
                       static_cast<const __bf16*>(a), coef, xx, T, H, d, D,
                       static_cast<__bf16*>(As));
  else
    hipLaunchKernelGGL(scale_a_kernel<float>, dim3(blocks), dim3(256), 0, st,
                       static_cast<const float*>(a), coef, xx, T, H, d, D,
                       static_cast<float*>(As));
  return hipGetLastError();
}

int64_t loo_tokens_padded(int64_t T) { return (T + 7) / 8 * 8; }

int loo_r_chunk(int64_t T) {
  const int64_t tp = loo_tokens_padded(T);
  int64_t s = T / 4096;
  s = s < 1 ? 1 : (s > 8 ? 8 : s);
  const int64_t kc = ((tp + s - 1) / s + 63) / 64 * 64;
  return (int)(kc < 64 ? 64 : kc);
}

int loo_r_parts(int64_t T) {
  const int64_t tp = loo_tokens_padded(T), kc = loo_r_chunk(T);
  return (int)((tp + kc - 1) / kc);
}

hipError_t launch_scale_cols(const float* R, int parts, const float* gamma, int HD, int D,
                             void* Rs, int dtype, hipStream_t st) {
  const int64_t n = (int64_t)HD * D;
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n / 4 + 255) / 256));
  if (dtype == 1)
    hipLaunchKernelGGL(scale_cols_kernel<__bf16>, grid, dim3(256), 0, st, R, parts, gamma, D, n,
                       static_cast<__bf16*>(Rs));
  else
    hipLaunchKernelGGL(scale_cols_kernel<float>, grid, dim3(256), 0, st, R, parts, gamma, D, n,
                       static_cast<float*>(Rs));
  return hipGetLastError();
}

bool loo_coef_fused(int d, int dtype) { return dtype == 1 && d % 32 == 0 && d >= 32 && d <= 128; }
bool loo_dot_epilogue(int d, int dtype) { return dtype == 1 && (d == 64 || d == 128); }

hipError_t launch_loo_coef_fused(const void* a, const void* Z, const float* xo_part, void* ZAT,
                                 const void* Q, const float* xx, int64_t T, int H, int d, int D,
                                 float2* coef, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int64_t n_tiles = (T + 15) / 16;
  const int64_t bx = (n_tiles + 3) / 4;
  const int64_t Tp = loo_tokens_padded(T);
  const dim3 grid((unsigned)(bx < kCoefBlocksPerHead ? bx : kCoefBlocksPerHead), (unsigned)H);
  const auto* ab = static_cast<const __bf16*>(a);
  const auto* zb = static_cast<const __bf16*>(Z);
  auto* zt = static_cast<__bf16*>(ZAT);
  const auto* qb = static_cast<const __bf16*>(Q);
  if (xo_part != nullptr) {
    // partial planes of x . o_h (head dims 64 and 128)
    switch (d) {
      case 64: hipLaunchKernelGGL((loo_coef_mfma_kernel<2, true>), grid, dim3(256), 0, st, ab, zb, xo_part, zt, qb, xx, T, Tp, H, D, coef); break;
      case 128: hipLaunchKernelGGL((loo_coef_mfma_kernel<4, true>), grid, dim3(256), 0, st, ab, zb, xo_part, zt, qb, xx, T, Tp, H, D, coef); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  switch (d / 32) {
    case 1: hipLaunchKernelGGL((loo_coef_mfma_kernel<1, false>), grid, dim3(256), 0, st, ab, zb, xo_part, zt, qb, xx, T, Tp, H, D, coef); break;
    case 2: hipLaunchKernelGGL((loo_coef_mfma_kernel<2, false>), grid, dim3(256), 0, st, ab, zb, xo_part, zt, qb, xx, T, Tp, H, D, coef); break;
    case 3: hipLaunchKernelGGL((loo_coef_mfma_kernel<3, false>), grid, dim3(256), 0, st, ab, zb, xo_part, zt, qb, xx, T, Tp, H, D, coef); break;
    case 4: hipLaunchKernelGGL((loo_coef_mfma_kernel<4, false>), grid, dim3(256), 0, st, ab, zb, xo_part, zt, qb, xx, T, Tp, H, D, coef); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int t1_chunks(int64_t T) { return (int)((T + kT1Chunk - 1) / kT1Chunk); }

hipError_t launch_t1(const void* g, const void* u, const float2* coef, int64_t T, int H, int I,
                     float* t1, int dtype, hipStream_t st) {
  if (T == 0 || I == 0) return hipSuccess;
  const bool vec = I % 8 == 0;
  const int tiles = (I + kT1Cols - 1) / kT1Cols;
  const dim3 grid(t1_chunks(T), (tiles + 3) / 4);
  if (dtype == 1) {
    const auto* gb = static_cast<const __bf16*>(g);
    const auto* ub = static_cast<const __bf16*>(u);
    if (vec) hipLaunchKernelGGL((t1_kernel<__bf16, true>), grid, dim3(256), 0, st, gb, ub, coef, T, H, I, t1);
    else hipLaunchKernelGGL((t1_kernel<__bf16, false>), grid, dim3(256), 0, st, gb, ub, coef, T, H, I, t1);
  } else {
    const auto* gf = static_cast<const float*>(g);
    const auto* uf = static_cast<const float*>(u);
    if (vec) hipLaunchKernelGGL((t1_kernel<float, true>), grid, dim3(256), 0, st, gf, uf, coef, T, H, I, t1);
    else hipLaunchKernelGGL((t1_kernel<float, false>), grid, dim3(256), 0, st, gf, uf, coef, T, H, I, t1);
  }
  return hipGetLastError();
}

hipError_t launch_t1_reduce(const float* t1, int n_tc, int64_t HI, double* t1r, hipStream_t st) {
  if (HI == 0) return hipSuccess;
  hipLaunchKernelGGL(t1_reduce_kernel, dim3((unsigned)((HI + 63) / 64)), dim3(256), 0, st, t1,
                     n_tc, HI, t1r);
  return hipGetLastError();
}

hipError_t launch_loo_combine(const LooCombineParams& p, int dtype, hipStream_t st) {
  const dim3 grid((unsigned)p.KB, (unsigned)p.G);
  if (dtype == 1) hipLaunchKernelGGL(loo_combine_kernel<__bf16>, grid, dim3(64), 0, st, p);
  else hipLaunchKernelGGL(loo_combine_kernel<float>, grid, dim3(64), 0, st, p);
  return hipGetLastError();
}

}  // namespace hna
