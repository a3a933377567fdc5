// Scaled "NT" GEMM on the matrix cores, C[m, n] = sum_c X[m, c] s[c] Y[n, c],
// with X [Mrows, K] and Y [N, K] row-major (c contiguous).  Two uses, both
// from section 3 ("Affinity scores") of the affinity-aware sharding paper:
//   * weight fold: X = W_o^T (rows h*d+j), Y = W_gate or W_up, s = gamma;
//     C = M_h[j, k], written in the fragment order the affinity kernel reads;
//   * down edge: X = W_down^T (rows k), Y = one d'-row segment of W_q, W_k or
//     W_v, s = gamma'; the epilogue squares C and sums over the segment's
//     rows, so b_gk itself is never stored.
// bf16 inputs: X is exact in bf16; s*Y is formed in fp32 and split into a
// bf16 high part and a bf16 remainder, and both are multiplied (2 MFMAs), so
// the product is accurate to fp32 accumulation.  fp32 inputs use fp32 MFMA.
// Tile 128 x 128 x 32, 4 waves (2 x 2, 64 x 64 each), LDS double buffer with
// XOR-swizzled 16-byte chunks.
#include "hna_internal.h"

namespace hna {
namespace {

constexpr int BM = 128, BN = 128, BK = 32;

template <typename T> struct GT;
template <> struct GT<__bf16> {
  static constexpr int kBytes = 2, kCR = 4, kCPS = 2, kQ = 1, kSplit = 2;
};
template <> struct GT<float> {
  static constexpr int kBytes = 4, kCR = 8, kCPS = 4, kQ = 2, kSplit = 1;
};

__device__ inline void mma(f32x16& c, const uint4 (&a)[1], const uint4 (&b)[1]) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[0]),
                                              __builtin_bit_cast(bf16x8, b[0]), c, 0, 0, 0);
}
__device__ inline void mma(f32x16& c, const uint4 (&a)[2], const uint4 (&b)[2]) {
  const float af[8] = {__uint_as_float(a[0].x), __uint_as_float(a[0].y), __uint_as_float(a[0].z),
                       __uint_as_float(a[0].w), __uint_as_float(a[1].x), __uint_as_float(a[1].y),
                       __uint_as_float(a[1].z), __uint_as_float(a[1].w)};
  const float bf[8] = {__uint_as_float(b[0].x), __uint_as_float(b[0].y), __uint_as_float(b[0].z),
                       __uint_as_float(b[0].w), __uint_as_float(b[1].x), __uint_as_float(b[1].y),
                       __uint_as_float(b[1].z), __uint_as_float(b[1].w)};
#pragma unroll
  for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(af[e], bf[e], c, 0, 0, 0);
}

template <int CR>
__device__ inline int swz(int row, int col) {
  return row * CR + (col ^ ((row / (8 / CR)) % CR));
}

template <typename T, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmParams p) {
  using Tr = GT<T>;
  constexpr int CR = Tr::kCR;            // 16-byte chunks per BK row
  constexpr int CPT = BM * CR / 256;     // chunks per thread per operand tile
  constexpr int EPC = 16 / Tr::kBytes;   // elements per chunk
  constexpr int NSPLIT = Tr::kSplit;
  constexpr int Q = Tr::kQ;
  constexpr int TILE_CHUNKS = BM * CR;

  __shared__ uint4 xs[2][TILE_CHUNKS];
  __shared__ uint4 ys[2][NSPLIT][TILE_CHUNKS];
  __shared__ float red[2][BM];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int wm = w >> 1, wn = w & 1;

  int m0, n0, gu = 0, seg = 0;
  const T* Y;
  int Nrows;
  if (EPI == kEpiFold) {
    n0 = blockIdx.x * BN;
    m0 = blockIdx.y * BM;
    gu = blockIdx.z;
    Y = static_cast<const T*>(p.Y[gu]);
    Nrows = p.Nvalid;
  } else {
    m0 = blockIdx.x * BM;
    n0 = 0;
    seg = blockIdx.y;
    int which = 0, r0 = seg;
    if (seg >= p.H_next + p.G_next) { which = 2; r0 = seg - p.H_next - p.G_next; }
    else if (seg >= p.H_next) { which = 1; r0 = seg - p.H_next; }
    Y = static_cast<const T*>(p.Y[which]) + (int64_t)r0 * p.d_next * p.ldy;
    Nrows = p.d_next;
  }
  const T* X = static_cast<const T*>(p.X);
  const int K = p.K;

  uint4 xr[CPT], yr[CPT][NSPLIT];
  auto load = [&](int k0) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int q = tid + 256 * c;
      const int row = q / CR, col = q % CR;
      const int kc = k0 + col * EPC;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m0 + row < p.Mrows && kc < K)
        v = *reinterpret_cast<const uint4*>(X + (int64_t)(m0 + row) * p.ldx + kc);
      xr[c] = v;
      float f[8];
      const bool ok = n0 + row < Nrows && kc < K;
      if constexpr (NSPLIT == 2) {
        uint4 yv = make_uint4(0, 0, 0, 0);
        if (ok) yv = *reinterpret_cast<const uint4*>(Y + (int64_t)(n0 + row) * p.ldy + kc);
        const uint32_t wv[4] = {yv.x, yv.y, yv.z, yv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[2 * e] = bf16_bits_to_f32(wv[e] & 0xffffu);
          f[2 * e + 1] = bf16_bits_to_f32(wv[e] >> 16);
        }
        uint32_t hi[4], lo[4];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float sv = ok ? f[e] * p.s[kc + e] : 0.f;
          const uint32_t hb = f32_to_bf16_bits(sv);
          const uint32_t lb = f32_to_bf16_bits(sv - bf16_bits_to_f32(hb));
          if (e & 1) { hi[e >> 1] |= hb << 16; lo[e >> 1] |= lb << 16; }
          else { hi[e >> 1] = hb; lo[e >> 1] = lb; }
        }
        yr[c][0] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        yr[c][1] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      } else {
        float4 yv = make_float4(0.f, 0.f, 0.f, 0.f);
        if (ok) {
          yv = *reinterpret_cast<const float4*>(Y + (int64_t)(n0 + row) * p.ldy + kc);
          yv.x *= p.s[kc]; yv.y *= p.s[kc + 1]; yv.z *= p.s[kc + 2]; yv.w *= p.s[kc + 3];
        }
        yr[c][0] = make_uint4(__float_as_uint(yv.x), __float_as_uint(yv.y),
                              __float_as_uint(yv.z), __float_as_uint(yv.w));
        (void)f;
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int q = tid + 256 * c;
      const int row = q / CR, col = q % CR;
      const int o = swz<CR>(row, col);
      xs[buf][o] = xr[c];
#pragma unroll
      for (int sp = 0; sp < NSPLIT; ++sp) ys[buf][sp][o] = yr[c][sp];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int nk = (K + BK - 1) / BK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * BK);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      uint4 af[2][Q], bf[2][NSPLIT][Q];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ra = wm * 64 + i * 32 + (l & 31);
        const int rb = wn * 64 + i * 32 + (l & 31);
#pragma unroll
        for (int qq = 0; qq < Q; ++qq) {
          const int col = s * Tr::kCPS + (l >> 5) * Q + qq;
          af[i][qq] = xs[buf][swz<CR>(ra, col)];
#pragma unroll
          for (int sp = 0; sp < NSPLIT; ++sp) bf[i][sp][qq] = ys[buf][sp][swz<CR>(rb, col)];
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int sp = 0; sp < NSPLIT; ++sp) mma(acc[i][j], af[i], bf[j][sp]);
    }
    if (kt + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }

  if (EPI == kEpiFold) {
    T* Mout = static_cast<T*>(p.M);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int m = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
          const int n = n0 + wn * 64 + j * 32 + (l & 31);
          if (m < p.Mrows && n < p.N) {
            const int h = m / p.d, jj = m - h * p.d;
            const int64_t o = folded_index(h, jj, n, gu, p.KB, p.S);
            if constexpr (Tr::kBytes == 2)
              reinterpret_cast<uint16_t*>(Mout)[o] = (uint16_t)f32_to_bf16_bits(acc[i][j][v]);
            else
              reinterpret_cast<float*>(Mout)[o] = acc[i][j][v];
          }
        }
  } else {
    // sum of squares over this segment's rows n (columns of C)
    float sq[2][16];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        sq[i][v] = acc[i][0][v] * acc[i][0][v] + acc[i][1][v] * acc[i][1][v];
#pragma unroll
    for (int off = 1; off < 32; off <<= 1)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) sq[i][v] += __shfl_xor(sq[i][v], off);
    if ((l & 31) == 0) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          red[wn][wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3)] = sq[i][v];
    }
    __syncthreads();
    if (tid < BM && m0 + tid < p.Mrows)
      p.seg_part[(int64_t)seg * p.Mrows + m0 + tid] = red[0][tid] + red[1][tid];
  }
}

}  // namespace

hipError_t launch_gemm(const GemmParams& p, int dtype, int epilogue, dim3 grid, hipStream_t st) {
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return hipSuccess;
  if (dtype == 1) {
    if (epilogue == kEpiFold) hipLaunchKernelGGL((gemm_kernel<__bf16, kEpiFold>), grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL((gemm_kernel<__bf16, kEpiSegSq>), grid, dim3(256), 0, st, p);
  } else {
    if (epilogue == kEpiFold) hipLaunchKernelGGL((gemm_kernel<float, kEpiFold>), grid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL((gemm_kernel<float, kEpiSegSq>), grid, dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace hna
