// fp32 "NT" GEMM on the matrix cores, C[m, n] = sum_k X[m, k] Y[n, k] with X
// and Y row-major (k contiguous), for fp32 inputs (bf16 inputs run the
// k_mm.hip kernel).  Three epilogues, the same as the bf16 kernel's:
//   * weight fold (section 3, "Affinity scores": M_h = W_o^(h)T diag(gamma)
//     W^T): X = the gamma-scaled transpose of W_o, Y = W_gate or W_up; C is
//     written in the fragment order the affinity kernel reads;
//   * down edge: X = the gamma'-scaled transpose of W_down, Y = one d'-row
//     segment of W_q, W_k or W_v; the epilogue squares C and sums over the
//     segment's rows, so b_gk itself is never stored;
//   * plain store of C transposed (C[m, n] at n * ldc + m; the leave-one-out
//     score's token and weight products), per batch entry or per K chunk.
// Eight 32x32x2 fp32 MFMAs per 16-wide K step.  Tile 128 x 128 x 32, 4 waves
// (2 x 2, 64 x 64 each), register-staged loads into an LDS double buffer with
// XOR-swizzled 16-byte chunks.
// The transposition kernel (scale_transpose) also serves the bf16 path.
#include "hna_internal.h"

namespace hna {
namespace {

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int CR = 8;                    // 16-byte chunks per BK row (fp32)

// Chunk position of (row, 16-byte column) in a tile of CR chunks per row.  The
// XOR spreads the chunks that one fragment read touches (16 consecutive rows,
// one column) over 16 distinct 16-byte bank slots, and any 8 consecutive rows
// over 8 distinct slots of a 128-byte line.
template <int CR>
__device__ inline int swz(int row, int col) {
  return row * CR + (col ^ (((row / (8 / CR)) ^ (row >> 3)) % CR));
}

// out[c, r] = s[r] * in[r, c] (s may be null: no scaling) for in [rows, cols]
// row-major, out rows of length ldo >= rows (a multiple of 16 bytes; entries
// rows .. ldo - 1 are written as zeros), bf16 output rounded to nearest even.
// 64 x 64 tiles through LDS; VEC reads the input rows in 16-byte pieces
// (needs cols % (16 / sizeof(E)) == 0).
constexpr int PT = 64;
template <typename E, bool VEC>
__global__ __launch_bounds__(256) void scale_transpose_kernel(const E* __restrict__ in,
                                                              const float* __restrict__ s,
                                                              E* __restrict__ out, int rows, int cols,
                                                              int ldo) {
  constexpr int EPC = 16 / sizeof(E);
  constexpr bool kBf = sizeof(E) == 2;
  __shared__ float tile[PT][PT + 1];
  const int r0 = blockIdx.x * PT, c0 = blockIdx.y * PT, tid = threadIdx.x;
  if constexpr (VEC) {
#pragma unroll
    for (int it = 0; it < PT * PT / EPC / 256; ++it) {
      const int q = tid + 256 * it;
      const int cc = q % (PT / EPC), rl = q / (PT / EPC);
      const int r = r0 + rl, c = c0 + cc * EPC;
      float f[EPC];
      if (r < rows && c < cols) {
        const uint4 v = *reinterpret_cast<const uint4*>(in + (int64_t)r * cols + c);
        const float sv = s ? s[r] : 1.f;
        const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
        if constexpr (kBf) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            f[2 * e] = bf16_bits_to_f32(wv[e] & 0xffffu) * sv;
            f[2 * e + 1] = bf16_bits_to_f32(wv[e] >> 16) * sv;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(wv[e]) * sv;
        }
      } else {
#pragma unroll
        for (int e = 0; e < EPC; ++e) f[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < EPC; ++e) tile[rl][cc * EPC + e] = f[e];
    }
  } else {
    const int tx = tid & 63, ty = tid >> 6;
    for (int i = ty; i < PT; i += 4) {
      const int r = r0 + i, c = c0 + tx;
      float v = 0.f;
      if (r < rows && c < cols) {
        if constexpr (kBf)
          v = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(in)[(int64_t)r * cols + c]);
        else
          v = in[(int64_t)r * cols + c];
        if (s) v *= s[r];
      }
      tile[i][tx] = v;
    }
  }
  __syncthreads();
#pragma unroll
  for (int it = 0; it < PT * PT / EPC / 256; ++it) {
    const int q = tid + 256 * it;
    const int kq = q % (PT / EPC), cl = q / (PT / EPC);
    const int c = c0 + cl, r = r0 + kq * EPC;
    if (c >= cols || r >= ldo) continue;
    float f[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) f[e] = tile[kq * EPC + e][cl];
    E* o = out + (int64_t)c * ldo + r;
    if constexpr (kBf) {
      uint32_t v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = f32_to_bf16_bits(f[2 * e]) | (f32_to_bf16_bits(f[2 * e + 1]) << 16);
      *reinterpret_cast<uint4*>(o) = make_uint4(v[0], v[1], v[2], v[3]);
    } else {
      *reinterpret_cast<float4*>(o) = make_float4(f[0], f[1], f[2], f[3]);
    }
  }
}

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const GemmParams p) {
  constexpr int CPT = BM * CR / 256;     // chunks per thread per operand tile
  constexpr int EPC = 4;                 // elements per chunk
  constexpr int TILE_CHUNKS = BM * CR;

  __shared__ uint4 xs[2][TILE_CHUNKS];
  __shared__ uint4 ys[2][TILE_CHUNKS];
  __shared__ float red[2][BM];

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int wm = w >> 1, wn = w & 1;

  // fold: x = neuron tile, y = row tile, z = gate / up; segment square: x =
  // row tile, y = segment of W_q, W_k, W_v; store: x = column tile, y = row
  // tile, z = batch entry or K chunk
  int m0, n0, z = 0;
  const float* X = static_cast<const float*>(p.X);
  const float* Y;
  int Nrows, kbeg = 0, kend = p.K;
  if constexpr (EPI == kEpiFold) {
    n0 = blockIdx.x * BN;
    m0 = blockIdx.y * BM;
    z = blockIdx.z;
    Y = static_cast<const float*>(p.Y[z]);
    Nrows = p.Nvalid;
  } else if constexpr (EPI == kEpiSegSq) {
    m0 = blockIdx.x * BM;
    n0 = 0;
    z = blockIdx.y;
    int which = 0, r0 = z;
    if (z >= p.H_next + p.G_next) { which = 2; r0 = z - p.H_next - p.G_next; }
    else if (z >= p.H_next) { which = 1; r0 = z - p.H_next; }
    Y = static_cast<const float*>(p.Y[which]) + (int64_t)r0 * p.d_next * p.ldy;
    Nrows = p.d_next;
  } else {
    n0 = blockIdx.x * BN;
    m0 = blockIdx.y * BM;
    z = blockIdx.z;
    Y = static_cast<const float*>(p.Y[0]);
    Nrows = p.N;
    if (p.k_split > 0) {
      kbeg = z * p.k_split;
      kend = min(p.K, kbeg + p.k_split);
    } else {
      X += (int64_t)z * p.bx;
      Y += (int64_t)z * p.by;
    }
  }

  uint4 xr[CPT], yr[CPT];
  auto load = [&](int k0) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int q = tid + 256 * c;
      const int row = q / CR, col = q % CR;
      const int kc = k0 + col * EPC;
      const bool okx = m0 + row < p.Mrows && kc < kend;
      xr[c] = okx ? *reinterpret_cast<const uint4*>(X + (int64_t)(m0 + row) * p.ldx + kc)
                  : make_uint4(0, 0, 0, 0);
      const bool oky = n0 + row < Nrows && kc < kend;
      yr[c] = oky ? *reinterpret_cast<const uint4*>(Y + (int64_t)(n0 + row) * p.ldy + kc)
                  : make_uint4(0, 0, 0, 0);
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      const int q = tid + 256 * c;
      const int o = swz<CR>(q / CR, q % CR);
      xs[buf][o] = xr[c];
      ys[buf][o] = yr[c];
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
  if (nk > 0) {
    load(kbeg);
    store(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load(kbeg + (kt + 1) * BK);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      uint4 af[2][2], bf[2][2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ra = wm * 64 + i * 32 + (l & 31);
        const int rb = wn * 64 + i * 32 + (l & 31);
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
          const int col = s * 4 + (l >> 5) * 2 + qq;
          af[i][qq] = xs[buf][swz<CR>(ra, col)];
          bf[i][qq] = ys[buf][swz<CR>(rb, col)];
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) mma(acc[i][j], af[i], bf[j]);
    }
    if (kt + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }

  // lane l holds column l % 32 and rows 8a + 4(l/32) + {0..3} (a = 0..3) of
  // each 32x32 tile
  if constexpr (EPI == kEpiFold) {
    // lanes l and l^32 swap halves so each lane owns two whole 8-row groups
    // (even a for l < 32, odd a otherwise); a group of 8 consecutive j of one
    // neuron is one contiguous 32-byte piece of the fold layout
    const int up = l >> 5;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        uint32_t mine[4][4];
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int v = 0; v < 4; ++v) mine[a][v] = __float_as_uint(acc[i][j][4 * a + v]);
        const int n = n0 + wn * 64 + j * 32 + (l & 31);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int ka = 2 * b + up;  // the group this lane keeps
          uint32_t lo_w[4], hi_w[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const uint32_t send = up ? mine[2 * b][v] : mine[2 * b + 1][v];
            const uint32_t recv = (uint32_t)__shfl_xor((int)send, 32);
            const uint32_t keep = up ? mine[2 * b + 1][v] : mine[2 * b][v];
            lo_w[v] = up ? recv : keep;
            hi_w[v] = up ? keep : recv;
          }
          const int m = m0 + wm * 64 + i * 32 + 8 * ka;
          if (m < p.Mrows && n < p.N) {
            const int h = m / p.d, jj = m - h * p.d;
            const int64_t o = folded_index(h, jj, n, z, p.KB, p.S);
            uint4* dst = reinterpret_cast<uint4*>(static_cast<float*>(p.M) + o);
            dst[0] = make_uint4(lo_w[0], lo_w[1], lo_w[2], lo_w[3]);
            dst[1] = make_uint4(hi_w[0], hi_w[1], hi_w[2], hi_w[3]);
          }
        }
      }
  } else if constexpr (EPI == kEpiSegSq) {
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
      p.seg_part[(int64_t)z * p.Mrows + m0 + tid] = red[0][tid] + red[1][tid];
  } else {
    // C[m, n] at n * ldc + m: a lane's 4 consecutive rows m are one 16-byte store
    float* C = static_cast<float*>(p.C) + (int64_t)z * p.bc;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + wn * 64 + j * 32 + (l & 31);
        if (n >= p.N) continue;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int mb = m0 + wm * 64 + i * 32 + 8 * a + 4 * (l >> 5);
          if (mb >= p.Mrows) continue;
          float* o = C + (int64_t)n * p.ldc + mb;
          if (mb + 4 <= p.Mrows) {
            *reinterpret_cast<float4*>(o) = make_float4(acc[i][j][4 * a], acc[i][j][4 * a + 1],
                                                        acc[i][j][4 * a + 2], acc[i][j][4 * a + 3]);
          } else {
            for (int e = 0; e < p.Mrows - mb; ++e) o[e] = acc[i][j][4 * a + e];
          }
        }
      }
  }
}

}  // namespace

hipError_t launch_scale_transpose(const void* in, const float* s, void* out, int rows, int cols,
                                  int ldo, int dtype, hipStream_t st) {
  if (rows == 0 || cols == 0) return hipSuccess;
  dim3 grid((ldo + PT - 1) / PT, (cols + PT - 1) / PT);
  if (dtype == 1) {
    const auto* i = static_cast<const __bf16*>(in);
    auto* o = static_cast<__bf16*>(out);
    if (cols % 8 == 0) hipLaunchKernelGGL((scale_transpose_kernel<__bf16, true>), grid, dim3(256), 0, st, i, s, o, rows, cols, ldo);
    else hipLaunchKernelGGL((scale_transpose_kernel<__bf16, false>), grid, dim3(256), 0, st, i, s, o, rows, cols, ldo);
  } else {
    const auto* i = static_cast<const float*>(in);
    auto* o = static_cast<float*>(out);
    if (cols % 4 == 0) hipLaunchKernelGGL((scale_transpose_kernel<float, true>), grid, dim3(256), 0, st, i, s, o, rows, cols, ldo);
    else hipLaunchKernelGGL((scale_transpose_kernel<float, false>), grid, dim3(256), 0, st, i, s, o, rows, cols, ldo);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_f32(const GemmParams& p, int epilogue, int ny, hipStream_t st) {
  if (p.Mrows == 0 || ny == 0) return hipSuccess;
  const unsigned mt = (unsigned)((p.Mrows + BM - 1) / BM);
  if (epilogue == kEpiFold) {
    const dim3 grid((unsigned)((p.N + BN - 1) / BN), mt, (unsigned)ny);
    hipLaunchKernelGGL(gemm_f32_kernel<kEpiFold>, grid, dim3(256), 0, st, p);
  } else if (epilogue == kEpiSegSq) {
    hipLaunchKernelGGL(gemm_f32_kernel<kEpiSegSq>, dim3(mt, (unsigned)ny), dim3(256), 0, st, p);
  } else {
    if (p.N == 0) return hipSuccess;
    const dim3 grid((unsigned)((p.N + BN - 1) / BN), mt, (unsigned)ny);
    hipLaunchKernelGGL(gemm_f32_kernel<kEpiStore>, grid, dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace hna
