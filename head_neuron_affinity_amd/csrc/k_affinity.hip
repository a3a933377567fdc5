// The hot pass: first-order damage (eq. 5) and the FO / ADD up scores of
// "Affinity-Aware Sharding for Delayed Tensor Parallelism", section 3,
// paragraph "Affinity scores", plus the token moment of the down edge.
//
// Work decomposition (gfx950, wave64, 1 wave per SIMD):
//   * a workgroup owns 128 neurons (4 waves x 32) and a chunk of up to 8
//     consecutive token tiles of 128 tokens;
//   * per token tile each lane computes, once, the operating-point
//     coefficients A = silu'(g) u / r and B = silu(g) / r for the 64 (t, k)
//     pairs it holds in the MFMA C layout, and the down-edge moment;
//   * then for every head h (in KV-group order) the wave runs a 128 x 32 x d
//     contraction a_h . M_h on the matrix cores for gate and up columns
//     (8 MFMA 32x32 tiles), giving (p_h.w^g_k, p_h.w^u_k) * r in registers;
//   * the epilogue forms Delta = A Pg + B Pu and accumulates Delta^2 and
//     (Pg^2 + Pu^2) / r^2 into per-lane running sums; when the KV group
//     changes the sums are added to a per-(group, lane) LDS slot;
//   * nothing of size T x H x I leaves registers: each workgroup writes one
//     [2G+1, 128] block of fp32 partial sums, reduced later in fixed order.
// The head's a tile is double-buffered in LDS (XOR-swizzled 16-byte chunks,
// conflict-free fragment reads); the folded weights stream straight from
// global memory in fragment order.  Workgroups are mapped to XCDs so that the
// 32 concurrent workgroups of one XCD cover 4 neuron tiles x 8 token chunks
// and share a and M in that XCD's L2.
#include "hna_internal.h"

namespace hna {
namespace {

template <typename T> struct Traits;
template <> struct Traits<__bf16> {
  static constexpr int kBytes = 2;
  static constexpr int kChunksPerStep = 2;  // 16 values of d = 32 bytes
  static constexpr int kQuads = 1;          // 16 bytes per lane per fragment
};
template <> struct Traits<float> {
  static constexpr int kBytes = 4;
  static constexpr int kChunksPerStep = 4;  // 16 values of d = 64 bytes
  static constexpr int kQuads = 2;          // 32 bytes per lane per fragment
};

__device__ inline void mma(f32x16& c, const uint4 (&a)[1], const uint4 (&b)[1]) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[0]),
                                              __builtin_bit_cast(bf16x8, b[0]), c, 0, 0, 0);
}
// fp32: eight K=2 MFMAs.  MFMA e pairs element e of the lower lane half
// (d index 16s+e) with element e of the upper half (16s+8+e).
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

__device__ inline float load_elem(const __bf16* p, int64_t i) {
  return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
}
__device__ inline float load_elem(const float* p, int64_t i) { return p[i]; }

constexpr int pow2_slots(int cpr) { return cpr <= 8 ? 8 : (cpr <= 16 ? 16 : 32); }

// LDS per-token vectors of one tile: 1/r, 1/r^2, 1/r_next.
constexpr int kTokVec = 3 * kTileTokens;

template <typename E, int S>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void affinity_up_kernel(const UpParams p) {
  using T = E;
  using Tr = Traits<E>;
  constexpr int Q = Tr::kQuads;
  constexpr int CPS = Tr::kChunksPerStep;
  constexpr int CPR = S * CPS;              // 16-byte chunks per row of a_h
  constexpr int SLOTS = pow2_slots(CPR);
  constexpr int ROWB = SLOTS * 16;
  constexpr int BUFB = kTileTokens * ROWB;
  constexpr int CPT = CPR / 2;              // chunks staged per thread per tile

  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  unsigned char* abuf = lds;                                    // [2][128][ROWB]
  float* tokvec = reinterpret_cast<float*>(lds + 2 * BUFB);     // [2][3][128]
  float* accl = tokvec + 2 * kTokVec;                           // [2G][256]

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
  const int nb = kt * 4 + w;                 // this wave's block of 32 neurons
  const int nbc = nb < KB ? nb : KB - 1;     // clamped so that M reads stay in bounds
  const int k = nb * 32 + (l & 31);
  const bool kvalid = nb < KB && k < I;
  const T* a = static_cast<const T*>(p.a);
  const T* gp = static_cast<const T*>(p.g);
  const T* up = static_cast<const T*>(p.u);
  const T* M = static_cast<const T*>(p.M);
  const bool want_c = p.r_next != nullptr;

  for (int x = tid; x < 2 * G * 256; x += 256) accl[x] = 0.f;

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
  auto stage_tokvec = [&](int ti, int buf) {
    if (tid < kTileTokens) {
      const int64_t t = (int64_t)(tt0 + ti) * kTileTokens + tid;
      float ri = 0.f, rn = 0.f;
      if (t < NT) {
        ri = 1.0f / p.r[t];
        if (want_c) rn = 1.0f / p.r_next[t];
      }
      float* tv = tokvec + buf * kTokVec;
      tv[tid] = ri;
      tv[kTileTokens + tid] = ri * ri;
      tv[2 * kTileTokens + tid] = rn;
    }
  };

  // prologue: first (tile, head) in LDS buffer 0
  load_stage(0);
  stage_tokvec(0, 0);
  store_stage(0);
  __syncthreads();

  f32x16 accG[4], accU[4];
  float coefA[4][16], coefB[4][16];
  float fo_run[4] = {0.f, 0.f, 0.f, 0.f}, add_run[4] = {0.f, 0.f, 0.f, 0.f};
  float c_acc = 0.f;
  const int64_t slab = (int64_t)64 * 8;            // elements per (h, kb, gu, s)
  const T* Mw = M + (int64_t)nbc * 2 * S * slab + l * 8;

  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    const int ti = step / H, hi = step - ti * H;
    const int h = p.head_order[hi];
    const int grp = p.head_group[hi];
    const bool has_next = step + 1 < nsteps;
    if (has_next) load_stage(step + 1);

    if (hi == 0) {
      // operating-point coefficients of this tile, shared by all heads
      const float* tv = tokvec + (ti & 1) * kTokVec;
      const int64_t tbase = (int64_t)(tt0 + ti) * kTileTokens;
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = tb * 32 + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
          const int64_t t = tbase + row;
          float A = 0.f, B = 0.f;
          if (kvalid && t < NT) {
            const float gv = load_elem(gp, t * I + k);
            const float uv = load_elem(up, t * I + k);
            const float ri = tv[row];
            const float sg = 1.0f / (1.0f + __expf(-gv));   // logistic sigma(g)
            const float silu = gv * sg;
            const float dsilu = fmaf(silu, 1.0f - sg, sg);   // sigma (1 + g (1 - sigma))
            A = dsilu * uv * ri;
            B = silu * ri;
            if (want_c) {
              const float al = silu * uv * tv[2 * kTileTokens + row];
              c_acc = fmaf(al, al, c_acc);
            }
          }
          coefA[tb][v] = A;
          coefB[tb][v] = B;
        }
      }
    }
    if (hi == H - 1 && ti + 1 < ntile) stage_tokvec(ti + 1, (ti + 1) & 1);

    // a_h (128 x d) . M_h (d x [32 gate | 32 up]) on the matrix cores
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      accG[tb] = f32x16{};
      accU[tb] = f32x16{};
    }
    const unsigned char* ab = abuf + buf * BUFB;
    const T* Mh = Mw + (int64_t)h * KB * 2 * S * slab;
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

    // fused epilogue: eq. (5), its square, and the ADD terms
    const float* r2 = tokvec + (ti & 1) * kTokVec + kTileTokens;
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        const float4 rr = *reinterpret_cast<const float4*>(r2 + tb * 32 + 8 * vq + 4 * (l >> 5));
        const float rv[4] = {rr.x, rr.y, rr.z, rr.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int v = vq * 4 + i;
          const float pg = accG[tb][v], pu = accU[tb][v];
          const float dl = fmaf(coefA[tb][v], pg, coefB[tb][v] * pu);
          fo_run[tb] = fmaf(dl, dl, fo_run[tb]);
          const float q2 = fmaf(pg, pg, pu * pu);
          add_run[tb] = fmaf(q2, rv[i], add_run[tb]);
        }
      }
    }
    if (hi == H - 1 || p.head_group[hi + 1] != grp) {
      accl[grp * 256 + tid] += (fo_run[0] + fo_run[1]) + (fo_run[2] + fo_run[3]);
      accl[(G + grp) * 256 + tid] += (add_run[0] + add_run[1]) + (add_run[2] + add_run[3]);
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) fo_run[tb] = add_run[tb] = 0.f;
    }
    if (has_next) store_stage(buf ^ 1);
    __syncthreads();
  }

  // lanes l and l+32 hold the same neuron: combine and write the partial sums
  c_acc += __shfl_xor(c_acc, 32);
  if (l < 32 && nb < KB) {
    const int kk = nb * 32 + l;
    float* out = p.part + (int64_t)chunk * (2 * G + 1) * p.I32;
    for (int gg = 0; gg < 2 * G; ++gg)
      out[(int64_t)gg * p.I32 + kk] = accl[gg * 256 + tid] + accl[gg * 256 + tid + 32];
    out[(int64_t)2 * G * p.I32 + kk] = c_acc;
  }
}

// Fixed-order reduction of the partial sums (float64 accumulation).
__global__ __launch_bounds__(256) void finalize_up_kernel(const float* __restrict__ part,
                                                          int n_chunks, int G, int I, int I32,
                                                          const float* __restrict__ wd_sq,
                                                          float scale, int accumulate,
                                                          float* S_fo, float* S_add,
                                                          float* c_down) {
  const int rows = 2 * G + (c_down ? 1 : 0);
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)rows * I) return;
  const int row = (int)(idx / I), k = (int)(idx - (int64_t)row * I);
  double s = 0.0;
  for (int c = 0; c < n_chunks; ++c) s += part[((int64_t)c * (2 * G + 1) + row) * I32 + k];
  float* dst;
  double v = s * (double)scale;
  if (row < G) {
    v *= (double)wd_sq[k];
    dst = S_fo + (int64_t)row * I + k;
  } else if (row < 2 * G) {
    dst = S_add + (int64_t)(row - G) * I + k;
  } else {
    dst = c_down + k;
  }
  *dst = accumulate ? *dst + (float)v : (float)v;
}

template <typename T, int S>
hipError_t launch_typed(const UpParams& p, size_t lds, int grid, hipStream_t st) {
  auto fn = affinity_up_kernel<T, S>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(256), lds, st, p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_by_steps(const UpParams& p, size_t lds, int grid, hipStream_t st) {
  switch (p.d / 16) {
    case 1: return launch_typed<T, 1>(p, lds, grid, st);
    case 2: return launch_typed<T, 2>(p, lds, grid, st);
    case 3: return launch_typed<T, 3>(p, lds, grid, st);
    case 4: return launch_typed<T, 4>(p, lds, grid, st);
    case 5: return launch_typed<T, 5>(p, lds, grid, st);
    case 6: return launch_typed<T, 6>(p, lds, grid, st);
    case 7: return launch_typed<T, 7>(p, lds, grid, st);
    case 8: return launch_typed<T, 8>(p, lds, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

UpGeometry up_geometry(int64_t T, int H, int G, int d, int I, int dtype) {
  UpGeometry g{};
  g.I32 = round_up(I, 32);
  g.n_tt = (int)((T + kTileTokens - 1) / kTileTokens);
  g.n_kt = (g.I32 + kTileNeurons - 1) / kTileNeurons;
  g.n_chunks = (g.n_tt + kTilesPerChunk - 1) / kTilesPerChunk;
  g.n_ktg = (g.n_kt + kSuperKt - 1) / kSuperKt;
  g.n_cg = (g.n_chunks + kSuperChunks - 1) / kSuperChunks;
  g.n_st = g.n_ktg * g.n_cg;
  g.grid = round_up(g.n_st, 8) * 32;
  g.part_floats = (size_t)g.n_chunks * (2 * G + 1) * g.I32;
  const int cpr = (d / 16) * (dtype == 1 ? 2 : 4);
  const int slots = pow2_slots(cpr);
  g.lds_bytes = (size_t)2 * kTileTokens * slots * 16 + (size_t)2 * kTokVec * 4 +
                (size_t)2 * G * 256 * 4;
  return g;
}

hipError_t launch_affinity_up(const UpParams& p, int dtype, size_t lds_bytes, int grid,
                              hipStream_t st) {
  if (grid == 0) return hipSuccess;
  return dtype == 1 ? launch_by_steps<__bf16>(p, lds_bytes, grid, st)
                    : launch_by_steps<float>(p, lds_bytes, grid, st);
}

hipError_t launch_finalize_up(const float* part, int n_chunks, int G, int I, int I32,
                              const float* wd_sq, float scale, int accumulate, float* S_fo,
                              float* S_add, float* c_down, hipStream_t st) {
  const int64_t n = (int64_t)(2 * G + (c_down ? 1 : 0)) * I;
  const int blocks = (int)((n + 255) / 256);
  hipLaunchKernelGGL(finalize_up_kernel, dim3(blocks), dim3(256), 0, st, part, n_chunks, G, I,
                     I32, wd_sq, scale, accumulate, S_fo, S_add, c_down);
  return hipGetLastError();
}

}  // namespace hna
