// The hot pass: first-order damage (eq. 5) and the FO up score of
// "Affinity-Aware Sharding for Delayed Tensor Parallelism", section 3,
// paragraph "Affinity scores", plus the token moment of the down edge.
// (The ADD score is linear in per-head Gram matrices and is formed from them
// in k_gram.hip; this kernel does not touch it.)
//
// Work decomposition (gfx950, wave64, 8 waves = 2 per SIMD):
//   * a workgroup owns 128 neurons and a chunk of up to 8 consecutive token
//     tiles of 128 tokens; wave w covers 64 tokens (w >> 2) x 32 neurons
//     (w & 3);
//   * per token tile each lane computes, once, the operating-point
//     coefficients A = silu'(g) u / r and B = silu(g) / r for the 32 (t, k)
//     pairs it holds in the MFMA C layout, and the down-edge moment;
//   * then for every head h (in KV-group order) the wave runs a 64 x 32 x d
//     contraction a_h . M_h on the matrix cores for gate and up columns,
//     giving r * (p_h.w^g_k, p_h.w^u_k) in registers;
//   * the epilogue forms Delta = A Pg + B Pu and accumulates Delta^2 into
//     per-lane running sums (three VALU operations per pair); when the KV
//     group changes the sums are added to a per-(group, lane) LDS slot.  The
//     two waves of a SIMD overlap one's epilogue with the other's MFMAs;
//   * nothing of size T x H x I leaves registers: each workgroup writes one
//     [G+1, 128] block of fp32 partial sums, reduced later in fixed order.
// The head's a tile is double-buffered in LDS by asynchronous LDS DMA
// (XOR-swizzled 16-byte chunks, conflict-free fragment reads); the g/u tile
// of the next token tile is copied the same way; the folded weights stream
// straight from global memory into a register ring in fragment order.
// Workgroups are mapped to XCDs so that the 32 concurrent workgroups of one
// XCD cover 4 neuron tiles x 8 token chunks and share a and M in that XCD's L2.
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

__device__ inline float load_elem(const __bf16* p, int64_t i) {
  return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(p)[i]);
}
__device__ inline float load_elem(const float* p, int64_t i) { return p[i]; }

constexpr int pow2_slots(int cpr) { return cpr <= 8 ? 8 : (cpr <= 16 ? 16 : 32); }

// LDS per-token vectors of one tile: 1/r, 1/r_next.
constexpr int kTokVec = 2 * kTileTokens;

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (LGKM and export counters untouched).
constexpr int vm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

typedef __attribute__((address_space(3))) void* lds_ptr;

// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes
// return zeros (hardware range check), so tile edges need no clamping.
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000 /* 32-bit data format, no swizzle */);
}
constexpr uint32_t kOutOfRange = 0x7ffffff0u;   // offset past any resource: reads zeros

// Asynchronous 16-byte buffer -> LDS copy: lane l copies the 16 bytes at
// voff + soff and writes them at dst + 16 l.  Only voff is range checked.
__device__ inline void dma16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff,
                             unsigned char* dst_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)dst_wave_base, 16, voff, soff, 0, 0);
}

constexpr int kWaves = 8;             // 2 per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kTB = 2;                // 32-token blocks per wave (64 tokens)

template <typename E, int S, bool GULDS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void affinity_up_kernel(const UpParams p) {
  using T = E;
  using Tr = Traits<E>;
  constexpr int Q = Tr::kQuads;
  constexpr int CPS = Tr::kChunksPerStep;
  constexpr int EPC = 16 / Tr::kBytes;      // elements per 16-byte chunk
  constexpr int CPR = S * CPS;              // 16-byte chunks per row of a_h
  constexpr int SLOTS = pow2_slots(CPR);
  constexpr int ROWB = SLOTS * 16;
  constexpr int BUFB = kTileTokens * ROWB;
  constexpr int DMA_A = kTileTokens * SLOTS / kThreads;   // a-tile copies per thread per step
  constexpr int DMA_GU = GULDS ? 2 * kTileTokens * 16 / kThreads : 0;
  constexpr int GU_BYTES = GULDS ? 2 * kTileTokens * 256 : 16;

  // Distinct static LDS objects: the compiler can tell a pending copy into one
  // a-tile buffer (or the g/u tile) from reads of the other buffer.
  __shared__ __attribute__((aligned(16))) unsigned char abuf0[BUFB];
  __shared__ __attribute__((aligned(16))) unsigned char abuf1[BUFB];
  __shared__ __attribute__((aligned(16))) unsigned char gubuf[GU_BYTES];
  __shared__ __attribute__((aligned(16))) float tokvec[2 * kTokVec];
  __shared__ __attribute__((aligned(16))) float cbuf[2 * kTileNeurons];
  extern __shared__ __attribute__((aligned(16))) float accl[];   // [G][2][128] FO sums

  // workgroup -> (neuron tile, token chunk); consecutive ids alternate XCDs
  const int id = blockIdx.x;
  const int xcd = id & 7, wi = id >> 3;
  const int st = xcd + 8 * (wi >> 5), mem = wi & 31;
  if (st >= p.n_st) return;
  const int kt = (st % p.n_ktg) * kSuperKt + (mem & 3);
  const int chunk = (st / p.n_ktg) * kSuperChunks + (mem >> 2);
  if (kt >= p.n_kt || chunk >= p.n_chunks) return;

  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int wn = w & 3, wt = w >> 2;         // neuron block, token half
  const int H = p.H, G = p.G, I = p.I, d = p.d;
  const int64_t NT = p.T;
  const int KB = p.I32 >> 5;
  const int nb = kt * 4 + wn;                // this wave's block of 32 neurons
  const int nbc = nb < KB ? nb : KB - 1;     // clamped so that M reads stay in bounds
  const int k = nb * 32 + (l & 31);
  const int kc = k < I ? k : I - 1;          // clamped neuron for direct g/u reads
  const T* a = static_cast<const T*>(p.a);
  const T* gp = static_cast<const T*>(p.g);
  const T* up = static_cast<const T*>(p.u);
  const T* M = static_cast<const T*>(p.M);
  const bool want_c = p.want_c != 0;

  for (int x = tid; x < G * 2 * kTileNeurons; x += kThreads) accl[x] = 0.f;

  const int tt0 = chunk * kTilesPerChunk;
  const int ntile = min(kTilesPerChunk, p.n_tt - tt0);
  const int nsteps = ntile * H;

  // ---- asynchronous copies into LDS --------------------------------------
  // a tile of a (token tile, head) step: slot q of the buffer holds row
  // q / SLOTS, chunk (q % SLOTS) ^ (row % SLOTS).  A wave copies 64
  // consecutive slots (64 / SLOTS whole rows); rows past T and unused slots
  // read zeros through the buffer range check.
  auto dma_a = [&](int step, unsigned char* buf) {
    const int ti = step / H;
    const int h = p.head_order[step - ti * H];
    const int64_t t0 = (int64_t)(tt0 + ti) * kTileTokens;
    const int rows = (int)min((int64_t)kTileTokens, NT - t0);
    const uint32_t row_bytes = (uint32_t)(H * d * Tr::kBytes);
    const auto rs = buffer_rsrc(a + (t0 * H + h) * d,
                                (uint32_t)(rows - 1) * row_bytes + (uint32_t)(d * Tr::kBytes));
#pragma unroll
    for (int i = 0; i < DMA_A; ++i) {
      const int slot0 = (i * kWaves + w) * 64;
      const int row0 = slot0 / SLOTS;                       // wave-uniform
      const int row = row0 + l / SLOTS, sl = l % SLOTS;
      const int c = sl ^ (row & (SLOTS - 1));
      // the whole offset goes in voff: the range check does not cover soff
      const uint32_t voff = c < CPR ? (uint32_t)row * row_bytes + (uint32_t)(c * 16) : kOutOfRange;
      dma16(rs, voff, 0u, buf + slot0 * 16);
    }
  };
  // g and u tiles (bf16, 128 tokens x 128 neurons each; row = 16 chunks of 8
  // neurons, chunk c of row r in slot c ^ (r & 4): conflict-free reads).  A
  // wave copies 4 whole rows per instruction; rows past T read zeros.
  auto dma_gu = [&](int ti) {
    if constexpr (GULDS) {
      const int64_t t0 = (int64_t)(tt0 + ti) * kTileTokens;
      const int rows = (int)min((int64_t)kTileTokens, NT - t0);
      const int n0 = kt * kTileNeurons;
      const uint32_t row_bytes = (uint32_t)I * 2u;
      const uint32_t bytes = (uint32_t)rows * row_bytes - (uint32_t)n0 * 2u;
      const auto rg = buffer_rsrc(gp + t0 * I + n0, bytes);
      const auto ru = buffer_rsrc(up + t0 * I + n0, bytes);
#pragma unroll
      for (int i = 0; i < DMA_GU; ++i) {
        const int slot0 = (i * kWaves + w) * 64;   // slot index over [g tile | u tile]
        const int which = slot0 >= kTileTokens * 16;
        const int row0 = (slot0 - which * kTileTokens * 16) >> 4;
        const int row = row0 + (l >> 4);
        const int c = (l & 15) ^ (row & 4);
        const uint32_t voff = (uint32_t)row * row_bytes + (uint32_t)(c * 16);
        dma16(which ? ru : rg, voff, 0u, gubuf + slot0 * 16);
      }
    }
  };
  auto stage_tokvec = [&](int ti, int tb) {
    if (tid < kTileTokens) {
      const int64_t t = (int64_t)(tt0 + ti) * kTileTokens + tid;
      float ri = 0.f, rn = 0.f;
      if (t < NT) {
        ri = __builtin_amdgcn_rcpf(p.r[t]);
        if (want_c) rn = __builtin_amdgcn_rcpf(p.r_next[t]);
      }
      float* tv = tokvec + tb * kTokVec;
      tv[tid] = ri;
      tv[kTileTokens + tid] = rn;
    }
  };

  // ---- registers ------------------------------------------------------------
  f32x16 accG[kTB], accU[kTB];
  float coefA[kTB][16], coefB[kTB][16];
  float fo_run[kTB];
#pragma unroll
  for (int tb = 0; tb < kTB; ++tb) fo_run[tb] = 0.f;
  float c_acc = 0.f;
  constexpr int kSlabBytes = 64 * 8 * Tr::kBytes;      // one (h, kb, gu, s) fragment slab
  const char* Mbytes = reinterpret_cast<const char*>(M);
  const uint32_t mlane = (uint32_t)l * 8u * Tr::kBytes;
  // M fragments stream through a ring of D register slots: K-step s of a
  // step uses slot s % D, and right after its MFMAs the slot is refilled with
  // the K-step D positions later (in this step or the next one).
  constexpr int D = (S % 2 == 0) ? S / 2 : S;
  constexpr int NM = 2 * D * Q;   // M loads that may be outstanding at a step boundary
  uint4 mreg[D][2][Q];
  auto load_m = [&](int slot, int s, int h) {
    // wave-uniform base of (h, this wave's neuron block), per-lane 32-bit offset
    const char* Mh = Mbytes + ((int64_t)h * KB + nbc) * 2 * S * kSlabBytes;
#pragma unroll
    for (int qq = 0; qq < Q; ++qq) {
      mreg[slot][0][qq] = *reinterpret_cast<const uint4*>(Mh + mlane + s * kSlabBytes + qq * 16);
      mreg[slot][1][qq] = *reinterpret_cast<const uint4*>(Mh + mlane + (S + s) * kSlabBytes + qq * 16);
    }
  };
  const int row0 = wt * 64;                            // first token row of this wave

  // operating-point coefficients of tile ti (shared by all heads)
  auto coefficients = [&](int ti) {
    const float* tv = tokvec + (ti & 1) * kTokVec;
    const int64_t tbase = (int64_t)(tt0 + ti) * kTileTokens;
    const int nl = wn * 32 + (l & 31);                  // neuron within the tile
#pragma unroll
    for (int tb = 0; tb < kTB; ++tb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = row0 + tb * 32 + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
        float gv, uv;
        if constexpr (GULDS) {
          const int off = row * 256 + (((nl >> 3) ^ (row & 4)) << 4) + (nl & 7) * 2;
          gv = bf16_bits_to_f32(*reinterpret_cast<const uint16_t*>(gubuf + off));
          uv = bf16_bits_to_f32(*reinterpret_cast<const uint16_t*>(gubuf + kTileTokens * 256 + off));
        } else {
          const int last = (int)min((int64_t)kTileTokens, NT - tbase) - 1;
          const int rr = row < last ? row : last;
          const uint32_t off = (uint32_t)rr * (uint32_t)I + (uint32_t)kc;
          gv = load_elem(gp + tbase * I, off);
          uv = load_elem(up + tbase * I, off);
        }
        const float ri = tv[row];
        const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * gv);
        const float sg = __builtin_amdgcn_rcpf(1.0f + e);     // logistic sigma(g)
        const float silu = gv * sg;
        const float dsilu = fmaf(silu, 1.0f - sg, sg);         // sigma (1 + g (1 - sigma))
        coefA[tb][v] = dsilu * uv * ri;
        coefB[tb][v] = silu * ri;
        const float al = silu * uv * tv[kTileTokens + row];
        c_acc = fmaf(al, al, c_acc);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // one (token tile, head) step reading a-tile buffer `ab`
  auto step_body = [&](int step, const unsigned char* ab, unsigned char* ab_next) {
    const int ti = step / H, hi = step - ti * H;
    const int grp = p.head_group[hi];
    const int h = p.head_order[hi];
    const bool has_next = step + 1 < nsteps;
    // head of the next step (the last step refills with its own head: the
    // loads stay in bounds and are simply not used)
    const int hn = has_next ? p.head_order[(hi + 1) % H] : h;
    if (has_next) dma_a(step + 1, ab_next);
    const bool gu_now = GULDS && hi == 0 && ti + 1 < ntile;
    if (gu_now) dma_gu(ti + 1);
    if (hi == 0 && ti + 1 < ntile) stage_tokvec(ti + 1, (ti + 1) & 1);

#pragma unroll
    for (int tb = 0; tb < kTB; ++tb) {
      accG[tb] = f32x16{};
      accU[tb] = f32x16{};
    }
#pragma unroll
    for (int s = 0; s < S; ++s) {
#pragma unroll
      for (int tb = 0; tb < kTB; ++tb) {
        const int row = row0 + tb * 32 + (l & 31);
        uint4 af[Q];
#pragma unroll
        for (int qq = 0; qq < Q; ++qq) {
          const int col = s * CPS + (l >> 5) * Q + qq;
          af[qq] = *reinterpret_cast<const uint4*>(ab + row * ROWB + ((col ^ (row & (SLOTS - 1))) << 4));
        }
        mma(accG[tb], af, mreg[s % D][0]);
        mma(accU[tb], af, mreg[s % D][1]);
      }
      if (s + D < S) load_m(s % D, s + D, h);
      else load_m(s % D, s + D - S, hn);
      __builtin_amdgcn_sched_barrier(0);
    }

    // fused epilogue: eq. (5) and its square
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int tb = 0; tb < kTB; ++tb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float pg = accG[tb][v], pu = accU[tb][v];
        const float dl = fmaf(coefA[tb][v], pg, coefB[tb][v] * pu);
        fo_run[tb] = fmaf(dl, dl, fo_run[tb]);
      }
    }
    if (hi == H - 1 || p.head_group[hi + 1] != grp) {
      // lanes l and l + 32 hold the same neuron (other token rows)
      float fo = fo_run[0];
#pragma unroll
      for (int tb = 1; tb < kTB; ++tb) fo += fo_run[tb];
      fo += __shfl_xor(fo, 32);
      if (l < 32) accl[(grp * 2 + wt) * kTileNeurons + wn * 32 + l] += fo;
#pragma unroll
      for (int tb = 0; tb < kTB; ++tb) fo_run[tb] = 0.f;
    }
    // publish the next a tile (unless the next step opens a new token tile,
    // whose coefficient phase waits and synchronises instead)
    if (has_next && hi + 1 < H) {
      if (gu_now) __builtin_amdgcn_s_waitcnt(vm_wait(NM + DMA_GU));
      else __builtin_amdgcn_s_waitcnt(vm_wait(NM));
      __syncthreads();
    }
  };

  // ---- prologue ------------------------------------------------------------
  dma_a(0, abuf0);
  dma_gu(0);
  stage_tokvec(0, 0);
#pragma unroll
  for (int s = 0; s < D; ++s) load_m(s, s, p.head_order[0]);

  for (int step = 0; step < nsteps; ++step) {
    if (step % H == 0) {
      // new token tile: its a tile, g/u tile and token vectors must be in LDS
      __builtin_amdgcn_s_waitcnt(vm_wait(NM));
      __syncthreads();
      coefficients(step / H);
      __syncthreads();   // g/u tile fully read before it is refilled
    }
    if ((step & 1) == 0) step_body(step, abuf0, abuf1);
    else step_body(step, abuf1, abuf0);
  }

  // write this workgroup's partial sums (token halves added in fixed order)
  __builtin_amdgcn_s_waitcnt(vm_wait(0));   // drain the last (unused) M refills
  c_acc += __shfl_xor(c_acc, 32);
  if (l < 32) cbuf[wt * kTileNeurons + wn * 32 + l] = c_acc;
  __syncthreads();
  if (wt == 0 && l < 32 && nb < KB) {
    const int kk = nb * 32 + l, nl = wn * 32 + l;
    float* out = p.part + (int64_t)chunk * (G + 1) * p.I32;
    for (int gg = 0; gg < G; ++gg)
      out[(int64_t)gg * p.I32 + kk] =
          accl[(gg * 2 + 0) * kTileNeurons + nl] + accl[(gg * 2 + 1) * kTileNeurons + nl];
    out[(int64_t)G * p.I32 + kk] = cbuf[nl] + cbuf[kTileNeurons + nl];
  }
}

// Fixed-order reduction of the partial sums (float64 accumulation).
__global__ __launch_bounds__(256) void finalize_up_kernel(const float* __restrict__ part,
                                                          const float* __restrict__ add,
                                                          int n_chunks, int G, int I, int I32,
                                                          const float* __restrict__ wd_sq,
                                                          float scale, int accumulate,
                                                          float* S_fo, float* S_add,
                                                          float* c_down) {
  const int rows = 2 * G + (c_down ? 1 : 0);
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)rows * I) return;
  const int row = (int)(idx / I), k = (int)(idx - (int64_t)row * I);
  float* dst;
  double v;
  if (row < G || row == 2 * G) {
    const int prow = row < G ? row : G;
    double s = 0.0;
    for (int c = 0; c < n_chunks; ++c) s += part[((int64_t)c * (G + 1) + prow) * I32 + k];
    v = s * (double)scale;
    if (row < G) {
      v *= (double)wd_sq[k];
      dst = S_fo + (int64_t)row * I + k;
    } else {
      dst = c_down + k;
    }
  } else {
    v = n_chunks > 0 ? (double)add[(int64_t)(row - G) * I32 + k] * (double)scale : 0.0;
    dst = S_add + (int64_t)(row - G) * I + k;
  }
  *dst = accumulate ? *dst + (float)v : (float)v;
}

template <typename T, int S, bool GULDS>
hipError_t launch_typed(const UpParams& p, size_t lds, int grid, hipStream_t st) {
  auto fn = affinity_up_kernel<T, S, GULDS>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(kThreads), lds, st, p);
  return hipGetLastError();
}

template <typename T, bool GULDS>
hipError_t launch_by_steps(const UpParams& p, size_t lds, int grid, hipStream_t st) {
  switch (p.d / 16) {
    case 1: return launch_typed<T, 1, GULDS>(p, lds, grid, st);
    case 2: return launch_typed<T, 2, GULDS>(p, lds, grid, st);
    case 3: return launch_typed<T, 3, GULDS>(p, lds, grid, st);
    case 4: return launch_typed<T, 4, GULDS>(p, lds, grid, st);
    case 5: return launch_typed<T, 5, GULDS>(p, lds, grid, st);
    case 6: return launch_typed<T, 6, GULDS>(p, lds, grid, st);
    case 7: return launch_typed<T, 7, GULDS>(p, lds, grid, st);
    case 8: return launch_typed<T, 8, GULDS>(p, lds, grid, st);
    default: return hipErrorInvalidValue;
  }
}

size_t a256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

UpGeometry up_geometry(int64_t T, int H, int G, int d, int I, int dtype) {
  UpGeometry g{};
  const bool bf = dtype == 1;
  g.I32 = round_up(I, 32);
  g.n_tt = (int)((T + kTileTokens - 1) / kTileTokens);
  g.n_kt = (g.I32 + kTileNeurons - 1) / kTileNeurons;
  g.n_chunks = (g.n_tt + kTilesPerChunk - 1) / kTilesPerChunk;
  g.n_ktg = (g.n_kt + kSuperKt - 1) / kSuperKt;
  g.n_cg = (g.n_chunks + kSuperChunks - 1) / kSuperChunks;
  g.n_st = g.n_ktg * g.n_cg;
  g.grid = round_up(g.n_st, 8) * 32;
  g.gu_lds = bf && I % 8 == 0;
  // Gram kernel: enough (head, token chunk) workgroups to fill the chip
  if (T > 0) {
    const int64_t want = (512 + H - 1) / H;
    int64_t ct = (T + want - 1) / want;
    ct = (ct + kGramStage - 1) / kGramStage * kGramStage;
    if (ct < 4 * kGramStage) ct = 4 * kGramStage;
    g.gram_chunk = ct;
    g.n_gc = (int)((T + ct - 1) / ct);
  }
  g.part_bytes = a256((size_t)g.n_chunks * (G + 1) * g.I32 * sizeof(float));
  g.gram_part_bytes = a256((size_t)g.n_gc * H * d * d * sizeof(float));
  g.gram_bytes = a256((size_t)H * d * d * sizeof(float));
  g.add_bytes = a256((size_t)G * g.I32 * sizeof(float));
  g.off_gram_part = g.part_bytes;
  g.off_gram = g.off_gram_part + g.gram_part_bytes;
  g.off_add = g.off_gram + g.gram_bytes;
  g.ws_bytes = g.off_add + g.add_bytes;
  const int esize = bf ? 2 : 4;
  const int cpr = d * esize / 16;
  const size_t bufb = (size_t)kTileTokens * pow2_slots(cpr) * 16;
  const size_t gub = g.gu_lds ? 2 * kTileTokens * 256 : 16;
  g.dyn_lds_bytes = (size_t)G * 2 * kTileNeurons * sizeof(float);
  g.lds_bytes = 2 * bufb + gub + (2 * kTokVec + 2 * kTileNeurons) * sizeof(float) + g.dyn_lds_bytes;
  return g;
}

hipError_t launch_affinity_up(const UpParams& p, const UpGeometry& geo, int dtype,
                              hipStream_t st) {
  if (geo.grid == 0) return hipSuccess;
  if (dtype == 1) {
    return geo.gu_lds ? launch_by_steps<__bf16, true>(p, geo.dyn_lds_bytes, geo.grid, st)
                      : launch_by_steps<__bf16, false>(p, geo.dyn_lds_bytes, geo.grid, st);
  }
  return launch_by_steps<float, false>(p, geo.dyn_lds_bytes, geo.grid, st);
}

hipError_t launch_finalize_up(const float* part, const float* add, int n_chunks, int G, int I,
                              int I32, const float* wd_sq, float scale, int accumulate,
                              float* S_fo, float* S_add, float* c_down, hipStream_t st) {
  const int64_t n = (int64_t)(2 * G + (c_down ? 1 : 0)) * I;
  const int blocks = (int)((n + 255) / 256);
  hipLaunchKernelGGL(finalize_up_kernel, dim3(blocks), dim3(256), 0, st, part, add, n_chunks, G,
                     I, I32, wd_sq, scale, accumulate, S_fo, S_add, c_down);
  return hipGetLastError();
}

}  // namespace hna
