// The hot pass: first-order damage (eq. 5) and the FO up score of
// "Affinity-Aware Sharding for Delayed Tensor Parallelism", section 3,
// paragraph "Affinity scores", plus the token moment of the down edge.
// (The ADD score is linear in the per-head Gram matrices and is formed from
// them in k_gram.hip.)
//
// Work decomposition (gfx950, wave64, one wave per SIMD, 512 registers):
//   * a workgroup of 4 waves owns 128 neurons and a chunk of up to 8
//     consecutive token tiles of 128 tokens; wave w owns neurons 32w..32w+31
//     of the tile and all 128 tokens (4 blocks of 32 in the MFMA C layout);
//   * once per token tile each lane computes the operating-point
//     coefficients A = silu'(g) u / r and B = silu(g) / r of its 64 (t, k)
//     pairs (registers) and the down-edge moment (alpha / r_next)^2; on the
//     bf16 path they are kept as packed fp16 pairs, scaled by a power of two
//     s <= min r of the tile (so s / r <= 1 and they keep fp16's range for
//     any rms), and the tile's sums are divided by s^2 when they leave the
//     registers;
//   * per head h (in KV-group order) the wave runs the contraction a_h . M_h
//     on the matrix cores as two chain pairs (token blocks 0-1, then 2-3),
//     2 x 2 x d/16 MFMAs 32x32x16 each into gate and up accumulators, giving
//     r * (p_h.w^g_k, p_h.w^u_k); four independent accumulators are in flight;
//   * the epilogue of each chain pair, Delta = A Pg + B Pu and fo += Delta^2,
//     is spread over the MFMAs of the next pair (the second pair's over the
//     next head's first), so the VALU and the matrix cores overlap within the
//     wave; the folded-weight fragments of a head stay in registers for both
//     pairs and are refilled with the next head's during the second;
//   * at the end of a KV group the per-lane sums go to an LDS slot of that
//     group; nothing of size T x H x I leaves the chip: each workgroup writes
//     one [G+1, 128] block of fp32 partial sums, reduced later in fixed order.
// Data movement: the a tile of each (token tile, head) step arrives in LDS by
// asynchronous 16-byte buffer -> LDS DMA one step ahead (double buffered,
// XOR-swizzled rows: conflict-free fragment reads); the g/u tile of the next
// token tile is copied the same way a whole tile ahead; buffer range checks
// zero-fill past the tile edges.  Each wave reads the folded weights of its
// 32 neurons once per head (no duplicate reads within the workgroup).
// Workgroups are mapped to XCDs so that the 32 concurrent workgroups of one
// XCD cover 4 neuron tiles x 8 token chunks and share a and M in that XCD's L2.
#include "hna_internal.h"
#include "hna_hot.h"

#include <type_traits>

namespace hna {
namespace {

using namespace hot;

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

constexpr int kWaves = 4;              // one per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kTB = 4;                 // 32-token blocks per wave (the whole tile)
constexpr int kPairs = kTB * 16;       // (t, k) pairs per lane

template <int V> using IC = std::integral_constant<int, V>;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

template <typename E, int S, bool GULDS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void affinity_up_kernel(const UpParams p) {
  using Tr = Traits<E>;
  constexpr int EB = Tr::kBytes;
  constexpr int Q = Tr::kQuads;
  constexpr int CPS = Tr::kChunksPerStep;
  constexpr int CPR = S * CPS;              // 16-byte chunks per row of a_h
  constexpr int SLOTS = pow2_slots(CPR);
  constexpr int ROWB = SLOTS * 16;
  constexpr int BUFB = kTileTokens * ROWB;
  constexpr int DMA_A = kTileTokens * SLOTS / kThreads;           // per thread per step
  constexpr int DMA_GU = GULDS ? 2 * kTileTokens * 16 / kThreads : 0;
  constexpr int GU_BYTES = GULDS ? 2 * kTileTokens * 256 : 16;
  constexpr int NMS = 2 * S * Q;            // folded-weight loads per step
  constexpr int kSlabBytes = 64 * 8 * EB;   // one (h, kb, gu, s) fragment slab


  __shared__ __attribute__((aligned(16))) unsigned char abuf0[BUFB];
  __shared__ __attribute__((aligned(16))) unsigned char abuf1[BUFB];
  __shared__ __attribute__((aligned(16))) unsigned char gubuf[GU_BYTES];
  __shared__ __attribute__((aligned(16))) float tokinv[2 * kTileTokens];   // 1/r, 1/r_next
  __shared__ __attribute__((aligned(16))) float rraw[4 * kTileTokens];     // r, pad, r_next, pad
  extern __shared__ __attribute__((aligned(16))) float accl[];             // [G][128] FO sums
  __shared__ int8_t s_order[kMaxHeads], s_group[kMaxHeads];               // head tables
  __shared__ float s_rmin[2];                                              // per-wave min r of a tile

  // workgroup -> (neuron tile, token chunk); consecutive ids alternate XCDs
  const int id = blockIdx.x;
  const int xcd = id & 7, wi = id >> 3;
  const int st = xcd + 8 * (wi >> 5), mem = wi & 31;
  if (st >= p.n_st) return;
  const int kt = (st % p.n_ktg) * kSuperKt + (mem % kSuperKt);
  const int chunk = (st / p.n_ktg) * kSuperChunks + (mem / kSuperKt);
  if (kt >= p.n_kt || chunk >= p.n_chunks) return;

  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index (uniform)
  const int H = p.H, G = p.G, I = p.I, d = p.d;
  const int64_t NT = p.T;
  const int KB = p.I32 >> 5;
  const int nb = kt * 4 + w;                 // this wave's block of 32 neurons
  const int nbc = nb < KB ? nb : KB - 1;     // clamped so that M reads stay in bounds
  const int nl = w * 32 + (l & 31);          // this lane's neuron within the tile
  const int k = nb * 32 + (l & 31);
  const int kc = k < I ? k : I - 1;          // clamped neuron for direct g/u reads
  const E* gp = static_cast<const E*>(p.g);
  const E* up = static_cast<const E*>(p.u);

  for (int x = tid; x < G * kTileNeurons; x += kThreads) accl[x] = 0.f;
  if (tid < kMaxHeads) {
    s_order[tid] = p.head_order[tid];
    s_group[tid] = p.head_group[tid];
  }
  __syncthreads();

  const int tt0 = chunk * kTilesPerChunk;
  const int ntile = min(kTilesPerChunk, p.n_tt - tt0);
  const int nsteps = ntile * H;

  // ---- asynchronous copies ---------------------------------------------------
  // Per-wave LDS destinations: instruction i of wave w fills 64 slots of 16
  // bytes at byte offset (4 i + w) * 1024 of its buffer.
  const uint32_t lw = (uint32_t)w * 1024u;
  const uint32_t lds_a0 = lds_addr(abuf0) + lw, lds_a1 = lds_addr(abuf1) + lw;
  const uint32_t lds_gu = lds_addr(gubuf) + lw;
  const uint32_t lds_r = lds_addr(rraw);
  // a tile of one (token tile, head): slot q of the buffer holds row q / SLOTS,
  // chunk (q % SLOTS) ^ (row % SLOTS).  A wave copies 64 consecutive slots (64
  // / SLOTS whole rows) per instruction.  The per-lane offsets are the same
  // for every step; the resource selects the rows (rows past T, and every row
  // of the copy after the last step, read zeros).
  const uint32_t row_bytes_a = (uint32_t)(H * d * EB);
  auto voff_of = [&](int i) __attribute__((always_inline)) {
    const int slot0 = (i * kWaves + w) * 64;
    const int row = slot0 / SLOTS + l / SLOTS, sl = l % SLOTS;
    const int c = sl ^ (row & (SLOTS - 1));
    return c < CPR ? (uint32_t)row * row_bytes_a + (uint32_t)(c * 16) : kOutOfRange;
  };
  // kept in registers when there are few of them (bf16), else recomputed
  constexpr bool kKeepVoff = DMA_A <= 8;
  uint32_t voff_a[kKeepVoff ? DMA_A : 1];
  if constexpr (kKeepVoff) {
#pragma unroll
    for (int i = 0; i < DMA_A; ++i) voff_a[i] = voff_of(i);
  }
  const char* const abytes = static_cast<const char*>(p.a);
  // first byte and byte range of token tile ti's a rows (range 0 past the chunk)
  auto a_tile = [&](int ti, const char*& base, uint32_t& nrec) __attribute__((always_inline)) {
    const int64_t t0 = (int64_t)(tt0 + ti) * kTileTokens;
    base = abytes + t0 * row_bytes_a;
    nrec = ti < ntile ? (uint32_t)(min((int64_t)kTileTokens, NT - t0) - 1) * row_bytes_a + (uint32_t)(d * EB)
                      : 0u;
  };
  auto dma_a_part = [&](__amdgpu_buffer_rsrc_t rs, uint32_t lds, auto lo, auto hi) __attribute__((always_inline)) {
    static_for<decltype(lo)::value, decltype(hi)::value>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      if constexpr (kKeepVoff) dma16<i * kWaves * 1024>(rs, voff_a[i], lds);
      else dma16<i * kWaves * 1024>(rs, voff_of(i), lds);
    });
  };
  auto dma_a = [&](__amdgpu_buffer_rsrc_t rs, uint32_t lds) __attribute__((always_inline)) {
    static_for<0, DMA_A>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      if constexpr (kKeepVoff) dma16<i * kWaves * 1024>(rs, voff_a[i], lds);
      else dma16<i * kWaves * 1024>(rs, voff_of(i), lds);
    });
  };
  // g and u tiles of token tile ti (bf16, 128 tokens x 128 neurons each; a row
  // is 16 chunks of 8 neurons, chunk c of row r in slot c ^ (r & 4)).  A wave
  // copies 4 whole rows per instruction; rows past T read zeros.  Instruction
  // i covers rows 16 (i % 8) + 4 w + l / 16 of g (i < 8) or of u.
  const uint32_t row_bytes_gu = (uint32_t)I * 2u;
  uint32_t voff_gu = 0;
  if constexpr (GULDS) {
    const int row = 4 * w + (l >> 4);
    voff_gu = (uint32_t)row * row_bytes_gu + (uint32_t)(((l & 15) ^ (row & 4)) * 16);
  }
  auto dma_gu = [&](int ti) __attribute__((always_inline)) {
    if constexpr (GULDS) {
      const int64_t t0 = (int64_t)(tt0 + ti) * kTileTokens;
      const int rows = (int)min((int64_t)kTileTokens, NT - t0);
      const int n0 = kt * kTileNeurons;
      const uint32_t bytes = (uint32_t)rows * row_bytes_gu - (uint32_t)n0 * 2u;
      const auto rg = buffer_rsrc(gp + t0 * I + n0, bytes);
      const auto ru = buffer_rsrc(up + t0 * I + n0, bytes);
      static_for<0, DMA_GU>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        const uint32_t voff = voff_gu + (uint32_t)(16 * (i % 8)) * row_bytes_gu;
        dma16<i * kWaves * 1024>(i < DMA_GU / 2 ? rg : ru, voff, lds_gu);
      });
    }
  };
  // r and r_next of token tile ti (wave 0; 32 lanes x 16 bytes each, the
  // other 32 lanes read zeros into padding); tokens past T read zeros
  auto dma_tok = [&](int ti) __attribute__((always_inline)) {
    if (w == 0) {
      const int64_t t0 = (int64_t)(tt0 + ti) * kTileTokens;
      const uint32_t bytes = (uint32_t)min((int64_t)kTileTokens, NT - t0) * 4u;
      const uint32_t voff = l < 32 ? (uint32_t)l * 16u : kOutOfRange;
      dma16<0>(buffer_rsrc(p.r + t0, bytes), voff, lds_r);
      dma16<2 * kTileTokens * 4>(buffer_rsrc(p.r_next + t0, bytes), voff, lds_r);
    }
  };

  // ---- registers ---------------------------------------------------------------
  f32x16 accG[kTB], accU[kTB];
  // (A, B) of each pair: a packed fp16 pair on the bf16 path (one register,
  // rounded to nearest; the epilogue widens it inside v_fma_mix), fp32 on the
  // fp32 path
  using Coef = std::conditional_t<sizeof(E) == 2, half2_t, float2_t>;
  Coef cAB[kTB][16];
  float fo_run[kTB];
#pragma unroll
  for (int tb = 0; tb < kTB; ++tb) fo_run[tb] = 0.f;
  float c_acc = 0.f;
  // 1 / s^2 of the token tile whose sums fo_run holds (bf16 path: the tile's
  // coefficients carry the factor s)
  float inv_s2 = 1.f;
  const char* Mbytes = static_cast<const char*>(p.M);
  const uint32_t mlane = (uint32_t)l * 8u * EB;
  // The head's folded-weight fragments, all d-steps.  They are loaded with
  // untracked loads (gload16) and waited for with exact counts (wait_m), so
  // the a-tile copies issued between a refill and its use are not waited for.
  u32x4 mreg[S][2][Q];
  // this wave's neuron block of head 0, and the distance between heads
  const char* const Mw = Mbytes + (int64_t)nbc * 2 * S * kSlabBytes;
  const int64_t m_head = (int64_t)KB * 2 * S * kSlabBytes;
  // resource over the 2 S slabs of (head h, this wave's neuron block)
  auto m_rsrc = [&](int h) __attribute__((always_inline)) {
    return buffer_rsrc(Mw + (int64_t)h * m_head, 2 * S * kSlabBytes);
  };
  auto load_m = [&](auto sc, __amdgpu_buffer_rsrc_t rs) __attribute__((always_inline)) {
    constexpr int s = decltype(sc)::value;
    static_for<0, Q>([&](auto qc) __attribute__((always_inline)) {
      constexpr int qq = decltype(qc)::value;
      bload16_at<s * kSlabBytes + qq * 16>(mreg[s][0][qq], rs, mlane);
      bload16_at<(S + s) * kSlabBytes + qq * 16>(mreg[s][1][qq], rs, mlane);
    });
  };
  // Wait until d-step s's fragments have landed, given that `newer` untracked
  // loads were issued after them (the fragments pass through the wait, so no
  // use can be scheduled before it).
  auto wait_m = [&](int s, auto newer) __attribute__((always_inline)) {
    constexpr int N = decltype(newer)::value;
    if constexpr (Q == 1) vm_wait_tied<N>(mreg[s][0][0], mreg[s][1][0]);
    else vm_wait_tied<N>(mreg[s][0][0], mreg[s][0][1], mreg[s][1][0], mreg[s][1][1]);
  };

  // operating-point coefficients of token tile ti (shared by all heads)
  auto burst = [&](int ti) __attribute__((always_inline)) {
    // this tile's g/u copies completed before the step-start wait; the
    // barrier makes every wave's copies visible
    __syncthreads();
    {
      const int64_t t = (int64_t)(tt0 + ti) * kTileTokens + (tid & (kTileTokens - 1));
      const bool ok = t < NT && (tid < kTileTokens || p.want_c);
      const float rv = rraw[(tid < kTileTokens ? 0 : 2 * kTileTokens) + (tid & (kTileTokens - 1))];
      float sc = 1.f;
      if constexpr (sizeof(E) == 2) {
        // tile scale: the largest power of two s <= min r over the tile's
        // tokens (waves 0 and 1 hold the 128 r values), exponent clamped so
        // that 1 / s^2 stays a normal fp32 value
        if (tid < kTileTokens) {
          float m = ok ? rv : __builtin_inff();
#pragma unroll
          for (int o = 32; o >= 1; o >>= 1) m = fminf(m, __shfl_xor(m, o));
          if (l == 0) s_rmin[w] = m;
        }
        __syncthreads();
        const float rmin = fminf(s_rmin[0], s_rmin[1]);
        int e = rmin > 0.f && rmin < __builtin_inff() ? __builtin_amdgcn_frexp_expf(rmin) - 1 : 0;
        e = max(-60, min(60, e));
        if (tid < kTileTokens) sc = __builtin_ldexpf(1.f, e);
        inv_s2 = __builtin_ldexpf(1.f, -2 * e);
      }
      tokinv[tid] = ok ? __builtin_amdgcn_rcpf(rv) * sc : 0.f;
    }
    __syncthreads();
    int64_t tbase = (int64_t)(tt0 + ti) * kTileTokens;
    // opaque to the optimizer: the direct g/u addresses below are formed here,
    // once per tile, rather than hoisted out of the head loop (which would
    // keep all 64 of them live through every step)
    asm volatile("" : "+s"(tbase));
    const int last = (int)min((int64_t)kTileTokens, NT - tbase) - 1;
    // Every row this lane reads has (row & 4) == 4 (l >> 5), so the swizzled
    // g/u address is a per-lane base plus a compile-time row offset (nothing
    // per (row, lane) to keep live across the step loop).
    const int half = l >> 5;
    const unsigned char* gu_lane =
        gubuf + half * 4 * 256 + ((((nl >> 3) ^ (half * 4)) << 4) | ((nl & 7) * 2));
    const float* tok_lane = tokinv + 4 * half;
#pragma unroll
    for (int tb = 0; tb < kTB; ++tb) {
#pragma unroll
      for (int vq = 0; vq < 4; ++vq) {
        const int rowb = tb * 32 + 8 * vq;                 // + 4 (l >> 5)
        const float4 ri4 = *reinterpret_cast<const float4*>(tok_lane + rowb);
        const float4 rn4 = *reinterpret_cast<const float4*>(tok_lane + kTileTokens + rowb);
        const float ri[4] = {ri4.x, ri4.y, ri4.z, ri4.w};
        const float rn[4] = {rn4.x, rn4.y, rn4.z, rn4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = rowb + 4 * half + i, v = vq * 4 + i;
          float gv, uv;
          if constexpr (GULDS) {
            const int roff = (rowb + i) * 256;
            gv = bf16_bits_to_f32(*reinterpret_cast<const uint16_t*>(gu_lane + roff));
            uv = bf16_bits_to_f32(*reinterpret_cast<const uint16_t*>(gu_lane + kTileTokens * 256 + roff));
          } else {
            const int rr = row < last ? row : last;
            const int64_t off = (tbase + rr) * I + kc;
            if constexpr (sizeof(E) == 2) {
              gv = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(gp)[off]);
              uv = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(up)[off]);
            } else {
              gv = gp[off];
              uv = up[off];
            }
          }
          const float ex = __builtin_amdgcn_exp2f(-1.4426950408889634f * gv);
          const float sg = __builtin_amdgcn_rcpf(1.0f + ex);     // logistic sigma(g)
          const float silu = gv * sg;
          const float dsilu = fmaf(silu, 1.0f - sg, sg);         // sigma (1 + g (1 - sigma))
          using CT = std::conditional_t<sizeof(E) == 2, _Float16, float>;
          cAB[tb][v] = Coef{(CT)(dsilu * uv * ri[i]), (CT)(silu * ri[i])};
          const float al = silu * uv * rn[i];
          c_acc = fmaf(al, al, c_acc);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();                            // g/u tile and 1/r read by every wave
    if (ti + 1 < ntile) {
      dma_tok(ti + 1);
      dma_gu(ti + 1);
    }
  };

  // epilogue of pair v of token block tb
  auto epi_pair = [&](int tb, int v) __attribute__((always_inline)) {
    const float pg = accG[tb][v], pu = accU[tb][v];
    const Coef c = cAB[tb][v];
    const float dl = fmaf((float)c.x, pg, fmaf((float)c.y, pu, 0.0f));
    fo_run[tb] = fmaf(dl, dl, fo_run[tb]);
  };
  // KV group grp ends: fold the lane sums into its LDS slot (lanes l and l+32
  // hold the same neuron)
  auto flush = [&](int grp) __attribute__((always_inline)) {
    float fo = (fo_run[0] + fo_run[1]) + (fo_run[2] + fo_run[3]);
    fo += __shfl_xor(fo, 32);
    if (l < 32) accl[grp * kTileNeurons + nl] += fo * inv_s2;
#pragma unroll
    for (int tb = 0; tb < kTB; ++tb) fo_run[tb] = 0.f;
  };

  // ---- one (token tile, head) step ------------------------------------------------
  // s = ti * H + hi; a_cur / r_cur and a_nxt / r_nxt: the a rows of token
  // tiles ti and ti + 1 (see a_tile)
  auto step = [&](int s, int ti, int hi, const char* a_cur, uint32_t r_cur, const char* a_nxt,
                  uint32_t r_nxt) __attribute__((always_inline)) {
    const bool last_h = hi + 1 == H;
    const int hn = __builtin_amdgcn_readfirstlane(s_order[last_h ? 0 : hi + 1]);   // next head
    // Vector-memory loads complete in issue order.  The last NMS loads this
    // wave issued are this head's folded-weight fragments (refilled during
    // the previous step's last chain); everything before them has landed
    // once at most NMS are outstanding: the a tile of this step (copied one
    // step earlier) and the g/u, r and r_next copies of the next tile.  The
    // compiler waits for each weight fragment itself just before its first
    // MFMA, so the refills issued last keep most of a chain of lead time.
    // The copy of the next a tile is issued after this wait and overlaps the
    // whole step.
    __builtin_amdgcn_s_waitcnt(vm_wait(NMS));
    __syncthreads();
    const bool odd = (s & 1) != 0;
    const unsigned char* ab = odd ? abuf1 : abuf0;
    // the next step's a tile (after the last step the range is empty: the
    // copy reads nothing and fills the idle buffer with zeros, so every step
    // issues the same number of loads)
    const auto rs_next =
        buffer_rsrc((last_h ? a_nxt : a_cur) + (int64_t)hn * d * EB, last_h ? r_nxt : r_cur);
    const uint32_t lds_next = odd ? lds_a0 : lds_a1;
    const auto rs_m = m_rsrc(hn);   // the next head's weights (refilled during pair 1)

    // Two token blocks' chains run together (four independent accumulators,
    // enough to keep the matrix pipeline full); the a fragments go through a
    // 3-slot register ring, read two contraction steps ahead so that LDS
    // latency hides behind the MFMAs.
    constexpr int NQ = 2 * S;   // (chain pair, d-step)
    uint4 afr[3][2][Q];
    auto read_af = [&](int q, uint4 (&dst)[2][Q]) __attribute__((always_inline)) {
      const int ks = q % S;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = (2 * (q / S) + j) * 32 + (l & 31);
#pragma unroll
        for (int qq = 0; qq < Q; ++qq) {
          const int col = ks * CPS + (l >> 5) * Q + qq;
          dst[j][qq] =
              *reinterpret_cast<const uint4*>(ab + row * ROWB + ((col ^ (row & (SLOTS - 1))) << 4));
        }
      }
    };
    read_af(0, afr[0]);
    if (NQ > 1) read_af(1, afr[1]);
    auto body = [&](auto qc) __attribute__((always_inline)) {
      constexpr int q = decltype(qc)::value;
      constexpr int pr = q / S, ks = q % S;
      // the chain pair before this one: pair 0 of this head, or the previous
      // head's pair 1 (token blocks 2 and 3)
      constexpr int ppr = pr == 0 ? 1 : 0;
      if (q + 2 < NQ) read_af(q + 2, afr[(q + 2) % 3]);
      if (ks == 0) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          accG[2 * pr + j] = f32x16{};
          accU[2 * pr + j] = f32x16{};
        }
      }
      // a slice of the previous pair's epilogue (other accumulators; before the
      // first head they and the coefficients are zero, adding nothing).  The
      // slice's pairs go through each stage together, so no result is read
      // by the very next instruction.
      {
        constexpr int x0 = ks * 32 / S, x1 = (ks + 1) * 32 / S, nx = x1 - x0;
        float t[nx > 0 ? nx : 1];
#pragma unroll
        for (int x = x0; x < x1; ++x)
          t[x - x0] = fmaf((float)cAB[2 * ppr + (x >> 4)][x & 15].y, accU[2 * ppr + (x >> 4)][x & 15], 0.0f);
#pragma unroll
        for (int x = x0; x < x1; ++x)
          t[x - x0] = fmaf((float)cAB[2 * ppr + (x >> 4)][x & 15].x, accG[2 * ppr + (x >> 4)][x & 15], t[x - x0]);
#pragma unroll
        for (int x = x0; x < x1; ++x)
          fo_run[2 * ppr + (x >> 4)] = fmaf(t[x - x0], t[x - x0], fo_run[2 * ppr + (x >> 4)]);
      }
      // first use of d-step ks's fragments: issued after them are the later
      // d-steps' refills and this step's copy of the next a tile
      // the copies of the next a tile are spread over pair 0, after each
      // d-step's MFMAs (DMA_A / S per d-step, the rest with the last one)
      constexpr int dma_lo = ks * (DMA_A / S), dma_hi = ks + 1 == S ? DMA_A : (ks + 1) * (DMA_A / S);
      if constexpr (pr == 0) wait_m(ks, IC<2 * Q * (S - 1 - ks) + dma_lo>{});
      uint4 mg[Q], mu[Q];
#pragma unroll
      for (int qq = 0; qq < Q; ++qq) {
        mg[qq] = __builtin_bit_cast(uint4, mreg[ks][0][qq]);
        mu[qq] = __builtin_bit_cast(uint4, mreg[ks][1][qq]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        mma(accG[2 * pr + j], afr[q % 3][j], mg);
        mma(accU[2 * pr + j], afr[q % 3][j], mu);
      }
      if constexpr (pr == 0) dma_a_part(rs_next, lds_next, IC<dma_lo>{}, IC<dma_hi>{});
      // after the last pair's use, refill with the next head's fragments
      // (after the last step too, into registers that are drained after the
      // loop: every step issues the same loads)
      if constexpr (pr == 1) load_m(IC<ks>{}, rs_m);
      __builtin_amdgcn_sched_barrier(0);
    };
    // pair 0 (token blocks 0, 1), which also finishes the previous head
    static_for<0, S>(body);
    if (s > 0) {
      // the previous head is complete: flush if it ends its KV group
      const int hp = hi == 0 ? H - 1 : hi - 1;
      const int grp = s_group[hp];
      if (hp == H - 1 || s_group[hp + 1] != grp) flush(grp);
    }
    if (hi == 0) burst(ti);   // coefficients of this tile, used from pair 1 on
    // pair 1 (token blocks 2, 3)
    static_for<S, NQ>(body);
  };

  // ---- prologue and step loop ----------------------------------------------------
  // The first step's pair 0 runs the epilogue of a "previous" pair that does
  // not exist: zero accumulators and coefficients make it add nothing.
#pragma unroll
  for (int tb = 0; tb < kTB; ++tb) {
    accG[tb] = f32x16{};
    accU[tb] = f32x16{};
#pragma unroll
    for (int v = 0; v < 16; ++v) cAB[tb][v] = Coef{0, 0};
  }
  const char* a_cur;
  uint32_t r_cur;
  a_tile(0, a_cur, r_cur);
  const int h0 = __builtin_amdgcn_readfirstlane(s_order[0]);
  dma_gu(0);
  dma_tok(0);
  dma_a(buffer_rsrc(a_cur + (int64_t)h0 * d * EB, r_cur), lds_a0);
  {
    const auto rs0 = m_rsrc(h0);
    static_for<0, S>([&](auto kc) __attribute__((always_inline)) { load_m(kc, rs0); });
  }

  for (int ti = 0, s = 0; ti < ntile; ++ti) {
    const char* a_nxt;
    uint32_t r_nxt;
    a_tile(ti + 1, a_nxt, r_nxt);
    for (int hi = 0; hi < H; ++hi, ++s) step(s, ti, hi, a_cur, r_cur, a_nxt, r_nxt);
    a_cur = a_nxt;
    r_cur = r_nxt;
  }

  // the refills issued by the last step land before their registers can be
  // reused (they pass through the wait)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int ks = 0; ks < S; ++ks)
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int qq = 0; qq < Q; ++qq) tie(mreg[ks][g][qq]);

  // epilogue of the last pair (its head ends the last KV group)
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    epi_pair(kTB - 2, v);
    epi_pair(kTB - 1, v);
  }
  flush(s_group[H - 1]);

  // ---- write this workgroup's partial sums ----------------------------------------
  c_acc += __shfl_xor(c_acc, 32);
  if (l < 32 && nb < KB) {
    float* out = p.part + (int64_t)chunk * (G + 1) * p.I32 + nb * 32 + l;
    for (int gg = 0; gg < G; ++gg) out[(int64_t)gg * p.I32] = accl[gg * kTileNeurons + nl];
    out[(int64_t)G * p.I32] = c_acc;
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
    // chunks in order; eight loads in flight before they are added
    const float* src = part + (int64_t)prow * I32 + k;
    const int64_t stride = (int64_t)(G + 1) * I32;
    double s = 0.0;
    int c = 0;
    for (; c + 8 <= n_chunks; c += 8) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = src[(c + j) * stride];
#pragma unroll
      for (int j = 0; j < 8; ++j) s += (double)v[j];
    }
    for (; c < n_chunks; ++c) s += (double)src[c * stride];
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
  g.add_part_bytes = a256((size_t)H * g.I32 * sizeof(float));
  g.off_add = g.off_gram + g.gram_bytes;
  g.off_add_part = g.off_add + g.add_bytes;
  g.ws_bytes = g.off_add_part + g.add_part_bytes;
  const int esize = bf ? 2 : 4;
  const int cpr = d * esize / 16;
  const size_t bufb = (size_t)kTileTokens * pow2_slots(cpr) * 16;
  const size_t gub = g.gu_lds ? 2 * kTileTokens * 256 : 16;
  g.dyn_lds_bytes = (size_t)G * kTileNeurons * sizeof(float);
  // a double buffer, g/u tile, 1/r and 1/r_next, raw r and r_next, head tables
  g.lds_bytes = 2 * bufb + gub + 6 * kTileTokens * sizeof(float) + 2 * kMaxHeads + g.dyn_lds_bytes;
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
