// bf16 "NT" GEMM on the matrix cores for the weight products of the affinity
// pass and of the leave-one-out score: C[m, n] = sum_k X[m, k] Y[n, k], X and Y
// row-major with k contiguous, fp32 accumulation.  Four epilogues:
//   * fold (section 3, "Affinity scores": M_h = W_o^(h)T diag(gamma) W^T): C is
//     written in the fragment order of the folded weights;
//   * segment square (the down edge's ||b_gk||^2): C^2 summed over the rows n
//     of one W_q / W_k / W_v segment, b never stored;
//   * plain store of C transposed (C[m, n] at n * ldc + m, m contiguous),
//     fp32 or bf16, per batch entry or per K chunk;
//   * dot (the leave-one-out score's x . o_h = (x W_o^(h)) . a_h): each 64-row
//     block of C's column n dotted with a token operand's row n, C never
//     stored.
// Workgroup tile BM x BN x BK on WGM x WGN waves, each wave (BM/WGM) x
// (BN/WGN) as 32x32 MFMA tiles (every LDS fragment read feeds several MFMAs).
// The fold (256 x 256, or 256 x 192 or 192 x 256 where that fills the CUs
// better) and the large stores run 8-wave tiles in ping-pong:
// the two waves of a SIMD alternate between an MFMA phase and a memory phase
// (LDS fragment reads, copies), barrier to barrier; so do the segment
// squares of 128-, 96- or 64-wide segments, two to a tile (one per wave
// column).  Other segment squares and the small stores run 128 x 128 tiles on
// 4 waves, two workgroups per CU.
// Both operand tiles arrive in LDS by asynchronous 16-byte buffer -> LDS
// copies into a ring of NST stages: the copies of K step k + NST - 1 are
// issued before the MFMAs of step k (BK = 64 with two stages measured faster
// than BK = 32 with three or four).  LDS rows of 64 elements (128 bytes) hold
// their 16-byte chunks XOR-swizzled by the row index, so the 16 rows that a
// fragment read serves at once hit 16 distinct bank slots (the bank-conflict
// counter reads 0).  Rows past M or N and elements past K read zeros (buffer
// range check, chunk masking); K must be a multiple of 8.
// Workgroup ids map tiles XCD by XCD, in groups of 4 tile rows, so the
// workgroups that share an XCD's L2 at one time share operand panels.
#include "hna_internal.h"
#include "hna_hot.h"

namespace hna {
namespace {

using namespace hot;

constexpr uint32_t kMaxResourceBytes = 0x7ffff000u;   // below the out-of-range offset


// Asynchronous 16-byte buffer -> LDS copy with a scalar offset soff added to
// the address (voff is what the range check covers); lane l writes LDS
// m0 + 16 l.  The resource is passed as its four descriptor words.
__device__ inline void dma16s(u32x4 rs, uint32_t voff, uint32_t soff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :: "s"(m0), "v"(voff), "s"(rs), "s"(soff) : "memory");
}

// Raw buffer descriptor words (32-bit data format, no swizzle, stride 0) over
// [base, base + bytes), built from values the compiler may not see as uniform
// (they are): each word goes through readfirstlane, so the descriptor lives
// in scalar registers.
__device__ inline u32x4 uniform_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4 d;
  d.x = __builtin_amdgcn_readfirstlane((uint32_t)a);
  d.y = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) & 0xffffu;
  d.z = __builtin_amdgcn_readfirstlane(bytes);
  d.w = 0x00020000u;
  return d;
}

// XOR applied to the 16-byte chunk index in row r of a stage whose rows hold
// CPR chunks: any 8 consecutive rows put one chunk column in 8 distinct
// 16-byte slots of the 128-byte lines they span

template <int CPR>
__device__ inline int swz(int r) {
  // 128-byte rows: a 64-bank LDS serves 16 lanes (16 rows) of a 16-byte read
  // at once, so every 16 rows must also cover 16 distinct slots of the
  // 256-byte lines they span
  if constexpr (CPR == 8) return (r & 7) ^ ((r >> 3) & 1);
  return (r / (8 / CPR)) % CPR;
}

template <int BM, int BN, int BK, int WGM, int WGN, int NST, int EPI, bool PP>
__global__ __launch_bounds__(64 * WGM * WGN) void mm_bf16_kernel(const GemmParams p) {
  static_assert(BK == 32 || BK == 64, "K step of 32 or 64");
  static_assert(!PP || (WGM * WGN == 8 && NST == 2), "ping-pong: 8 waves, two stages");
  static_assert(NST >= 2 && NST <= 4, "two to four stages");
  constexpr int NW = WGM * WGN;               // waves, WGM x WGN
  constexpr int WM = BM / WGM, WN = BN / WGN; // wave tile
  constexpr int TM = WM / 32, TN = WN / 32;   // 32x32 tiles per wave
  constexpr int ROWS = BM + BN;
  constexpr int ROWB = 2 * BK;                // bytes per LDS row
  constexpr int CPR = BK / 8;                 // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;               // rows one wave's copy fills
  constexpr int STAGE = ROWS * ROWB;          // bytes per stage
  constexpr int NCP = ROWS / (RPI * NW);      // copies per thread per stage
  constexpr int NCX = BM / (RPI * NW);        // of which X rows
  static_assert(BM % (RPI * NW) == 0 && BN % (RPI * NW) == 0, "copy rounds cover whole rows");
  // segment squares: one segment per tile (BN = 128 >= d'), or, on the
  // ping-pong kernel, one per wave column (WGN per tile; the host launches it
  // only when the segment width d' is WN)
  constexpr int SEGS = (EPI == kEpiSegSq && PP) ? WGN : 1;
  static_assert(EPI != kEpiSegSq || (!PP && BN == 128 && BM <= 64 * NW) || PP,
                "a segment is a tile column or a wave column");

  static_assert((NST - 2) * NCP <= 63, "copies in flight must fit the wait counter");
  __shared__ __attribute__((aligned(16))) unsigned char lds[NST * STAGE];
  __shared__ float red[WGN][BM];

  const int tid = threadIdx.x, l = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w / WGN, wn = w % WGN;

  // ---- tile of this workgroup ----
  const int N = EPI == kEpiSegSq ? SEGS * p.d_next : p.N;
  const int ntm = (p.Mrows + BM - 1) / BM, ntn = (N + BN - 1) / BN;
  const int ntiles = ntm * ntn;
  const int per_xcd = (ntiles + 7) / 8;
  const int t = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (t >= ntiles) return;
  // tiles in groups of GM tile rows, column by column within a group: the
  // workgroups an XCD runs at once cover a few rows and columns of tiles
  constexpr int GM = 4;
  const int gsize = GM * ntn;
  const int g0 = (t / gsize) * GM, gm = min(GM, ntm - g0), tg = t - (g0 / GM) * gsize;
  const int tm = g0 + tg % gm, tn = tg / gm;
  const int m0 = tm * BM, n0 = tn * BN;
  const int z = blockIdx.y;

  // Y: the gate (z = 0) or up (z = 1) matrix (fold); for the segment square
  // segment z of W_q (z < H'), W_k, then W_v (d' rows each); batch or K chunk
  // z (store)
  const __bf16* X = static_cast<const __bf16*>(p.X);
  const __bf16* Y;
  int Nrows;
  int kbeg = 0, kend = p.K;
  if constexpr (EPI == kEpiFold) {
    Y = static_cast<const __bf16*>(z ? p.Y[1] : p.Y[0]);
    Nrows = p.Nvalid;
  } else if constexpr (EPI == kEpiSegSq) {
    // segments SEGS z .. SEGS z + SEGS - 1 (of one matrix: the host keeps
    // H', G' multiples of SEGS)
    const int sz = SEGS * z;
    const int c = sz < p.H_next ? 0 : (sz < p.H_next + p.G_next ? 1 : 2);
    const int zs = sz - (c == 0 ? 0 : (c == 1 ? p.H_next : p.H_next + p.G_next));
    Y = static_cast<const __bf16*>(c == 0 ? p.Y[0] : (c == 1 ? p.Y[1] : p.Y[2])) +
        (int64_t)zs * p.d_next * p.ldy;
    Nrows = SEGS * p.d_next;
  } else {
    Y = static_cast<const __bf16*>(p.Y[0]);
    Nrows = p.N;
    if (p.k_split > 0) {
      kbeg = z * p.k_split;
      kend = min(p.K, kbeg + p.k_split);
    } else {
      X += (int64_t)z * p.bx;
      Y += (int64_t)z * p.by;
    }
  }
  // resources over the rows from m0 / n0 on (rows past the end read zeros)
  const uint32_t lim = kMaxResourceBytes;
  const int64_t xb = (int64_t)max(0, p.Mrows - m0) * p.ldx * 2;
  const int64_t yb = (int64_t)max(0, Nrows - n0) * p.ldy * 2;
  const uint32_t xbytes = xb > (int64_t)lim ? lim : (uint32_t)xb;
  const uint32_t ybytes = yb > (int64_t)lim ? lim : (uint32_t)yb;
  const u32x4 rx = uniform_rsrc(X + (int64_t)m0 * p.ldx, xbytes);
  const u32x4 ry = uniform_rsrc(Y + (int64_t)n0 * p.ldy, ybytes);

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};
  const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
  constexpr int NKS = BK / 16;
  // fragment reads of K sub-step ks of the stage at sb
  auto rd = [&](const unsigned char* sb, int ks, uint4 (&fa)[TM][1], uint4 (&fb)[TN][1])
      __attribute__((always_inline)) {
    const int col = 2 * ks + (l >> 5);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int r = wm * WM + i * 32 + (l & 31);
      fa[i][0] = *reinterpret_cast<const uint4*>(sb + r * ROWB + ((col ^ swz<CPR>(r)) << 4));
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int r = BM + wn * WN + j * 32 + (l & 31);
      fb[j][0] = *reinterpret_cast<const uint4*>(sb + r * ROWB + ((col ^ swz<CPR>(r)) << 4));
    }
  };

  if constexpr (PP) {
    // ---- ping-pong: waves 0-3 (group A, one per SIMD) and 4-7 (group B)
    // alternate between a memory phase (LDS fragment reads of a whole K step
    // into registers; group A also issues every copy of the next stage) and
    // an MFMA phase, separated by workgroup barriers: while one wave of a
    // SIMD runs its MFMAs the other reads.  Group B starts one phase late.
    // Barrier sequence, phase by phase (A | B):
    //   copy stage 0, wait | -            barrier 1
    //   mem(0)             | -            barrier 2
    //   mfma(0), wait      | mem(0)       barrier 3
    //   mem(1)             | mfma(0)      barrier 4 ...
    //   mfma(k), wait      | mem(k)       barrier 2k + 3
    //   -                  | mfma(nk - 1) barrier 2 nk + 2
    // so both groups pass 2 nk + 2 barriers.  Group A's copies of stage k + 1
    // (issued in mem(k)) overwrite the buffer of stage k - 1, whose last reads
    // (B's mem(k - 1)) ended at barrier 2k + 1; A waits for them at the end
    // of mfma(k), so they are visible from barrier 2k + 3 on, before either
    // group reads them.  Each memory phase waits for its own LDS reads before
    // its barrier.
    constexpr int NWC = 4;                          // copying waves
    constexpr int NCPA = ROWS / (RPI * NWC);        // copies per group-A thread
    constexpr int NCXA = BM / (RPI * NWC);
    static_assert(BM % (RPI * NWC) == 0 && BN % (RPI * NWC) == 0, "copy rounds cover whole rows");
    const bool grp_a = w < NWC;
    const int wa = w & (NWC - 1);
    // copy i of A-wave wa fills rows RPI (4 i + wa) .. + RPI - 1; the lane's
    // chunk is the same for every i (rows 32 apart share their swizzle)
    const int r0 = RPI * wa + l / CPR;
    const int c0 = (l % CPR) ^ swz<CPR>(r0);
    const int kc0 = 8 * c0;
    const uint32_t vx0 = (uint32_t)((int64_t)r0 * p.ldx * 2 + 16 * c0);
    const uint32_t vy0 = (uint32_t)((int64_t)r0 * p.ldy * 2 + 16 * c0);
    const uint32_t sx = __builtin_amdgcn_readfirstlane((uint32_t)(RPI * NWC * p.ldx * 2));
    const uint32_t sy = __builtin_amdgcn_readfirstlane((uint32_t)(RPI * NWC * p.ldy * 2));
    const uint32_t lds0 = lds_addr(lds) + (uint32_t)wa * 1024u;
    auto issue = [&](int k0, int buf) __attribute__((always_inline)) {
      const uint32_t base = lds0 + (uint32_t)(buf * STAGE);
      const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)(k0 * 2));
      const bool drop = k0 + BK > kend && k0 + kc0 >= kend;
#pragma unroll
      for (int i = 0; i < NCPA; ++i) {
        const uint32_t v = drop ? kOutOfRange
                                : (i < NCXA ? vx0 + (uint32_t)i * sx : vy0 + (uint32_t)(i - NCXA) * sy);
        dma16s(i < NCXA ? rx : ry, v, soff, base + (uint32_t)(i * NWC * 1024));
      }
    };
    auto barrier = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };
    if (grp_a) {
      if (nk > 0) issue(kbeg, 0);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    barrier();                       // 1
    if (!grp_a) barrier();           // 2 (group B's idle phase)
    for (int kt = 0; kt < nk; ++kt) {
      const unsigned char* sb = lds + (kt & 1) * STAGE;
      // memory phase
      if (grp_a && kt + 1 < nk) issue(kbeg + (kt + 1) * BK, (kt + 1) & 1);
      uint4 af[NKS][TM][1], bfr[NKS][TN][1];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) rd(sb, ks, af[ks], bfr[ks]);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      barrier();
      // MFMA phase
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) mma(acc[i][j], af[ks][i], bfr[ks][j]);
      if (grp_a) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      barrier();
    }
    if (grp_a) barrier();            // group A's last barrier (B's last mfma)
  } else {
    // ---- copies: copy i of wave w fills rows 8 (4 i + w) .. + 7 of the stage
    // (X rows first, then Y rows); lane l: row + l / 8, slot l % 8 holding
    // chunk (l % 8) ^ (row & 7) ----
    uint32_t voff[NCP];
    int kc[NCP];   // element offset of the lane's chunk within the stage
  #pragma unroll
    for (int i = 0; i < NCP; ++i) {
      const int r = RPI * (NW * i + w) + l / CPR;
      const int c = (l % CPR) ^ swz<CPR>(r);
      kc[i] = 8 * c;
      voff[i] = i < NCX ? (uint32_t)((int64_t)r * p.ldx * 2 + 16 * c)
                        : (uint32_t)((int64_t)(r - BM) * p.ldy * 2 + 16 * c);
    }
    const uint32_t lds0 = lds_addr(lds) + (uint32_t)w * 1024u;
    auto issue = [&](int k0, int buf) __attribute__((always_inline)) {
      const uint32_t base = lds0 + (uint32_t)(buf * STAGE);
      const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)(k0 * 2));
      const bool tail = k0 + BK > kend;
  #pragma unroll
      for (int i = 0; i < NCP; ++i) {
        const uint32_t v = tail && k0 + kc[i] >= kend ? kOutOfRange : voff[i];
        dma16s(i < NCX ? rx : ry, v, soff, base + (uint32_t)(i * NW * 1024));
      }
    };

  #pragma unroll
    for (int st = 0; st < NST - 1; ++st)
      if (st < nk) issue(kbeg + st * BK, st);
    for (int kt = 0; kt < nk; ++kt) {
      // step kt has landed once at most the copies of the steps after it that
      // are in flight remain (copies complete in issue order); the barrier
      // makes it visible to every wave and ends every wave's reads of step
      // kt - 1, whose stage the next copies overwrite
      const int ahead = min(NST - 2, nk - 1 - kt);
      if (NST >= 4 && ahead >= 2) __builtin_amdgcn_s_waitcnt(vm_wait(2 * NCP));
      else if (NST >= 3 && ahead >= 1) __builtin_amdgcn_s_waitcnt(vm_wait(NCP));
      else __builtin_amdgcn_s_waitcnt(vm_wait(0));
      __syncthreads();
      if (kt + NST - 1 < nk) issue(kbeg + (kt + NST - 1) * BK, (kt + NST - 1) % NST);
      const unsigned char* sb = lds + (kt % NST) * STAGE;
  #pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        uint4 af[TM][1], bfr[TN][1];
        rd(sb, ks, af, bfr);
  #pragma unroll
        for (int i = 0; i < TM; ++i)
  #pragma unroll
          for (int j = 0; j < TN; ++j) mma(acc[i][j], af[i], bfr[j]);
      }
    }
  }

  // ---- epilogues: lane l holds column (l & 31) and rows
  // 8 (v / 4) + 4 (l / 32) + (v % 4) of each 32x32 tile ----
  if constexpr (EPI == kEpiFold) {
    // lanes l and l ^ 32 swap halves so that each lane owns two whole groups
    // of 8 rows (8 consecutive j of one neuron: one 16-byte piece of the
    // folded layout)
    const int upl = l >> 5;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        uint32_t mine[4][2];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          mine[a][0] = f32_to_bf16_bits(acc[i][j][4 * a]) | (f32_to_bf16_bits(acc[i][j][4 * a + 1]) << 16);
          mine[a][1] = f32_to_bf16_bits(acc[i][j][4 * a + 2]) | (f32_to_bf16_bits(acc[i][j][4 * a + 3]) << 16);
        }
        const int n = n0 + wn * WN + j * 32 + (l & 31);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int ka = 2 * b + upl;
          uint32_t lo_w[2], hi_w[2];
#pragma unroll
          for (int v = 0; v < 2; ++v) {
            const uint32_t send = upl ? mine[2 * b][v] : mine[2 * b + 1][v];
            const uint32_t recv = (uint32_t)__shfl_xor((int)send, 32);
            const uint32_t keep = upl ? mine[2 * b + 1][v] : mine[2 * b][v];
            lo_w[v] = upl ? recv : keep;
            hi_w[v] = upl ? keep : recv;
          }
          const int m = m0 + wm * WM + i * 32 + 8 * ka;
          if (m < p.Mrows && n < p.N) {
            const int h = m / p.d, jj = m - h * p.d;
            const int64_t o = folded_index(h, jj, n, z, p.KB, p.S);
            *reinterpret_cast<uint4*>(static_cast<__bf16*>(p.M) + o) =
                make_uint4(lo_w[0], lo_w[1], hi_w[0], hi_w[1]);
          }
        }
      }
  } else if constexpr (EPI == kEpiSegSq) {
    // sum of squares over this segment's rows n (the tile's columns)
    float sq[TM][16];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float s2 = 0.f;
#pragma unroll
        for (int j = 0; j < TN; ++j) s2 = fmaf(acc[i][j][v], acc[i][j][v], s2);
        sq[i][v] = s2;
      }
#pragma unroll
    for (int off = 1; off < 32; off <<= 1)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) sq[i][v] += __shfl_xor(sq[i][v], off);
    if ((l & 31) == 0) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          red[wn][wm * WM + i * 32 + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3)] = sq[i][v];
    }
    __syncthreads();
    if (tid < BM && m0 + tid < p.Mrows) {
      if constexpr (SEGS == 1) {
        float t = 0.f;
#pragma unroll
        for (int q = 0; q < WGN; ++q) t += red[q][tid];
        p.seg_part[(int64_t)z * p.Mrows + m0 + tid] = t;
      } else {
        static_assert(SEGS == WGN, "one segment per wave column");
#pragma unroll
        for (int q = 0; q < WGN; ++q) p.seg_part[(int64_t)(SEGS * z + q) * p.Mrows + m0 + tid] = red[q][tid];
      }
    }
  } else if constexpr (EPI == kEpiDot) {
    // x . o_h without storing Z: C[m][n] = Z[n][m] (m = h d + j) dotted with
    // A_tok[n][m] over each wave's 64 rows, one partial per (64-row block,
    // head, token).  The tile's A_tok block (256 tokens x 256 columns, bf16)
    // is copied into the idle operand stages: row t holds 32 chunks of 16
    // bytes, chunk c in slot c ^ (t % 32), so that the 32 tokens one read
    // serves land in distinct slots.
    static_assert(PP && BM == 256 && BN == 256 && WM == 64 && WN == 128, "the 256 x 256 ping-pong tile");
    static_assert(NST * STAGE >= 256 * 512, "the operand block fits the stages");
    __syncthreads();
    const int64_t lda2 = p.dot_lda * 2;                 // bytes per token row of A_tok
    const int64_t rows_left = (int64_t)p.N - n0;
    const int cols = min(256, p.Mrows - m0);           // columns of A_tok this tile covers
    // the range ends at the last needed byte: rows past N and columns past
    // Mrows read zeros
    const int64_t ab = rows_left > 0 ? (rows_left - 1) * lda2 + (int64_t)cols * 2 : 0;
    const u32x4 ra = uniform_rsrc(static_cast<const char*>(p.dot_a) + (int64_t)n0 * lda2 + (int64_t)m0 * 2,
                                  ab > (int64_t)lim ? lim : (uint32_t)ab);
    const uint32_t lds_a = lds_addr(lds);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      // copy k of wave w fills tile rows 2 (16 w + k) and + 1 (512 bytes each)
      const int r = 2 * (16 * w + k) + (l >> 5), c = (l & 31) ^ (r & 31);
      dma16s(ra, (uint32_t)((int64_t)r * lda2) + (uint32_t)(c * 16), 0u, lds_a + (uint32_t)(16 * w + k) * 1024u);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int half = l >> 5;
    const int mrow = m0 + wm * WM;                      // the wave's first row
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int t = wn * WN + j * 32 + (l & 31);       // tile row of A_tok (token)
      const unsigned char* arow = lds + t * 512;
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int hd = wm * WM + i * 32 + 8 * a + 4 * half;   // tile column: 4 consecutive
          const uint2 v = *reinterpret_cast<const uint2*>(arow + (((hd >> 3) ^ (t & 31)) << 4) + (hd & 7) * 2);
          const f32x16& cc = acc[i][j];
          s = fmaf(cc[4 * a], __uint_as_float(v.x << 16), s);
          s = fmaf(cc[4 * a + 1], __uint_as_float(v.x & 0xffff0000u), s);
          s = fmaf(cc[4 * a + 2], __uint_as_float(v.y << 16), s);
          s = fmaf(cc[4 * a + 3], __uint_as_float(v.y & 0xffff0000u), s);
        }
      s += __shfl_xor(s, 32);
      const int n = n0 + t;
      if (l < 32 && n < p.N && mrow < p.Mrows) {
        const int h = mrow / p.dot_d, q = (mrow - h * p.dot_d) / 64;
        p.dot_out[((int64_t)q * p.dot_H + h) * p.N + n] = s;
      }
    }
  } else {
    char* Cb = static_cast<char*>(p.C) + (int64_t)z * p.bc * (p.out_bf16 ? 2 : 4);
    if constexpr (PP && WM == 64 && WN % 64 == 0) {
      // output of the 256 x 256 kernel, bf16: each wave stages its 64-row
      // block through LDS, 64 columns at a time (the operand stages are idle
      // once every wave has passed the loop's last barrier), so that eight
      // lanes write one column's 64 consecutive rows (128 bytes) with 16-byte
      // stores instead of 64 scattered 8-byte pieces per instruction
      if (p.out_bf16 && p.ldc % 8 == 0 && p.bc % 8 == 0) {
        constexpr int PITCH = 144;   // bytes per staged column: 128 + 16
        static_assert(NW * 64 * PITCH <= NST * STAGE, "staging fits the operand stages");
        __syncthreads();
        unsigned char* stg = lds + w * 64 * PITCH;
        uint16_t* Cs = reinterpret_cast<uint16_t*>(Cb);
#pragma unroll
        for (int jh = 0; jh < WN / 64; ++jh) {
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int jj = 0; jj < 2; ++jj)
#pragma unroll
              for (int a = 0; a < 4; ++a) {
                const f32x16& c = acc[i][2 * jh + jj];
                const int nn = jj * 32 + (l & 31), mm = i * 32 + 8 * a + 4 * (l >> 5);
                *reinterpret_cast<uint2*>(stg + nn * PITCH + mm * 2) =
                    make_uint2(f32_to_bf16_bits(c[4 * a]) | (f32_to_bf16_bits(c[4 * a + 1]) << 16),
                               f32_to_bf16_bits(c[4 * a + 2]) | (f32_to_bf16_bits(c[4 * a + 3]) << 16));
              }
          // a wave's LDS operations run in order; the wait and the clobber
          // keep the compiler's order too
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int c = l + 64 * k, nn = c >> 3, q = c & 7;
            const uint4 v = *reinterpret_cast<const uint4*>(stg + nn * PITCH + q * 16);
            const int n = n0 + wn * WN + jh * 64 + nn;
            const int m = m0 + wm * WM + 8 * q;
            if (n >= p.N || m >= p.Mrows) continue;
            const int64_t o = (int64_t)n * p.ldc + m;
            if (m + 8 <= p.Mrows) {
              *reinterpret_cast<uint4*>(Cs + o) = v;
            } else {
              const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
              for (int e = 0; e < p.Mrows - m; ++e) Cs[o + e] = (uint16_t)(wv[e >> 1] >> (16 * (e & 1)));
            }
          }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
        return;
      }
      // fp32 output (the token-chunk parts of R): the same through LDS, 32
      // columns at a time, sixteen lanes writing one column's 64 rows (256
      // bytes)
      if (!p.out_bf16 && p.ldc % 4 == 0 && p.bc % 4 == 0) {
        constexpr int PITCH = 272;   // bytes per staged column: 256 + 16
        static_assert(NW * 32 * PITCH <= NST * STAGE, "staging fits the operand stages");
        __syncthreads();
        unsigned char* stg = lds + w * 32 * PITCH;
        float* Cf = reinterpret_cast<float*>(Cb);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int a = 0; a < 4; ++a) {
              const f32x16& c = acc[i][j];
              const int nn = l & 31, mm = i * 32 + 8 * a + 4 * (l >> 5);
              *reinterpret_cast<float4*>(stg + nn * PITCH + mm * 4) =
                  make_float4(c[4 * a], c[4 * a + 1], c[4 * a + 2], c[4 * a + 3]);
            }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
          for (int k = 0; k < 8; ++k) {
            const int c = l + 64 * k, nn = c >> 4, q = c & 15;
            const float4 v = *reinterpret_cast<const float4*>(stg + nn * PITCH + q * 16);
            const int n = n0 + wn * WN + j * 32 + nn;
            const int m = m0 + wm * WM + 4 * q;
            if (n >= p.N || m >= p.Mrows) continue;
            const int64_t o = (int64_t)n * p.ldc + m;
            if (m + 4 <= p.Mrows) {
              *reinterpret_cast<float4*>(Cf + o) = v;
            } else {
              const float vv[4] = {v.x, v.y, v.z, v.w};
              for (int e = 0; e < p.Mrows - m; ++e) Cf[o + e] = vv[e];
            }
          }
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        }
        return;
      }
    }
    // C[m, n] at n * ldc + m: a lane's 4 consecutive rows m (e = 0..3) are one
    // 8-byte (bf16) or 16-byte (fp32) store
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WN + j * 32 + (l & 31);
        if (n >= p.N) continue;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int mb = m0 + wm * WM + i * 32 + 8 * a + 4 * (l >> 5);
          if (mb >= p.Mrows) continue;
          const int64_t o = (int64_t)n * p.ldc + mb;
          const float v0 = acc[i][j][4 * a], v1 = acc[i][j][4 * a + 1];
          const float v2 = acc[i][j][4 * a + 2], v3 = acc[i][j][4 * a + 3];
          if (mb + 4 <= p.Mrows) {
            if (p.out_bf16)
              *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(Cb) + o) =
                  make_uint2(f32_to_bf16_bits(v0) | (f32_to_bf16_bits(v1) << 16),
                             f32_to_bf16_bits(v2) | (f32_to_bf16_bits(v3) << 16));
            else
              *reinterpret_cast<float4*>(reinterpret_cast<float*>(Cb) + o) = make_float4(v0, v1, v2, v3);
          } else {
            const float v[4] = {v0, v1, v2, v3};
            for (int e = 0; e < p.Mrows - mb; ++e) {
              if (p.out_bf16) reinterpret_cast<uint16_t*>(Cb)[o + e] = (uint16_t)f32_to_bf16_bits(v[e]);
              else reinterpret_cast<float*>(Cb)[o + e] = v[e];
            }
          }
        }
      }
  }
}

template <int BM, int BN, int BK, int WGM, int WGN, int NST, int EPI, bool PP = false>
hipError_t launch_t(const GemmParams& p, int ny, hipStream_t st) {
  // a tile's rows must lie within the 32-bit range of its buffer resource
  if ((int64_t)BM * p.ldx * 2 > kMaxResourceBytes || (int64_t)BN * p.ldy * 2 > kMaxResourceBytes)
    return hipErrorInvalidValue;
  const int N = EPI == kEpiSegSq ? (PP ? WGN : 1) * p.d_next : p.N;
  const int ntiles = ((p.Mrows + BM - 1) / BM) * ((N + BN - 1) / BN);
  const dim3 grid(8 * ((ntiles + 7) / 8), ny);
  hipLaunchKernelGGL((mm_bf16_kernel<BM, BN, BK, WGM, WGN, NST, EPI, PP>), grid, dim3(64 * WGM * WGN), 0, st, p);
  return hipGetLastError();
}

}  // namespace

// rounds of `slots` concurrent workgroups (one per CU) times the work of one
// tile (its area, at equal K): the cost of a tiling
static int64_t tiling_cost(int64_t tiles, int slots, int area) { return (tiles + slots - 1) / slots * area; }

hipError_t launch_mm_bf16(const GemmParams& p, int epilogue, int ny, hipStream_t st) {
  if (ny == 0 || p.Mrows == 0) return hipSuccess;
  const int64_t ntm256 = (p.Mrows + 255) / 256;
  if (epilogue == kEpiSegSq) {
    // segments two to a ping-pong tile whose wave columns are one segment
    // wide (d' = 128, 96 or 64) when the segment counts of W_q and of W_k,
    // W_v are even; else one per 128 x 128 tile (192-row tiles, ping-pong or
    // not, measured 4-36% slower than these)
    if (p.H_next % 2 == 0 && p.G_next % 2 == 0 && ny % 2 == 0) {
      if (p.d_next == 128) return launch_t<256, 256, 64, 4, 2, 2, kEpiSegSq, true>(p, ny / 2, st);
      if (p.d_next == 96) return launch_t<256, 192, 64, 4, 2, 2, kEpiSegSq, true>(p, ny / 2, st);
      if (p.d_next == 64) return launch_t<256, 128, 64, 4, 2, 2, kEpiSegSq, true>(p, ny / 2, st);
    }
    return launch_t<128, 128, 64, 2, 2, 2, kEpiSegSq>(p, ny, st);
  }
  if (epilogue == kEpiDot) return launch_t<256, 256, 64, 4, 2, 2, kEpiDot, true>(p, ny, st);
  if (epilogue == kEpiFold) {
    // the ping-pong tile (256 x 256, 256 x 192 or 192 x 256) that needs the
    // least work per CU: the Qwen3-0.6B-shaped fold gets 256 x 192 and the
    // Danube3-500M-shaped one 192 x 256 (256 tiles on 256 CUs instead of 192)
    const int64_t c_sq = tiling_cost(ntm256 * ((p.N + 255) / 256) * ny, 256, 256 * 256);
    const int64_t c_n192 = tiling_cost(ntm256 * ((p.N + 191) / 192) * ny, 256, 256 * 192);
    const int64_t c_m192 = tiling_cost((p.Mrows + 191) / 192 * ((p.N + 255) / 256) * ny, 256, 192 * 256);
    if (c_n192 < c_sq && c_n192 <= c_m192) return launch_t<256, 192, 64, 4, 2, 2, kEpiFold, true>(p, ny, st);
    if (c_m192 < c_sq) return launch_t<192, 256, 64, 2, 4, 2, kEpiFold, true>(p, ny, st);
    return launch_t<256, 256, 64, 4, 2, 2, kEpiFold, true>(p, ny, st);
  }
  if (p.N == 0) return hipSuccess;
  // 256 x 256 tiles when both sides fill them and there is a tile per CU
  if (p.Mrows >= 256 && p.N >= 256 &&
      (int64_t)((p.Mrows + 255) / 256) * ((p.N + 255) / 256) * ny >= 256)
    return launch_t<256, 256, 64, 4, 2, 2, kEpiStore, true>(p, ny, st);
  return launch_t<128, 128, 64, 2, 2, 2, kEpiStore>(p, ny, st);
}

}  // namespace hna
