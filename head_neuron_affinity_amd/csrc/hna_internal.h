// Internal declarations shared by the HIP translation units of libhna.
// Everything here is gfx950-only device code or host-side launch plumbing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hna {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kMaxHeads = 128;
constexpr int kLdsBytes = 160 * 1024;   // LDS per CU on gfx950

// ---------------------------------------------------------------------------
// Folded up-weights M_h = W_o^(h)T diag(gamma) [W_gate; W_up]^T, stored in the
// operand order of the 32x32 MFMA B fragments the affinity kernel consumes:
//   M[h][kb][gu][s][lane][e],  e in 0..7,
// kb = neuron block of 32 (neuron k = 32 kb + (lane & 31)), gu = 0 gate / 1 up,
// s = step of 16 along d (j = 16 s + 8 (lane >> 5) + e).  One (h, kb, gu, s)
// slab is 64 lanes x 8 elements, contiguous, so every fragment load of a wave
// is one fully coalesced 1 KiB (bf16) or 2 KiB (f32) read.  Neurons are padded
// to a multiple of 32 with zeros.
__host__ __device__ inline int64_t folded_index(int h, int j, int k, int gu, int KB, int S) {
  const int s = j >> 4, half = (j >> 3) & 1, e = j & 7;
  const int kb = k >> 5, lane = (k & 31) + 32 * half;
  return (((((int64_t)h * KB + kb) * 2 + gu) * S + s) * 64 + lane) * 8 + e;
}

inline int round_up(int x, int m) { return (x + m - 1) / m * m; }

// bf16 <-> f32 (round to nearest even; the inputs here are finite).
__device__ inline float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }
__device__ inline uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats to packed bf16 (low half = a), round to nearest even, one
// v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// MFMA helpers shared by the kernels that consume folded-layout fragments.
// bf16: one 32x32x16 MFMA per 16-wide step of the contraction.
__device__ inline void mma(f32x16& c, const uint4 (&a)[1], const uint4 (&b)[1]) {
  c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[0]),
                                              __builtin_bit_cast(bf16x8, b[0]), c, 0, 0, 0);
}
// f32: eight 32x32x2 MFMAs per 16-wide step; MFMA e pairs element e of the
// lower lane half (index 16s+e of the step) with element e of the upper half
// (16s+8+e), so both operands use the same per-lane element order as bf16.
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

// ------------------------------------------------------------- affinity pass
constexpr int kTileTokens = 128;   // tokens per tile
constexpr int kTileNeurons = 128;  // neurons per workgroup (4 waves x 32)
constexpr int kTilesPerChunk = 8;  // token tiles accumulated by one workgroup
constexpr int kSuperKt = 4;        // neuron tiles per XCD super-tile
constexpr int kSuperChunks = 8;    // token chunks per XCD super-tile
constexpr int kGramStage = 64;     // tokens per LDS stage of the Gram kernel

struct UpParams {
  const void* a;
  const void* g;
  const void* u;
  const float* r;
  const float* r_next;    // r when the down moment is not wanted (want_c = 0)
  const void* M;
  float* part;            // [n_chunks][G+1][I32]: per-group FO sums, then the down moment
  int64_t T;
  int H, G, d, I, I32;
  int n_tt, n_kt, n_chunks, n_ktg, n_st;
  int want_c;
  int8_t head_order[kMaxHeads];  // heads sorted by KV group (stable)
  int8_t head_group[kMaxHeads];  // group of head_order[i]
};

// Gram matrices C_h = sum_t a_th a_th^T / r_t^2 ([H, d, d] fp32), in partial
// sums over token chunks.
struct GramParams {
  const void* a;
  const float* r;
  const float2* coef;     // [T][H] (alpha, beta): weights beta^2 instead of 1/r^2 (or NULL)
  float* part;            // [n_gc][H][d][d]
  int64_t T;
  int H, d, n_gc;
  int64_t chunk_tokens;   // multiple of kGramStage
};

// add[g][k] = sum_{h in g} sum_{gate, up} m_hk^T C_h m_hk, m_hk = column k of M_h
// (per head into add_part, then summed over each group's heads in order).
struct QuadParams {
  const void* C;          // [H][d][d]: bf16 high plane then remainder plane, or fp32
  const void* M;          // folded weights
  float* add;             // [G][KB * 32]
  float* add_part;        // [H][KB * 32]: per-head sums before the group sum
  int H, G, d, KB;
  int8_t head_order[kMaxHeads];       // heads sorted by KV group
  int16_t group_start[kMaxHeads + 1]; // group g owns head_order[group_start[g] .. group_start[g+1])
};

struct UpGeometry {
  int I32, n_tt, n_kt, n_chunks, n_ktg, n_cg, n_st, grid;
  int n_gc;               // token chunks of the Gram kernel
  int64_t gram_chunk;     // tokens per Gram chunk
  bool gu_lds;            // g/u staged in LDS (bf16 with I % 8 == 0)
  size_t part_bytes, gram_part_bytes, gram_bytes, add_bytes, add_part_bytes, ws_bytes;
  size_t lds_bytes, dyn_lds_bytes;
  // byte offsets of the regions inside the workspace
  size_t off_gram_part, off_gram, off_add, off_add_part;
};
UpGeometry up_geometry(int64_t T, int H, int G, int d, int I, int dtype);

hipError_t launch_affinity_up(const UpParams& p, const UpGeometry& geo, int dtype, hipStream_t st);
hipError_t launch_finalize_up(const float* part, const float* add, int n_chunks, int G, int I,
                              int I32, const float* wd_sq, float scale, int accumulate,
                              float* S_fo, float* S_add, float* c_down, hipStream_t st);
hipError_t launch_gram(const GramParams& p, int dtype, hipStream_t st);
hipError_t launch_gram_reduce(const float* part, int n_gc, int64_t n, void* C, int dtype,
                              hipStream_t st);
hipError_t launch_quad(const QuadParams& p, int dtype, hipStream_t st);

// --------------------------------------------------------------- small kernels
hipError_t launch_col_sqnorm(const void* W, int rows, int cols, int dtype, float* out,
                             hipStream_t st);
hipError_t launch_down_group_sum(const float* seg_part, const int16_t* seg_list,
                                 const int16_t* group_start, int G_next, int I, float* n,
                                 hipStream_t st);
hipError_t launch_down_combine(const float* c, const float* n, int I, int G_next,
                               float* S_down, hipStream_t st);

// ----------------------------------------------------------- layout objective
hipError_t launch_unit_mass(const float* S, int64_t count, int n_mat, float* out, hipStream_t st);
hipError_t launch_mfma_rate(const void* seed, int n_wg, int iters, int shape, float* out,
                            hipStream_t st);
int max_objective_layers();
hipError_t launch_layout_objective(const float* S_up, const float* S_down, const int32_t* heads,
                                   const int32_t* neurons, int N, int G, int I, double* frac_up,
                                   double* frac_down, double* J, hipStream_t st);

// ------------------------------------------------- neuron step of the layout search
constexpr int kLayoutMaxDevices = 8;
constexpr int kLayoutMaxNpt = 16;                 // neurons per thread: I <= 16384
constexpr size_t kLayoutMaxLds = 128 * 1024;      // the fp64 gain M [L][I] in LDS
enum { kLayoutOk = 0, kLayoutBadHeads = 1, kLayoutSwapLimit = 2, kLayoutNoMove = 3 };

struct NeuronStepParams {
  const float* S_up;      // [N][G][I]
  const float* S_down;    // [N-1][I][G]
  const int32_t* heads;   // [N][G], devices 0..L-1
  int32_t* neurons;       // [N][I] out
  int32_t* stats;         // [N][4] out: status, excess after the dual ascent, moves, swaps
  int N, G, I, L, iters, max_swaps;
  int qtab;               // set by the launcher: the dual quotients come from an LDS table
};
size_t neuron_step_lds_bytes(int I, int L);
hipError_t launch_neuron_step(const NeuronStepParams& p, hipStream_t st);

// head step: G <= 16 groups, at most 2^24 balanced partitions
constexpr int kHeadMaxGroups = 16;
constexpr int kHeadMaxParts = 1 << 24;
enum { kLayoutBadNeurons = 4 };
struct HeadStepParams {
  const float* S_up;       // [N][G][I]
  const float* S_down;     // [N-1][I][G]
  const int32_t* neurons;  // [N][I], devices 0..L-1
  int32_t* heads;          // [N][G] out
  double* score;           // [N] out: the best partition's score
  int32_t* status;         // [N] out
  int N, G, I, L;
  int n_parts;             // G! / ((G/L)!)^L
};
hipError_t launch_head_step(const HeadStepParams& p, hipStream_t st);

// --------------------------------------------------------- NT GEMM (MFMA)
// C[m, n] = sum_c X[m, c] * Y[n, c]; X [Mrows, K] and Y [N, K] row-major with
// c contiguous.  launch_scale_transpose makes X[m, c] = s[c] * W[c, m] from a
// row-major W [K, Mrows].  Epilogues: write the folded layout, sum C^2 over
// the n of a segment, or store C[m, n] (fp32, or bf16 from the bf16 kernel)
// at C + n * ldc + m (C transposed: m contiguous, ldc and m0 multiples of 4),
// or (dot) dot each 64-row block of C's column n with the matching entries of
// a row-major token operand A_tok [N][lda]: out[q][h][n] = sum over the 64
// rows m = h d + 64 q + i of C[m, n] A_tok[n][m] (d a multiple of 64).
enum GemmEpilogue { kEpiFold = 0, kEpiSegSq = 1, kEpiStore = 2, kEpiDot = 3 };

struct GemmParams {
  const void* X;       // Xs [Mrows, K]
  const void* Y[3];    // fold: Y[0] = W_gate, Y[1] = W_up; segsq: W_q, W_k, W_v; store: Y[0]
  int64_t ldx, ldy;
  int Mrows, N, K;     // fold: N = I32 (rows of Y beyond Nvalid are zero)
  int Nvalid;
  // fold output
  void* M;
  int d, KB, S;
  // segment-square output
  float* seg_part;     // [n_seg][Mrows]
  int H_next, G_next, d_next;
  // plain-store output; grid.y indexes batches (X, Y and C advance by bx, by,
  // bc elements) or, when k_split > 0, chunks of k_split along K (C advances
  // by bc, one fp32 part per chunk)
  void* C;
  int64_t ldc, bx, by, bc;
  int k_split;
  int out_bf16;        // store in bf16 (fp32 otherwise)
  // dot output: A_tok (bf16, [N][dot_lda]) and out ([d / 64][dot_H][N] fp32)
  const void* dot_a;
  float* dot_out;
  int64_t dot_lda;
  int dot_H, dot_d;
};
// The bf16 GEMM (k_mm.hip): grid y runs over gate / up (fold, ny = 2), the
// H' + 2 G' segments of W_q, W_k, W_v (segment square), or batches / K chunks
// of Y[0] (store).  X, Y rows 16-byte aligned (ldx, ldy multiples of 8), K and
// k_split multiples of 8.
hipError_t launch_mm_bf16(const GemmParams& p, int epilogue, int ny, hipStream_t st);


// The leave-one-out score through its split T1 + 2 T2 + T3 (see k_loo.hip).
struct LooCombineParams {
  const void* M;          // folded weights
  const float* Y;         // [2][I][H*d]: Y^g then Y^u, column-major H*d x I
  const double* t1r;      // [H][I]: T1 summed over the token chunks (NULL: no tokens)
  const float* t3;        // [G][I32]: the group sums of the weighted quadratic forms
  float* S_loo;           // [G][I]
  float scale;
  int H, G, d, I, I32, KB, S;
  int8_t head_order[kMaxHeads];
  int16_t group_start[kMaxHeads + 1];
};
hipError_t launch_t1_reduce(const float* t1, int n_tc, int64_t HI, double* t1r, hipStream_t st);
// |x|^2, x in bf16 (xl, when not null) and x transposed into [D][Tp] (GEMM
// dtype, zero padding tokens) in one pass
hipError_t launch_x_prep(const float* x, int64_t T, int D, int64_t Tp, float* xx, void* xl,
                         void* xT, int dtype, hipStream_t st);
hipError_t launch_loo_coef(const void* a, const void* Z, const void* U, const float* xx, int64_t T,
                           int H, int d, int D, float2* coef, int dtype, hipStream_t st);
// bf16 with d a multiple of 32 up to 128: the moments (|o_h|^2 on the matrix
// cores from Q_h = W_o^(h)T W_o^(h)), alpha and beta, and (alpha beta / r) a
// written transposed, ZAT [H d][Tp], in one kernel.  x . o_h is Z_h . a_h
// from Z = x W_o, or (xo_part non-null; d = 64 or 128) the sum of the d / 64
// planes xo_part[q][h][t] that the GEMM's dot epilogue wrote.
bool loo_coef_fused(int d, int dtype);
bool loo_dot_epilogue(int d, int dtype);
hipError_t launch_loo_coef_fused(const void* a, const void* Z, const float* xo_part, void* ZAT,
                                 const void* Q, const float* xx, int64_t T, int H, int d, int D,
                                 float2* coef, hipStream_t st);
hipError_t launch_scale_a(const void* a, const float2* coef, const float* xx, int64_t T, int H,
                          int d, int D, void* As, int dtype, hipStream_t st);
// Tokens padded to a multiple of 8 (the K length of the token GEMM)
int64_t loo_tokens_padded(int64_t T);
// R = ((alpha beta / r) a)^T x over the tokens runs in K chunks of this many
// padded tokens (a multiple of 64), one fp32 part per chunk, so that its few
// output tiles still fill the chip
int loo_r_chunk(int64_t T);
int loo_r_parts(int64_t T);
// Rs = (sum of `parts` parts of R) diag(gamma) in the input dtype, each part
// row-major [HD][D] fp32
hipError_t launch_scale_cols(const float* R, int parts, const float* gamma, int HD, int D,
                             void* Rs, int dtype, hipStream_t st);
int t1_chunks(int64_t T);
hipError_t launch_t1(const void* g, const void* u, const float2* coef, int64_t T, int H, int I,
                     float* t1, int dtype, hipStream_t st);
hipError_t launch_loo_combine(const LooCombineParams& p, int dtype, hipStream_t st);
// out[c, r] = s[r] in[r, c] (s null: no scaling) for in [rows, cols]
// row-major; out rows have length ldo >= rows (ldo a multiple of 8), the
// entries past rows are written as zeros
hipError_t launch_scale_transpose(const void* in, const float* s, void* out, int rows, int cols,
                                  int ldo, int dtype, hipStream_t st);
// The fp32 GEMM (k_gemm.hip): ny = gate / up (fold), segments (segment square)
// or batches / K chunks (store); K and k_split multiples of 4
hipError_t launch_gemm_f32(const GemmParams& p, int epilogue, int ny, hipStream_t st);

}  // namespace hna
