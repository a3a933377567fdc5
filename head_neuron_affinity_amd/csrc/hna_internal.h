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

// ------------------------------------------------------------- affinity pass
constexpr int kTileTokens = 128;   // tokens per tile (4 MFMA row blocks of 32)
constexpr int kTileNeurons = 128;  // neurons per workgroup (4 waves x 32)
constexpr int kTilesPerChunk = 8;  // token tiles accumulated by one workgroup
constexpr int kSuperKt = 4;        // neuron tiles per XCD super-tile
constexpr int kSuperChunks = 8;    // token chunks per XCD super-tile

struct UpParams {
  const void* a;
  const void* g;
  const void* u;
  const float* r;
  const float* r_next;
  const void* M;
  float* part;          // [n_chunks][2G+1][I32]
  int64_t T;
  int H, G, d, I, I32;
  int n_tt, n_kt, n_chunks, n_ktg, n_st;
  int8_t head_order[kMaxHeads];  // heads sorted by KV group (stable)
  int8_t head_group[kMaxHeads];  // group of head_order[i]
};

struct UpGeometry {
  int I32, n_tt, n_kt, n_chunks, n_ktg, n_cg, n_st, grid;
  size_t part_floats;
  size_t lds_bytes;       // total LDS per workgroup (static + dynamic)
  size_t dyn_lds_bytes;   // dynamic part (per-group accumulators)
  bool gu_lds;            // g/u tiles staged through LDS (bf16 with I % 8 == 0)
};
UpGeometry up_geometry(int64_t T, int H, int G, int d, int I, int dtype);

hipError_t launch_affinity_up(const UpParams& p, int dtype, size_t dyn_lds_bytes, int grid,
                              hipStream_t st);
hipError_t launch_finalize_up(const float* part, int n_chunks, int G, int I, int I32,
                              const float* wd_sq, float scale, int accumulate, float* S_fo,
                              float* S_add, float* c_down, hipStream_t st);

// --------------------------------------------------------------- small kernels
hipError_t launch_transpose(const void* in, void* out, int rows, int cols, int esize,
                            hipStream_t st);
hipError_t launch_col_sqnorm(const void* W, int rows, int cols, int dtype, float* out,
                             hipStream_t st);
hipError_t launch_down_group_sum(const float* seg_part, const int16_t* seg_list,
                                 const int16_t* group_start, int G_next, int I, float* n,
                                 hipStream_t st);
hipError_t launch_down_combine(const float* c, const float* n, int I, int G_next,
                               float* S_down, hipStream_t st);

// ------------------------------------------------------ scaled NT GEMM (MFMA)
// C[m, n] = sum_c X[m, c] * s[c] * Y[n, c]; X [Mrows, K] and Y [N, K] row-major
// with c contiguous.  Epilogues: write the folded layout, or sum C^2 over the
// n of a segment.
enum GemmEpilogue { kEpiFold = 0, kEpiSegSq = 1 };

struct GemmParams {
  const void* X;       // [Mrows, K]
  const void* Y[3];    // fold: Y[0] = W_gate, Y[1] = W_up; segsq: W_q, W_k, W_v
  const float* s;      // [K]
  int64_t ldx, ldy;
  int Mrows, N, K;     // fold: N = I32 (rows of Y beyond Nvalid are zero)
  int Nvalid;
  // fold output
  void* M;
  int d, KB, S;
  // segment-square output
  float* seg_part;     // [n_seg][Mrows]
  int H_next, G_next, d_next;
};
hipError_t launch_gemm(const GemmParams& p, int dtype, int epilogue, dim3 grid,
                       hipStream_t st);

}  // namespace hna
