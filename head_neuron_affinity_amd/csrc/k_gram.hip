// The ADD up score of "Affinity-Aware Sharding for Delayed Tensor
// Parallelism", section 3, paragraph "Affinity scores", through per-head Gram
// matrices.
//
// With p_h = gamma * (a_h W_o^(h)T) / r and the folded weights M_h (column
// m_hk = W_o^(h)T diag(gamma) w^g_k for the gate, likewise for the up
// projection), p_h . w^g_k = (a_h . m_hk) / r, so
//   sum_t (p_h . w^g_k)^2 = m_hk^T C_h m_hk,   C_h = sum_t a_th a_th^T / r_t^2.
// The identity is exact (linearity of the sum), so ADD needs one d x d Gram
// matrix per head instead of a per-(token, head, neuron) square:
//   gram_kernel   C_h = sum_t (a_th / r_t)(a_th / r_t)^T over a token chunk,
//                 on the matrix cores: a / r is staged once through LDS,
//                 transposed (token index contiguous), and serves as both MFMA
//                 operands (16-byte fragments);
//   gram_reduce   fixed-order sum over the token chunks;
//   quad_kernel   Y = C_h M_h(:, block) on the matrix cores, then
//                 add[g][k] = sum_{h in g} sum_{gate, up} m_hk . Y(:, k).
// bf16 path: a / r is rounded to bf16 once (an unbiased relative error <= 2^-9
// per element, <= 2^-8 per product, averaged over the token sum), and the
// reduced fp32 Gram entries are split into two bf16 terms (hi + lo) for the
// quadratic forms, a relative error near 2^-16 there.  f32 path: fp32 MFMA
// throughout.  A weight w_th per (token, head) in place of 1 / r_t^2 (the
// leave-one-out score's beta^2) scales by sqrt(w) = beta the same way.
#include "hna_internal.h"

namespace hna {
namespace {

constexpr int kGThreads = 256;

template <typename E> struct GramLds;
template <> struct GramLds<__bf16> {
  static constexpr int kPitch = kGramStage + 8;   // elements; 144-byte rows
  static constexpr int kQ = 1;
};
template <> struct GramLds<float> {
  static constexpr int kPitch = kGramStage + 4;   // 272-byte rows
  static constexpr int kQ = 2;
};

__device__ inline uint16_t bf16_rn(float x) { return (uint16_t)f32_to_bf16_bits(x); }

// Output tiles of 32 x 32 owned by wave w (NT x NT tiles in all): with NT >= 3
// a 2 x 2 block, tiles (2 (w / 2) + x, 2 (w % 2) + y), so that each MFMA
// operand fragment read from LDS serves two MFMAs; with NT <= 2 the single
// tile (w / NT, w % NT).  Slot s of the wave's accumulators is (x, y) =
// (s / 2, s % 2); tiles past NT are skipped.
template <int NT>
__device__ inline bool gram_tile(int w, int s, int& it, int& jt) {
  if constexpr (NT >= 3) {
    it = 2 * (w >> 1) + (s >> 1);
    jt = 2 * (w & 1) + (s & 1);
    return NT == 4 || (it < NT && jt < NT);   // NT = 4: every slot (w < 4)
  } else {
    it = w / NT;
    jt = w % NT;
    return s == 0 && w < NT * NT;
  }
}

// grid: n_gc * H workgroups (head fastest); C_part[gc][h] = sum over chunk gc.
// NT = ceil(d / 32).
template <typename E, int NT>
__global__ __launch_bounds__(kGThreads) void gram_kernel(const GramParams p) {
  using L = GramLds<E>;
  constexpr int TP = L::kPitch;
  constexpr int Q = L::kQ;
  __shared__ __attribute__((aligned(16))) E xs[128 * TP];   // a / r, transposed

  const int h = blockIdx.x % p.H;
  const int gc = blockIdx.x / p.H;
  const int d = p.d;
  const int d32 = 32 * NT;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int64_t t_begin = (int64_t)gc * p.chunk_tokens;
  const int64_t t_end = min(p.T, t_begin + p.chunk_tokens);
  const int64_t H = p.H;

  // rows d .. d32-1 stay zero
  for (int x = tid; x < (d32 - d) * TP; x += kGThreads) xs[d * TP + x] = E(0.f);

  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x16{};

  // One (4 tokens) x (8 features) item per thread (d <= 128).  Items are
  // loaded into registers two stages ahead (two register sets in turn), so
  // that two stages' loads are in flight under each stage's MFMAs.
  const int items = (kGramStage / 4) * (d / 8);
  const bool has_item = tid < items;
  const int tq = tid % (kGramStage / 4), fo = tid / (kGramStage / 4);
  constexpr int NV = sizeof(E) == 2 ? 1 : 2;   // 16-byte loads per token
  uint4 rawA[4][NV], rawB[4][NV];
  float rrA[4], rrB[4];
  int okA, okB;   // bit j: token j of the item lies in the chunk
  // the weight per token: 1/r^2 from r, or beta^2 per (token, head) from the
  // coefficient table (its second component)
  const bool weighted = p.coef != nullptr;
  const float* wsrc = weighted ? reinterpret_cast<const float*>(p.coef) + 2 * h + 1 : p.r;
  const int64_t wstride = weighted ? 2 * H : 1;
  const int fo_c = has_item ? fo : 0;
  // The loads are unconditional: a token outside the chunk reads row t_begin
  // (which always exists), and its in-chunk bit is applied where the data is
  // used.  Nothing then waits on a load at issue time, and the wait before a
  // stage's LDS writes covers that stage only, not the one loading behind it.
  // pa0 / pw0: this thread's first token of the first stage (t_begin + 4 tq).
  const int64_t rs = H * d;
  const E* pa_safe = static_cast<const E*>(p.a) + (t_begin * H + h) * d + 8 * fo_c;
  const E* pa0 = pa_safe + 4 * tq * rs;
  const float* pw_safe = wsrc + t_begin * wstride;
  const float* pw0 = pw_safe + 4 * tq * wstride;
  auto load_item = [&](uint4 (&raw)[4][NV], float (&rr)[4], int& ok, int64_t ts) __attribute__((always_inline)) {
    const int64_t o = ts - t_begin;
    const E* pa = pa0 + o * rs;
    const float* pw = pw0 + o * wstride;
    const int64_t tq0 = ts + 4 * tq;
    ok = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool in = has_item && tq0 + j < t_end;
      ok |= (int)in << j;
      rr[j] = *(in ? pw + j * wstride : pw_safe);
      const uint4* src = reinterpret_cast<const uint4*>(in ? pa + j * rs : pa_safe);
#pragma unroll
      for (int v = 0; v < NV; ++v) raw[j][v] = src[v];
    }
  };
  auto stage = [&](uint4 (&raw)[4][NV], float (&rr)[4], int& ok, int64_t ts) __attribute__((always_inline)) {
    // (ok is refilled by the load of stage ts + 2 kGramStage below)
    __syncthreads();   // the previous stage has been read
    if (has_item) {
      // tokens outside the chunk get weight 0 (their finite values, from row
      // t_begin, then add nothing)
#pragma unroll
      for (int j = 0; j < 4; ++j) rr[j] = ((ok >> j) & 1) ? rr[j] : 0.f;
      float sw[4];   // sqrt of the weight: 1 / r_t, or beta_th
#pragma unroll
      for (int j = 0; j < 4; ++j)
        // hardware reciprocal (about 1 ulp): the product is rounded to bf16
        // on the bf16 path, and 1 ulp is far inside the fp32 tolerance
        sw[j] = weighted ? rr[j] : (rr[j] != 0.f ? __builtin_amdgcn_rcpf(rr[j]) : 0.f);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int base = (8 * fo + e) * TP + 4 * tq;
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float xv;
          if constexpr (sizeof(E) == 2) {
            const uint32_t wv = e < 2 ? raw[j][0].x : e < 4 ? raw[j][0].y : e < 6 ? raw[j][0].z : raw[j][0].w;
            xv = (e & 1) ? __uint_as_float(wv & 0xffff0000u) : __uint_as_float(wv << 16);
          } else {
            const uint32_t wv[8] = {raw[j][0].x, raw[j][0].y, raw[j][0].z, raw[j][0].w,
                                    raw[j][NV - 1].x, raw[j][NV - 1].y, raw[j][NV - 1].z,
                                    raw[j][NV - 1].w};
            xv = __uint_as_float(wv[e]);
          }
          y[j] = xv * sw[j];
        }
        if constexpr (sizeof(E) == 2)
          *reinterpret_cast<uint2*>(&xs[base]) = make_uint2(pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]));
        else
          *reinterpret_cast<float4*>(&xs[base]) = make_float4(y[0], y[1], y[2], y[3]);
      }
    }
    __syncthreads();
    load_item(raw, rr, ok, ts + 2 * kGramStage);   // past the chunk: masked off
    // C[i][j] += sum_t (x[i][t] / r_t) (x[j][t] / r_t): A rows i, B rows j
#pragma unroll
    for (int q = 0; q < kGramStage / 16; ++q) {
      const int col = 16 * q + 8 * (l >> 5);
      uint4 af[2][Q], bh[2][Q];
      // the fragments of the wave's row tiles (A) and column tiles (B)
      auto frag = [&](uint4 (&f)[Q], int tile) __attribute__((always_inline)) {
#pragma unroll
        for (int qq = 0; qq < Q; ++qq)
          f[qq] = *reinterpret_cast<const uint4*>(&xs[(tile * 32 + (l & 31)) * TP + col] +
                                                  qq * (16 / sizeof(E)));
      };
      if constexpr (NT >= 3) {
        const int it0 = 2 * (w >> 1), jt0 = 2 * (w & 1);
#pragma unroll
        for (int x = 0; x < 2; ++x) {
          if (it0 + x < NT) frag(af[x], it0 + x);
          if (jt0 + x < NT) frag(bh[x], jt0 + x);
        }
      } else if (w < NT * NT) {
        frag(af[0], w / NT);
        frag(bh[0], w % NT);
      }
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        int it, jt;
        if (gram_tile<NT>(w, sl, it, jt)) mma(acc[sl], af[sl >> 1], bh[sl & 1]);
      }
    }
  };
  load_item(rawA, rrA, okA, t_begin);
  load_item(rawB, rrB, okB, t_begin + kGramStage);
  // two stages per trip (a stage past the chunk adds zeros)
  for (int64_t ts = t_begin; ts < t_end; ts += 2 * kGramStage) {
    stage(rawA, rrA, okA, ts);
    stage(rawB, rrB, okB, ts + kGramStage);
  }
  // write the tiles (C layout: column l & 31, row 8 (v / 4) + 4 (l / 32) + v % 4)
  float* out = p.part + ((int64_t)gc * p.H + h) * d * d;
#pragma unroll
  for (int sl = 0; sl < 4; ++sl) {
    int it, jt;
    if (gram_tile<NT>(w, sl, it, jt)) {
      const int j = jt * 32 + (l & 31);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = it * 32 + 8 * (v >> 2) + 4 * (l >> 5) + (v & 3);
        if (i < d && j < d) out[(int64_t)i * d + j] = acc[sl][v];
      }
    }
  }
}

// C = sum over the token chunks in chunk order (4 entries per thread).  bf16
// path: C is written as two bf16 planes (high part, then remainder), the form
// the quadratic-form kernel multiplies; fp32 path: fp32.
template <bool BF>
__global__ __launch_bounds__(256) void gram_reduce_kernel(const float* __restrict__ part, int n_gc,
                                                          int64_t n, void* __restrict__ C) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;   // n is a multiple of 16 (d % 16 == 0)
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  int c = 0;
  for (; c + 4 <= n_gc; c += 4) {
    float4 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = *reinterpret_cast<const float4*>(part + (int64_t)(c + j) * n + i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s.x += v[j].x; s.y += v[j].y; s.z += v[j].z; s.w += v[j].w;
    }
  }
  for (; c < n_gc; ++c) {
    const float4 v = *reinterpret_cast<const float4*>(part + (int64_t)c * n + i);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  if constexpr (BF) {
    const uint32_t h01 = pack_bf16x2(s.x, s.y), h23 = pack_bf16x2(s.z, s.w);
    const uint32_t l01 = pack_bf16x2(s.x - bf16_bits_to_f32(h01 & 0xffffu), s.y - __uint_as_float(h01 & 0xffff0000u));
    const uint32_t l23 = pack_bf16x2(s.z - bf16_bits_to_f32(h23 & 0xffffu), s.w - __uint_as_float(h23 & 0xffff0000u));
    uint16_t* c16 = static_cast<uint16_t*>(C);
    *reinterpret_cast<uint2*>(c16 + i) = make_uint2(h01, h23);
    *reinterpret_cast<uint2*>(c16 + n + i) = make_uint2(l01, l23);
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(C) + i) = s;
  }
}

// grid (H, ceil(KB / 4)), 4 waves: head blockIdx.x; wave w handles neuron block
// blockIdx.y * 4 + w and writes add_part[h][32 kb + l] (gate and up summed).
// C_h (bf16 high and remainder planes, or fp32) is copied into LDS; Y = C_h M
// for the wave's 32 neurons comes out of the MFMAs in the C layout (column
// l % 32, rows 8 (v / 4) + 4 (l / 32) + v % 4 of a 32-row tile), and each lane
// takes the dot product of its Y entries with the matching folded-weight
// entries: rows with (row / 8) % 2 == l / 32 are in its own fragment, the
// others in the fragment of lane l ^ 32 (one exchange per d-step).
constexpr int kQWaves = 4;
template <typename E, int S>
__global__ __launch_bounds__(64 * kQWaves) void quad_kernel(const QuadParams p) {
  constexpr bool BF = sizeof(E) == 2;
  constexpr int Q = BF ? 1 : 2;
  constexpr int DD = 16 * S;                          // d
  constexpr int D32 = (DD + 31) & ~31;
  constexpr int NT = D32 / 32;
  constexpr int CP = DD + (BF ? 8 : 4);               // LDS pitch of C (elements)
  constexpr int EPC = 16 / sizeof(E);                 // elements per 16 bytes
  constexpr int kSlabBytes = 64 * 8 * sizeof(E);
  constexpr int NB = BF ? 2 : 1;                      // C planes
  constexpr int NTH = 64 * kQWaves;
  __shared__ __attribute__((aligned(16))) E cs[NB][D32 * CP];

  const int h = blockIdx.x;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, half = l >> 5;
  const int kb = blockIdx.y * kQWaves + w;
  const bool active = kb < p.KB;
  const int kbc = active ? kb : p.KB - 1;
  const char* Mbytes = static_cast<const char*>(p.M);
  float q = 0.f;

  for (int x = tid; x < (D32 - DD) * CP; x += NTH)
#pragma unroll
    for (int b = 0; b < NB; ++b) cs[b][DD * CP + x] = E(0.f);
  {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const E* C = static_cast<const E*>(p.C) + ((int64_t)b * p.H + h) * DD * DD;
      for (int x = tid; x < DD * DD / EPC; x += NTH) {
        const int i = (x * EPC) / DD, jj = (x * EPC) % DD;
        *reinterpret_cast<uint4*>(&cs[b][i * CP + jj]) = reinterpret_cast<const uint4*>(C)[x];
      }
    }
    __syncthreads();
#pragma unroll
    for (int gu = 0; gu < 2; ++gu) {
      const char* Mb = Mbytes + (((int64_t)h * p.KB + kbc) * 2 + gu) * S * kSlabBytes +
                       (uint32_t)l * 8u * sizeof(E);
      uint4 bfr[S][Q];
#pragma unroll
      for (int s = 0; s < S; ++s)
#pragma unroll
        for (int qq = 0; qq < Q; ++qq)
          bfr[s][qq] = *reinterpret_cast<const uint4*>(Mb + s * kSlabBytes + qq * 16);
      // per d-step: this lane's fragment entries 4 half .. 4 half + 3 (own
      // rows) and the partner's (rows of the other half), as floats
      float own[S][4], oth[S][4];
#pragma unroll
      for (int s = 0; s < S; ++s) {
        float mv[8];
        if constexpr (BF) {
          const uint32_t wv[4] = {bfr[s][0].x, bfr[s][0].y, bfr[s][0].z, bfr[s][0].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            mv[2 * e] = bf16_bits_to_f32(wv[e] & 0xffffu);
            mv[2 * e + 1] = bf16_bits_to_f32(wv[e] >> 16);
          }
        } else {
          const uint32_t wv[8] = {bfr[s][0].x, bfr[s][0].y, bfr[s][0].z, bfr[s][0].w,
                                  bfr[s][Q - 1].x, bfr[s][Q - 1].y, bfr[s][Q - 1].z, bfr[s][Q - 1].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) mv[e] = __uint_as_float(wv[e]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          own[s][r] = half ? mv[4 + r] : mv[r];
          const float send = half ? mv[r] : mv[4 + r];   // what the partner needs
          oth[s][r] = __shfl_xor(send, 32);
        }
      }
#pragma unroll
      for (int it = 0; it < NT; ++it) {
        f32x16 acc = f32x16{};
#pragma unroll
        for (int s = 0; s < S; ++s) {
          const int off = (it * 32 + (l & 31)) * CP + 16 * s + 8 * half;
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            uint4 ah[Q];
#pragma unroll
            for (int qq = 0; qq < Q; ++qq)
              ah[qq] = *reinterpret_cast<const uint4*>(&cs[b][off] + qq * EPC);
            mma(acc, ah, bfr[s]);
          }
        }
        // rows it*32 + 8 a + 4 half + r (v = 4 a + r): d-step 2 it + a / 2,
        // entry r of own (a % 2 == half) or of the partner's
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int a = v >> 2, r = v & 3, s = 2 * it + (a >> 1);
          if (s < S) q = fmaf((a & 1) == half ? own[s][r] : oth[s][r], acc[v], q);
        }
      }
    }
  }
  q += __shfl_xor(q, 32);
  if (active && l < 32) p.add_part[(int64_t)h * p.KB * 32 + kb * 32 + l] = q;
}

// add[g][k] = sum of add_part[h][k] over the heads h of KV group g, in head
// order (fixed-order sum).
__global__ __launch_bounds__(256) void quad_group_sum_kernel(const QuadParams p) {
  const int64_t n = (int64_t)p.KB * 32;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)p.G * n) return;
  const int g = (int)(idx / n);
  const int64_t k = idx - g * n;
  float s = 0.f;
  for (int hh = p.group_start[g]; hh < p.group_start[g + 1]; ++hh)
    s += p.add_part[(int64_t)p.head_order[hh] * n + k];
  p.add[idx] = s;
}

template <typename E, int S>
hipError_t launch_quad_t(const QuadParams& p, hipStream_t st) {
  const dim3 grid(p.H, (p.KB + kQWaves - 1) / kQWaves);
  hipLaunchKernelGGL((quad_kernel<E, S>), grid, dim3(64 * kQWaves), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)p.G * p.KB * 32;
  hipLaunchKernelGGL(quad_group_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_quad_e(const QuadParams& p, hipStream_t st) {
  switch (p.d / 16) {
    case 1: return launch_quad_t<E, 1>(p, st);
    case 2: return launch_quad_t<E, 2>(p, st);
    case 3: return launch_quad_t<E, 3>(p, st);
    case 4: return launch_quad_t<E, 4>(p, st);
    case 5: return launch_quad_t<E, 5>(p, st);
    case 6: return launch_quad_t<E, 6>(p, st);
    case 7: return launch_quad_t<E, 7>(p, st);
    case 8: return launch_quad_t<E, 8>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_gram(const GramParams& p, int dtype, hipStream_t st) {
  if (p.n_gc == 0) return hipSuccess;
  const dim3 grid(p.n_gc * p.H);
  const int nt = (p.d + 31) / 32;
#define HNA_GRAM(NT)                                                                    \
  if (dtype == 1) hipLaunchKernelGGL((gram_kernel<__bf16, NT>), grid, dim3(kGThreads), 0, st, p); \
  else hipLaunchKernelGGL((gram_kernel<float, NT>), grid, dim3(kGThreads), 0, st, p);
  switch (nt) {
    case 1: HNA_GRAM(1) break;
    case 2: HNA_GRAM(2) break;
    case 3: HNA_GRAM(3) break;
    case 4: HNA_GRAM(4) break;
    default: return hipErrorInvalidValue;
  }
#undef HNA_GRAM
  return hipGetLastError();
}

hipError_t launch_gram_reduce(const float* part, int n_gc, int64_t n, void* C, int dtype,
                              hipStream_t st) {
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n / 4 + 255) / 256));
  if (dtype == 1) hipLaunchKernelGGL(gram_reduce_kernel<true>, grid, dim3(256), 0, st, part, n_gc, n, C);
  else hipLaunchKernelGGL(gram_reduce_kernel<false>, grid, dim3(256), 0, st, part, n_gc, n, C);
  return hipGetLastError();
}

hipError_t launch_quad(const QuadParams& p, int dtype, hipStream_t st) {
  return dtype == 1 ? launch_quad_e<__bf16>(p, st) : launch_quad_e<float>(p, st);
}

}  // namespace hna
