// Neuron step of the layout search of "Affinity-Aware Sharding for Delayed
// Tensor Parallelism", section 3, paragraph "Optimiser" (iteration count and
// step decay from appendix A).  Given the KV-group devices h_i and h_{i+1},
// layer i's neurons go to devices by a balanced linear assignment on the gain
//   M[k, l] = sum_{g: h_i(g) = l} S_up_i[g, k] + sum_{g: h_{i+1}(g) = l} S_down_i[k, g]
// solved by dual ascent on L device offsets, a capacity fix-up and pairwise
// swaps.
//
// One 1024-thread workgroup per layer (the layers are independent given the
// head devices); neuron k = j * 1024 + thread.  M lives in LDS as fp64
// [L][I].  Every decision compares fp64 values produced by the same
// operations in the same order as the plain definition (contraction is off in
// this file), so the assignment is exactly reproducible:
//   * M sums its up terms in increasing g, then its down terms;
//   * the offsets move by step * (count_l - cap) / cap, the first step being
//     a tenth of max(M) - min(M), decaying by 0.98 per iteration;
//   * the fix-up moves the neuron, from an over-full to an under-full device,
//     that loses least (ties: lowest neuron, then lowest device);
//   * a swap round performs the best swap over device pairs l1 < l2 if it
//     gains (ties: first pair, lowest neurons).
// The head step (given nu_{i-1} and nu_i, the best balanced KV-group map h_i
// by exhaustive scoring of the labelled balanced partitions) is here too.
#include <climits>
#include <cmath>

#include "hna_internal.h"

#pragma clang fp contract(off)

namespace hna {
namespace {

constexpr int kLThreads = 1024;
constexpr int kLWaves = kLThreads / 64;
constexpr int kMaxPairs = kLayoutMaxDevices * (kLayoutMaxDevices - 1);

constexpr double kStepFrac = 0.1;
constexpr double kStepDecay = 0.98;

// (d, i) beats (bd, bi): larger d, then smaller i
__device__ inline bool better(double d, int i, double bd, int bi) {
  return d > bd || (d == bd && i < bi);
}

// value of lane l (uniform l) in every lane
__device__ inline double readlane_f64(double v, int l) {
  const unsigned long long u = __double_as_longlong(v);
  const unsigned lo = __builtin_amdgcn_readlane((unsigned)u, l);
  const unsigned hi = __builtin_amdgcn_readlane((unsigned)(u >> 32), l);
  return __longlong_as_double(((unsigned long long)hi << 32) | lo);
}

__device__ inline void wave_best(double& d, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const double od = __shfl_xor(d, o);
    const int oi = __shfl_xor(i, o);
    if (better(od, oi, d, i)) {
      d = od;
      i = oi;
    }
  }
}

// NPT_MAX neurons per thread and LMAX devices at most.  CACHE keeps the
// thread's gains in registers as well, for the argmax of the dual ascent; the
// thread then owns exactly NPT_MAX neuron slots, and the devices L..LMAX-1
// take an offset of +inf so that they never win the argmax.
template <int NPT_MAX, int LMAX, bool CACHE>
__global__ __launch_bounds__(kLThreads) void neuron_step_kernel(NeuronStepParams p) {
  extern __shared__ double Ms[];  // [L][I]
  __shared__ int hs[kMaxHeads], hn[kMaxHeads];
  __shared__ int cnt_w[2][kLWaves][LMAX];  // per-wave device counts, two buffers in turn
  __shared__ double red_d[2][kLWaves][kMaxPairs];
  __shared__ int red_i[2][kLWaves][kMaxPairs];
  __shared__ double mm[2][kLWaves];
  __shared__ int bad;

  const int layer = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int G = p.G, I = p.I, L = p.L, cap = I / L;
  const bool has_down = layer + 1 < p.N;
  const int npt = CACHE ? NPT_MAX : (I + kLThreads - 1) / kLThreads;
  int32_t* out = p.neurons + (int64_t)layer * I;
  int32_t* st = p.stats + (int64_t)layer * 4;

  // ---- head devices of this layer and the next; ids outside [0, L) fail the layer
  if (t == 0) bad = 0;
  __syncthreads();
  if (t < G) {
    const int a = p.heads[(int64_t)layer * G + t];
    hs[t] = a;
    if (a < 0 || a >= L) bad = 1;
    if (has_down) {
      const int b = p.heads[(int64_t)(layer + 1) * G + t];
      hn[t] = b;
      if (b < 0 || b >= L) bad = 1;
    }
  }
  __syncthreads();
  if (bad) {
    for (int k = t; k < I; k += kLThreads) out[k] = -1;
    if (t == 0) {
      st[0] = kLayoutBadHeads;
      st[1] = st[2] = st[3] = 0;
    }
    return;
  }

  // ---- gain M and its range
  const float* Su = p.S_up + (int64_t)layer * G * I;
  const float* Sd = has_down ? p.S_down + (int64_t)layer * I * G : nullptr;
  double mx = -INFINITY, mn = INFINITY;
  for (int j = 0; j < npt; ++j) {
    const int k = j * kLThreads + t;
    if (k >= I) break;
    double acc[LMAX];
#pragma unroll
    for (int l = 0; l < LMAX; ++l) acc[l] = 0.0;
    for (int g = 0; g < G; ++g) {
      const double v = (double)Su[(int64_t)g * I + k];
      const int dv = hs[g];
#pragma unroll
      for (int l = 0; l < LMAX; ++l)
        if (l == dv) acc[l] += v;
    }
    if (has_down) {
      for (int g = 0; g < G; ++g) {
        const double v = (double)Sd[(int64_t)k * G + g];
        const int dv = hn[g];
#pragma unroll
        for (int l = 0; l < LMAX; ++l)
          if (l == dv) acc[l] += v;
      }
    }
#pragma unroll
    for (int l = 0; l < LMAX; ++l) {
      if (l < L) {
        Ms[l * I + k] = acc[l];
        mx = fmax(mx, acc[l]);
        mn = fmin(mn, acc[l]);
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    mx = fmax(mx, __shfl_xor(mx, o));
    mn = fmin(mn, __shfl_xor(mn, o));
  }
  if (lane == 0) {
    mm[0][w] = mx;
    mm[1][w] = mn;
  }
  // The dual step's quotient (c - cap) / cap takes only the values c = 0..I:
  // when LDS allows, they are divided once here and looked up in the loop
  // (the same fp64 division, so the same values)
  double* qtab = Ms + (size_t)L * I;
  if (p.qtab)
    for (int c = t; c <= I; c += kLThreads) qtab[c] = (double)(c - cap) / (double)cap;
  __syncthreads();  // also publishes Ms and the quotients
  mx = mm[0][0];
  mn = mm[1][0];
  for (int i = 1; i < kLWaves; ++i) {
    mx = fmax(mx, mm[0][i]);
    mn = fmin(mn, mm[1][i]);
  }

  // ---- per-thread assignment (-1 past the last neuron)
  int a[NPT_MAX];
  double lam[LMAX];
#pragma unroll
  for (int l = 0; l < LMAX; ++l) lam[l] = l < L ? 0.0 : INFINITY;
  int buf = 0;
  double mr[CACHE ? NPT_MAX : 1][CACHE ? LMAX : 1];
  if constexpr (CACHE) {
#pragma unroll
    for (int j = 0; j < NPT_MAX; ++j)
#pragma unroll
      for (int l = 0; l < LMAX; ++l) {
        const int k = j * kLThreads + t;
        mr[j][l] = (j < npt && l < L && k < I) ? Ms[l * I + k] : 0.0;
      }
  }
  auto gain_of = [&](int j, int l, int k) -> double {
    if constexpr (CACHE) return mr[j][l];
    else return Ms[l * I + k];
  };

  auto assign_argmax = [&]() {
    if constexpr (CACHE) {
      // straight-line: every slot and device is evaluated, padding never wins
#pragma unroll
      for (int j = 0; j < NPT_MAX; ++j) {
        double best = mr[j][0] - lam[0];
        int bl = 0;
#pragma unroll
        for (int l = 1; l < LMAX; ++l) {
          const double v = mr[j][l] - lam[l];
          if (v > best) {
            best = v;
            bl = l;
          }
        }
        a[j] = j * kLThreads + t < I ? bl : -1;
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < NPT_MAX; ++j) {
      if (j < npt) {
        const int k = j * kLThreads + t;
        int bl = -1;
        if (k < I) {
          double best = gain_of(j, 0, k) - lam[0];
          bl = 0;
#pragma unroll
          for (int l = 1; l < LMAX; ++l) {
            if (l < L) {
              const double v = gain_of(j, l, k) - lam[l];
              if (v > best) {
                best = v;
                bl = l;
              }
            }
          }
        }
        a[j] = bl;
      }
    }
  };
  // Device counts: each wave writes its ballot counts of the L devices into
  // its own slot of cnt_w[rot] (every slot is rewritten, so nothing is
  // cleared), one barrier, then each reader adds the waves' slots in wave
  // order (integers: exact).  Two buffers alternate: a wave writes a buffer
  // again only after passing the next barrier, which every reader of that
  // buffer reaches after its reads.
  int cnt[LMAX];
  int rot = 0;
  // returns the count of device `lane` (cap in lanes >= L); fills cnt[] if asked
  auto count = [&](bool all) -> int {
#pragma unroll
    for (int l = 0; l < LMAX; ++l) {
      if (CACHE || l < L) {   // (padding devices count zero and are never read)
        int c = 0;
#pragma unroll
        for (int j = 0; j < NPT_MAX; ++j)
          if (j < npt) c += __popcll(__ballot(a[j] == l));
        if (lane == 0) cnt_w[rot][w][l] = c;
      }
    }
    __syncthreads();
    int mine = cap;
    if (lane < L) {
      mine = 0;
#pragma unroll
      for (int v = 0; v < kLWaves; ++v) mine += cnt_w[rot][v][lane];
    }
    if (all) {
#pragma unroll
      for (int l = 0; l < LMAX; ++l) {
        int c = 0;
        if (l < L)
#pragma unroll
          for (int v = 0; v < kLWaves; ++v) c += cnt_w[rot][v][l];
        cnt[l] = c;
      }
    }
    rot ^= 1;
    return mine;
  };

  // ---- 1. dual ascent on the device offsets.  Lane l of every wave updates
  // offset l (lanes >= L add an exact zero), then the offsets are broadcast.
  double step = kStepFrac * (mx - mn);
  double lam_lane = 0.0;
  for (int it = 0; it < p.iters; ++it) {
    assign_argmax();
    const int c = count(false);
    const double q = p.qtab ? qtab[c] : (double)(c - cap) / (double)cap;   // 0 <= c <= I
    lam_lane = lam_lane + step * q;
#pragma unroll
    for (int l = 0; l < LMAX; ++l) lam[l] = l < L ? readlane_f64(lam_lane, l) : INFINITY;
    step = step * kStepDecay;
  }
  assign_argmax();
  count(true);
  int excess = 0;
#pragma unroll
  for (int l = 0; l < LMAX; ++l)
    if (l < L && cnt[l] > cap) excess += cnt[l] - cap;

  // ---- 2. capacity fix-up: one least-loss move per round
  int moves = 0, status = kLayoutOk;
  for (;;) {
    int over = 0, under = 0;
#pragma unroll
    for (int l = 0; l < LMAX; ++l) {
      if (l < L && cnt[l] > cap) over |= 1 << l;
      if (l < L && cnt[l] < cap) under |= 1 << l;
    }
    if (!over) break;
    double bd = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int j = 0; j < NPT_MAX; ++j) {
      if (j < npt && a[j] >= 0 && ((over >> a[j]) & 1)) {
        const int k = j * kLThreads + t;
        const double own = Ms[a[j] * I + k];
        for (int l = 0; l < L; ++l) {
          if ((under >> l) & 1) {
            const double d = Ms[l * I + k] - own;
            const int idx = ((k * L + l) << 4) | a[j];   // order: k, then l
            if (better(d, idx, bd, bi)) {
              bd = d;
              bi = idx;
            }
          }
        }
      }
    }
    wave_best(bd, bi);
    if (lane == 0) {
      red_d[buf][w][0] = bd;
      red_i[buf][w][0] = bi;
    }
    __syncthreads();
    bd = red_d[buf][0][0];
    bi = red_i[buf][0][0];
    for (int i = 1; i < kLWaves; ++i)
      if (better(red_d[buf][i][0], red_i[buf][i][0], bd, bi)) {
        bd = red_d[buf][i][0];
        bi = red_i[buf][i][0];
      }
    buf ^= 1;
    if (bi == INT_MAX) {  // no comparable candidate (non-finite gains)
      status = kLayoutNoMove;
      break;
    }
    const int src = bi & 15, kl = bi >> 4, k = kl / L, dst = kl - k * L;
#pragma unroll
    for (int j = 0; j < NPT_MAX; ++j)
      if (j < npt && j * kLThreads + t == k) a[j] = dst;
#pragma unroll
    for (int l = 0; l < LMAX; ++l) {
      if (l == src) --cnt[l];
      if (l == dst) ++cnt[l];
    }
    ++moves;
  }

  // ---- 3. pairwise swaps: best swap per round while it gains
  int swaps = 0;
  bool hit = status == kLayoutOk;
  while (status == kLayoutOk && swaps < p.max_swaps) {
    // best one-way move of every ordered pair (l1 -> l2), per wave
    int q = 0;
    for (int l1 = 0; l1 < L; ++l1) {
      for (int l2 = 0; l2 < L; ++l2) {
        if (l2 == l1) continue;
        double bd = -INFINITY;
        int bk = INT_MAX;
#pragma unroll
        for (int j = 0; j < NPT_MAX; ++j) {
          if (j < npt && a[j] == l1) {
            const int k = j * kLThreads + t;
            const double d = Ms[l2 * I + k] - Ms[l1 * I + k];
            if (better(d, k, bd, bk)) {
              bd = d;
              bk = k;
            }
          }
        }
        wave_best(bd, bk);
        if (lane == 0) {
          red_d[buf][w][q] = bd;
          red_i[buf][w][q] = bk;
        }
        ++q;
      }
    }
    __syncthreads();
    double best_gain = 0.0;
    int k1 = -1, k2 = -1, d1v = 0, d2v = 0;
    for (int l1 = 0; l1 < L; ++l1) {
      for (int l2 = l1 + 1; l2 < L; ++l2) {
        const int q12 = l1 * (L - 1) + (l2 - 1);      // l1 -> l2 (l2 > l1)
        const int q21 = l2 * (L - 1) + l1;            // l2 -> l1 (l1 < l2)
        double e1 = red_d[buf][0][q12], e2 = red_d[buf][0][q21];
        int i1 = red_i[buf][0][q12], i2 = red_i[buf][0][q21];
        for (int i = 1; i < kLWaves; ++i) {
          if (better(red_d[buf][i][q12], red_i[buf][i][q12], e1, i1)) {
            e1 = red_d[buf][i][q12];
            i1 = red_i[buf][i][q12];
          }
          if (better(red_d[buf][i][q21], red_i[buf][i][q21], e2, i2)) {
            e2 = red_d[buf][i][q21];
            i2 = red_i[buf][i][q21];
          }
        }
        if (i1 == INT_MAX || i2 == INT_MAX) continue;   // a device with no neuron
        const double gain = e1 + e2;
        if (gain > best_gain) {
          best_gain = gain;
          k1 = i1;
          k2 = i2;
          d1v = l2;
          d2v = l1;
        }
      }
    }
    buf ^= 1;
    if (k1 < 0) {
      hit = false;
      break;
    }
#pragma unroll
    for (int j = 0; j < NPT_MAX; ++j) {
      if (j < npt) {
        const int k = j * kLThreads + t;
        if (k == k1) a[j] = d1v;
        else if (k == k2) a[j] = d2v;
      }
    }
    ++swaps;
  }
  if (status == kLayoutOk && hit) status = kLayoutSwapLimit;

#pragma unroll
  for (int j = 0; j < NPT_MAX; ++j) {
    if (j < npt) {
      const int k = j * kLThreads + t;
      if (k < I) out[k] = a[j];
    }
  }
  if (t == 0) {
    st[0] = status;
    st[1] = excess;
    st[2] = moves;
    st[3] = swaps;
  }
}

// ---------------------------------------------------------------- head step
// Exact quotient x / n for x a multiple of n, 1 <= n <= 16, in 32-bit
// integers: the power of two of n is shifted out and the odd part's inverse
// mod 2^32 multiplies (Newton-Hensel iteration x <- x (2 - o x), which doubles
// the correct low bits from 3 to 48 in four steps)
struct ExactDiv {
  uint32_t tz, inv;
};
__device__ inline ExactDiv exact_div_by(uint32_t n) {
  const uint32_t tz = (uint32_t)__builtin_ctz(n), o = n >> tz;
  uint32_t x = o;
#pragma unroll
  for (int i = 0; i < 4; ++i) x *= 2u - o * x;
  return {tz, x};
}
__device__ inline uint32_t exact_div(uint32_t x, ExactDiv d) { return (x >> d.tz) * d.inv; }

// One 1024-thread workgroup per layer.  A[g][l] (fp64, LDS): each group is
// summed by 16/G waves (one for G > 8); each lane adds its strided neurons, up
// terms then down terms, a fixed butterfly combines the lanes and the waves'
// parts are added in order.  Every balanced
// partition is then scored by unranking its lexicographic rank (multiset
// permutations of G/L copies of each device), the score being
// sum_g A[g][h(g)] in increasing g; the best (ties: lowest rank) wins.
// LMAX: a compile-time bound on L (4 for the usual shapes, else 8), so the
// unrolled per-device steps carry no dead devices
template <int LMAX>
__global__ __launch_bounds__(kLThreads) void head_step_kernel(HeadStepParams p) {
  __shared__ double A[kHeadMaxGroups * kLayoutMaxDevices];
  __shared__ double Apart[kLWaves * kLayoutMaxDevices];   // per-wave partial sums
  __shared__ double red_d[kLWaves];
  __shared__ int red_i[kLWaves];
  __shared__ int bad;

  const int layer = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int G = p.G, I = p.I, L = p.L;
  const bool has_prev = layer > 0;
  const int32_t* nu = p.neurons + (int64_t)layer * I;
  const int32_t* nu_prev = has_prev ? p.neurons + (int64_t)(layer - 1) * I : nullptr;

  if (t == 0) bad = 0;
  __syncthreads();
  for (int k = t; k < I; k += kLThreads) {
    const int a = nu[k];
    if (a < 0 || a >= L) bad = 1;
    if (has_prev) {
      const int b = nu_prev[k];
      if (b < 0 || b >= L) bad = 1;
    }
  }
  __syncthreads();
  if (bad) {
    if (t < G) p.heads[(int64_t)layer * G + t] = -1;
    if (t == 0) {
      p.status[layer] = kLayoutBadNeurons;
      p.score[layer] = 0.0;
    }
    return;
  }

  // A[g][l]: the waves split into 16/G parts per group (1 for G > 8); part q
  // of group g takes the neurons q*64 + lane, stepping by parts*64; the parts
  // are then added in order
  const float* Su = p.S_up + (int64_t)layer * G * I;
  const float* Sd = has_prev ? p.S_down + (int64_t)(layer - 1) * I * G : nullptr;
  const int parts = G <= kLWaves / 2 ? kLWaves / G : 1;
  for (int wg = w; wg < G * parts; wg += kLWaves) {
    const int g = wg / parts, q = wg - g * parts;
    double acc[LMAX];
#pragma unroll
    for (int l = 0; l < LMAX; ++l) acc[l] = 0.0;
#pragma unroll 4
    for (int k = q * 64 + lane; k < I; k += parts * 64) {
      const double v = (double)Su[(int64_t)g * I + k];
      const int dv = nu[k];
#pragma unroll
      for (int l = 0; l < LMAX; ++l)
        if (l == dv) acc[l] += v;
    }
    if (has_prev) {
#pragma unroll 4
      for (int k = q * 64 + lane; k < I; k += parts * 64) {
        const double v = (double)Sd[(int64_t)k * G + g];
        const int dv = nu_prev[k];
#pragma unroll
        for (int l = 0; l < LMAX; ++l)
          if (l == dv) acc[l] += v;
      }
    }
#pragma unroll
    for (int l = 0; l < LMAX; ++l) {
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) acc[l] += __shfl_xor(acc[l], o);
      if (lane == 0 && l < L) Apart[(g * parts + q) * L + l] = acc[l];
    }
  }
  __syncthreads();
  if (t < G * L) {
    const int g = t / L, l = t - g * L;
    double a = Apart[(g * parts) * L + l];
    for (int q = 1; q < parts; ++q) a += Apart[(g * parts + q) * L + l];
    A[g * L + l] = a;
  }
  __syncthreads();

  // score the partitions r = t, t + 1024, ...  (ranks fit in an int: at most 2^24)
  const int per = G / L;
  const uint32_t total = (uint32_t)p.n_parts;
  double bd = -INFINITY;
  int bi = INT_MAX;
  for (int r0 = t; r0 < p.n_parts; r0 += kLThreads) {
    int c[LMAX];
#pragma unroll
    for (int l = 0; l < LMAX; ++l) c[l] = l < L ? per : 0;
    uint32_t r = (uint32_t)r0, mc = total;
    double score = 0.0;
    for (int q = 0; q < G; ++q) {
      const ExactDiv dn = exact_div_by((uint32_t)(G - q));
      bool done = false;
#pragma unroll
      for (int v = 0; v < LMAX; ++v) {
        if (!done && c[v] > 0) {
          // completions with device v at position q: mc * c_v / n, an exact
          // integer (mc * c_v < 2^24 * 16 fits 32 bits)
          const uint32_t sub = exact_div(mc * (uint32_t)c[v], dn);
          if (r < sub) {
            score += A[q * L + v];
            mc = sub;
            --c[v];
            done = true;
          } else {
            r -= sub;
          }
        }
      }
    }
    if (better(score, r0, bd, bi)) {
      bd = score;
      bi = r0;
    }
  }
  wave_best(bd, bi);
  if (lane == 0) {
    red_d[w] = bd;
    red_i[w] = bi;
  }
  __syncthreads();
  if (t == 0) {
    for (int i = 1; i < kLWaves; ++i)
      if (better(red_d[i], red_i[i], bd, bi)) {
        bd = red_d[i];
        bi = red_i[i];
      }
    // unrank the winner into the head devices
    int c[LMAX];
#pragma unroll
    for (int l = 0; l < LMAX; ++l) c[l] = l < L ? per : 0;
    uint32_t r = (uint32_t)bi, mc = total;
    for (int q = 0; q < G; ++q) {
      const ExactDiv dn = exact_div_by((uint32_t)(G - q));
      bool done = false;
#pragma unroll
      for (int v = 0; v < LMAX; ++v) {
        if (!done && c[v] > 0) {
          const uint32_t sub = exact_div(mc * (uint32_t)c[v], dn);
          if (r < sub) {
            p.heads[(int64_t)layer * G + q] = v;
            mc = sub;
            --c[v];
            done = true;
          } else {
            r -= sub;
          }
        }
      }
    }
    p.score[layer] = bd;
    p.status[layer] = kLayoutOk;
  }
}

}  // namespace

hipError_t launch_head_step(const HeadStepParams& p, hipStream_t st) {
  if (p.L <= 4)
    hipLaunchKernelGGL(head_step_kernel<4>, dim3(p.N), dim3(kLThreads), 0, st, p);
  else
    hipLaunchKernelGGL(head_step_kernel<kLayoutMaxDevices>, dim3(p.N), dim3(kLThreads), 0, st, p);
  return hipGetLastError();
}

size_t neuron_step_lds_bytes(int I, int L) { return (size_t)I * L * sizeof(double); }

constexpr size_t kLdsPerWorkgroup = 160 * 1024;   // gfx950

template <int NPT_MAX, int LMAX, bool CACHE>
static hipError_t launch_ns(const NeuronStepParams& p0, hipStream_t st) {
  auto fn = neuron_step_kernel<NPT_MAX, LMAX, CACHE>;
  hipFuncAttributes attr;
  hipError_t e = hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(fn));
  if (e != hipSuccess) return e;
  // M, plus the quotient table when static + dynamic LDS still fit
  NeuronStepParams p = p0;
  size_t lds = neuron_step_lds_bytes(p.I, p.L);
  const size_t tab = (size_t)(p.I + 1) * sizeof(double);
  p.qtab = attr.sharedSizeBytes + lds + tab <= kLdsPerWorkgroup;
  if (p.qtab) lds += tab;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(p.N), dim3(kLThreads), lds, st, p);
  return hipGetLastError();
}

hipError_t launch_neuron_step(const NeuronStepParams& p, hipStream_t st) {
  const int npt = (p.I + kLThreads - 1) / kLThreads;
  if (p.L <= 4) {
    switch (npt) {
      case 1: return launch_ns<1, 4, true>(p, st);
      case 2: return launch_ns<2, 4, true>(p, st);
      case 3: return launch_ns<3, 4, true>(p, st);
      case 4: return launch_ns<4, 4, true>(p, st);
      default: break;
    }
  }
  return launch_ns<kLayoutMaxNpt, kLayoutMaxDevices, false>(p, st);
}

}  // namespace hna
