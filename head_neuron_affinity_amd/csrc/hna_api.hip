// C ABI of libhna: argument validation, workspace sizing and kernel dispatch.
// Every check runs on the host before anything is enqueued; failures return a
// negative status and leave a thread-local message (see include/hna.h).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <climits>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/hna.h"
#include "hna_internal.h"

using namespace hna;

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(HNA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool debug_sync() {
  static const bool on = [] {
    const char* v = std::getenv("HNA_DEBUG_SYNC");
    return v && v[0] == '1';
  }();
  return on;
}

int finish(hipError_t e, hipStream_t st, const char* where) {
  if (e != hipSuccess) return hip_fail(e, where);
  if (debug_sync()) {
    e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_fail(e, where);
  }
  g_last_error.clear();
  return HNA_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int esize_of(int dtype) { return dtype == HNA_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE_PTR(p)                                                               \
  do {                                                                               \
    if (!(p)) return fail(HNA_ERR_INVALID_ARG, "%s: %s is NULL", fn, #p);            \
    if (!aligned16(p)) return fail(HNA_ERR_ALIGNMENT, "%s: %s is not 16-byte aligned", fn, #p); \
  } while (0)

int check_dtype(const char* fn, int dtype) {
  if (dtype != HNA_F32 && dtype != HNA_BF16)
    return fail(HNA_ERR_INVALID_ARG, "%s: unknown dtype %d", fn, dtype);
  return HNA_OK;
}

int check_heads(const char* fn, int hidden, int H, int G, int d) {
  if (hidden < 1 || H < 1 || G < 1 || d < 1)
    return fail(HNA_ERR_INVALID_ARG, "%s: dimensions must be positive (hidden=%d H=%d G=%d d=%d)",
                fn, hidden, H, G, d);
  if (H % G != 0)
    return fail(HNA_ERR_INVALID_ARG, "%s: H=%d is not a multiple of G=%d", fn, H, G);
  if (H > kMaxHeads) return fail(HNA_ERR_UNSUPPORTED, "%s: H=%d > %d", fn, H, kMaxHeads);
  if (d % 16 != 0 || d > 128)
    return fail(HNA_ERR_UNSUPPORTED, "%s: head dim d=%d must be a multiple of 16 and <= 128", fn, d);
  if (hidden % 8 != 0)
    return fail(HNA_ERR_UNSUPPORTED, "%s: hidden=%d must be a multiple of 8", fn, hidden);
  return HNA_OK;
}

int check_dims(const char* fn, const hna_dims* dm) {
  if (!dm) return fail(HNA_ERR_INVALID_ARG, "%s: dims is NULL", fn);
  int rc = check_dtype(fn, dm->dtype);
  if (rc) return rc;
  if (dm->T < 0) return fail(HNA_ERR_INVALID_ARG, "%s: T=%lld < 0", fn, (long long)dm->T);
  if (dm->I < 1) return fail(HNA_ERR_INVALID_ARG, "%s: I=%d < 1", fn, dm->I);
  // Token counts are held in 32-bit tile counts by the kernels' geometry.
  if (dm->T > (int64_t)INT32_MAX)
    return fail(HNA_ERR_UNSUPPORTED, "%s: T=%lld > 2^31 - 1", fn, (long long)dm->T);
  if (dm->I > (1 << 22)) return fail(HNA_ERR_UNSUPPORTED, "%s: I=%d > 2^22", fn, dm->I);
  rc = check_heads(fn, dm->hidden, dm->H, dm->G, dm->d);
  if (rc) return rc;
  // the hot kernel's grid (computed in 64 bits): at most 2^24 workgroups, so
  // that its 256-thread workgroups stay within 2^32 threads
  const int64_t n_tt = (dm->T + kTileTokens - 1) / kTileTokens;
  const int64_t n_chunks = (n_tt + kTilesPerChunk - 1) / kTilesPerChunk;
  const int64_t n_cg = (n_chunks + kSuperChunks - 1) / kSuperChunks;
  const int64_t n_kt = ((int64_t)round_up(dm->I, 32) + kTileNeurons - 1) / kTileNeurons;
  const int64_t n_ktg = (n_kt + kSuperKt - 1) / kSuperKt;
  const int64_t grid = (n_ktg * n_cg + 7) / 8 * 8 * 32;
  if (grid > ((int64_t)1 << 24))
    return fail(HNA_ERR_UNSUPPORTED, "%s: T=%lld with I=%d needs %lld workgroups > 2^24", fn,
                (long long)dm->T, dm->I, (long long)grid);
  return HNA_OK;
}

int check_map(const char* fn, const int32_t* map, int H, int G) {
  if (!map) return fail(HNA_ERR_INVALID_ARG, "%s: group map is NULL", fn);
  for (int h = 0; h < H; ++h)
    if (map[h] < 0 || map[h] >= G)
      return fail(HNA_ERR_INVALID_ARG, "%s: group_of_head[%d]=%d outside [0, %d)", fn, h, map[h], G);
  return HNA_OK;
}

size_t fold_ws_bytes(const hna_dims* dm) {
  return align256((size_t)dm->H * dm->d * dm->hidden * esize_of(dm->dtype));
}

size_t up_ws_bytes(const hna_dims* dm) {
  return up_geometry(dm->T, dm->H, dm->G, dm->d, dm->I, dm->dtype).ws_bytes;
}

size_t down_ws_transposed(const hna_down_dims* dm) {
  return align256((size_t)dm->I * dm->hidden * esize_of(dm->dtype));
}
size_t down_ws_bytes(const hna_down_dims* dm) {
  return down_ws_transposed(dm) + align256((size_t)(dm->H + 2 * dm->G) * dm->I * sizeof(float));
}

}  // namespace

extern "C" {

int hna_abi_version(void) { return HNA_ABI_VERSION; }

const char* hna_status_string(int status) {
  switch (status) {
    case HNA_OK: return "HNA_OK";
    case HNA_ERR_INVALID_ARG: return "HNA_ERR_INVALID_ARG";
    case HNA_ERR_UNSUPPORTED: return "HNA_ERR_UNSUPPORTED";
    case HNA_ERR_ALIGNMENT: return "HNA_ERR_ALIGNMENT";
    case HNA_ERR_WORKSPACE: return "HNA_ERR_WORKSPACE";
    case HNA_ERR_HIP: return "HNA_ERR_HIP";
    default: return "HNA_ERR_UNKNOWN";
  }
}

const char* hna_last_error(void) { return g_last_error.c_str(); }

size_t hna_folded_bytes(const hna_dims* dm) {
  if (check_dims("hna_folded_bytes", dm)) return 0;
  return (size_t)dm->H * dm->d * 2 * round_up(dm->I, 32) * esize_of(dm->dtype);
}

size_t hna_fold_workspace_bytes(const hna_dims* dm) {
  if (check_dims("hna_fold_workspace_bytes", dm)) return 0;
  return fold_ws_bytes(dm);
}

int hna_fold_up_weights(const hna_dims* dm, const void* W_o, const float* gamma,
                        const void* W_gate, const void* W_up, void* M, size_t M_bytes,
                        void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "hna_fold_up_weights";
  int rc = check_dims(fn, dm);
  if (rc) return rc;
  REQUIRE_PTR(W_o);
  REQUIRE_PTR(gamma);
  REQUIRE_PTR(W_gate);
  REQUIRE_PTR(W_up);
  REQUIRE_PTR(M);
  REQUIRE_PTR(workspace);
  const size_t need_m = hna_folded_bytes(dm);
  if (M_bytes < need_m)
    return fail(HNA_ERR_WORKSPACE, "%s: M has %zu bytes, needs %zu", fn, M_bytes, need_m);
  const size_t need_ws = fold_ws_bytes(dm);
  if (workspace_bytes < need_ws)
    return fail(HNA_ERR_WORKSPACE, "%s: workspace has %zu bytes, needs %zu", fn, workspace_bytes, need_ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int Hd = dm->H * dm->d;
  hipError_t e = launch_scale_transpose(W_o, gamma, workspace, dm->hidden, Hd, dm->hidden,
                                        dm->dtype, st);
  if (e != hipSuccess) return hip_fail(e, fn);
  GemmParams p{};
  p.X = workspace;
  p.Y[0] = W_gate;
  p.Y[1] = W_up;
  p.ldx = dm->hidden;
  p.ldy = dm->hidden;
  p.Mrows = Hd;
  p.N = round_up(dm->I, 32);
  p.Nvalid = dm->I;
  p.K = dm->hidden;
  p.M = M;
  p.d = dm->d;
  p.KB = p.N / 32;
  p.S = dm->d / 16;
  e = dm->dtype == HNA_BF16 ? launch_mm_bf16(p, kEpiFold, 2, st) : launch_gemm_f32(p, kEpiFold, 2, st);
  return finish(e, st, fn);
}

int hna_down_col_sqnorm(const hna_dims* dm, const void* W_down, float* wd_sq, void* stream) {
  const char* fn = "hna_down_col_sqnorm";
  int rc = check_dims(fn, dm);
  if (rc) return rc;
  REQUIRE_PTR(W_down);
  REQUIRE_PTR(wd_sq);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return finish(launch_col_sqnorm(W_down, dm->hidden, dm->I, dm->dtype, wd_sq, st), st, fn);
}

size_t hna_up_workspace_bytes(const hna_dims* dm) {
  if (check_dims("hna_up_workspace_bytes", dm)) return 0;
  return up_ws_bytes(dm);
}

int hna_affinity_up(const hna_dims* dm, const void* a, const void* g, const void* u,
                    const float* r, const float* r_next, const void* M,
                    const int32_t* group_of_head, void* workspace, size_t workspace_bytes,
                    void* stream) {
  const char* fn = "hna_affinity_up";
  int rc = check_dims(fn, dm);
  if (rc) return rc;
  rc = check_map(fn, group_of_head, dm->H, dm->G);
  if (rc) return rc;
  REQUIRE_PTR(M);
  const UpGeometry geo = up_geometry(dm->T, dm->H, dm->G, dm->d, dm->I, dm->dtype);
  if (geo.lds_bytes > (size_t)kLdsBytes)
    return fail(HNA_ERR_UNSUPPORTED, "%s: needs %zu bytes of LDS (G=%d, d=%d, dtype %d) > %d",
                fn, geo.lds_bytes, dm->G, dm->d, dm->dtype, kLdsBytes);
  if (dm->T == 0) {
    g_last_error.clear();
    return HNA_OK;
  }
  REQUIRE_PTR(a);
  REQUIRE_PTR(g);
  REQUIRE_PTR(u);
  REQUIRE_PTR(r);
  if (r_next && !aligned16(r_next))
    return fail(HNA_ERR_ALIGNMENT, "%s: r_next is not 16-byte aligned", fn);
  REQUIRE_PTR(workspace);
  const size_t need = up_ws_bytes(dm);
  if (workspace_bytes < need)
    return fail(HNA_ERR_WORKSPACE, "%s: workspace has %zu bytes, needs %zu", fn, workspace_bytes, need);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  UpParams p{};
  p.a = a;
  p.g = g;
  p.u = u;
  p.r = r;
  p.r_next = r_next ? r_next : r;
  p.want_c = r_next ? 1 : 0;
  p.M = M;
  p.part = reinterpret_cast<float*>(ws);
  p.T = dm->T;
  p.H = dm->H;
  p.G = dm->G;
  p.d = dm->d;
  p.I = dm->I;
  p.I32 = geo.I32;
  p.n_tt = geo.n_tt;
  p.n_kt = geo.n_kt;
  p.n_chunks = geo.n_chunks;
  p.n_ktg = geo.n_ktg;
  p.n_st = geo.n_st;
  int n = 0;
  for (int gg = 0; gg < dm->G; ++gg)
    for (int h = 0; h < dm->H; ++h)
      if (group_of_head[h] == gg) {
        p.head_order[n] = (int8_t)h;
        p.head_group[n] = (int8_t)gg;
        ++n;
      }
  // FO sums and the down-edge moment
  return finish(launch_affinity_up(p, geo, dm->dtype, st), st, fn);
}

int hna_affinity_add(const hna_dims* dm, const void* a, const float* r, const void* M,
                     const int32_t* group_of_head, void* workspace, size_t workspace_bytes,
                     void* stream) {
  const char* fn = "hna_affinity_add";
  int rc = check_dims(fn, dm);
  if (rc) return rc;
  rc = check_map(fn, group_of_head, dm->H, dm->G);
  if (rc) return rc;
  REQUIRE_PTR(M);
  if (dm->T == 0) {
    g_last_error.clear();
    return HNA_OK;
  }
  REQUIRE_PTR(a);
  REQUIRE_PTR(r);
  REQUIRE_PTR(workspace);
  const UpGeometry geo = up_geometry(dm->T, dm->H, dm->G, dm->d, dm->I, dm->dtype);
  if (workspace_bytes < geo.ws_bytes)
    return fail(HNA_ERR_WORKSPACE, "%s: workspace has %zu bytes, needs %zu", fn, workspace_bytes,
                geo.ws_bytes);
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  QuadParams qp{};
  int n = 0;
  for (int gg = 0; gg < dm->G; ++gg) {
    qp.group_start[gg] = (int16_t)n;
    for (int h = 0; h < dm->H; ++h)
      if (group_of_head[h] == gg) qp.head_order[n++] = (int8_t)h;
  }
  qp.group_start[dm->G] = (int16_t)n;
  // C_h = sum_t a_th a_th^T / r_t^2 per head, in token-chunk partial sums
  GramParams gp{};
  gp.a = a;
  gp.r = r;
  gp.part = reinterpret_cast<float*>(ws + geo.off_gram_part);
  gp.T = dm->T;
  gp.H = dm->H;
  gp.d = dm->d;
  gp.n_gc = geo.n_gc;
  gp.chunk_tokens = geo.gram_chunk;
  hipError_t e = launch_gram(gp, dm->dtype, st);
  if (e != hipSuccess) return hip_fail(e, fn);
  void* C = ws + geo.off_gram;   // H d d fp32, or two bf16 planes of H d d
  e = launch_gram_reduce(gp.part, geo.n_gc, (int64_t)dm->H * dm->d * dm->d, C, dm->dtype, st);
  if (e != hipSuccess) return hip_fail(e, fn);
  // ADD[g][k] = sum_{h in g} (m^g_hk . C_h m^g_hk + m^u_hk . C_h m^u_hk)
  qp.C = C;
  qp.M = M;
  qp.add = reinterpret_cast<float*>(ws + geo.off_add);
  qp.add_part = reinterpret_cast<float*>(ws + geo.off_add_part);
  qp.H = dm->H;
  qp.G = dm->G;
  qp.d = dm->d;
  qp.KB = geo.I32 / 32;
  return finish(launch_quad(qp, dm->dtype, st), st, fn);
}

int hna_finalize_up(const hna_dims* dm, const float* wd_sq, float scale, int flags,
                    const void* workspace, size_t workspace_bytes, float* S_fo, float* S_add,
                    float* c_down, void* stream) {
  const char* fn = "hna_finalize_up";
  int rc = check_dims(fn, dm);
  if (rc) return rc;
  if (flags & ~HNA_ACCUMULATE) return fail(HNA_ERR_INVALID_ARG, "%s: unknown flags 0x%x", fn, flags);
  REQUIRE_PTR(wd_sq);
  REQUIRE_PTR(S_fo);
  REQUIRE_PTR(S_add);
  if (c_down && !aligned16(c_down))
    return fail(HNA_ERR_ALIGNMENT, "%s: c_down is not 16-byte aligned", fn);
  const UpGeometry geo = up_geometry(dm->T, dm->H, dm->G, dm->d, dm->I, dm->dtype);
  if (geo.n_chunks > 0) {
    REQUIRE_PTR(workspace);
    const size_t need = up_ws_bytes(dm);
    if (workspace_bytes < need)
      return fail(HNA_ERR_WORKSPACE, "%s: workspace has %zu bytes, needs %zu", fn, workspace_bytes, need);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const char* ws = static_cast<const char*>(workspace);
  return finish(launch_finalize_up(reinterpret_cast<const float*>(ws),
                                   reinterpret_cast<const float*>(ws + geo.off_add), geo.n_chunks,
                                   dm->G, dm->I, geo.I32, wd_sq, scale, flags & HNA_ACCUMULATE,
                                   S_fo, S_add, c_down, st),
                st, fn);
}

// ------------------------------------------------ allocation-free up pass
// Scratch of hna_affinity_up_static: a fixed array in device memory, one copy
// per GPU the library runs on, held until the process ends.  Host code never
// names the array itself (its host-side name is not a device address): the
// address comes from hipGetSymbolAddress once per device and is kept below.
}  // extern "C"

namespace {
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
constexpr int kMaxScratchDevices = 64;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// The current device's copy of `scratch` (looked up on the first call on that
// device, with that device current).
int static_scratch(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, fn);
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(HNA_ERR_UNSUPPORTED, "%s: device %d beyond the %d devices with a scratch copy", fn,
                dev, kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, fn);
    if (!ptr) return fail(HNA_ERR_HIP, "%s: no device address for the scratch array", fn);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return HNA_OK;
}
}  // namespace

extern "C" {

size_t hna_static_scratch_bytes(void) { return kStaticScratchBytes; }

int hna_affinity_up_static(const hna_dims* dm, const void* a, const void* g, const void* u,
                           const float* r, const float* r_next, const void* M, const float* wd_sq,
                           const int32_t* group_of_head, float scale, int flags, float* S_fo,
                           float* S_add, float* c_down, void* stream) {
  const char* fn = "hna_affinity_up_static";
  int rc = check_dims(fn, dm);
  if (rc) return rc;
  rc = check_map(fn, group_of_head, dm->H, dm->G);
  if (rc) return rc;
  if (flags & ~HNA_ACCUMULATE) return fail(HNA_ERR_INVALID_ARG, "%s: unknown flags 0x%x", fn, flags);
  if (!r_next != !c_down)
    return fail(HNA_ERR_INVALID_ARG, "%s: r_next and c_down must both be given or both be NULL", fn);
  const size_t need = up_ws_bytes(dm);
  if (need > kStaticScratchBytes)
    return fail(HNA_ERR_WORKSPACE,
                "%s: T=%lld needs %zu bytes of scratch, more than the fixed %zu: pass fewer "
                "tokens per call (HNA_ACCUMULATE adds the calls up)",
                fn, (long long)dm->T, need, kStaticScratchBytes);
  void* ws = nullptr;
  rc = static_scratch(fn, &ws);
  if (rc) return rc;
  // The same three steps as hna_affinity_up, hna_affinity_add and
  // hna_finalize_up, on the scratch instead of a caller's workspace.  Every
  // region they read is written first in the same call, so nothing needs
  // clearing.
  rc = hna_affinity_up(dm, a, g, u, r, r_next, M, group_of_head, ws, kStaticScratchBytes, stream);
  if (rc) return rc;
  rc = hna_affinity_add(dm, a, r, M, group_of_head, ws, kStaticScratchBytes, stream);
  if (rc) return rc;
  return hna_finalize_up(dm, wd_sq, scale, flags, ws, kStaticScratchBytes, S_fo, S_add, c_down,
                         stream);
}

size_t hna_down_workspace_bytes(const hna_down_dims* dm) {
  if (!dm || check_dtype("hna_down_workspace_bytes", dm->dtype) ||
      check_heads("hna_down_workspace_bytes", dm->hidden, dm->H, dm->G, dm->d) || dm->I < 1)
    return 0;
  return down_ws_bytes(dm);
}

int hna_down_weight_norms(const hna_down_dims* dm, const void* W_q, const void* W_k,
                          const void* W_v, const float* gamma_next, const void* W_down,
                          const int32_t* group_of_head_next, float* n, void* workspace,
                          size_t workspace_bytes, void* stream) {
  const char* fn = "hna_down_weight_norms";
  if (!dm) return fail(HNA_ERR_INVALID_ARG, "%s: dims is NULL", fn);
  int rc = check_dtype(fn, dm->dtype);
  if (rc) return rc;
  rc = check_heads(fn, dm->hidden, dm->H, dm->G, dm->d);
  if (rc) return rc;
  if (dm->I < 1) return fail(HNA_ERR_INVALID_ARG, "%s: I=%d < 1", fn, dm->I);
  rc = check_map(fn, group_of_head_next, dm->H, dm->G);
  if (rc) return rc;
  REQUIRE_PTR(W_q);
  REQUIRE_PTR(W_k);
  REQUIRE_PTR(W_v);
  REQUIRE_PTR(gamma_next);
  REQUIRE_PTR(W_down);
  REQUIRE_PTR(n);
  REQUIRE_PTR(workspace);
  const size_t need = down_ws_bytes(dm);
  if (workspace_bytes < need)
    return fail(HNA_ERR_WORKSPACE, "%s: workspace has %zu bytes, needs %zu", fn, workspace_bytes, need);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = launch_scale_transpose(W_down, gamma_next, workspace, dm->hidden, dm->I,
                                        dm->hidden, dm->dtype, st);
  if (e != hipSuccess) return hip_fail(e, fn);
  float* seg_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + down_ws_transposed(dm));
  GemmParams p{};
  p.X = workspace;
  p.Y[0] = W_q;
  p.Y[1] = W_k;
  p.Y[2] = W_v;
  p.ldx = dm->hidden;
  p.ldy = dm->hidden;
  p.Mrows = dm->I;
  p.N = dm->d;
  p.Nvalid = dm->d;
  p.K = dm->hidden;
  p.seg_part = seg_part;
  p.H_next = dm->H;
  p.G_next = dm->G;
  p.d_next = dm->d;
  const int nseg = dm->H + 2 * dm->G;
  // segments of W_q (one per query head), then of W_k and W_v (one per group)
  e = dm->dtype == HNA_BF16 ? launch_mm_bf16(p, kEpiSegSq, nseg, st)
                            : launch_gemm_f32(p, kEpiSegSq, nseg, st);
  if (e != hipSuccess) return hip_fail(e, fn);
  // segments of group g': its query heads (ascending), then its k rows, then its v rows
  int16_t seg_list[3 * kMaxHeads];
  int16_t start[kMaxHeads + 1];
  int c = 0;
  for (int gg = 0; gg < dm->G; ++gg) {
    start[gg] = (int16_t)c;
    for (int h = 0; h < dm->H; ++h)
      if (group_of_head_next[h] == gg) seg_list[c++] = (int16_t)h;
    seg_list[c++] = (int16_t)(dm->H + gg);
    seg_list[c++] = (int16_t)(dm->H + dm->G + gg);
  }
  start[dm->G] = (int16_t)c;
  return finish(launch_down_group_sum(seg_part, seg_list, start, dm->G, dm->I, n, st), st, fn);
}

int hna_down_combine(int32_t I, int32_t G_next, const float* c_down, const float* n,
                     float* S_down, void* stream) {
  const char* fn = "hna_down_combine";
  if (I < 1 || G_next < 1)
    return fail(HNA_ERR_INVALID_ARG, "%s: I=%d and G_next=%d must be positive", fn, I, G_next);
  REQUIRE_PTR(c_down);
  REQUIRE_PTR(n);
  REQUIRE_PTR(S_down);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return finish(launch_down_combine(c_down, n, I, G_next, S_down, st), st, fn);
}

int hna_unit_mass(const float* S, int64_t count, int32_t n_matrices, float* out, void* stream) {
  const char* fn = "hna_unit_mass";
  if (count < 0 || n_matrices < 0)
    return fail(HNA_ERR_INVALID_ARG, "%s: count=%lld and n_matrices=%d must be >= 0", fn,
                (long long)count, n_matrices);
  if (count == 0 || n_matrices == 0) {
    g_last_error.clear();
    return HNA_OK;
  }
  REQUIRE_PTR(S);
  REQUIRE_PTR(out);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return finish(launch_unit_mass(S, count, n_matrices, out, st), st, fn);
}

int hna_mfma_rate_probe(int32_t n_workgroups, int32_t iters, int32_t shape, const void* seed,
                        float* out, void* stream) {
  const char* fn = "hna_mfma_rate_probe";
  if (shape != 0 && shape != 1)
    return fail(HNA_ERR_INVALID_ARG, "%s: shape=%d is neither 0 (32x32x16) nor 1 (16x16x32)", fn, shape);
  if (n_workgroups < 1 || n_workgroups > 65536)
    return fail(HNA_ERR_INVALID_ARG, "%s: n_workgroups=%d outside [1, 65536]", fn, n_workgroups);
  if (iters < 1 || iters > 1000000)
    return fail(HNA_ERR_INVALID_ARG, "%s: iters=%d outside [1, 1000000]", fn, iters);
  REQUIRE_PTR(seed);
  REQUIRE_PTR(out);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return finish(launch_mfma_rate(seed, n_workgroups, iters, shape, out, st), st, fn);
}

int hna_layout_objective(int32_t N, int32_t G, int32_t I, const float* S_up, const float* S_down,
                         const int32_t* head_device, const int32_t* neuron_device,
                         double* frac_up, double* frac_down, double* J, void* stream) {
  const char* fn = "hna_layout_objective";
  if (N < 1 || G < 1 || I < 1)
    return fail(HNA_ERR_INVALID_ARG, "%s: N=%d, G=%d and I=%d must be positive", fn, N, G, I);
  if (N > max_objective_layers())
    return fail(HNA_ERR_UNSUPPORTED, "%s: N=%d exceeds %d layers", fn, N, max_objective_layers());
  if ((int64_t)G * I > (int64_t)1 << 31)
    return fail(HNA_ERR_UNSUPPORTED, "%s: G*I=%lld exceeds 2^31 entries per matrix", fn,
                (long long)G * I);
  REQUIRE_PTR(S_up);
  REQUIRE_PTR(head_device);
  REQUIRE_PTR(neuron_device);
  REQUIRE_PTR(frac_up);
  REQUIRE_PTR(J);
  if (N > 1) {
    REQUIRE_PTR(S_down);
    REQUIRE_PTR(frac_down);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  return finish(launch_layout_objective(S_up, S_down, head_device, neuron_device, N, G, I,
                                        frac_up, frac_down, J, st),
                st, fn);
}

static_assert(HNA_LAYOUT_OK == kLayoutOk && HNA_LAYOUT_BAD_HEADS == kLayoutBadHeads &&
                  HNA_LAYOUT_SWAP_LIMIT == kLayoutSwapLimit &&
                  HNA_LAYOUT_NO_MOVE == kLayoutNoMove && HNA_LAYOUT_BAD_NEURONS == kLayoutBadNeurons,
              "layout status codes");

int hna_neuron_step(int32_t N, int32_t G, int32_t I, int32_t L, const float* S_up_hat,
                    const float* S_down_hat, const int32_t* head_device, int32_t iters,
                    int32_t max_swaps, int32_t* neuron_device, int32_t* stats, void* stream) {
  const char* fn = "hna_neuron_step";
  if (N < 1 || G < 1 || I < 1 || L < 1)
    return fail(HNA_ERR_INVALID_ARG, "%s: N=%d, G=%d, I=%d and L=%d must be positive", fn, N, G,
                I, L);
  if (G % L || I % L)
    return fail(HNA_ERR_INVALID_ARG, "%s: G=%d and I=%d must be multiples of L=%d", fn, G, I, L);
  if (iters < 0 || max_swaps < 0)
    return fail(HNA_ERR_INVALID_ARG, "%s: iters=%d and max_swaps=%d must be >= 0", fn, iters,
                max_swaps);
  if (L > kLayoutMaxDevices || G > kMaxHeads || I > kLayoutMaxNpt * 1024 ||
      neuron_step_lds_bytes(I, L) > kLayoutMaxLds)
    return fail(HNA_ERR_UNSUPPORTED,
                "%s: L=%d, G=%d, I=%d outside L <= %d, G <= %d, I <= %d, I*L <= %d", fn, L, G, I,
                kLayoutMaxDevices, kMaxHeads, kLayoutMaxNpt * 1024,
                (int)(kLayoutMaxLds / sizeof(double)));
  REQUIRE_PTR(S_up_hat);
  REQUIRE_PTR(head_device);
  REQUIRE_PTR(neuron_device);
  REQUIRE_PTR(stats);
  if (N > 1) REQUIRE_PTR(S_down_hat);
  NeuronStepParams p{S_up_hat, S_down_hat, head_device, neuron_device, stats,
                     N, G, I, L, iters, max_swaps};
  hipStream_t st = static_cast<hipStream_t>(stream);
  return finish(launch_neuron_step(p, st), st, fn);
}

}  // extern "C"

namespace {

struct LooWorkspace {
  size_t xx, xl, xT, WoT, Z, ZAT, U, Q, coef, R, Rs, Y, t1, t1r, gram_part, gram, t3, t3_part,
      total;
  int n_tc;
};
LooWorkspace loo_workspace(const hna_dims* dm) {
  const UpGeometry geo = up_geometry(dm->T, dm->H, dm->G, dm->d, dm->I, dm->dtype);
  const size_t es = esize_of(dm->dtype);
  const size_t HD = (size_t)dm->H * dm->d, D = (size_t)dm->hidden;
  const size_t thd = (size_t)dm->T * HD;
  const size_t tp = (size_t)loo_tokens_padded(dm->T);
  LooWorkspace w;
  w.n_tc = t1_chunks(dm->T);
  size_t o = 0;
  w.xx = o;        o += align256((size_t)dm->T * sizeof(float));
  w.xl = o;        o += dm->dtype == HNA_BF16 ? align256((size_t)dm->T * D * 2) : 0;
  w.xT = o;        o += align256(D * tp * es);      // x^T, padded tokens
  w.WoT = o;       o += align256(HD * D * es);      // W_o^T
  // x W_o (then a scaled, unfused path); with the dot epilogue only the
  // d / 64 fp32 planes of x . o_h
  w.Z = o;
  o += loo_coef_fused(dm->d, dm->dtype) && loo_dot_epilogue(dm->d, dm->dtype)
           ? align256((size_t)(dm->d / 64) * dm->H * dm->T * sizeof(float))
           : align256(thd * es);
  w.ZAT = o;       o += align256(HD * tp * es);     // (alpha beta / r) a, transposed
  w.U = o;         o += loo_coef_fused(dm->d, dm->dtype) ? 0 : align256(thd * es);
  w.Q = o;         o += align256(HD * dm->d * es);
  w.coef = o;      o += align256((size_t)dm->T * dm->H * 2 * sizeof(float));
  w.R = o;         o += align256((size_t)loo_r_parts(dm->T) * HD * D * sizeof(float));
  w.Rs = o;        o += align256(HD * D * es);
  w.Y = o;         o += align256((size_t)2 * HD * dm->I * sizeof(float));
  w.t1 = o;        o += align256((size_t)w.n_tc * dm->H * dm->I * sizeof(float));
  w.t1r = o;       o += align256((size_t)dm->H * dm->I * sizeof(double));
  w.gram_part = o; o += geo.gram_part_bytes;
  w.gram = o;      o += geo.gram_bytes;
  w.t3 = o;        o += geo.add_bytes;
  w.t3_part = o;   o += geo.add_part_bytes;
  w.total = o;
  return w;
}

// G! / ((G/L)!)^L, or -1 above kHeadMaxParts
long long partition_count(int G, int L) {
  // multiply in the multinomial one factor at a time: C(n, per) for each device
  const int per = G / L;
  long long total = 1;
  int n = G;
  for (int l = 0; l < L; ++l) {
    long long c = 1;
    for (int j = 1; j <= per; ++j) c = c * (n - per + j) / j;   // C(n, per), exact at each step
    total *= c;
    if (total > kHeadMaxParts) return -1;
    n -= per;
  }
  return total;
}

int check_layout_dims(const char* fn, int N, int G, int I, int L) {
  if (N < 1 || G < 1 || I < 1 || L < 1)
    return fail(HNA_ERR_INVALID_ARG, "%s: N=%d, G=%d, I=%d and L=%d must be positive", fn, N, G,
                I, L);
  if (G % L || I % L)
    return fail(HNA_ERR_INVALID_ARG, "%s: G=%d and I=%d must be multiples of L=%d", fn, G, I, L);
  return HNA_OK;
}

int check_head_dims(const char* fn, int G, int L) {
  if (L > kLayoutMaxDevices || G > kHeadMaxGroups || partition_count(G, L) < 0)
    return fail(HNA_ERR_UNSUPPORTED,
                "%s: G=%d, L=%d outside L <= %d, G <= %d and at most %d balanced partitions", fn,
                G, L, kLayoutMaxDevices, kHeadMaxGroups, kHeadMaxParts);
  return HNA_OK;
}

// J, the neuron-step stats [N][4] and the head-step statuses [N] sit in one
// block, so that a sweep reads them back with one copy
struct SearchWorkspace {
  size_t heads, neurons, hscore, frac_up, frac_down, report, J, stats, hstatus, report_bytes, total;
};
SearchWorkspace search_workspace(int N, int G, int I) {
  SearchWorkspace w;
  size_t o = 0;
  w.heads = o;     o += align256((size_t)N * G * 4);
  w.neurons = o;   o += align256((size_t)N * I * 4);
  w.hscore = o;    o += align256((size_t)N * 8);
  w.frac_up = o;   o += align256((size_t)N * 8);
  w.frac_down = o; o += align256((size_t)N * 8);
  w.report = o;
  w.J = o;
  w.stats = w.J + 8;
  w.hstatus = w.stats + (size_t)N * 16;
  w.report_bytes = 8 + (size_t)N * 20;
  o += align256(w.report_bytes);
  w.total = o;
  return w;
}

}  // namespace

extern "C" {

int hna_head_step(int32_t N, int32_t G, int32_t I, int32_t L, const float* S_up_hat,
                  const float* S_down_hat, const int32_t* neuron_device, int32_t* head_device,
                  double* score, int32_t* status, void* stream) {
  const char* fn = "hna_head_step";
  int rc = check_layout_dims(fn, N, G, I, L);
  if (rc != HNA_OK) return rc;
  rc = check_head_dims(fn, G, L);
  if (rc != HNA_OK) return rc;
  REQUIRE_PTR(S_up_hat);
  REQUIRE_PTR(neuron_device);
  REQUIRE_PTR(head_device);
  REQUIRE_PTR(score);
  REQUIRE_PTR(status);
  if (N > 1) REQUIRE_PTR(S_down_hat);
  HeadStepParams p{S_up_hat, S_down_hat, neuron_device, head_device, score, status,
                   N, G, I, L, (int)partition_count(G, L)};
  hipStream_t st = static_cast<hipStream_t>(stream);
  return finish(launch_head_step(p, st), st, fn);
}

size_t hna_loo_workspace_bytes(const hna_dims* dm) {
  if (check_dims("hna_loo_workspace_bytes", dm)) return 0;
  return loo_workspace(dm).total;
}

int hna_affinity_loo(const hna_dims* dm, const void* a, const void* g, const void* u,
                     const float* x, const void* W_o, const float* gamma, const void* W_gate,
                     const void* W_up, const void* M, const int32_t* group_of_head, float scale,
                     float* S_loo, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "hna_affinity_loo";
  int rc = check_dims(fn, dm);
  if (rc) return rc;
  rc = check_map(fn, group_of_head, dm->H, dm->G);
  if (rc) return rc;
  // the token GEMM reads 256-row tiles of the transposed operands (rows of
  // T padded tokens) through 32-bit buffer offsets
  constexpr int64_t kLooMaxTokens = 4000000;
  if ((int64_t)dm->T > kLooMaxTokens)
    return fail(HNA_ERR_UNSUPPORTED, "%s: T=%lld exceeds %lld tokens per call", fn,
                (long long)dm->T, (long long)kLooMaxTokens);
  REQUIRE_PTR(M);
  REQUIRE_PTR(S_loo);
  REQUIRE_PTR(workspace);
  const LooWorkspace wl = loo_workspace(dm);
  if (workspace_bytes < wl.total)
    return fail(HNA_ERR_WORKSPACE, "%s: workspace has %zu bytes, needs %zu", fn, workspace_bytes,
                wl.total);
  if (dm->T > 0) {
    REQUIRE_PTR(a);
    REQUIRE_PTR(g);
    REQUIRE_PTR(u);
    REQUIRE_PTR(x);
    REQUIRE_PTR(W_o);
    REQUIRE_PTR(gamma);
    REQUIRE_PTR(W_gate);
    REQUIRE_PTR(W_up);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float* xx = reinterpret_cast<float*>(ws + wl.xx);
  void* xl = ws + wl.xl;
  void* xT = ws + wl.xT;
  void* WoT = ws + wl.WoT;
  void* Z = ws + wl.Z;
  void* ZAT = ws + wl.ZAT;
  void* U = ws + wl.U;
  void* Q = ws + wl.Q;
  float2* coef = reinterpret_cast<float2*>(ws + wl.coef);
  float* Y = reinterpret_cast<float*>(ws + wl.Y);
  float* R = reinterpret_cast<float*>(ws + wl.R);
  void* Rs = ws + wl.Rs;
  float* t1 = reinterpret_cast<float*>(ws + wl.t1);
  const UpGeometry geo = up_geometry(dm->T, dm->H, dm->G, dm->d, dm->I, dm->dtype);
  const int HD = dm->H * dm->d, dt = dm->dtype, T = (int)dm->T, d = dm->d, D = dm->hidden;
  const int Tp = (int)loo_tokens_padded(dm->T);
  const bool bf = dt == HNA_BF16;

  // heads in KV-group order (shared by the quadratic forms and the combine)
  QuadParams qp{};
  LooCombineParams cp{};
  int n = 0;
  for (int gg = 0; gg < dm->G; ++gg) {
    qp.group_start[gg] = cp.group_start[gg] = (int16_t)n;
    for (int h = 0; h < dm->H; ++h)
      if (group_of_head[h] == gg) {
        qp.head_order[n] = cp.head_order[n] = (int8_t)h;
        ++n;
      }
  }
  qp.group_start[dm->G] = cp.group_start[dm->G] = (int16_t)n;

  // C[m, n] = sum_k X[m, k] Yo[n, k], stored at C + n * ldc + m, over ny batch
  // entries (X, Yo, C advance by bx, by, bc) or K chunks of k_split; C in the
  // input dtype or fp32
  auto gemm = [&](const void* X, int ldx, const void* Yo, int ldy, int Mr, int N, int K, void* C,
                  int ldc, bool c_in_dtype, int ny, int64_t bx, int64_t by, int64_t bc,
                  int k_split) {
    GemmParams p{};
    p.X = X;
    p.Y[0] = Yo;
    p.ldx = ldx;
    p.ldy = ldy;
    p.Mrows = Mr;
    p.N = N;
    p.Nvalid = N;
    p.K = K;
    p.C = C;
    p.ldc = ldc;
    p.bx = bx;
    p.by = by;
    p.bc = bc;
    p.k_split = k_split;
    p.out_bf16 = bf && c_in_dtype;
    return bf ? launch_mm_bf16(p, kEpiStore, ny, st) : launch_gemm_f32(p, kEpiStore, ny, st);
  };

  hipError_t e;
  if (dm->T > 0) {
    // 1. |x|^2, x in bf16 and x^T [hidden][Tp] in one pass; W_o^T [HD][hidden];
    //    the moments x . o_h and |o_h|^2 through Z = x W_o [T][HD],
    //    Q_h = W_o^(h)T W_o^(h) [d][d] and U_h = a_h Q_h [T][HD]
    if ((e = launch_x_prep(x, dm->T, D, Tp, xx, bf ? xl : nullptr, xT, dt, st)) != hipSuccess)
      return hip_fail(e, fn);
    const void* xg = bf ? xl : static_cast<const void*>(x);
    const bool fused = loo_coef_fused(d, dt);
    // bf16, d = 64 or 128: x . o_h straight from the GEMM (Z never stored;
    // its buffer holds the d / 64 fp32 partial planes [q][H][T] instead)
    const bool dot = fused && loo_dot_epilogue(d, dt);
    float* xo_part = dot ? static_cast<float*>(Z) : nullptr;
    auto gemm_dot = [&]() {
      GemmParams p{};
      p.X = WoT;
      p.Y[0] = xg;
      p.ldx = D;
      p.ldy = D;
      p.Mrows = HD;
      p.N = T;
      p.Nvalid = T;
      p.K = D;
      p.dot_a = a;
      p.dot_out = xo_part;
      p.dot_lda = HD;
      p.dot_H = dm->H;
      p.dot_d = d;
      return launch_mm_bf16(p, kEpiDot, 1, st);
    };
    if ((e = launch_scale_transpose(W_o, nullptr, WoT, D, HD, D, dt, st)) != hipSuccess ||
        (e = dot ? gemm_dot() : gemm(WoT, D, xg, D, HD, T, D, Z, HD, true, 1, 0, 0, 0, 0)) != hipSuccess ||
        (e = gemm(WoT, D, WoT, D, d, d, D, Q, d, true, dm->H, (int64_t)d * D, (int64_t)d * D,
                  (int64_t)d * d, 0)) != hipSuccess ||
        (!fused && (e = gemm(Q, d, a, HD, d, T, d, U, HD, true, dm->H, (int64_t)d * d, d, d,
                             0)) != hipSuccess))
      return hip_fail(e, fn);
    // 2. T2: Y^g = (alpha beta a)^T g and Y^u likewise.  With g_t = W_g (gamma x_t) / r_t,
    //    Y^g = R diag(gamma) W_g^T where R = ((alpha beta / r) a)^T x: the scaled
    //    head outputs, transposed (ZAT), and x^T make R one GEMM over the tokens
    //    (HD x hidden, in K chunks), and Y^g, Y^u are two GEMMs over hidden
    if (fused) {
      if ((e = launch_loo_coef_fused(a, Z, xo_part, ZAT, Q, xx, dm->T, dm->H, d, D, coef, st)) != hipSuccess)
        return hip_fail(e, fn);
    } else if ((e = launch_loo_coef(a, Z, U, xx, dm->T, dm->H, d, D, coef, dt, st)) != hipSuccess ||
               (e = launch_scale_a(a, coef, xx, dm->T, dm->H, d, D, Z, dt, st)) != hipSuccess ||
               (e = launch_scale_transpose(Z, nullptr, ZAT, T, HD, Tp, dt, st)) != hipSuccess) {
      return hip_fail(e, fn);
    }
    const int r_parts = loo_r_parts(dm->T);
    if ((e = gemm(xT, Tp, ZAT, Tp, D, HD, Tp, R, D, false, r_parts, 0, 0, (int64_t)HD * D,
                  loo_r_chunk(dm->T))) != hipSuccess ||
        (e = launch_scale_cols(R, r_parts, gamma, HD, D, Rs, dt, st)) != hipSuccess)
      return hip_fail(e, fn);
    // Y^g [I][HD] = W_g Rs^T: row k is sum_c W_g[k][c] Rs[j][c]
    for (int gu = 0; gu < 2; ++gu)
      if ((e = gemm(Rs, D, gu ? W_up : W_gate, D, HD, dm->I, D, Y + (int64_t)gu * HD * dm->I, HD,
                    false, 1, 0, 0, 0, 0)) != hipSuccess)
        return hip_fail(e, fn);
    // 3. T1
    if ((e = launch_t1(g, u, coef, dm->T, dm->H, dm->I, t1, dm->dtype, st)) != hipSuccess ||
        (e = launch_t1_reduce(t1, wl.n_tc, (int64_t)dm->H * dm->I,
                              reinterpret_cast<double*>(ws + wl.t1r), st)) != hipSuccess)
      return hip_fail(e, fn);
    // 4. T3: Gram matrices weighted by beta^2, their quadratic forms, group sums
    GramParams gp{};
    gp.a = a;
    gp.r = nullptr;
    gp.coef = coef;
    gp.part = reinterpret_cast<float*>(ws + wl.gram_part);
    gp.T = dm->T;
    gp.H = dm->H;
    gp.d = dm->d;
    gp.n_gc = geo.n_gc;
    gp.chunk_tokens = geo.gram_chunk;
    if ((e = launch_gram(gp, dm->dtype, st)) != hipSuccess) return hip_fail(e, fn);
    void* C = ws + wl.gram;
    if ((e = launch_gram_reduce(gp.part, geo.n_gc, (int64_t)dm->H * dm->d * dm->d, C, dm->dtype,
                                st)) != hipSuccess)
      return hip_fail(e, fn);
    qp.C = C;
    qp.M = M;
    qp.add = reinterpret_cast<float*>(ws + wl.t3);
    qp.add_part = reinterpret_cast<float*>(ws + wl.t3_part);
    qp.H = dm->H;
    qp.G = dm->G;
    qp.d = dm->d;
    qp.KB = geo.I32 / 32;
    if ((e = launch_quad(qp, dm->dtype, st)) != hipSuccess) return hip_fail(e, fn);
  }
  // 5. S_loo = scale * (sum over the group's heads of T1 + 2 T2, plus T3); with
  // no tokens the same kernel writes zeros (no terms)
  const bool any = dm->T > 0;
  cp.M = M;
  cp.Y = any ? Y : nullptr;
  cp.t1r = any ? reinterpret_cast<const double*>(ws + wl.t1r) : nullptr;
  cp.t3 = any ? reinterpret_cast<const float*>(ws + wl.t3) : nullptr;
  cp.S_loo = S_loo;
  cp.scale = scale;
  cp.H = dm->H;
  cp.G = dm->G;
  cp.d = dm->d;
  cp.I = dm->I;
  cp.I32 = geo.I32;
  cp.KB = geo.I32 / 32;
  cp.S = dm->d / 16;
  return finish(launch_loo_combine(cp, dm->dtype, st), st, fn);
}

size_t hna_layout_search_workspace_bytes(int32_t N, int32_t G, int32_t I) {
  if (N < 1 || G < 1 || I < 1) return 0;
  return search_workspace(N, G, I).total;
}

int hna_layout_search(int32_t N, int32_t G, int32_t I, int32_t L, const float* S_up_hat,
                      const float* S_down_hat, int32_t iters, int32_t max_swaps,
                      int32_t max_sweeps, int32_t* head_device, int32_t* neuron_device,
                      int32_t* neuron_stats, double* J_history, int32_t* n_sweeps,
                      void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "hna_layout_search";
  int rc = check_layout_dims(fn, N, G, I, L);
  if (rc != HNA_OK) return rc;
  rc = check_head_dims(fn, G, L);
  if (rc != HNA_OK) return rc;
  if (iters < 0 || max_swaps < 0 || max_sweeps < 1)
    return fail(HNA_ERR_INVALID_ARG, "%s: iters=%d, max_swaps=%d must be >= 0, max_sweeps=%d >= 1",
                fn, iters, max_swaps, max_sweeps);
  if (L > kLayoutMaxDevices || I > kLayoutMaxNpt * 1024 ||
      neuron_step_lds_bytes(I, L) > kLayoutMaxLds)
    return fail(HNA_ERR_UNSUPPORTED, "%s: I=%d, L=%d outside the neuron step's limits", fn, I, L);
  if (N > max_objective_layers())
    return fail(HNA_ERR_UNSUPPORTED, "%s: N=%d exceeds %d layers", fn, N, max_objective_layers());
  REQUIRE_PTR(S_up_hat);
  if (N > 1) REQUIRE_PTR(S_down_hat);
  REQUIRE_PTR(head_device);
  REQUIRE_PTR(neuron_device);
  REQUIRE_PTR(neuron_stats);
  REQUIRE_PTR(workspace);
  if (!J_history || !n_sweeps)
    return fail(HNA_ERR_INVALID_ARG, "%s: J_history and n_sweeps are required host pointers", fn);
  const SearchWorkspace wl = search_workspace(N, G, I);
  if (workspace_bytes < wl.total)
    return fail(HNA_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, workspace_bytes, wl.total);
  char* ws = static_cast<char*>(workspace);
  int32_t* h_new = reinterpret_cast<int32_t*>(ws + wl.heads);
  int32_t* nu_new = reinterpret_cast<int32_t*>(ws + wl.neurons);
  int32_t* st_new = reinterpret_cast<int32_t*>(ws + wl.stats);
  double* hscore = reinterpret_cast<double*>(ws + wl.hscore);
  int32_t* hstatus = reinterpret_cast<int32_t*>(ws + wl.hstatus);
  double* fu = reinterpret_cast<double*>(ws + wl.frac_up);
  double* fd = reinterpret_cast<double*>(ws + wl.frac_down);
  double* Jd = reinterpret_cast<double*>(ws + wl.J);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int parts = (int)partition_count(G, L);

  *n_sweeps = 0;
  double bestJ = 0.0;
  std::vector<char> report(wl.report_bytes);
  for (int s = 0; s < max_sweeps; ++s) {
    // neuron step from the kept heads, head step from the new neurons, then J
    NeuronStepParams np{S_up_hat, S_down_hat, head_device, nu_new, st_new,
                        N, G, I, L, iters, max_swaps};
    hipError_t e = launch_neuron_step(np, st);
    if (e != hipSuccess) return hip_fail(e, fn);
    HeadStepParams hp{S_up_hat, S_down_hat, nu_new, h_new, hscore, hstatus, N, G, I, L, parts};
    e = launch_head_step(hp, st);
    if (e != hipSuccess) return hip_fail(e, fn);
    e = launch_layout_objective(S_up_hat, S_down_hat, h_new, nu_new, N, G, I, fu, fd, Jd, st);
    if (e != hipSuccess) return hip_fail(e, fn);
    if ((e = hipMemcpyAsync(report.data(), ws + wl.report, wl.report_bytes, hipMemcpyDeviceToHost,
                            st)) != hipSuccess ||
        (e = hipStreamSynchronize(st)) != hipSuccess)
      return hip_fail(e, fn);
    double J;
    std::memcpy(&J, report.data(), sizeof(double));
    const int32_t* nst = reinterpret_cast<const int32_t*>(report.data() + (wl.stats - wl.report));
    const int32_t* hst = reinterpret_cast<const int32_t*>(report.data() + (wl.hstatus - wl.report));
    for (int i = 0; i < N; ++i) {
      const int ns = nst[(size_t)i * 4];
      if (ns == HNA_LAYOUT_BAD_HEADS)
        return fail(HNA_ERR_INVALID_ARG, "%s: head devices of layer %d or %d outside [0, %d)", fn,
                    i, i + 1 < N ? i + 1 : i, L);
      if (ns == HNA_LAYOUT_NO_MOVE || hst[i] != HNA_LAYOUT_OK)
        return fail(HNA_ERR_INVALID_ARG, "%s: layer %d: non-finite scores", fn, i);
    }
    J_history[s] = J;
    *n_sweeps = s + 1;
    if (s > 0 && !(J > bestJ)) break;
    bestJ = J;
    if ((e = hipMemcpyAsync(head_device, h_new, (size_t)N * G * 4, hipMemcpyDeviceToDevice, st)) !=
            hipSuccess ||
        (e = hipMemcpyAsync(neuron_device, nu_new, (size_t)N * I * 4, hipMemcpyDeviceToDevice,
                            st)) != hipSuccess ||
        (e = hipMemcpyAsync(neuron_stats, st_new, (size_t)N * 16, hipMemcpyDeviceToDevice, st)) !=
            hipSuccess)
      return hip_fail(e, fn);
  }
  return finish(hipSuccess, st, fn);
}

}  // extern "C"
