/*
 * hna.h -- C ABI of the head-to-neuron affinity library (gfx950 / MI355X).
 *
 * The library computes the calibration scores of "Affinity-Aware Sharding for
 * Delayed Tensor Parallelism" (E. de Reynal, arXiv:2609.13846), section 3,
 * paragraph "Affinity scores" and equation (5):
 *
 *   p_h      = gamma * (a_h W_o^(h)T) / r        head h's piece of the FFN input
 *   Delta_hk = silu'(g_k) u_k (p_h . w^g_k) + silu(g_k) (p_h . w^u_k)     (5)
 *   S_fo[g,k]  = sum_{h in g} E_t[Delta_hk^2] ||w^d_k||^2          [G x I]
 *   S_add[g,k] = sum_{h in g} E_t[(p_h . w^g_k)^2 + (p_h . w^u_k)^2] [G x I]
 *   S_down[k,g'] = E_t[alpha_k^2 / r'^2] ||W^qkv_g' (gamma' * w^d_k)||^2
 *                  with alpha_k = silu(g_k) u_k                     [I x G']
 *
 * Conventions shared by every call
 *   - Matrices are row-major, linear-layer (out, in) order:
 *       W_o [hidden, H*d]  (head h owns columns h*d .. h*d+d-1)
 *       W_gate, W_up [I, hidden]  (row k is w^g_k, w^u_k)
 *       W_down [hidden, I]        (column k is w^d_k)
 *       W_q [H'*d', hidden], W_k, W_v [G'*d', hidden]  (next layer)
 *     Activations: a [T, H, d] (token-major), g, u [T, I]; r, r_next [T].
 *   - dtype HNA_BF16: a, g, u and all weight matrices are bfloat16; HNA_F32:
 *     they are float32.  gamma, gamma_next, r, r_next, wd_sq and every output
 *     are float32 in both cases.  Accumulation is float32.
 *   - Every tensor pointer is a device pointer owned by the caller; the
 *     library allocates no memory and keeps no state between calls (the
 *     allocation-free entry point's static device array aside, see there).
 *     Scratch space is the caller's workspace.  group maps are host arrays, read
 *     during the call only.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = the default
 *     stream) and runs asynchronously; nothing synchronises the host except
 *     hna_layout_search (once per sweep) and, for every call, the
 *     environment variable HNA_DEBUG_SYNC=1.
 *   - Every argument is validated on the host before anything is enqueued.
 *     On failure a negative hna_status is returned, a thread-local message
 *     is available from hna_last_error(), and nothing has been launched.
 *     Launch failures return HNA_ERR_HIP.  Nothing prints, aborts or throws.
 *   - Device pointers must be 16-byte aligned (HNA_ERR_ALIGNMENT otherwise).
 *   - The library is reentrant; its only global mutable state is the
 *     thread-local error text (and that static array).  Calls
 *     that share a workspace or an output must be ordered on one stream by
 *     the caller.
 *
 * Supported shapes: H <= 128, 1 <= G <= H, H % G == 0, 0 <= group_of_head[h]
 * < G; d a multiple of 16 with d <= 128; hidden a positive multiple of 8;
 * 1 <= I <= 2^22; 0 <= T <= 2^31 - 1, and T and I such that the hot kernel
 * needs at most 2^24 workgroups (about 2^31 tokens at I = 3072).  Others
 * return HNA_ERR_UNSUPPORTED (HNA_ERR_INVALID_ARG for non-positive sizes).
 */
#ifndef HNA_H
#define HNA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HNA_ABI_VERSION 2

typedef enum hna_status {
  HNA_OK = 0,
  HNA_ERR_INVALID_ARG = -1,  /* bad dimension, null pointer, bad map, bad flag */
  HNA_ERR_UNSUPPORTED = -2,  /* valid but outside the supported shapes/dtypes */
  HNA_ERR_ALIGNMENT = -3,    /* a device pointer is not 16-byte aligned */
  HNA_ERR_WORKSPACE = -4,    /* workspace or output buffer too small */
  HNA_ERR_HIP = -5           /* the HIP runtime reported an error */
} hna_status;

typedef enum hna_dtype { HNA_F32 = 0, HNA_BF16 = 1 } hna_dtype;

/* flags for hna_finalize_up */
enum { HNA_ACCUMULATE = 1 }; /* add into S_fo/S_add/c_down instead of overwriting */

/* Shape of one layer's up edge (heads of layer i -> neurons of layer i). */
typedef struct hna_dims {
  int64_t T;       /* calibration tokens in this call */
  int32_t hidden;  /* residual width */
  int32_t H;       /* query heads */
  int32_t G;       /* KV groups */
  int32_t d;       /* head dim */
  int32_t I;       /* FFN neurons */
  int32_t dtype;   /* hna_dtype */
} hna_dims;

/* Shape of one down edge (neurons of layer i -> KV groups of layer i+1). */
typedef struct hna_down_dims {
  int32_t hidden;  /* residual width (shared by both layers) */
  int32_t I;       /* neurons of layer i (columns of W_down) */
  int32_t H;       /* query heads of layer i+1 */
  int32_t G;       /* KV groups of layer i+1 */
  int32_t d;       /* head dim of layer i+1 */
  int32_t dtype;   /* hna_dtype of W_q, W_k, W_v, W_down */
} hna_down_dims;

int hna_abi_version(void);
const char* hna_status_string(int status);
/* Message of the calling thread's most recent failure ("" if none). */
const char* hna_last_error(void);

/* ---------------------------------------------------------------- up edge */

/* Bytes of the folded weight M for `dims` (see hna_fold_up_weights). */
size_t hna_folded_bytes(const hna_dims* dims);
/* Bytes of workspace hna_fold_up_weights needs: gamma * W_o transposed, in
 * the input dtype. */
size_t hna_fold_workspace_bytes(const hna_dims* dims);

/*
 * Weight fold.  Because p_h . w_k = (1/r) a_h . (W_o^(h)T (gamma * w_k)) (the
 * decomposition of section 3, "Affinity scores", with the two finite sums
 * exchanged), the folded weights
 *     M_h = W_o^(h)T diag(gamma) [W_gate; W_up]^T          [H, d, 2I]
 * turn the per-head pieces into one short contraction over d per token.
 * Writes M (hna_folded_bytes(dims) bytes, dtype of `dims`) in the internal
 * layout the affinity kernel reads; callers treat it as opaque.  Float32
 * accumulation; bf16 output is rounded once at the end.
 */
int hna_fold_up_weights(const hna_dims* dims, const void* W_o, const float* gamma,
                        const void* W_gate, const void* W_up,
                        void* M, size_t M_bytes,
                        void* workspace, size_t workspace_bytes, void* stream);

/* wd_sq[k] = ||w^d_k||^2, the squared norm of column k of W_down [hidden, I]. */
int hna_down_col_sqnorm(const hna_dims* dims, const void* W_down, float* wd_sq,
                        void* stream);

/*
 * Bytes of workspace hna_affinity_up, hna_affinity_add and hna_finalize_up
 * share for `dims`: the FO and down-moment partial sums of each 1024-token
 * block of neurons, the per-head Gram partials and sums, and the ADD sums.
 */
size_t hna_up_workspace_bytes(const hna_dims* dims);

/*
 * The hot pass (equation (5) and the FO score).  For every token t of this
 * call, head h and neuron k it forms (p_h . w^g_k, p_h . w^u_k) from a and M,
 * the operating-point coefficients silu'(g)u/r and silu(g)/r, the damage
 * Delta_hk, and accumulates sum_t Delta^2 over the query heads of each KV
 * group, plus sum_t (silu(g)u/r_next)^2 when r_next is not NULL.  Partial
 * sums go to `workspace` (>= hna_up_workspace_bytes); nothing of size
 * T x H x I is ever written.
 *   a [T,H,d], g, u [T,I] (dtype of dims); r [T], r_next [T] or NULL (fp32);
 *   M from hna_fold_up_weights with the same dims;
 *   group_of_head: host int32 [H], values in [0, G).
 * T = 0 is allowed and yields zero sums.
 */
int hna_affinity_up(const hna_dims* dims, const void* a, const void* g, const void* u,
                    const float* r, const float* r_next, const void* M,
                    const int32_t* group_of_head,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * The ADD score of the same section ("ignores the operating point"):
 *   sum_t sum_{h in g} (p_h.w^g_k)^2 + (p_h.w^u_k)^2
 *     = sum_{h in g} m^g_hk . C_h m^g_hk + m^u_hk . C_h m^u_hk,
 *   C_h = sum_t a_th a_th^T / r_t^2  (d x d),
 * where m^g_hk, m^u_hk are columns of the folded weights M_h (exact by
 * linearity of the sum over tokens).  Reads a, r and M; writes the Gram
 * matrices and the ADD sums into `workspace`, the same workspace as
 * hna_affinity_up, for hna_finalize_up.  Arguments as for hna_affinity_up.
 */
int hna_affinity_add(const hna_dims* dims, const void* a, const float* r, const void* M,
                     const int32_t* group_of_head,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Fixed-order reduction of the sums left by hna_affinity_up and
 * hna_affinity_add (both must have run on this workspace):
 *   S_fo[g*I+k]  (+)= scale * wd_sq[k] * sum_t sum_{h in g} Delta^2
 *   S_add[g*I+k] (+)= scale * sum_t sum_{h in g} ((p.w^g)^2 + (p.w^u)^2)
 *   c_down[k]    (+)= scale * sum_t (silu(g_k) u_k / r_next)^2   (if not NULL)
 * `scale` is 1/T_total (the mean over all calibration tokens, possibly fed in
 * several chunks with HNA_ACCUMULATE).  S_fo, S_add [G, I] and c_down [I]
 * are fp32; c_down may be NULL (then r_next must have been NULL).  The result
 * is deterministic: no atomics, fixed summation order.
 */
int hna_finalize_up(const hna_dims* dims, const float* wd_sq, float scale, int flags,
                    const void* workspace, size_t workspace_bytes,
                    float* S_fo, float* S_add, float* c_down, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the three
 * calls above in one, hna_affinity_up + hna_affinity_add + hna_finalize_up
 * with the same arguments and results, whose partial sums live in a fixed
 * scratch array of hna_static_scratch_bytes() (64 MiB) compiled into the
 * library instead of a caller's workspace.  Nothing is allocated: each GPU
 * the library runs on holds its own copy of the array from the first call on
 * it until the process ends (its address is looked up once per device, with
 * that device current).
 *   Outputs: S_fo, S_add [G, I] and, when r_next is given, c_down [I]
 *   (r_next and c_down are both given or both NULL); flags and scale as for
 *   hna_finalize_up (HNA_ACCUMULATE adds token chunks up).
 * Calls that need more scratch than the array holds (about 100 MB for
 * 131,072 tokens of a 32-head, 14,336-neuron layer) return
 * HNA_ERR_WORKSPACE: split the tokens over calls with HNA_ACCUMULATE.  Every
 * call on one GPU uses that GPU's one array and leaves its contents behind;
 * each call writes every region it reads before reading it, so no clearing
 * is needed.  Calls on one GPU that overlap (concurrent streams, or threads
 * without ordering) race on the array: order them on one stream.
 */
size_t hna_static_scratch_bytes(void);
int hna_affinity_up_static(const hna_dims* dims, const void* a, const void* g, const void* u,
                           const float* r, const float* r_next, const void* M, const float* wd_sq,
                           const int32_t* group_of_head, float scale, int flags, float* S_fo,
                           float* S_add, float* c_down, void* stream);

/* -------------------------------------------------------------- down edge */

/* Bytes of workspace hna_down_weight_norms needs. */
size_t hna_down_workspace_bytes(const hna_down_dims* dims);

/*
 * Down-edge weight part (section 3, "Affinity scores"):
 *   n[g', k] = ||b_g'k||^2,  b_g'k = W^qkv_g' (gamma_next * w^d_k)
 * where W^qkv_g' stacks the W_q rows of the next-layer query heads h' with
 * group_of_head_next[h'] = g', then rows g'*d'..g'*d'+d'-1 of W_k and of W_v.
 * n is fp32 [G', I].  b is never stored.
 */
int hna_down_weight_norms(const hna_down_dims* dims, const void* W_q, const void* W_k,
                          const void* W_v, const float* gamma_next, const void* W_down,
                          const int32_t* group_of_head_next, float* n,
                          void* workspace, size_t workspace_bytes, void* stream);

/* S_down[k*G'+g'] = c_down[k] * n[g'*I+k]   (fp32, [I, G']). */
int hna_down_combine(int32_t I, int32_t G_next, const float* c_down, const float* n,
                     float* S_down, void* stream);

/* ------------------------------------------------ exact leave-one-out score */

/* Bytes of workspace hna_affinity_loo needs (0 for invalid dims). */
size_t hna_loo_workspace_bytes(const hna_dims* dims);

/*
 * Exact leave-one-out score of the pre-activations (section 3, "Affinity
 * scores": the variant that keeps the change of the norm's rms when a head
 * is removed):
 *   o_h = a_h W_o^(h)T,  r = rms(x),  r_h = rms(x - o_h)
 *   g_k^(-h) = (gamma * (x - o_h) / r_h) . w^g_k   (u likewise)
 *   S_loo[g, k] = scale * sum_{h in g} sum_t ((g_k - g_k^(-h))^2 + (u_k - u_k^(-h))^2)
 * (scale = 1/T gives the mean over tokens).  Computed exactly through
 *   g_k - g_k^(-h) = alpha_th g_k + beta_th (a_h . m_hk),
 *   alpha_th = 1 - r/r_h,  beta_th = 1/r_h,
 * with m_hk the folded weights of hna_fold_up_weights (M) and r_h from |x|^2,
 * x . o_h and |o_h|^2; the square is summed as three terms (alpha^2 g^2, the
 * cross term, beta^2 P^2 through weighted Gram matrices).  The cross term
 * uses g_t = W_gate (gamma * x_t) / r_t: sum_t alpha beta a_th g_tk equals
 * (R_h diag(gamma) w^g_k) with R_h = sum_t (alpha beta / r_t) a_th x_t^T, one
 * GEMM over the tokens of width hidden (shared by gate and up) followed by
 * two GEMMs over hidden.
 *   a [T, H, d], g, u [T, I], W_o [hidden, H*d], W_gate, W_up [I, hidden], M:
 *     the input dtype; gamma fp32 [hidden] (the pre-norm weight of the fold)
 *   x fp32 [T, hidden]: the residual entering the FFN pre-norm (the g and u
 *     given must be its pre-activations, g = W_gate (gamma * x / rms(x)))
 *   S_loo fp32 [G, I] output (written, also for T = 0: zeros)
 * A token whose residual vanishes without head h (r_h = 0) contributes
 * nothing for that head.  Limits: those of hna_affinity_up and T <= 4,000,000
 * per call (HNA_ERR_UNSUPPORTED above: the token GEMM addresses 256-row tiles
 * of the transposed operands through 32-bit offsets).  Deterministic: every
 * sum, the plain GEMMs included, runs in a fixed order in the library's own
 * kernels (no BLAS library is used).
 */
int hna_affinity_loo(const hna_dims* dims, const void* a, const void* g, const void* u,
                     const float* x, const void* W_o, const float* gamma, const void* W_gate,
                     const void* W_up, const void* M, const int32_t* group_of_head, float scale,
                     float* S_loo, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------- layout objective */

/*
 * Unit-mass normalisation (section 3, paragraph "Objective"): S holds
 * n_matrices consecutive fp32 matrices of `count` entries each; every one is
 * divided by its own sum, taken in fp64 in a fixed order, and the quotient is
 * rounded to fp32 into out.  A matrix whose sum is 0 becomes all zeros.  out
 * may equal S (in place).  count == 0 or n_matrices == 0 is a no-op.
 */
int hna_unit_mass(const float* S, int64_t count, int32_t n_matrices, float* out, void* stream);

/*
 * Layout objective J of eq. (6) (section 3, paragraph "Objective") over a
 * stack of N layers:
 *   S_up   fp32 [N, G, I]: up-edge scores of layer i (KV group g, neuron k)
 *   S_down fp32 [N-1, I, G]: down-edge scores from layer i's neuron k to
 *          layer i+1's KV group g; may be NULL when N == 1
 *   head_device   int32 [N, G]: device of KV group g of layer i
 *   neuron_device int32 [N, I]: device of neuron k of layer i
 * Outputs (fp64, device memory):
 *   frac_up[i]   = mass of unit-mass S_up[i] on entries (g, k) with
 *                  head_device[i, g] == neuron_device[i, k]
 *   frac_down[i] = mass of unit-mass S_down[i] on entries (k, g) with
 *                  neuron_device[i, k] == head_device[i+1, g]   (N-1 values;
 *                  may be NULL when N == 1)
 *   J[0]         = sum of the N + (N-1) fractions, in that order
 * The scores need not be normalised beforehand: each fraction is the
 * matrix's co-located sum over its total sum, both accumulated in fp64 in a
 * fixed order (0 for a matrix whose total is 0), so results are reproducible
 * bit for bit.  Device ids are only compared for equality, never used as
 * indices: any int32 values are valid.  Requires G*I <= 2^31 and
 * N <= 2048 (HNA_ERR_UNSUPPORTED otherwise).
 */
int hna_layout_objective(int32_t N, int32_t G, int32_t I, const float* S_up, const float* S_down,
                         const int32_t* head_device, const int32_t* neuron_device,
                         double* frac_up, double* frac_down, double* J, void* stream);

/* ------------------------------------------- neuron step of the layout search */

/* Per-layer status written by hna_neuron_step into stats[i*4 + 0]. */
enum hna_layout_status {
  HNA_LAYOUT_OK = 0,
  HNA_LAYOUT_BAD_HEADS = 1,   /* a head device of layer i or i+1 is outside [0, L) */
  HNA_LAYOUT_SWAP_LIMIT = 2,  /* the swap phase stopped at max_swaps swaps */
  HNA_LAYOUT_NO_MOVE = 3,     /* non-finite gains left the fix-up without a move */
  HNA_LAYOUT_BAD_NEURONS = 4  /* a neuron device of layer i or i-1 is outside [0, L) */
};

/*
 * Neuron step of the layout search (section 3, paragraph "Optimiser";
 * iteration count and step decay from appendix A), for every layer of an
 * N-layer stack at once, given the KV-group devices of all layers:
 *   M_i[k, l] = sum_{g: h_i(g) = l} S_up_hat_i[g, k]
 *             + sum_{g: h_{i+1}(g) = l} S_down_hat_i[k, g]     (no down term for i = N-1)
 *   nu_i = a balanced assignment (I/L neurons per device) maximising
 *          sum_k M_i[k, nu_i(k)]
 * solved by dual ascent on the L device offsets (`iters` iterations; the
 * pages use 300), a fix-up to the capacities and pairwise swaps (at most
 * max_swaps per layer).  Inputs (device memory):
 *   S_up_hat   fp32 [N, G, I] unit-mass up-edge scores (see hna_unit_mass)
 *   S_down_hat fp32 [N-1, I, G] unit-mass down-edge scores; may be NULL if N == 1
 *   head_device int32 [N, G], values in [0, L)
 * Outputs (device memory):
 *   neuron_device int32 [N, I]: nu_i(k) in [0, L); all -1 for a layer whose
 *                 head devices (of layer i or i+1) fall outside [0, L)
 *   stats int32 [N, 4]: hna_layout_status, the load in excess of the
 *                 capacities after the dual ascent, fix-up moves, swaps
 * Every decision compares fp64 values computed in a fixed order (M sums its
 * up terms in increasing g, then its down terms; the offsets move by
 * step*(count-cap)/cap with a first step of (max M - min M)/10 decaying by
 * 0.98; ties go to the lowest device or neuron), so the result is exactly
 * reproducible.  Limits: 1 <= L <= 8, G and I multiples of L, G <= 128,
 * I <= 16384 and I*L <= 16384 (HNA_ERR_UNSUPPORTED otherwise).  Per-layer
 * failures are reported in stats, not in the return value.
 */
int hna_neuron_step(int32_t N, int32_t G, int32_t I, int32_t L, const float* S_up_hat,
                    const float* S_down_hat, const int32_t* head_device, int32_t iters,
                    int32_t max_swaps, int32_t* neuron_device, int32_t* stats, void* stream);

/* ---------------------------------------------- head step and the sweeps */

/*
 * Head step of the layout search (section 3, paragraph "Optimiser"), for
 * every layer at once, given the neuron devices of all layers:
 *   A_i[g, l] = sum_{k: nu_i(k) = l} S_up_hat_i[g, k]
 *             + sum_{k: nu_{i-1}(k) = l} S_down_hat_{i-1}[k, g]   (no down term for i = 0)
 *   h_i = the balanced map (G/L groups per device) maximising sum_g A_i[g, h_i(g)],
 * found by scoring all G!/((G/L)!)^L labelled balanced partitions (2520 for
 * G = 8, L = 4).  Partitions are ranked in lexicographic order of
 * (h(0), ..., h(G-1)); ties go to the lowest rank.  A_i and the scores are
 * fp64.  Inputs (device): S_up_hat [N, G, I], S_down_hat [N-1, I, G] fp32
 * (S_down_hat may be NULL if N == 1), neuron_device int32 [N, I].  Outputs
 * (device): head_device int32 [N, G]; score fp64 [N], the best partition's
 * score (the co-located mass layer i's up edge and layer i-1's down edge
 * get); status int32 [N] (HNA_LAYOUT_OK, or HNA_LAYOUT_BAD_NEURONS with
 * head_device = -1 when a neuron device of layer i or i-1 is outside
 * [0, L)).  Limits: 1 <= L <= 8, G <= 16 and at most 2^24 partitions
 * (HNA_ERR_UNSUPPORTED otherwise), G and I multiples of L.
 */
int hna_head_step(int32_t N, int32_t G, int32_t I, int32_t L, const float* S_up_hat,
                  const float* S_down_hat, const int32_t* neuron_device, int32_t* head_device,
                  double* score, int32_t* status, void* stream);

/* Bytes of device workspace hna_layout_search needs (0 for bad sizes). */
size_t hna_layout_search_workspace_bytes(int32_t N, int32_t G, int32_t I);

/*
 * The layout search (section 3, paragraph "Optimiser"): coordinate ascent
 * over the chain of layers.  Each sweep runs hna_neuron_step for every layer
 * from the kept head devices, then hna_head_step for every layer from the new
 * neuron devices, then J (eq. 6) of the new layout.  A sweep is kept while J
 * strictly increases; the first sweep that does not raise J ends the search
 * and is discarded, as is everything after max_sweeps sweeps.
 *   head_device   int32 [N, G] device memory: in, the starting head devices
 *                 (the pages start from the contiguous map g / (G/L)); out,
 *                 the kept layout's
 *   neuron_device int32 [N, I] device memory, out: the kept layout's
 *   neuron_stats  int32 [N, 4] device memory, out: hna_neuron_step's stats of
 *                 the kept sweep
 *   J_history     fp64 [max_sweeps] HOST memory, out: J after each sweep run
 *   n_sweeps      HOST int32, out: sweeps run (the last one is discarded if it
 *                 did not raise J)
 *   workspace     device memory of hna_layout_search_workspace_bytes(N, G, I)
 * iters and max_swaps are passed to hna_neuron_step (the pages: 300).
 * Unlike the other calls, this one synchronises `stream` once per sweep to
 * read J.  Head devices outside [0, L) in the starting map return
 * HNA_ERR_INVALID_ARG.  Limits: those of hna_neuron_step, hna_head_step and
 * hna_layout_objective.
 */
int hna_layout_search(int32_t N, int32_t G, int32_t I, int32_t L, const float* S_up_hat,
                      const float* S_down_hat, int32_t iters, int32_t max_swaps,
                      int32_t max_sweeps, int32_t* head_device, int32_t* neuron_device,
                      int32_t* neuron_stats, double* J_history, int32_t* n_sweeps,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------ measurement */

/*
 * Sustained bf16 matrix-core rate (a measurement aid, not a step of the
 * method; it reads the dense rate the affinity kernel's MFMA throughput is
 * compared with).  n_workgroups workgroups of 256 threads each run `iters`
 * rounds of independent bf16 MFMAs per wave: four 32x32x16
 * (v_mfma_f32_32x32x16_bf16, 32768 FLOP each) for shape 0, eight 16x16x32
 * (v_mfma_f32_16x16x32_bf16, 16384 FLOP each, accumulators k and k + 4 on
 * operand pair k) for shape 1; n_workgroups * 4 * iters * 131072 FLOP in all
 * either way.  Thread t of
 * the grid loads its four operand pairs from seed[8 t .. 8 t + 7] (16-byte
 * items of bf16: seed holds n_workgroups * 256 * 128 bytes; random values
 * give the power draw, and the clock, of real data) and writes the sum of its
 * accumulators to out[t] (n_workgroups * 256 floats).  Both buffers are
 * caller-owned device memory, 16-byte aligned.  Limits: 1 <= n_workgroups <=
 * 65536, 1 <= iters <= 1,000,000 and shape 0 or 1, else HNA_ERR_INVALID_ARG.
 */
int hna_mfma_rate_probe(int32_t n_workgroups, int32_t iters, int32_t shape, const void* seed,
                        float* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* HNA_H */
