"""Float64 CPU oracle of the head-to-neuron affinity pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module; only the tests, the smoke check and the benchmark's CPU
baseline do.  It shares no code with the HIP library and imports nothing from
it.

Source: "Affinity-Aware Sharding for Delayed Tensor Parallelism" (E. de Reynal,
arXiv:2609.13846), section 3, paragraph "Affinity scores", equation (5), in the
PDF text and in the HTML copy of the same paper.  Notation follows the paper:

  x        residual entering the FFN pre-norm, r = rms(x), gamma the norm gain
  a_h      head h's attention output, W_o^(h) its slice of the output
           projection (columns h*d .. h*d+d-1 of W_o, stored (out, in))
  p_h      = gamma * (a_h W_o^(h)T) / r, head h's additive piece of the
           normalised FFN input
  w^g_k, w^u_k  row k of the gate / up projections; w^d_k column k of W_down
  g_k, u_k the neuron's gate / up pre-activations
  Delta_hk = silu'(g_k) u_k (p_h . w^g_k) + silu(g_k) (p_h . w^u_k)   (eq. 5)
  S_fo[g,k]  = sum_{h in group g} E_t[Delta_hk^2] * ||w^d_k||^2
  S_add[g,k] = sum_{h in group g} E_t[(p_h . w^g_k)^2 + (p_h . w^u_k)^2]
  b_gk     = W^qkv_g (gamma' * w^d_k)    (next layer's q/k/v rows of group g)
  S_down[k,g] = E_t[alpha_k^2 / r'^2] * ||b_gk||^2,  alpha_k = silu(g_k) u_k

Readings where the pages leave a step open (each is listed with its reason in
the design notes): silu' is the exact derivative sigma(g)(1 + g(1 - sigma(g)));
E_t is the plain mean over every calibration token; a group's score is the sum
of its query heads' scores (not the removal of the whole group); the norm
multiplies by gamma (not 1 + gamma); W^qkv_g stacks the group's query-head rows
of W_q, then its rows of W_k, then of W_v; r and r' are inputs, so both sides
use the same values.

Everything here is float64 numpy with the literal definitions: per head the
piece p_h is formed in full, then dotted with the neuron weights.  Matrix
products are library calls (numpy matmul).  There is no weight folding, no
fusion and no reordering of the sums.  Work is split over token chunks only
to bound memory; chunk partial sums are added in order.

Parity status: every function below is pinned by tests that do not retype its
formulas (ablation by removing a head from a genuine forward pass, central
finite differences of the neuron output, an independent Gram-matrix closed
form, permutation equivariance, scaling and special cases).
"""
from __future__ import annotations

from typing import Iterable, Optional, Sequence

import numpy as np

__all__ = [
    "silu_parts", "head_piece", "first_order_damage", "affinity_up",
    "down_moment", "down_weight_norms", "affinity_down", "affinity_layer",
    "down_col_sqnorm",
]


def _f64(x) -> np.ndarray:
    """Exact conversion to float64 (bf16 and fp32 values are representable)."""
    if hasattr(x, "detach"):  # a torch tensor (bf16 -> f64 is exact)
        import torch
        x = x.detach().to(device="cpu", dtype=torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def silu_parts(g: np.ndarray):
    """sigma(g), silu(g) = g sigma(g) and its exact derivative.

    silu'(g) = sigma(g) + g sigma(g) (1 - sigma(g)) = sigma(g) (1 + g (1 - sigma(g))).
    Paper section 3, eq. (5) uses silu' at the operating point g_k.
    """
    g = np.asarray(g, dtype=np.float64)
    # logistic sigmoid 1 / (1 + e^-g), evaluated on the branch where the
    # exponential cannot overflow and no cancellation occurs
    e = np.exp(-np.abs(g))
    sig = np.where(g >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    silu = g * sig
    dsilu = sig * (1.0 + g * (1.0 - sig))
    return sig, silu, dsilu


def head_piece(a_h: np.ndarray, r: np.ndarray, gamma: np.ndarray,
               W_o: np.ndarray, h: int) -> np.ndarray:
    """p_h = gamma * (a_h W_o^(h)T) / r for a block of tokens.

    a_h [Tc, d] is head h's attention output, W_o [hidden, H*d] the output
    projection (out, in); head h owns its columns h*d .. h*d+d-1.  Paper
    section 3 ("Affinity scores"): the normalised FFN input decomposes as
    sum_h p_h + (rest).
    """
    d = a_h.shape[1]
    W_oh = W_o[:, h * d:(h + 1) * d]                   # [hidden, d]
    return (a_h @ W_oh.T) * gamma[None, :] / r[:, None]


def first_order_damage(a, g, u, r, gamma, W_o, W_gate, W_up) -> np.ndarray:
    """Delta[t, h, k] of eq. (5) for every token, head and neuron (small inputs).

    Delta_hk = silu'(g_k) u_k (p_h . w^g_k) + silu(g_k) (p_h . w^u_k).
    """
    a, g, u, r = _f64(a), _f64(g), _f64(u), _f64(r)
    gamma, W_o, W_gate, W_up = _f64(gamma), _f64(W_o), _f64(W_gate), _f64(W_up)
    T, H, d = a.shape
    _, silu, dsilu = silu_parts(g)
    out = np.empty((T, H, W_gate.shape[0]))
    for h in range(H):
        p = head_piece(a[:, h, :], r, gamma, W_o, h)
        pg = p @ W_gate.T
        pu = p @ W_up.T
        out[:, h, :] = dsilu * u * pg + silu * pu
    return out


def down_col_sqnorm(W_down) -> np.ndarray:
    """||w^d_k||^2 for every neuron k (column k of W_down [hidden, I])."""
    W_down = _f64(W_down)
    return np.einsum("ck,ck->k", W_down, W_down)


def affinity_up(a, g, u, r, gamma, W_o, W_gate, W_up, W_down, group_of_head,
                G: Optional[int] = None, groups: Optional[Sequence[int]] = None,
                neurons: Optional[Sequence[int]] = None, token_chunk: int = 4096):
    """S_fo and S_add [G, I] (paper section 3, "Affinity scores").

    S_fo[g,k]  = sum_{h: group(h)=g} mean_t(Delta_thk^2) * ||w^d_k||^2
    S_add[g,k] = sum_{h: group(h)=g} mean_t((p_h.w^g_k)^2 + (p_h.w^u_k)^2)

    ``groups`` / ``neurons`` restrict the computation to a subset of rows and
    columns (the same literal arithmetic on fewer heads and neurons); the
    returned arrays then have shape [len(groups), len(neurons)].
    ``g``/``u`` and the weight rows must still be indexed by the full neuron
    range; only the selected columns are read.
    """
    a, r, gamma, W_o = _f64(a), _f64(r), _f64(gamma), _f64(W_o)
    grp = np.asarray(group_of_head, dtype=np.int64).reshape(-1)
    T, H, d = a.shape
    if G is None:
        G = int(grp.max()) + 1
    I_full = W_gate.shape[0]
    ks = np.arange(I_full) if neurons is None else np.asarray(neurons, dtype=np.int64)
    gs = list(range(G)) if groups is None else [int(x) for x in groups]
    row_of = {gg: i for i, gg in enumerate(gs)}
    W_gate_k = _f64(W_gate)[ks]                      # [n, hidden]
    W_up_k = _f64(W_up)[ks]
    wd2 = down_col_sqnorm(_f64(W_down)[:, ks])        # [n]
    fo = np.zeros((len(gs), len(ks)))
    add = np.zeros((len(gs), len(ks)))
    heads = [h for h in range(H) if int(grp[h]) in row_of]
    for t0 in range(0, T, token_chunk):
        t1 = min(T, t0 + token_chunk)
        g_c = _f64(g[t0:t1])[:, ks]
        u_c = _f64(u[t0:t1])[:, ks]
        _, silu, dsilu = silu_parts(g_c)
        A = dsilu * u_c
        for h in heads:
            p = head_piece(a[t0:t1, h, :], r[t0:t1], gamma, W_o, h)   # [Tc, hidden]
            pg = p @ W_gate_k.T                                        # p_h . w^g_k
            pu = p @ W_up_k.T                                          # p_h . w^u_k
            delta = A * pg + silu * pu                                 # eq. (5)
            row = row_of[int(grp[h])]
            fo[row] += np.sum(delta * delta, axis=0)
            add[row] += np.sum(pg * pg + pu * pu, axis=0)
    S_fo = fo / T * wd2[None, :]
    S_add = add / T
    return S_fo, S_add


def down_moment(g, u, r_next, token_chunk: int = 8192,
                neurons: Optional[Sequence[int]] = None) -> np.ndarray:
    """c_k = E_t[alpha_k^2 / r'^2] with alpha_k = silu(g_k) u_k (paper section 3).

    ``neurons`` restricts the result to those columns (same arithmetic)."""
    r_next = _f64(r_next)
    T = r_next.shape[0]
    acc = None
    for t0 in range(0, T, token_chunk):
        t1 = min(T, t0 + token_chunk)
        g_c, u_c = _f64(g[t0:t1]), _f64(u[t0:t1])
        if neurons is not None:
            ks = np.asarray(neurons, dtype=np.int64)
            g_c, u_c = g_c[:, ks], u_c[:, ks]
        _, silu, _ = silu_parts(g_c)
        q = silu * u_c / r_next[t0:t1, None]
        s = np.sum(q * q, axis=0)
        acc = s if acc is None else acc + s
    return acc / T


def qkv_rows_of_group(group_of_head_next, G_next: int, d_next: int, gp: int):
    """Row indices of W_q, W_k and W_v that make up W^qkv_g for next-layer group gp."""
    grp = np.asarray(group_of_head_next, dtype=np.int64).reshape(-1)
    q_rows = [h * d_next + j for h in range(grp.shape[0]) if grp[h] == gp
              for j in range(d_next)]
    kv_rows = list(range(gp * d_next, (gp + 1) * d_next))
    return q_rows, kv_rows


def down_weight_norms(W_q, W_k, W_v, gamma_next, W_down, group_of_head_next,
                      G_next: Optional[int] = None,
                      neurons: Optional[Sequence[int]] = None) -> np.ndarray:
    """n[g, k] = ||b_gk||^2 with b_gk = W^qkv_g (gamma' * w^d_k) (paper section 3).

    ``neurons`` restricts the result to those columns of W_down (same arithmetic)."""
    W_q, W_k, W_v = _f64(W_q), _f64(W_k), _f64(W_v)
    gamma_next, W_down = _f64(gamma_next), _f64(W_down)
    if neurons is not None:
        W_down = W_down[:, np.asarray(neurons, dtype=np.int64)]
    grp = np.asarray(group_of_head_next, dtype=np.int64).reshape(-1)
    if G_next is None:
        G_next = int(grp.max()) + 1
    d_next = W_k.shape[0] // G_next
    scaled = gamma_next[:, None] * W_down                  # column k = gamma' * w^d_k
    I = W_down.shape[1]
    n = np.zeros((G_next, I))
    for gp in range(G_next):
        q_rows, kv_rows = qkv_rows_of_group(grp, G_next, d_next, gp)
        W_g = np.concatenate([W_q[q_rows], W_k[kv_rows], W_v[kv_rows]], axis=0)
        b = W_g @ scaled                                   # [rows, I]: b_gk per column
        n[gp] = np.sum(b * b, axis=0)
    return n


def affinity_down(c: np.ndarray, n: np.ndarray) -> np.ndarray:
    """S_down[k, g] = c_k * n[g, k]."""
    return np.asarray(c)[:, None] * np.asarray(n).T


def affinity_layer(layer, token_chunk: int = 4096):
    """All three scores for one synthetic layer dict (keys as produced by synth)."""
    H = layer["a"].shape[1]
    grp = np.asarray(layer["group_of_head"]).reshape(-1)
    G = int(grp.max()) + 1
    S_fo, S_add = affinity_up(layer["a"], layer["g"], layer["u"], layer["r"],
                              layer["gamma"], layer["W_o"], layer["W_gate"],
                              layer["W_up"], layer["W_down"], grp, G=G,
                              token_chunk=token_chunk)
    out = {"S_fo": S_fo, "S_add": S_add}
    if "r_next" in layer and layer["r_next"] is not None:
        grp_n = np.asarray(layer["group_of_head_next"]).reshape(-1)
        Gn = int(grp_n.max()) + 1
        c = down_moment(layer["g"], layer["u"], layer["r_next"])
        n = down_weight_norms(layer["W_q"], layer["W_k"], layer["W_v"],
                              layer["gamma_next"], layer["W_down"], grp_n, G_next=Gn)
        out.update({"c_down": c, "n_down": n, "S_down": affinity_down(c, n)})
    return out
