"""Float64 CPU oracle of the exact leave-one-out score of the pre-activations.

TEST INFRASTRUCTURE ONLY (like affinity.py): imported by the tests, the smoke
check and the benchmark's CPU leg, never by the product path; it shares no code
with the HIP library.

Source: "Affinity-Aware Sharding for Delayed Tensor Parallelism", section 3,
paragraph "Affinity scores": besides ADD, the pages compute exact leave-one-out
ablation scores of the pre-activations, which differ from ADD only in keeping
the change of the norm's rms when a head is removed.  Written out, with the
notation of affinity.py:

  o_h       = a_h W_o^(h)T                 head h's write into the residual
  x^(-h)    = x - o_h,   r^(-h) = rms(x^(-h))
  g^(-h)    = (gamma * x^(-h) / r^(-h)) W_gate^T,  u^(-h) likewise
  g         = (gamma * x / r) W_gate^T with r = rms(x),  u likewise
  S_loo[g,k] = sum_{h in group g} E_t[(g_k - g_k^(-h))^2 + (u_k - u_k^(-h))^2]

Readings: the ablated pass recomputes the rms of the residual (no epsilon) and
keeps gamma and the weights; the full pass is recomputed from the same x (the
layer's stored pre-activations are not used here); E_t is the plain mean over
the tokens; a group's score is the sum over its query heads, as for ADD; a
token whose residual vanishes without head h (r^(-h) = 0) contributes nothing
for that head.

Everything is the literal computation: for every head the residual is
ablated, renormalised and projected in full with numpy matmuls, token chunk by
token chunk (chunk sums added in order).

Parity status: pinned by tests/test_loo_pins.py (a hand-computed two-
dimensional example, equality with ADD of affinity.py when removing the head
leaves the rms unchanged, the algebraic split into a rescaled pre-activation
plus the rescaled head piece of affinity.py, zero heads, group sums of head
rows, token duplication).
"""
from __future__ import annotations

import numpy as np

__all__ = ["loo_scores"]


def _f64(t) -> np.ndarray:
    if hasattr(t, "detach"):
        t = t.detach().cpu()
        if str(t.dtype) == "torch.bfloat16":
            t = t.float()
        t = t.numpy()
    return np.asarray(t, dtype=np.float64)


def _rms(v: np.ndarray) -> np.ndarray:
    return np.sqrt((v * v).mean(axis=1))


def loo_scores(a, x, gamma, W_o, W_gate, W_up, group_of_head, G: int | None = None,
               token_chunk: int = 2048, neurons=None) -> np.ndarray:
    """S_loo [G, I] float64.  a [T, H, d], x [T, hidden], W_o [hidden, H*d],
    W_gate, W_up [I, hidden], gamma [hidden], group_of_head [H].  ``neurons``
    restricts the output to those columns (the same arithmetic on fewer
    neurons; the result is then [G, len(neurons)])."""
    a, x, gamma = _f64(a), _f64(x), _f64(gamma)
    W_o, W_gate, W_up = _f64(W_o), _f64(W_gate), _f64(W_up)
    if neurons is not None:
        W_gate, W_up = W_gate[np.asarray(neurons)], W_up[np.asarray(neurons)]
    grp = np.asarray(group_of_head).reshape(-1)
    T, H, d = a.shape
    I = W_gate.shape[0]
    if G is None:
        G = int(grp.max()) + 1
    acc = np.zeros((G, I))
    for t0 in range(0, T, token_chunk):
        xs = x[t0:t0 + token_chunk]
        y = gamma[None, :] * xs / _rms(xs)[:, None]
        g_full, u_full = y @ W_gate.T, y @ W_up.T
        for h in range(H):
            o = a[t0:t0 + token_chunk, h, :] @ W_o[:, h * d:(h + 1) * d].T
            xm = xs - o
            rm = _rms(xm)
            keep = rm > 0
            ym = gamma[None, :] * xm[keep] / rm[keep][:, None]
            dg = g_full[keep] - ym @ W_gate.T
            du = u_full[keep] - ym @ W_up.T
            acc[grp[h]] += (dg * dg + du * du).sum(axis=0)
    return acc / T
