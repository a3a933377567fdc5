"""Float64 CPU oracle of the layout search: the neuron step (the gain of
placing each neuron on each device, and the balanced assignment that
maximises it), the head step (the best balanced partition of each layer's KV
groups) and the coordinate-ascent sweeps that alternate them.

TEST INFRASTRUCTURE ONLY (like affinity.py and objective.py): imported by the
tests, the smoke check and the benchmark's CPU leg, never by the product path;
it shares no code with the HIP library.

Source: "Affinity-Aware Sharding for Delayed Tensor Parallelism", section 3,
paragraph "Optimiser", and appendix A (the iteration count and the step
decay).  Notation as in objective.py; L devices, cap = I / L neurons each.

Gain.  Given the head devices h_i of layer i and h_{i+1} of layer i+1,
    M[k, l] = sum_{g: h_i(g) = l} S_hat_up_i[g, k]
            + sum_{g: h_{i+1}(g) = l} S_hat_down_i[k, g]
(the last layer has no down edge).  For a balanced nu_i,
sum_k M[k, nu_i(k)] is the co-located mass layer i contributes to J through
its up edge and its down edge, so the best nu_i is a balanced linear
assignment on cap replicated slots per device.

Solver, in the pages' order:
  1. dual ascent on L device offsets lam_l: every neuron takes
     argmax_l (M[k, l] - lam_l), and each offset moves by the step times the
     device's excess load; 300 iterations, the step decaying by 0.98;
  2. a fix-up that meets the capacities exactly;
  3. pairwise swaps until no swap improves.

Readings where the pages are silent (each one stated where it is used):
  * M sums its up terms in increasing g, then its down terms in increasing g,
    starting from 0;
  * the excess load is normalised by the capacity, (count_l - cap) / cap, and
    the first step is one tenth of the range max(M) - min(M) of the layer's
    gains; the final assignment is the argmax under the offsets after the
    last update; ties go to the lowest device;
  * the fix-up repeatedly moves the single neuron, from a device above
    capacity to a device below it, that loses the least gain (ties: lowest
    neuron, then lowest target device);
  * a swap exchanges the devices of two neurons on different devices; each
    round takes the best swap of every device pair (l1 < l2), from the two
    separate best one-way moves, and performs the best of those if its gain
    is positive (ties: the first pair, then the lowest neurons); rounds stop
    when no swap improves or after max_swaps swaps.
Every decision compares float64 values computed by the operations written
here, in this order.

Head step.  Given nu_{i-1} and nu_i, putting KV group g of layer i on device
l gains
    A[g, l] = sum_{k: nu_i(k) = l} S_hat_up_i[g, k]
            + sum_{k: nu_{i-1}(k) = l} S_hat_down_{i-1}[k, g]
(the first layer has no down term), and the best balanced h_i maximises
sum_g A[g, h_i(g)] over all G! / ((G/L)!)^L labelled balanced partitions,
scored exhaustively.  Reading: the partitions are taken in lexicographic order
of (h(0), ..., h(G-1)) and ties go to the first.

Sweeps.  From the contiguous head assignment, one sweep runs the neuron step
of every layer (the layers are independent given all head devices), then the
head step of every layer (independent given all neuron devices), then
evaluates J.  Reading: sweeps continue while J strictly increases; the first
sweep that does not raise J is discarded and the search returns the layout
before it (also after max_sweeps sweeps).

Parity status: pinned by tests/test_layout_search_pins.py (the gain against
the co-located masses of the objective, the assignment against the Hungarian
solution on replicated slots and against enumeration of every balanced
assignment on tiny layers, swap-stability by exhaustive pair check, the fix-up
on tied gains, invariance under device relabelling; the partition count
2520, the head step against brute force over all L^G maps and against the
objective's co-located masses, J never falling across sweeps).
"""
from __future__ import annotations

import numpy as np

from .objective import layout_objective

__all__ = ["neuron_gain", "dual_ascent", "capacity_fixup", "pairwise_swaps", "neuron_step",
           "neuron_step_stack", "DUAL_ITERS", "DUAL_DECAY", "DUAL_STEP_FRAC",
           "balanced_partitions", "head_gain", "head_step", "head_step_stack", "layout_search"]

DUAL_ITERS = 300       # appendix A
DUAL_DECAY = 0.98      # appendix A
DUAL_STEP_FRAC = 0.1   # first step as a fraction of the gain range (reading)

# stats columns: status (0 ok, 2 swap limit reached), excess load left by the
# dual ascent, fix-up moves, swaps
STAT_OK, STAT_SWAP_LIMIT = 0, 2


def neuron_gain(S_up_hat, S_down_hat, heads, heads_next, L: int) -> np.ndarray:
    """M [I, L] float64.  S_up_hat [G, I]; S_down_hat [I, G] or None (last layer)."""
    S_up_hat = np.asarray(S_up_hat)
    G, I = S_up_hat.shape
    M = np.zeros((I, L), dtype=np.float64)
    for g in range(G):
        M[:, heads[g]] += S_up_hat[g].astype(np.float64)
    if S_down_hat is not None:
        S_down_hat = np.asarray(S_down_hat)
        for g in range(G):
            M[:, heads_next[g]] += S_down_hat[:, g].astype(np.float64)
    return M


def dual_ascent(M, L: int, iters: int = DUAL_ITERS, decay: float = DUAL_DECAY,
                step_frac: float = DUAL_STEP_FRAC):
    """Subgradient steps on the offsets; returns (assignment [I], offsets [L])."""
    I = M.shape[0]
    cap = I // L
    lam = np.zeros(L, dtype=np.float64)
    step = step_frac * (M.max() - M.min())
    for _ in range(iters):
        assign = np.argmax(M - lam, axis=1)            # first maximum = lowest device
        count = np.bincount(assign, minlength=L)
        lam = lam + step * ((count - cap) / cap)
        step = step * decay
    return np.argmax(M - lam, axis=1), lam


def capacity_fixup(M, assign, L: int):
    """Move neurons off over-full devices, least loss first; returns (assign, moves)."""
    I = M.shape[0]
    cap = I // L
    assign = np.array(assign, dtype=np.int64)
    moves = 0
    while True:
        count = np.bincount(assign, minlength=L)
        over, under = count > cap, count < cap
        if not over.any():
            return assign, moves
        own = M[np.arange(I), assign]
        cand = M - own[:, None]                        # gain change of moving k to l
        ok = over[assign][:, None] & under[None, :]
        cand = np.where(ok, cand, -np.inf)
        k, l = np.unravel_index(np.argmax(cand), cand.shape)   # row-major: lowest k, then l
        assign[k] = l
        moves += 1


def pairwise_swaps(M, assign, L: int, max_swaps: int):
    """Best-swap rounds until none improves; returns (assign, swaps, hit_limit)."""
    assign = np.array(assign, dtype=np.int64)
    swaps = 0
    while swaps < max_swaps:
        best_gain, best = 0.0, None
        for l1 in range(L):
            for l2 in range(l1 + 1, L):
                k1s = np.nonzero(assign == l1)[0]
                k2s = np.nonzero(assign == l2)[0]
                if len(k1s) == 0 or len(k2s) == 0:
                    continue
                d1 = M[k1s, l2] - M[k1s, l1]
                d2 = M[k2s, l1] - M[k2s, l2]
                i1, i2 = int(np.argmax(d1)), int(np.argmax(d2))
                gain = d1[i1] + d2[i2]
                if gain > best_gain:
                    best_gain, best = gain, (k1s[i1], k2s[i2])
        if best is None:
            return assign, swaps, False
        k1, k2 = best
        assign[k1], assign[k2] = assign[k2], assign[k1]
        swaps += 1
    return assign, swaps, True


def neuron_step(S_up_hat, S_down_hat, heads, heads_next, L: int, iters: int = DUAL_ITERS,
                max_swaps: int | None = None):
    """Best balanced neuron devices of one layer; returns (assign [I] int32, stats [4])."""
    M = neuron_gain(S_up_hat, S_down_hat, heads, heads_next, L)
    I = M.shape[0]
    if max_swaps is None:
        max_swaps = 4 * I
    a0, _ = dual_ascent(M, L, iters=iters)
    excess = int(np.maximum(np.bincount(a0, minlength=L) - I // L, 0).sum())
    a1, moves = capacity_fixup(M, a0, L)
    a2, swaps, hit = pairwise_swaps(M, a1, L, max_swaps)
    status = STAT_SWAP_LIMIT if hit else STAT_OK
    return a2.astype(np.int32), np.array([status, excess, moves, swaps], dtype=np.int32)


def neuron_step_stack(S_up_hat, S_down_hat, heads, L: int, iters: int = DUAL_ITERS,
                      max_swaps: int | None = None):
    """The neuron step of every layer of an N-layer stack, given all head devices.

    S_up_hat [N, G, I], S_down_hat [N-1, I, G], heads [N, G] (values in 0..L-1).
    Returns (neurons [N, I] int32, stats [N, 4] int32).
    """
    N = len(S_up_hat)
    out, stats = [], []
    for i in range(N):
        down = S_down_hat[i] if i + 1 < N else None
        nxt = heads[i + 1] if i + 1 < N else None
        a, st = neuron_step(S_up_hat[i], down, heads[i], nxt, L, iters, max_swaps)
        out.append(a)
        stats.append(st)
    return np.stack(out), np.stack(stats)


# ------------------------------------------------------------------ head step
def balanced_partitions(G: int, L: int) -> np.ndarray:
    """All maps {0..G-1} -> {0..L-1} with G/L groups per device, [P, G], in
    lexicographic order (built device by device, smallest first)."""
    per = G // L
    out = []

    def rec(prefix, left):
        if len(prefix) == G:
            out.append(list(prefix))
            return
        for v in range(L):
            if left[v]:
                left[v] -= 1
                prefix.append(v)
                rec(prefix, left)
                prefix.pop()
                left[v] += 1

    rec([], [per] * L)
    return np.array(out, dtype=np.int64).reshape(-1, G)


def head_gain(S_up_hat, S_down_prev, neurons, neurons_prev, L: int) -> np.ndarray:
    """A [G, L] float64.  S_up_hat [G, I] of layer i; S_down_prev [I, G] of
    layer i-1 (None for the first layer) with that layer's neuron devices."""
    S_up_hat = np.asarray(S_up_hat, dtype=np.float64)
    G = S_up_hat.shape[0]
    A = np.zeros((G, L), dtype=np.float64)
    for l in range(L):
        A[:, l] = S_up_hat[:, np.asarray(neurons) == l].sum(axis=1)
        if S_down_prev is not None:
            A[:, l] += np.asarray(S_down_prev, dtype=np.float64)[np.asarray(neurons_prev) == l].sum(axis=0)
    return A


def head_step(S_up_hat, S_down_prev, neurons, neurons_prev, L: int):
    """Best balanced head map of one layer by exhaustive scoring.

    Returns (h [G] int32, best score, second-best score (-inf if only one))."""
    A = head_gain(S_up_hat, S_down_prev, neurons, neurons_prev, L)
    G = A.shape[0]
    parts = balanced_partitions(G, L)
    scores = A[np.arange(G)[None, :], parts].sum(axis=1)
    best = int(np.argmax(scores))                   # first maximum in lexicographic order
    rest = np.delete(scores, best)
    second = float(rest.max()) if rest.size else -np.inf
    return parts[best].astype(np.int32), float(scores[best]), second


def head_step_stack(S_up_hat, S_down_hat, neurons, L: int):
    """The head step of every layer given all neuron devices.

    Returns (heads [N, G] int32, scores [N], second-best scores [N])."""
    N = len(S_up_hat)
    hs, sc, sec = [], [], []
    for i in range(N):
        prev = S_down_hat[i - 1] if i > 0 else None
        nprev = neurons[i - 1] if i > 0 else None
        h, b, s2 = head_step(S_up_hat[i], prev, neurons[i], nprev, L)
        hs.append(h)
        sc.append(b)
        sec.append(s2)
    return np.stack(hs), np.array(sc), np.array(sec)


# --------------------------------------------------------------------- sweeps
def layout_search(S_up_hat, S_down_hat, L: int, heads0=None, iters: int = DUAL_ITERS,
                  max_swaps: int | None = None, max_sweeps: int = 16):
    """Coordinate ascent over the chain of layers.

    Returns a dict: heads [N, G], neurons [N, I] (the best layout), J (its
    objective), J_history (J after every sweep run, the last one possibly not
    kept), sweeps (the number run), head_margin (the smallest relative gap
    between the best and second-best head partition over all head steps of
    the kept sweeps), neuron_stats [N, 4] of the last kept sweep."""
    S_up_hat = np.asarray(S_up_hat)
    N, G, I = S_up_hat.shape
    if heads0 is None:
        heads0 = np.tile(np.arange(G) // (G // L), (N, 1))
    heads = np.asarray(heads0, dtype=np.int64)
    best = None
    history = []
    margin = np.inf
    for _ in range(max_sweeps):
        nu, stats = neuron_step_stack(S_up_hat, S_down_hat, heads, L, iters, max_swaps)
        h_new, sc, sec = head_step_stack(S_up_hat, S_down_hat, nu, L)
        J, _, _ = layout_objective(S_up_hat, S_down_hat, h_new, nu)
        history.append(J)
        if best is not None and not J > best["J"]:
            break
        gap = np.min((sc - sec) / np.maximum(np.abs(sc), 1e-300))
        best = {"heads": h_new, "neurons": nu, "J": J, "neuron_stats": stats,
                "head_margin": min(margin, gap)}
        margin = best["head_margin"]
        heads = h_new
    best["J_history"] = np.array(history)
    best["sweeps"] = len(history)
    return best
