"""Float64 CPU oracle of the layout objective: unit-mass normalisation and the
total co-located affinity J.

TEST INFRASTRUCTURE ONLY (like affinity.py): imported by the tests, the smoke
check and the benchmark's CPU leg, never by the product path; it shares no code
with the HIP library.

Source: "Affinity-Aware Sharding for Delayed Tensor Parallelism", section 3,
paragraph "Objective", equation (6), and the caption of Table 3.  Notation:

  S_up_i  [G, I]   the up-edge scores of layer i (KV group g -> neuron k)
  S_down_i [I, G]  the down-edge scores from layer i's neurons to layer i+1's
                   KV groups (i = 0 .. N-2)
  h_i(g)           the device of KV group g in layer i
  nu_i(k)          the device of neuron k in layer i
  unit mass        S_hat = S / sum(S), per matrix
  J(h, nu) = sum_{i=0}^{N-1} sum_{g,k: h_i(g) = nu_i(k)} S_hat_up_i[g, k]
           + sum_{i=0}^{N-2} sum_{k,g: nu_i(k) = h_{i+1}(g)} S_hat_down_i[k, g]

Each of the 2N - 1 terms is the co-located fraction of one matrix, so J lies
in [0, 2N - 1] and a uniformly random balanced layout scores (2N - 1)/L in
expectation.  Readings where the pages are silent: a matrix whose total is 0
normalises to 0 (it adds nothing to J); device ids are compared for equality
only.

Parity status: pinned by tests/test_objective_pins.py (unit mass, the exact
random-layout expectation by enumeration, extreme layouts, the down edge's
use of the next layer's head devices, device relabelling, the printed random
expectations 13.75 and 7.75).
"""
from __future__ import annotations

import numpy as np

__all__ = ["unit_mass", "colocated_mass", "layout_objective"]


def unit_mass(S) -> np.ndarray:
    """S / sum(S) in float64 (0 where the total is 0)."""
    S = np.asarray(S, dtype=np.float64)
    tot = S.sum()
    return S / tot if tot != 0 else np.zeros_like(S)


def colocated_mass(S_hat, dev_rows, dev_cols) -> float:
    """Sum of S_hat[r, c] over the entries whose row and column devices match."""
    S_hat = np.asarray(S_hat, dtype=np.float64)
    same = np.asarray(dev_rows)[:, None] == np.asarray(dev_cols)[None, :]
    return float(S_hat[same].sum())


def layout_objective(S_up, S_down, heads, neurons):
    """J (eq. 6) and the per-matrix co-located fractions.

    S_up [N, G, I], S_down [N-1, I, G], heads [N, G], neurons [N, I].
    Returns (J, frac_up [N], frac_down [N-1]), all float64.
    """
    S_up = np.asarray(S_up, dtype=np.float64)
    S_down = np.asarray(S_down, dtype=np.float64)
    heads = np.asarray(heads)
    neurons = np.asarray(neurons)
    N = S_up.shape[0]
    if S_down.shape[0] != max(N - 1, 0):
        raise ValueError("S_down must hold N - 1 matrices")
    frac_up = np.array([colocated_mass(unit_mass(S_up[i]), heads[i], neurons[i]) for i in range(N)])
    frac_down = np.array([colocated_mass(unit_mass(S_down[i]), neurons[i], heads[i + 1])
                          for i in range(N - 1)])
    return float(frac_up.sum() + frac_down.sum()), frac_up, frac_down
