"""Pins of the layout-objective oracle (unit mass and J, eq. (6)).

None of these tests retypes the objective.  They check the oracle against the
random-layout expectation computed by exhaustive enumeration, against the
expectations the pages print (tests/golden), against layouts whose value is
known in closed form (all mass co-located: 2N - 1; none: 0), against the
down edge's dependence on the *next* layer's head devices, and against the
invariances the definition implies (device relabelling, score scaling).
Source: "Affinity-Aware Sharding for Delayed Tensor Parallelism", section 3,
paragraph "Objective", eq. (6), and the caption of Table 3.
"""
import itertools
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "objective_random_expectation.txt")


def balanced_assignments(n, L):
    """Every labelled balanced map of n items onto L devices (n/L each)."""
    per = n // L
    out = []
    for perm in set(itertools.permutations(sorted(list(range(L)) * per))):
        out.append(np.array(perm))
    return out


def test_unit_mass():
    S = np.random.default_rng(1).lognormal(size=(5, 7))
    Sh = oracle.unit_mass(S)
    assert abs(Sh.sum() - 1.0) < 1e-13
    assert np.all(Sh >= 0)
    assert np.allclose(Sh[2, 3] / Sh[4, 1], S[2, 3] / S[4, 1], rtol=1e-13)
    assert np.allclose(oracle.unit_mass(3.5 * S), Sh, rtol=1e-13)   # scale free
    assert np.all(oracle.unit_mass(np.zeros((3, 4))) == 0)           # reading: empty -> 0


def test_random_expectation_by_enumeration():
    # N = 2 layers, G = 4 groups, I = 4 neurons, L = 2 devices: every balanced
    # layout enumerated (6 choices per map, 6^4 layouts); the mean of J is
    # (2N - 1)/L exactly for any non-negative scores.
    N, G, I, L = 2, 4, 4, 2
    rng = np.random.default_rng(3)
    S_up = rng.lognormal(size=(N, G, I))
    S_down = rng.lognormal(size=(N - 1, I, G))
    hs, ns = balanced_assignments(G, L), balanced_assignments(I, L)
    assert len(hs) == 6 and len(ns) == 6
    tot, cnt = 0.0, 0
    for h0, h1, n0, n1 in itertools.product(hs, hs, ns, ns):
        J, _, _ = oracle.layout_objective(S_up, S_down, np.stack([h0, h1]), np.stack([n0, n1]))
        tot += J
        cnt += 1
    assert abs(tot / cnt - (2 * N - 1) / L) < 1e-12


def test_range_and_extremes():
    N, G, I, L = 3, 4, 8, 2
    heads, neurons = (t.numpy() for t in synth.random_balanced_layout(N, G, I, L, seed=5))
    rng = np.random.default_rng(9)
    S_up = rng.lognormal(size=(N, G, I))
    S_down = rng.lognormal(size=(N - 1, I, G))
    J, fu, fd = oracle.layout_objective(S_up, S_down, heads, neurons)
    assert 0 <= J <= 2 * N - 1 and np.all((0 <= fu) & (fu <= 1)) and np.all((0 <= fd) & (fd <= 1))
    # keep only co-located entries: every matrix is fully co-located
    up_c = S_up * (heads[:, :, None] == neurons[:, None, :])
    down_c = S_down * (neurons[:-1, :, None] == heads[1:, None, :])
    J1, fu1, fd1 = oracle.layout_objective(up_c, down_c, heads, neurons)
    assert abs(J1 - (2 * N - 1)) < 1e-12 and np.allclose(fu1, 1) and np.allclose(fd1, 1)
    # keep only split entries: nothing is co-located
    J0, _, _ = oracle.layout_objective(S_up - up_c, S_down - down_c, heads, neurons)
    assert J0 == 0.0


def test_down_edge_uses_next_layer_heads():
    # layer 0 and layer 1 place the groups differently; the down edge's mass
    # sits on (k, g) pairs co-located under layer 1's head map only
    G, I, L = 2, 2, 2
    heads = np.array([[0, 1], [1, 0]])
    neurons = np.array([[0, 1], [0, 1]])
    S_up = np.ones((2, G, I))
    S_down = np.zeros((1, I, G))
    S_down[0, 0, 1] = 2.0   # neuron 0 (device 0) -> next-layer group 1 (device 0 in layer 1)
    S_down[0, 1, 0] = 1.0   # neuron 1 (device 1) -> next-layer group 0 (device 1 in layer 1)
    _, fu, fd = oracle.layout_objective(S_up, S_down, heads, neurons)
    assert fd[0] == 1.0                   # under layer 0's map it would be 0
    assert np.allclose(fu, [0.5, 0.5])    # half of a uniform matrix is co-located


def test_device_relabelling_and_contiguous_layout():
    N, G, I, L = 4, 8, 16, 4
    heads, neurons = (t.numpy() for t in synth.random_balanced_layout(N, G, I, L, seed=11))
    S_up, S_down = (t.numpy() for t in synth.make_scores(N, G, I, seed=2))
    J, _, _ = oracle.layout_objective(S_up, S_down, heads, neurons)
    perm = np.array([2, 0, 3, 1])
    Jp, _, _ = oracle.layout_objective(S_up, S_down, perm[heads], perm[neurons])
    assert abs(J - Jp) < 1e-12
    # contiguous: storage-order slices; block-diagonal scores are fully co-located
    hc, nc = (t.numpy() for t in synth.contiguous_layout(N, G, I, L))
    assert np.array_equal(hc[0], np.repeat(np.arange(L), G // L))
    assert np.array_equal(nc[0], np.repeat(np.arange(L), I // L))
    blk_up = np.kron(np.eye(L), np.ones((G // L, I // L)))[None].repeat(N, 0)
    blk_down = np.kron(np.eye(L), np.ones((I // L, G // L)))[None].repeat(N - 1, 0)
    Jc, _, _ = oracle.layout_objective(blk_up, blk_down, hc, nc)
    assert abs(Jc - (2 * N - 1)) < 1e-12


def golden_rows():
    rows = []
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            name, N, L, G, I, ex = line.split()
            rows.append((name, int(N), int(L), int(G), int(I), float(ex)))
    return rows


@pytest.mark.parametrize("row", golden_rows(), ids=lambda r: r[0])
def test_printed_random_expectation(row):
    # the pages' printed expectations, reproduced by averaging J over seeded
    # random balanced layouts of synthetic scores of those shapes
    name, N, L, G, I, expect = row
    assert abs((2 * N - 1) / L - expect) < 1e-12   # the printed value is (2N - 1)/L
    S_up, S_down = (t.numpy() for t in synth.make_scores(N, G, I, seed=N))
    Js = []
    for seed in range(40):
        heads, neurons = (t.numpy() for t in synth.random_balanced_layout(N, G, I, L, seed=seed))
        Js.append(oracle.layout_objective(S_up, S_down, heads, neurons)[0])
    Js = np.array(Js)
    se = Js.std(ddof=1) / np.sqrt(len(Js))
    assert abs(Js.mean() - expect) < 5 * se + 1e-3, (Js.mean(), se)
