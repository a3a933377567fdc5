"""Pins of the neuron-step oracle (section 3, paragraph "Optimiser"; appendix A)
to facts outside its own code: the objective's co-located masses, the exact
Hungarian solution, exhaustive enumeration, exhaustive swap checks."""
import itertools

import numpy as np
import pytest
from scipy.optimize import linear_sum_assignment

import oracle
import synth


def unit_stack(N, G, I, seed, dtype=np.float32, **kw):
    S_up, S_down = synth.make_scores(N, G, I, seed, **kw)
    up = np.stack([oracle.unit_mass(S_up[i].numpy()) for i in range(N)]).astype(dtype)
    down = np.stack([oracle.unit_mass(S_down[i].numpy()) for i in range(N - 1)]).astype(dtype)
    return up, down


def value(M, a):
    return float(M[np.arange(M.shape[0]), a].sum())


def hungarian_value(M, L):
    cap = M.shape[0] // L
    C = np.repeat(M, cap, axis=1)              # column j is a slot of device j // cap
    r, c = linear_sum_assignment(C, maximize=True)
    return float(C[r, c].sum())


def test_gain_is_the_layers_colocated_mass():
    # for any balanced layout, sum_k M_i[k, nu_i(k)] is the co-located mass of
    # layer i's up edge plus its down edge, as the objective measures them
    N, G, I, L = 3, 8, 64, 4
    up, down = unit_stack(N, G, I, seed=1, dtype=np.float64)   # exactly unit mass
    heads, neurons = (t.numpy() for t in synth.random_balanced_layout(N, G, I, L, seed=1))
    _, fu, fd = oracle.layout_objective(up, down, heads, neurons)
    for i in range(N):
        M = oracle.neuron_gain(up[i], down[i] if i + 1 < N else None, heads[i],
                               heads[i + 1] if i + 1 < N else None, L)
        expect = fu[i] + (fd[i] if i + 1 < N else 0.0)
        assert abs(value(M, neurons[i]) - expect) < 1e-12
    # every neuron's gains sum to its share of both matrices
    M = oracle.neuron_gain(up[0], down[0], heads[0], heads[1], L)
    assert np.allclose(M.sum(1), up[0].sum(0) + down[0].sum(1), rtol=1e-12, atol=0)


@pytest.mark.parametrize("G,I,L,sigma,zero_frac,seed", [
    (8, 768, 4, 1.0, 0.0, 2), (8, 768, 4, 2.0, 0.0, 3), (8, 512, 4, 1.0, 0.5, 4),
    (8, 512, 2, 1.0, 0.0, 5), (8, 512, 8, 1.5, 0.0, 6)])
def test_matches_hungarian_on_replicated_slots(G, I, L, sigma, zero_frac, seed):
    # the pages report agreement with the Hungarian solution to 1e-6
    up, down = unit_stack(2, G, I, seed, sigma=sigma, zero_frac=zero_frac)
    heads, _ = (t.numpy() for t in synth.random_balanced_layout(2, G, I, L, seed))
    for i, (d, hn) in enumerate([(down[0], heads[1]), (None, None)]):
        M = oracle.neuron_gain(up[i], d, heads[i], hn, L)
        a, stats = oracle.neuron_step(up[i], d, heads[i], hn, L)
        assert np.array_equal(np.bincount(a, minlength=L), np.full(L, I // L))
        assert stats[0] == 0
        best = hungarian_value(M, L)
        assert (best - value(M, a)) <= 1e-6 * best


def test_matches_enumeration_on_a_tiny_layer():
    # I = 8 neurons on L = 4 devices: all 8!/(2!^4) = 2520 balanced assignments
    G, I, L = 4, 8, 4
    rng = np.random.default_rng(7)
    for trial in range(5):
        up = rng.lognormal(size=(G, I)).astype(np.float32)
        down = rng.lognormal(size=(I, G)).astype(np.float32)
        h, hn = rng.permutation(np.repeat(np.arange(L), G // L)), rng.permutation(np.repeat(np.arange(L), G // L))
        M = oracle.neuron_gain(up, down, h, hn, L)
        best = max(value(M, np.array(p)) for p in set(itertools.permutations(np.repeat(np.arange(L), I // L))))
        a, _ = oracle.neuron_step(up, down, h, hn, L)
        assert abs(value(M, a) - best) <= 1e-12 * best


def test_swaps_reach_a_swap_stable_assignment():
    # from a random balanced start (no dual ascent), the swap phase ends where
    # no exchange of two neurons on different devices gains, and never loses
    I, L = 96, 4
    rng = np.random.default_rng(8)
    M = rng.lognormal(size=(I, L))
    a0 = rng.permutation(np.repeat(np.arange(L), I // L))
    a, n, hit = oracle.pairwise_swaps(M, a0, L, max_swaps=10 * I)
    assert not hit and n > 0
    assert np.array_equal(np.bincount(a, minlength=L), np.bincount(a0, minlength=L))
    assert value(M, a) >= value(M, a0)
    own = M[np.arange(I), a]
    cross = M[:, a]                      # cross[k1, k2] = M[k1, a[k2]]
    gain = cross + cross.T - own[:, None] - own[None, :]
    assert gain.max() <= 1e-12
    # the swap limit is honoured and reported
    _, n2, hit2 = oracle.pairwise_swaps(M, a0, L, max_swaps=3)
    assert hit2 and n2 == 3


def test_fixup_on_tied_gains():
    # constant gains: the offsets never move (zero range), every neuron takes
    # device 0, and the fix-up moves (L-1) * cap of them, lowest neurons first
    I, L = 16, 4
    cap = I // L
    M = np.full((I, L), 0.25)
    a0, lam = oracle.dual_ascent(M, L)
    assert np.all(a0 == 0) and np.all(lam == 0)
    a, moves = oracle.capacity_fixup(M, a0, L)
    assert moves == (L - 1) * cap
    assert np.array_equal(np.bincount(a, minlength=L), np.full(L, cap))
    # ties go to the lowest neuron, then the lowest target: 0..3 -> 1, 4..7 -> 2, ...
    assert np.array_equal(a, np.r_[np.repeat(np.arange(1, L), cap), np.zeros(cap, int)])


def test_dual_ascent_balances_generic_layers():
    # with continuous scores the offsets alone reach the capacities (the fix-up
    # and the swaps then have nothing to do) on the pages' shapes
    up, down = unit_stack(2, 8, 3072, seed=9)
    heads, _ = (t.numpy() for t in synth.contiguous_layout(2, 8, 3072, 4))
    _, stats = oracle.neuron_step(up[0], down[0], heads[0], heads[1], 4)
    assert stats.tolist() == [0, 0, 0, 0]


def test_device_relabelling_permutes_the_assignment():
    G, I, L = 8, 256, 4
    up, down = unit_stack(2, G, I, seed=10)
    heads, _ = (t.numpy() for t in synth.random_balanced_layout(2, G, I, L, seed=10))
    perm = np.array([3, 1, 0, 2])
    a, _ = oracle.neuron_step(up[0], down[0], heads[0], heads[1], L)
    b, _ = oracle.neuron_step(up[0], down[0], perm[heads[0]], perm[heads[1]], L)
    assert np.array_equal(b, perm[a])


def test_stack_step_does_not_lower_the_objective():
    N, G, I, L = 4, 8, 512, 4
    up, down = unit_stack(N, G, I, seed=12)
    heads, neurons = (t.numpy() for t in synth.contiguous_layout(N, G, I, L))
    J0, _, _ = oracle.layout_objective(up, down, heads, neurons)
    nu, stats = oracle.neuron_step_stack(up, down, heads, L)
    J1, _, _ = oracle.layout_objective(up, down, heads, nu)
    assert J1 >= J0 and np.all(stats[:, 0] == 0)
    for i in range(N):
        assert np.array_equal(np.bincount(nu[i], minlength=L), np.full(L, I // L))


# ------------------------------------------------------------------ head step
def test_partition_count_and_order():
    # the pages count G!/((G/L)!)^L = 2520 labelled balanced partitions for G = 8, L = 4
    import math
    for G, L in [(8, 4), (6, 3), (4, 2), (8, 2), (8, 8), (4, 1)]:
        P = oracle.balanced_partitions(G, L)
        assert len(P) == math.factorial(G) // math.factorial(G // L) ** L
        assert np.all(np.stack([np.bincount(p, minlength=L) for p in P]) == G // L)
        assert len({tuple(p) for p in P}) == len(P)
        keys = [tuple(p) for p in P]
        assert keys == sorted(keys)
    assert len(oracle.balanced_partitions(8, 4)) == 2520


def test_head_step_against_brute_force_objective():
    # every map {0..G-1} -> {0..L-1} is tried; a balanced one's score is the
    # co-located mass it gives layer i's up edge and layer i-1's down edge, as
    # the objective measures them
    N, G, I, L = 3, 8, 96, 4
    up, down = unit_stack(N, G, I, seed=13, dtype=np.float64)
    heads, neurons = (t.numpy() for t in synth.random_balanced_layout(N, G, I, L, seed=13))
    for i in (0, 1, 2):
        h, best, second = oracle.head_step(up[i], down[i - 1] if i else None, neurons[i],
                                           neurons[i - 1] if i else None, L)
        top = -1.0
        for cand in itertools.product(range(L), repeat=G):
            cand = np.array(cand)
            if np.any(np.bincount(cand, minlength=L) != G // L):
                continue
            hh = heads.copy()
            hh[i] = cand
            _, fu, fd = oracle.layout_objective(up, down, hh, neurons)
            top = max(top, fu[i] + (fd[i - 1] if i else 0.0))
        assert abs(best - top) < 1e-12 and second <= best
        hh = heads.copy()
        hh[i] = h
        _, fu, fd = oracle.layout_objective(up, down, hh, neurons)
        assert abs(fu[i] + (fd[i - 1] if i else 0.0) - best) < 1e-12


def test_sweeps_raise_the_objective_and_stop():
    N, G, I, L = 6, 8, 512, 4
    up, down = unit_stack(N, G, I, seed=14)
    res = oracle.layout_search(up, down, L)
    hist = res["J_history"]
    kept = hist[:-1] if len(hist) > 1 and not hist[-1] > hist[-2] else hist
    assert np.all(np.diff(kept) > 0)                  # every kept sweep raised J
    assert res["J"] == kept[-1]
    assert 1 <= res["sweeps"] <= 16
    heads0, nu0 = (t.numpy() for t in synth.contiguous_layout(N, G, I, L))
    J0, _, _ = oracle.layout_objective(up, down, heads0, nu0)
    assert res["J"] > J0
    assert 0 <= res["J"] <= 2 * N - 1
    for i in range(N):
        assert np.all(np.bincount(res["heads"][i], minlength=L) == G // L)
        assert np.all(np.bincount(res["neurons"][i], minlength=L) == I // L)
    # the reported J is the objective of the returned layout
    J, _, _ = oracle.layout_objective(up, down, res["heads"], res["neurons"])
    assert abs(J - res["J"]) < 1e-12


def test_exact_division_by_odd_inverse():
    """The head step divides mc * c_v by n (1 <= n <= 16, the quotient an exact
    integer below 2^28) in 32-bit integers: n's power of two is shifted out,
    then the product is multiplied by the odd part's inverse mod 2^32, found by
    four Newton-Hensel steps x <- x (2 - o x) from x = o.  Checked here for
    every n and a range of quotients, including the largest."""
    M = 1 << 32
    for n in range(1, 17):
        tz = (n & -n).bit_length() - 1
        o = n >> tz
        x = o
        for _ in range(4):
            x = (x * (2 - o * x)) % M
        assert (o * x) % M == 1
        for q in list(range(0, 4096)) + [(1 << 24) - 1, (1 << 28) // n - 1]:
            assert (((q * n) >> tz) * x) % M == q
