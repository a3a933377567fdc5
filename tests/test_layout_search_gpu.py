"""Parity of the neuron step of the layout search (section 3, "Optimiser") on
the GPU, through the C ABI, against the float64 oracle.

Both sides take every decision on the same fp32 unit-mass inputs with fp64
values computed by the same operations in the same order, so the assignment
and the statistics (status, excess after the dual ascent, fix-up moves,
swaps) must agree exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hna():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_neuron_affinity_amd as m
    m.lib()
    return m


def unit_stack(N, G, I, seed, **kw):
    S_up, S_down = synth.make_scores(N, G, I, seed, **kw)
    up = np.stack([oracle.unit_mass(S_up[i].numpy()) for i in range(N)]).astype(np.float32)
    down = np.zeros((N - 1, I, G), np.float32)
    for i in range(N - 1):
        down[i] = oracle.unit_mass(S_down[i].numpy())
    return up, down


def gpu_step(hna, up, down, heads, L, **kw):
    N = up.shape[0]
    nu, st = hna.neuron_step(torch.from_numpy(up).cuda(),
                             torch.from_numpy(down).cuda() if N > 1 else None,
                             torch.from_numpy(np.ascontiguousarray(heads, dtype=np.int32)).cuda(),
                             L, **kw)
    torch.cuda.synchronize()
    return nu.cpu().numpy(), st.cpu().numpy()


def check(hna, up, down, heads, L, iters=oracle.DUAL_ITERS, max_swaps=None):
    N, G, I = up.shape
    kw = {} if max_swaps is None else {"max_swaps": max_swaps}
    nu, st = gpu_step(hna, up, down, heads, L, iters=iters, **kw)
    ref, rst = oracle.neuron_step_stack(up, down, heads, L, iters=iters, max_swaps=max_swaps)
    print(f"  N={N} G={G} I={I} L={L} iters={iters}: stats {st.sum(0).tolist()} "
          f"differing neurons {(nu != ref).sum()}", flush=True)
    assert np.array_equal(st, rst)
    assert np.array_equal(nu, ref)
    return nu, st


@pytest.mark.parametrize("N,G,I,L,seed,kw", [
    (4, 8, 3072, 4, 0, {}),                         # the Qwen3-0.6B layer shape
    (3, 8, 1000, 4, 1, {}),                         # a partial last row of threads
    (2, 16, 4096, 4, 2, {"sigma": 2.0}),            # the Danube3 width, skewed scores
    (2, 8, 2048, 8, 3, {}),                         # eight devices
    (1, 8, 512, 2, 4, {}),                          # one layer: no down edge
    (3, 8, 768, 4, 5, {"zero_frac": 0.5}),          # sparse scores
    (2, 4, 100, 1, 6, {}),                          # one device
])
def test_neuron_step_matches_oracle(hna, N, G, I, L, seed, kw):
    up, down = unit_stack(N, G, I, seed, **kw)
    heads, _ = synth.random_balanced_layout(N, G, I, L, seed)
    check(hna, up, down, heads.numpy(), L)


def test_fixup_and_swaps_without_dual_ascent(hna):
    # no dual iterations: the argmax start is far from balanced, so the fix-up
    # and the swap phase carry the whole solve
    up, down = unit_stack(3, 8, 512, seed=7)
    heads, _ = synth.random_balanced_layout(3, 8, 512, 4, seed=7)
    _, st = check(hna, up, down, heads.numpy(), 4, iters=0)
    assert st[:, 2].min() > 0 and st[:, 3].min() > 0
    _, st = check(hna, up, down, heads.numpy(), 4, iters=0, max_swaps=5)
    assert np.all(st[:, 0] == 2) and np.all(st[:, 3] == 5)


def test_tied_gains(hna):
    # constant scores: every gain is equal, the offsets never move and the
    # fix-up places every neuron by the tie rule
    N, G, I, L = 2, 8, 256, 4
    up = np.full((N, G, I), 1.0 / (G * I), np.float32)
    down = np.full((N - 1, I, G), 1.0 / (G * I), np.float32)
    heads, _ = synth.contiguous_layout(N, G, I, L)
    _, st = check(hna, up, down, heads.numpy(), L)
    assert np.all(st[:, 2] == (L - 1) * (I // L))


def test_bad_head_devices_fail_their_layers_only(hna):
    N, G, I, L = 3, 8, 512, 4
    up, down = unit_stack(N, G, I, seed=8)
    heads = synth.random_balanced_layout(N, G, I, L, seed=8)[0].numpy().copy()
    heads[1, 3] = L                      # layer 1's map is broken: layers 0 and 1 use it
    nu, st = gpu_step(hna, up, down, heads, L)
    assert st[0, 0] == st[1, 0] == 1 and np.all(nu[:2] == -1)
    ref, rst = oracle.neuron_step(up[2], None, heads[2], None, L)
    assert st[2].tolist() == rst.tolist() and np.array_equal(nu[2], ref)


def test_full_stack_determinism_and_objective(hna):
    # the 28-layer Qwen3-0.6B stack on 4 devices, from the contiguous heads
    N, G, I, L = 28, 8, 3072, 4
    up, down = unit_stack(N, G, I, seed=9)
    heads, neurons0 = (t.numpy() for t in synth.contiguous_layout(N, G, I, L))
    nu, st = check(hna, up, down, heads, L)
    nu2, st2 = gpu_step(hna, up, down, heads, L)
    assert np.array_equal(nu, nu2) and np.array_equal(st, st2)
    J0, _, _ = hna.layout_objective(torch.from_numpy(up).cuda(), torch.from_numpy(down).cuda(),
                                    torch.from_numpy(heads).cuda(), torch.from_numpy(neurons0).cuda())
    J1, _, _ = hna.layout_objective(torch.from_numpy(up).cuda(), torch.from_numpy(down).cuda(),
                                    torch.from_numpy(heads).cuda(), torch.from_numpy(nu).cuda())
    print(f"  J contiguous {float(J0.cpu()[0]):.4f} -> neuron step {float(J1.cpu()[0]):.4f}", flush=True)
    assert float(J1.cpu()[0]) > float(J0.cpu()[0])


# ------------------------------------------------------------------ head step
def oracle_head_check(up, down, nu, L, heads, score):
    """GPU head maps against the oracle: the best score to 1e-12 (relative);
    the map itself where the best partition is unique beyond rounding,
    otherwise the GPU's map must score within 1e-12 of the best."""
    N = up.shape[0]
    for i in range(N):
        prev, nprev = (down[i - 1], nu[i - 1]) if i else (None, None)
        h, best, second = oracle.head_step(up[i], prev, nu[i], nprev, L)
        assert abs(score[i] - best) <= 1e-12 * abs(best)
        if best - second > 1e-12 * abs(best):
            assert np.array_equal(heads[i], h), i
        else:
            A = oracle.head_gain(up[i], prev, nu[i], nprev, L)
            assert abs(A[np.arange(len(h)), heads[i]].sum() - best) <= 1e-12 * abs(best)
            assert np.all(np.bincount(heads[i], minlength=L) == len(h) // L)


@pytest.mark.parametrize("N,G,I,L,seed", [
    (4, 8, 3072, 4, 20),    # 2520 partitions, the pages' count
    (3, 8, 1000, 4, 21),
    (2, 16, 512, 2, 22),    # 12870 partitions
    (2, 8, 512, 8, 23),     # 40320 partitions
    (2, 12, 600, 4, 24),    # 369600 partitions: many per thread
    (1, 8, 512, 4, 25),     # one layer: no down term
    (3, 4, 100, 1, 26),     # one device: a single partition
])
def test_head_step_matches_oracle(hna, N, G, I, L, seed):
    up, down = unit_stack(N, G, I, seed)
    _, nu = synth.random_balanced_layout(N, G, I, L, seed)
    nu = nu.numpy()
    heads, score, status = hna.head_step(torch.from_numpy(up).cuda(),
                                         torch.from_numpy(down).cuda() if N > 1 else None,
                                         torch.from_numpy(nu).cuda(), L)
    torch.cuda.synchronize()
    heads, score, status = heads.cpu().numpy(), score.cpu().numpy(), status.cpu().numpy()
    print(f"  N={N} G={G} I={I} L={L}: scores {np.round(score, 4).tolist()}", flush=True)
    assert np.all(status == 0)
    oracle_head_check(up, down, nu, L, heads, score)


def test_head_step_bad_neuron_devices(hna):
    N, G, I, L = 4, 8, 256, 4
    up, down = unit_stack(N, G, I, seed=27)
    nu = synth.random_balanced_layout(N, G, I, L, seed=27)[1].numpy().copy()
    nu[1, 5] = -3                       # layers 1 and 2 read layer 1's neuron devices
    heads, score, status = hna.head_step(torch.from_numpy(up).cuda(), torch.from_numpy(down).cuda(),
                                         torch.from_numpy(nu).cuda(), L)
    torch.cuda.synchronize()
    heads, status = heads.cpu().numpy(), status.cpu().numpy()
    assert status.tolist() == [0, 4, 4, 0]
    assert np.all(heads[1:3] == -1)
    for i in (0, 3):
        h, _, _ = oracle.head_step(up[i], down[i - 1] if i else None, nu[i], nu[i - 1] if i else None, L)
        assert np.array_equal(heads[i], h)


# --------------------------------------------------------------------- sweeps
def run_search(hna, up, down, L, heads0=None):
    r = hna.layout_search(torch.from_numpy(up).cuda(), torch.from_numpy(down).cuda(), L,
                          head_device=None if heads0 is None else torch.from_numpy(heads0).cuda())
    torch.cuda.synchronize()
    return r


def check_search(hna, up, down, L, heads0=None):
    r = run_search(hna, up, down, L, heads0)
    ref = oracle.layout_search(up, down, L, heads0=heads0)
    print(f"  J {np.round(r['J_history'], 6).tolist()} vs {np.round(ref['J_history'], 6).tolist()}, "
          f"sweeps {r['sweeps']} vs {ref['sweeps']}, head margin {ref['head_margin']:.2e}", flush=True)
    assert ref["head_margin"] > 1e-9       # every head decision is unique beyond rounding
    assert r["sweeps"] == ref["sweeps"]
    assert np.allclose(r["J_history"], ref["J_history"], rtol=0, atol=1e-9)
    assert np.array_equal(r["heads"].cpu().numpy(), ref["heads"])
    assert np.array_equal(r["neurons"].cpu().numpy(), ref["neurons"])
    assert np.array_equal(r["neuron_stats"].cpu().numpy(), ref["neuron_stats"])
    return r, ref


def test_search_from_contiguous_heads_full_stack(hna):
    # the 28-layer Qwen3-0.6B stack on 4 devices, as the pages start it
    up, down = unit_stack(28, 8, 3072, seed=30)
    r, _ = check_search(hna, up, down, 4)
    assert 2 <= r["sweeps"] <= 4


def test_search_from_random_heads(hna):
    N, G, I, L = 6, 8, 512, 4
    up, down = unit_stack(N, G, I, seed=31)
    heads0 = synth.random_balanced_layout(N, G, I, L, seed=31)[0].numpy()
    check_search(hna, up, down, L, heads0)


def test_search_rejects_bad_start(hna):
    up, down = unit_stack(3, 8, 256, seed=32)
    heads0 = synth.contiguous_layout(3, 8, 256, 4)[0].numpy().copy()
    heads0[2, 0] = 9
    with pytest.raises(hna.HnaError):
        run_search(hna, up, down, 4, heads0)
