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
