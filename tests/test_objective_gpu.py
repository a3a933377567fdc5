"""Parity of the layout objective (eq. 6) on the GPU, through the C ABI,
against the float64 oracle.

Tolerances, derived from the arithmetic: both sides sum fp32 scores in fp64
(the orders differ), so a fraction in [0, 1] may differ by a few times
n * 2^-53 with n <= 2^15 entries per matrix: |d frac| <= 1e-11 and
|d J| <= 1e-11 * (2N - 1).  hna_unit_mass rounds the fp64 quotient to fp32,
so each entry is within half an fp32 ulp: |d| <= 2^-24 |S_hat| (plus the fp64
difference of the totals, far below that).
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

FRAC_TOL = 1e-11
UNIT_REL = 2.0 ** -24 * 1.01


@pytest.fixture(scope="module")
def hna():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_neuron_affinity_amd as m
    m.lib()
    return m


def gpu_objective(hna, S_up, S_down, heads, neurons):
    J, fu, fd = hna.layout_objective(S_up.cuda(), S_down.cuda() if S_up.shape[0] > 1 else None,
                                     heads.cuda(), neurons.cuda())
    torch.cuda.synchronize()
    return float(J.cpu()[0]), fu.cpu().numpy(), fd.cpu().numpy()


def check(hna, S_up, S_down, heads, neurons):
    J, fu, fd = gpu_objective(hna, S_up, S_down, heads, neurons)
    Jr, fur, fdr = oracle.layout_objective(S_up.numpy(), S_down.numpy(), heads.numpy(),
                                           neurons.numpy())
    N = S_up.shape[0]
    assert fu.shape == (N,) and fd.shape == (N - 1,)
    err = max(np.max(np.abs(fu - fur), initial=0), np.max(np.abs(fd - fdr), initial=0))
    print(f"  N={N} G={S_up.shape[1]} I={S_up.shape[2]}: J={J:.12f} ref={Jr:.12f} "
          f"max|dfrac|={err:.2e}", flush=True)
    assert err <= FRAC_TOL
    assert abs(J - Jr) <= FRAC_TOL * (2 * N - 1)
    # J is the in-order sum of the fractions the kernel wrote
    s = 0.0
    for f in list(fu) + list(fd):
        s += float(f)
    assert J == s
    return J, fu, fd


@pytest.mark.parametrize("N,G,I,L,seed", [
    (3, 8, 3072, 4, 0),     # one small stack of the Qwen3-0.6B shape
    (4, 3, 100, 1, 1),      # ragged: rows and columns divide nothing
    (5, 7, 1000, 7, 2),     # columns > 256, not a multiple of the block
    (2, 16, 37, 1, 3),
    (1, 8, 512, 4, 4),      # one layer: no down edge
    (3, 4, 12, 2, 9),       # vector path with rows much shorter than a workgroup
    (2, 8, 20000, 4, 10),   # many entries per thread
])
def test_objective_matches_oracle(hna, N, G, I, L, seed):
    S_up, S_down = synth.make_scores(N, G, I, seed)
    if L > 1 and G % L == 0 and I % L == 0:
        heads, neurons = synth.random_balanced_layout(N, G, I, L, seed)
    else:
        gen = torch.Generator().manual_seed(seed)
        heads = torch.randint(0, 3, (N, G), generator=gen, dtype=torch.int32)
        neurons = torch.randint(0, 3, (N, I), generator=gen, dtype=torch.int32)
    check(hna, S_up, S_down, heads, neurons)


def test_zero_mass_and_sparse_matrices(hna):
    S_up, S_down = synth.make_scores(4, 8, 640, seed=5, zero_frac=0.5)
    S_up[1] = 0
    S_down[2] = 0
    heads, neurons = synth.random_balanced_layout(4, 8, 640, 4, seed=5)
    J, fu, fd = check(hna, S_up, S_down, heads, neurons)
    assert fu[1] == 0.0 and fd[2] == 0.0


def test_extremes_and_arbitrary_ids(hna):
    N, G, I = 3, 4, 300
    S_up, S_down = synth.make_scores(N, G, I, seed=6)
    big = torch.tensor([-2 ** 31, 2 ** 31 - 1, 7, -5], dtype=torch.int32)
    gen = torch.Generator().manual_seed(6)
    # all on one device: every fraction is 1, J = 2N - 1
    J, _, _ = check(hna, S_up, S_down, torch.full((N, G), 7, dtype=torch.int32),
                    torch.full((N, I), 7, dtype=torch.int32))
    assert J == pytest.approx(2 * N - 1, abs=1e-12)
    # heads and neurons on disjoint ids: J = 0 exactly
    J, _, _ = check(hna, S_up, S_down, big[torch.randint(0, 2, (N, G), generator=gen)],
                    big[2 + torch.randint(0, 2, (N, I), generator=gen)])
    assert J == 0.0


def test_full_stack_and_determinism(hna):
    # 28 layers x 8 KV groups x 3072 neurons on 4 devices (the Qwen3-0.6B stack)
    N, G, I, L = 28, 8, 3072, 4
    S_up, S_down = synth.make_scores(N, G, I, seed=7)
    heads, neurons = synth.random_balanced_layout(N, G, I, L, seed=7)
    J, fu, fd = check(hna, S_up, S_down, heads, neurons)
    J2, fu2, fd2 = gpu_objective(hna, S_up, S_down, heads, neurons)
    assert J2 == J and np.array_equal(fu2, fu) and np.array_equal(fd2, fd)
    hc, nc = synth.contiguous_layout(N, G, I, L)
    check(hna, S_up, S_down, hc, nc)


@pytest.mark.parametrize("shape", [(3, 8, 3072), (2, 5, 33), (1, 1, 1), (4, 1000, 7)])
def test_unit_mass_matches_oracle(hna, shape):
    gen = torch.Generator().manual_seed(sum(shape))
    S = torch.exp(torch.randn(shape, generator=gen))
    if shape[0] > 1:
        S[1] = 0
    out = hna.unit_mass(S.cuda())
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    for m in range(shape[0]):
        ref = oracle.unit_mass(S[m].numpy())
        assert np.all(np.abs(got[m] - ref) <= UNIT_REL * np.abs(ref)), m
    # in place gives the same bits
    Sd = S.cuda()
    hna.unit_mass(Sd, out=Sd)
    torch.cuda.synchronize()
    assert torch.equal(Sd.cpu(), out.cpu())


def test_objective_of_unit_mass_input(hna):
    N, G, I, L = 4, 8, 1024, 4
    S_up, S_down = synth.make_scores(N, G, I, seed=8)
    heads, neurons = synth.random_balanced_layout(N, G, I, L, seed=8)
    Ju, fu, fd = gpu_objective(hna, hna.unit_mass(S_up.cuda()).cpu(),
                               hna.unit_mass(S_down.cuda()).cpu(), heads, neurons)
    Jr, fur, fdr = oracle.layout_objective(S_up.numpy(), S_down.numpy(), heads.numpy(),
                                           neurons.numpy())
    # the fp32 rounding of the normalised entries moves a fraction by <= 2^-24
    assert np.max(np.abs(fu - fur)) <= 1e-7 and np.max(np.abs(fd - fdr)) <= 1e-7
