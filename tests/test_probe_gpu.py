"""The matrix-core rate probe (hna_mfma_rate_probe) computes what it claims.

The probe is a measurement aid, not part of the method, so there is no oracle
function for it; its result is pinned by the algebra of one MFMA instead.
Each wave's accumulator k after one round is the 32 x 32 product of a 32 x 16
A (lane l supplies row l % 32, columns 8 (l / 32) .. + 7) and a 16 x 32 B
(lane l supplies column l % 32, the same rows).  The sum of all its entries
is sum_c colsum(A)[c] * rowsum(B)[c], computed here in float64 from the
seed.  After two rounds every checksum is twice that of one round, up to
fp32 rounding (the matrix core adds C into its dot products in its own
order, so the doubling is not exact).
"""
import pytest
import torch

import head_neuron_affinity_amd as hna

pytestmark = pytest.mark.gpu


def _seed(n_wg: int, gen_seed: int) -> torch.Tensor:
    g = torch.Generator().manual_seed(gen_seed)
    vals = torch.randn(n_wg * 256 * 64, generator=g).to(torch.bfloat16)
    return vals.cuda()


def _expected_wave_sums(seed_bf16: torch.Tensor, n_wg: int) -> torch.Tensor:
    # [waves, 64 lanes, 4 pairs, (a, b), 8 elements]
    v = seed_bf16.cpu().double().view(n_wg * 4, 64, 4, 2, 8)
    a, b = v[:, :, :, 0, :], v[:, :, :, 1, :]
    # column c = 8 * half + e of A: summed over the 32 lanes of that half
    a_col = a.view(n_wg * 4, 2, 32, 4, 8).sum(dim=2)        # [waves, half, pair, e]
    b_row = b.view(n_wg * 4, 2, 32, 4, 8).sum(dim=2)
    return (a_col * b_row).sum(dim=(1, 2, 3))               # all four accumulators


@pytest.mark.parametrize("n_wg", [1, 7])
def test_one_round_matches_the_product_sums(n_wg):
    seed = _seed(n_wg, 100 + n_wg)
    out = hna.mfma_rate_probe(seed, n_wg, 1)
    torch.cuda.synchronize()
    got = out.cpu().double().view(n_wg * 4, 64).sum(dim=1)
    want = _expected_wave_sums(seed, n_wg)
    assert torch.allclose(got, want, rtol=1e-4, atol=1e-3), (got - want).abs().max()


def test_rounds_accumulate():
    n_wg = 3
    seed = _seed(n_wg, 7)
    one = hna.mfma_rate_probe(seed, n_wg, 1).clone()
    two = hna.mfma_rate_probe(seed, n_wg, 2)
    torch.cuda.synchronize()
    assert torch.isfinite(one).all()
    assert torch.allclose(two, 2 * one, rtol=1e-5, atol=1e-4), (two - 2 * one).abs().max()
