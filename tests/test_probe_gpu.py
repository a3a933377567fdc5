"""The matrix-core rate probe (hna_mfma_rate_probe) computes what it claims.

The probe is a measurement aid, not part of the method, so there is no oracle
function for it; its result is pinned by the algebra of one MFMA instead.
Each wave's accumulator k after one round is the 32 x 32 product of a 32 x 16
A (lane l supplies row l % 32, columns 8 (l / 32) .. + 7) and a 16 x 32 B
(lane l supplies column l % 32, the same rows); with 16x16x32 MFMAs, of a
16 x 32 A and a 32 x 16 B (lane l: row or column l % 16, K indices
8 (l / 16) .. + 7), two accumulators per operand pair.  The sum of all its entries
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


def _expected_wave_sums(seed_bf16: torch.Tensor, n_wg: int, shape: int) -> torch.Tensor:
    # [waves, 64 lanes, 4 pairs, (a, b), 8 elements]
    v = seed_bf16.cpu().double().view(n_wg * 4, 64, 4, 2, 8)
    a, b = v[:, :, :, 0, :], v[:, :, :, 1, :]
    # the lanes that supply one group of 8 K indices: 32 per half (32x32x16,
    # K group l / 32) or 16 per quarter (16x16x32, K group l / 16); column c of
    # A is summed over them, and row c of B likewise
    groups = 2 if shape == 0 else 4
    a_col = a.reshape(n_wg * 4, groups, 64 // groups, 4, 8).sum(dim=2)
    b_row = b.reshape(n_wg * 4, groups, 64 // groups, 4, 8).sum(dim=2)
    # all accumulators (16x16x32: two per operand pair)
    return (a_col * b_row).sum(dim=(1, 2, 3)) * (1 if shape == 0 else 2)


@pytest.mark.parametrize("shape", [0, 1])
@pytest.mark.parametrize("n_wg", [1, 7])
def test_one_round_matches_the_product_sums(n_wg, shape):
    seed = _seed(n_wg, 100 + n_wg)
    out = hna.mfma_rate_probe(seed, n_wg, 1, shape=shape)
    torch.cuda.synchronize()
    got = out.cpu().double().view(n_wg * 4, 64).sum(dim=1)
    want = _expected_wave_sums(seed, n_wg, shape)
    assert torch.allclose(got, want, rtol=1e-4, atol=1e-3), (got - want).abs().max()


@pytest.mark.parametrize("shape", [0, 1])
def test_rounds_accumulate(shape):
    n_wg = 3
    seed = _seed(n_wg, 7)
    one = hna.mfma_rate_probe(seed, n_wg, 1, shape=shape).clone()
    two = hna.mfma_rate_probe(seed, n_wg, 2, shape=shape)
    torch.cuda.synchronize()
    assert torch.isfinite(one).all()
    assert torch.allclose(two, 2 * one, rtol=1e-5, atol=1e-4), (two - 2 * one).abs().max()
