"""Parity of the exact leave-one-out score (section 3, "Affinity scores") on the
GPU, through the C ABI, against the float64 oracle's literal ablation.

Tolerances as for the other scores: fp32 inputs, max|dS| / max|S| <= 1e-4;
bf16 inputs (fp32 accumulation), relative Frobenius <= 1e-2.  The GPU uses the
layer's stored g and u for the alpha^2 g^2 term and x with the gate and up
weights for the cross term; the oracle recomputes g and u from the same fp32
residual x, so the difference is the storage rounding of g and u.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

FP32_TOL = 1e-4
BF16_TOL = 1e-2


@pytest.fixture(scope="module")
def hna():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_neuron_affinity_amd as m
    m.lib()
    return m


def run_loo(hna, layer):
    ap = hna.pass_for_layer(layer, with_down=False)
    ap.fold(layer)
    S = ap.loo(layer, [int(x) for x in layer["group_of_head"].tolist()])
    torch.cuda.synchronize()
    return S.cpu().double().numpy()


def oracle_loo(layer, neurons=None):
    return oracle.loo_scores(layer["a"], layer["x_in"], layer["gamma"], layer["W_o"],
                             layer["W_gate"], layer["W_up"],
                             np.asarray(layer["group_of_head"]), neurons=neurons)


def check(got, ref, tol, metric):
    if metric == "max":
        err = float(np.max(np.abs(got - ref)) / np.max(np.abs(ref)))
    else:
        err = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    print(f"  LOO {metric}-rel err {err:.3e}", flush=True)
    assert err <= tol
    assert np.all(got >= 0)


@pytest.mark.parametrize("shape,tol,metric", [
    (synth.LayerShape("tiny-fp32", 256, 64, 4, 2, 16, 128, "f32", 0.5), FP32_TOL, "max"),
    (synth.LayerShape("ragged-fp32", 300, 96, 6, 3, 32, 100, "f32", 0.5), FP32_TOL, "max"),
    (synth.LayerShape("odd-I-fp32", 200, 64, 4, 2, 16, 102, "f32", 0.5), FP32_TOL, "max"),
    (synth.LayerShape("ragged-bf16", 1000, 136, 4, 2, 48, 200, "bf16", 0.5), BF16_TOL, "fro"),
    (synth.LayerShape("mid-bf16", 2048, 256, 8, 4, 64, 384, "bf16", 0.5), BF16_TOL, "fro"),
    # head dim 32 and a token count off the 32-token tile
    (synth.LayerShape("d32-ragged-bf16", 999, 128, 4, 2, 32, 200, "bf16", 0.5), BF16_TOL, "fro"),
    # token counts off the 8-token padding of the token GEMM's transposed
    # operands and off its K chunks (2 and 3 chunks, the last one short)
    (synth.LayerShape("split-remainder-bf16", 8195, 128, 4, 2, 32, 200, "bf16", 0.5), BF16_TOL, "fro"),
    (synth.LayerShape("split-remainder-fp32", 12289, 64, 4, 2, 16, 128, "f32", 0.5), FP32_TOL, "max"),
    (synth.LayerShape("d128-bf16", 512, 512, 16, 8, 128, 256, "bf16", 0.5), BF16_TOL, "fro"),
    # x . o_h from the GEMM's dot epilogue with partial tiles both ways: H d
    # below or past a multiple of 256, tokens not a multiple of 256
    (synth.LayerShape("d64-ragged-bf16", 777, 192, 3, 1, 64, 200, "bf16", 0.5), BF16_TOL, "fro"),
    (synth.LayerShape("d128-ragged-bf16", 1001, 320, 5, 1, 128, 136, "bf16", 0.5), BF16_TOL, "fro"),
    # fewer tokens than one 8-token pad group (one K step of 64, mostly zeros)
    (synth.LayerShape("five-tokens-bf16", 5, 128, 4, 2, 32, 64, "bf16", 0.5), BF16_TOL, "fro"),
    (synth.LayerShape("three-tokens-fp32", 3, 64, 4, 2, 16, 64, "f32", 0.5), FP32_TOL, "max"),
    # the Danube3-500M layer shape (head dim 96), fewer tokens and neurons
    (synth.LayerShape("danube-shape-bf16", 1024, 1536, 16, 8, 96, 512, "bf16", 0.5), BF16_TOL, "fro"),
    # neuron counts off 8 in bf16 (T1 with one-element loads, partial Y rows):
    # with Z stored (head dim 32) and with the dot epilogue (head dim 128)
    (synth.LayerShape("odd-I-bf16", 300, 128, 4, 2, 32, 100, "bf16", 0.5), BF16_TOL, "fro"),
    (synth.LayerShape("odd-I-d128-bf16", 259, 256, 2, 1, 128, 77, "bf16", 0.5), BF16_TOL, "fro"),
    # the fp32 path at the larger head dims (unfused coefficients, fp32 GEMMs)
    (synth.LayerShape("d128-fp32", 300, 256, 4, 2, 128, 100, "f32", 0.5), FP32_TOL, "max"),
    (synth.LayerShape("d96-fp32", 333, 192, 3, 3, 96, 130, "f32", 0.5), FP32_TOL, "max"),
], ids=lambda v: v.name if isinstance(v, synth.LayerShape) else str(v))
def test_loo_matches_oracle(hna, shape, tol, metric):
    layer = synth.make_layer(shape, seed=17, device="cuda", with_next=False, with_x=True)
    got = run_loo(hna, layer)
    ref = oracle_loo({k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in layer.items()})
    check(got, ref, tol, metric)


@pytest.mark.parametrize("config,cols", [
    # the 65,536-token Qwen3-0.6B-shaped layer in the benchmark's launch configuration
    (1, [0, 1, 517, 1024, 2047, 2048, 3000, 3071]),
    # the 65,536-token Danube3-500M-shaped layer (head dim 96, hidden 1536)
    (2, [0, 3, 1000, 2048, 3333, 4095]),
])
def test_loo_full_layer_sampled_neurons(hna, config, cols):
    # full token count; the oracle computes the sampled neurons over every token
    layer = synth.make_config_layer(config, device="cuda", with_next=False, with_x=True)
    got = run_loo(hna, layer)
    cols = np.array(cols)
    cpu = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in layer.items()}
    ref = oracle_loo(cpu, neurons=cols)
    check(got[:, cols], ref, BF16_TOL, "fro")


def test_loo_zero_tokens_and_determinism(hna):
    shape = synth.LayerShape("tiny-fp32", 256, 64, 4, 2, 16, 128, "f32", 0.5)
    layer = synth.make_layer(shape, seed=18, device="cuda", with_next=False, with_x=True)
    a1 = run_loo(hna, layer)
    a2 = run_loo(hna, layer)
    assert np.array_equal(a1, a2)
    empty = synth.make_layer(shape.with_tokens(0) if hasattr(shape, "with_tokens") else shape,
                             seed=18, device="cuda", with_next=False, with_x=True)
    assert np.all(run_loo(hna, empty) == 0.0)
