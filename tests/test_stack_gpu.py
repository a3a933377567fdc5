"""The affinity pass over a multi-layer stack (the 28-layer Qwen3-0.6B-shaped
workload's driver, head_neuron_affinity_amd.StackPass, at 4 layers and 1024
tokens) against the float64 oracle, layer by layer.

Each layer's S_fo and S_add, and each adjacent pair's S_down (layer i's
neurons to layer i+1's KV groups, through layer i+1's attention weights and
pre-norm gain, which the synthetic layer i carries as its next block), are
compared in full with oracle.affinity_layer at the bf16 tolerance (relative
Frobenius <= 1e-2).  The driver's side-stream overlap of the weight work must
not change a bit: the run without it gives identical scores.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

BF16_TOL = 1e-2
N_LAYERS = 4
T = 1024


@pytest.fixture(scope="module")
def hna():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_neuron_affinity_amd as m
    m.lib()
    return m


def fro_rel(x, ref):
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-300))


def test_stack_against_oracle(hna):
    layers = [synth.make_config_layer(3, layer=i, T=T) for i in range(N_LAYERS)]
    gpu_layers = [{k: (v.cuda() if isinstance(v, torch.Tensor) and not k.startswith("group_of")
                       else v) for k, v in L.items()} for L in layers]
    stack = hna.StackPass(gpu_layers, overlap=True)
    stack.run(gpu_layers)
    torch.cuda.synchronize()
    S_fo, S_add, S_down = (t.double().cpu().numpy() for t in stack.scores())
    assert S_fo.shape == (N_LAYERS, 8, 3072) and S_down.shape == (N_LAYERS - 1, 3072, 8)
    for i, L in enumerate(layers):
        print(f"layer {i}: oracle", flush=True)
        ref = oracle.affinity_layer(L)
        errs = {"S_fo": fro_rel(S_fo[i], ref["S_fo"]), "S_add": fro_rel(S_add[i], ref["S_add"])}
        if i + 1 < N_LAYERS:
            errs["S_down"] = fro_rel(S_down[i], ref["S_down"])
        for k, e in errs.items():
            print(f"  {k}: err={e:.3e}", flush=True)
            assert e <= BF16_TOL, f"layer {i} {k}: {e:.3e}"
    # the same stack without the side stream: bit-identical scores
    serial = hna.StackPass(gpu_layers, overlap=False)
    serial.run(gpu_layers)
    torch.cuda.synchronize()
    for a, b in zip(stack.scores(), serial.scores()):
        assert torch.equal(a, b)
