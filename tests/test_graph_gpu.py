"""One whole step of the affinity pass captured in a HIP graph.

The step (fold, ||w^d||^2, the hot kernel, ADD, the fixed-order reduction, the
down-edge weight norms and S_down) allocates nothing, sets no memory with
memset nodes and never synchronises, so a caller can capture it once and
replay it.  Each replay is checked bit for bit against an eager step of the
same inputs (every kernel sums in a fixed order), with eager work and
synchronisations between the replays.
"""
import pytest
import torch

import head_neuron_affinity_amd as hna
import synth

pytestmark = pytest.mark.gpu


def _outputs(P):
    return [t.clone() for t in (P.S_fo, P.S_add, P.c_down, P.n_down, P.S_down)]


@pytest.mark.parametrize("config,T", [(1, 4096), (2, 1000)])
def test_step_replays_match_eager(config, T):
    print(f"graph capture: config {config}, T={T}", flush=True)
    L = synth.make_config_layer(config, T=T, device="cuda")
    P = hna.pass_for_layer(L)
    grp = [int(x) for x in L["group_of_head"].tolist()]
    grp_n = [int(x) for x in L["group_of_head_next"].tolist()]

    def step():
        P.fold(L)
        P.hot(L, grp)
        P.add(L, grp)
        P.finalize(1.0 / T)
        P.down(L, grp_n)

    # eager reference; warm-up on a side stream, as stream capture expects
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    ref = _outputs(P)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        for t in (P.S_fo, P.S_add, P.c_down, P.n_down, P.S_down):
            t.fill_(float("nan"))          # a replay must rewrite every output
        g.replay()
        torch.cuda.synchronize()
        got = _outputs(P)
        for name, a, b in zip(("S_fo", "S_add", "c_down", "n_down", "S_down"), got, ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager step"
        step()                              # eager work between the replays
        torch.cuda.synchronize()
        for a, b in zip(_outputs(P), ref):
            assert torch.equal(a, b)
