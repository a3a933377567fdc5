"""The allocation-free entry point hna_affinity_up_static against the existing
calls it stands for (hna_affinity_up, hna_affinity_add, hna_finalize_up on a
caller's workspace), through the C ABI, on two calls in a row: the second
with fewer tokens, so that what the first left in the library's scratch
array must not leak into it.  The scores must agree bit for bit (same kernels,
same geometry, same summation order), which is stricter than the float64
oracle's tolerances; both runs are also checked against the oracle."""
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


def dev(layer):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) and not k.startswith("group_of") else v)
            for k, v in layer.items()}


def existing_calls(hna, L):
    """Scores from the three existing entry points on a fresh workspace."""
    ap = hna.pass_for_layer(L)
    ap.fold(L)
    grp = [int(x) for x in L["group_of_head"].tolist()]
    ap.hot(L, grp)
    ap.add(L, grp)
    ap.finalize(1.0 / L["a"].shape[0])
    return ap


def static_call(hna, L, ap):
    """The allocation-free call on the same folded weights; outputs allocated
    here, before the call (the call itself allocates nothing)."""
    G, I = ap.S_fo.shape
    S_fo = torch.full((G, I), float("nan"), device="cuda")
    S_add = torch.full((G, I), float("nan"), device="cuda")
    c_down = torch.full((I,), float("nan"), device="cuda")
    grp = [int(x) for x in L["group_of_head"].tolist()]
    hna.affinity_up_static(ap.dims, L["a"], L["g"], L["u"], L["r"], L["r_next"], ap.M, ap.wd_sq,
                           grp, 1.0 / L["a"].shape[0], S_fo, S_add, c_down)
    return S_fo, S_add, c_down


def fro_rel(x, ref):
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-300))


@pytest.mark.parametrize("config,T1,T2,tol", [(1, 3000, 700, 1e-2), (0, 256, 100, 1e-4)])
def test_static_matches_existing_calls_twice(hna, config, T1, T2, tol):
    for T in (T1, T2):
        print(f"config {config}, T={T}", flush=True)
        Lc = synth.make_config_layer(config, T=T)
        L = dev(Lc)
        ap = existing_calls(hna, L)
        S_fo, S_add, c_down = static_call(hna, L, ap)
        torch.cuda.synchronize()
        assert torch.equal(S_fo, ap.S_fo)
        assert torch.equal(S_add, ap.S_add)
        assert torch.equal(c_down, ap.c_down)
        ref = oracle.affinity_layer(Lc)
        for key, t in (("S_fo", S_fo), ("S_add", S_add), ("c_down", c_down)):
            err = fro_rel(t.double().cpu().numpy(), ref[key])
            print(f"  {key}: err={err:.3e}", flush=True)
            assert err <= tol


def test_static_rejects_more_than_its_scratch(hna):
    """131,072 tokens of the large 32-head, 14,336-neuron layer need about
    99 MiB of partial sums: refused before any launch."""
    dims = hna.make_dims(131072, 4096, 32, 8, 128, 14336, hna.HNA_BF16)
    assert hna.up_workspace_bytes(dims) > hna.static_scratch_bytes()
    t = torch.empty(16, dtype=torch.uint8, device="cuda")
    L = hna.lib()
    import ctypes
    vp = ctypes.c_void_p(t.data_ptr())
    grp = (ctypes.c_int32 * 32)(*[h // 4 for h in range(32)])
    rc = L.hna_affinity_up_static(ctypes.byref(dims), vp, vp, vp, vp, vp, vp, vp, grp, 1.0, 0,
                                  vp, vp, vp, None)
    assert rc == hna._binding.HNA_ERR_WORKSPACE
    assert "scratch" in hna.last_error()
