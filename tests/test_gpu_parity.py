"""Parity of the HIP path (through the C ABI) against the float64 oracle.

Tolerances: fp32 inputs, max|dS| / max|S| <= 1e-4 per output matrix; bf16
inputs with fp32 accumulation, relative Frobenius ||dS|| / ||S|| <= 1e-2.
Both sides consume exactly the same (rounded) inputs.
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


def dev(layer):
    return {k: (v.cuda() if isinstance(v, torch.Tensor) and not k.startswith("group_of") else v)
            for k, v in layer.items()}


def f64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def max_rel(x, ref):
    return float(np.max(np.abs(x - ref)) / max(np.max(np.abs(ref)), 1e-300))


def fro_rel(x, ref):
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-300))


def run(hna, layer):
    out = hna.affinity_layer(layer)
    torch.cuda.synchronize()
    return {k: f64(v) for k, v in out.items()}


def check_all(got, ref, tol, metric):
    for key in ("S_fo", "S_add", "c_down", "n_down", "S_down"):
        if key in ref:
            err = metric(got[key], ref[key])
            print(f"  {key}: err={err:.3e}", flush=True)
            assert err <= tol, f"{key}: {err:.3e} > {tol}"
            assert np.all(got[key] >= 0)


def layer_of(T, hidden, H, G, d, I, dtype, sigma=0.5, seed=1):
    sh = synth.LayerShape("t", T, hidden, H, G, d, I, dtype, sigma)
    return synth.make_layer(sh, seed)


# ------------------------------------------------------------- fp32 path
def test_tiny_fp32_config_full_parity(hna):
    L = synth.make_config_layer(0)
    got = run(hna, dev(L))
    check_all(got, oracle.affinity_layer(L), FP32_TOL, max_rel)


@pytest.mark.parametrize("shape", [
    (200, 64, 4, 2, 16, 100),     # ragged tokens and neurons
    (1, 64, 4, 2, 16, 128),       # one token
    (333, 48, 6, 3, 32, 70),      # hidden != H*d, ragged everything
    (130, 40, 2, 2, 16, 33),      # MHA-like (G == H)
    (257, 64, 8, 1, 48, 161),     # one KV group, d = 48
    (1100, 32, 2, 1, 128, 40),    # d = 128 in fp32, several token tiles
])
def test_fp32_ragged_shapes(hna, shape):
    T, hidden, H, G, d, I = shape
    print(f"shape {shape}", flush=True)
    L = layer_of(T, hidden, H, G, d, I, "f32", seed=T)
    got = run(hna, dev(L))
    check_all(got, oracle.affinity_layer(L), FP32_TOL, max_rel)


def test_fp32_custom_group_map(hna):
    L = layer_of(300, 64, 6, 3, 16, 96, "f32", seed=9)
    grp = torch.tensor([2, 0, 1, 0, 2, 1], dtype=torch.int32)
    L["group_of_head"] = grp
    L["group_of_head_next"] = torch.tensor([1, 1, 0, 2, 0, 2], dtype=torch.int32)
    got = run(hna, dev(L))
    check_all(got, oracle.affinity_layer(L), FP32_TOL, max_rel)


# ------------------------------------------------------------- bf16 path
def test_bf16_qwen_shape_reduced_tokens(hna):
    L = synth.make_config_layer(1, T=521)
    got = run(hna, dev(L))
    check_all(got, oracle.affinity_layer(L), BF16_TOL, fro_rel)
    # the fp32 accumulation keeps the bf16 path far inside the tolerance
    assert fro_rel(got["S_fo"], oracle.affinity_layer(L)["S_fo"]) < 2e-3


def sub_oracle(L, groups, neurons, T=None):
    """Oracle on a subset of KV groups and neurons (same literal arithmetic)."""
    grp = L["group_of_head"].tolist()
    d = L["a"].shape[2]
    ks = torch.as_tensor(neurons)
    rows_fo, rows_add = [], []
    for gg in groups:
        heads = [h for h in range(len(grp)) if grp[h] == gg]
        cols = torch.cat([torch.arange(h * d, (h + 1) * d) for h in heads])
        a_s = L["a"][:, heads, :]
        W_o_s = L["W_o"][:, cols.to(L["W_o"].device)]
        kd = ks.to(L["g"].device)
        fo, add = oracle.affinity_up(a_s, L["g"][:, kd], L["u"][:, kd], L["r"], L["gamma"], W_o_s,
                                     L["W_gate"][kd], L["W_up"][kd], L["W_down"][:, kd],
                                     np.zeros(len(heads), dtype=np.int64), G=1)
        rows_fo.append(fo[0])
        rows_add.append(add[0])
    kd = ks.to(L["g"].device)
    c = oracle.down_moment(L["g"][:, kd], L["u"][:, kd], L["r_next"])
    Gn = int(max(L["group_of_head_next"].tolist())) + 1
    n = oracle.down_weight_norms(L["W_q"], L["W_k"], L["W_v"], L["gamma_next"], L["W_down"][:, kd],
                                 L["group_of_head_next"], G_next=Gn)
    return np.array(rows_fo), np.array(rows_add), c, n


def check_sampled(got, ref, groups, neurons):
    fo, add, c, n = ref
    g_fo = got["S_fo"][np.ix_(groups, neurons)]
    g_add = got["S_add"][np.ix_(groups, neurons)]
    errs = {"S_fo": fro_rel(g_fo, fo), "S_add": fro_rel(g_add, add),
            "c_down": fro_rel(got["c_down"][neurons], c),
            "n_down": fro_rel(got["n_down"][:, neurons], n),
            "S_down": fro_rel(got["S_down"][neurons, :], c[:, None] * n.T)}
    for k, e in errs.items():
        print(f"  {k}: err={e:.3e}", flush=True)
        assert e <= BF16_TOL, f"{k}: {e:.3e}"


def test_bf16_danube_shape_reduced_tokens(hna):
    L = synth.make_config_layer(2, T=777)
    got = run(hna, dev(L))
    groups, neurons = [0, 3, 7], list(range(0, 4096, 61)) + [4095]
    check_sampled(got, sub_oracle(L, groups, neurons), groups, neurons)


def test_bf16_large_shape_reduced_tokens(hna):
    L = synth.make_config_layer(4, T=300)
    got = run(hna, dev(L))
    groups, neurons = [0, 5], list(range(7, 14336, 997)) + [14335]
    check_sampled(got, sub_oracle(L, groups, neurons), groups, neurons)


def test_bf16_identity_and_scattered_group_maps(hna):
    # G == H: every head is its own group
    L = layer_of(260, 128, 8, 8, 32, 200, "bf16", seed=4)
    got = run(hna, dev(L))
    check_all(got, oracle.affinity_layer(L), BF16_TOL, fro_rel)
    # a non-contiguous map for both layers
    L = layer_of(260, 128, 8, 4, 32, 200, "bf16", seed=5)
    L["group_of_head"] = torch.tensor([3, 1, 0, 2, 3, 1, 0, 2], dtype=torch.int32)
    L["group_of_head_next"] = torch.tensor([0, 0, 3, 3, 1, 2, 2, 1], dtype=torch.int32)
    got = run(hna, dev(L))
    check_all(got, oracle.affinity_layer(L), BF16_TOL, fro_rel)


# ------------------------------------------------------------- invariants
def test_deterministic_reruns(hna):
    L = dev(synth.make_config_layer(1, T=1000))
    a = run(hna, L)
    b = run(hna, L)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_neuron_and_group_permutation_bitwise(hna):
    """The paper's layout symmetry holds exactly on the GPU: permuting neurons
    (gate/up rows, down columns, g/u columns) or KV groups with their heads
    permutes the scores bit for bit (fixed per-neuron summation order)."""
    L = synth.make_config_layer(1, T=700)
    base = run(hna, dev(L))
    I = L["g"].shape[1]
    perm = torch.randperm(I, generator=torch.Generator().manual_seed(3))
    P = dict(L, W_gate=L["W_gate"][perm].contiguous(), W_up=L["W_up"][perm].contiguous(),
             W_down=L["W_down"][:, perm].contiguous(), g=L["g"][:, perm].contiguous(),
             u=L["u"][:, perm].contiguous())
    got = run(hna, dev(P))
    for key in ("S_fo", "S_add"):
        assert np.array_equal(got[key], base[key][:, perm.numpy()]), key
    assert np.array_equal(got["c_down"], base["c_down"][perm.numpy()])
    # groups: new group j is old group gperm[j], its heads moved with it
    gperm = [5, 2, 7, 0, 1, 6, 3, 4]
    d = L["a"].shape[2]
    heads = [2 * g + i for g in gperm for i in range(2)]
    cols = torch.cat([torch.arange(h * d, (h + 1) * d) for h in heads])
    Q = dict(L, a=L["a"][:, heads, :].contiguous(), W_o=L["W_o"][:, cols].contiguous())
    got = run(hna, dev(Q))
    for key in ("S_fo", "S_add"):
        assert np.array_equal(got[key], base[key][gperm]), key


def test_chunked_tokens_accumulate(hna):
    """Feeding the tokens in two calls with HNA_ACCUMULATE and scale 1/T_total
    equals the one-shot pass up to fp32 summation order."""
    L = dev(synth.make_config_layer(1, T=1500))
    full = run(hna, L)
    ap = hna.pass_for_layer(L)
    grp = L["group_of_head"].tolist()
    ap.fold(L)
    T1 = 640
    for i, (t0, t1) in enumerate([(0, T1), (T1, 1500)]):
        part = {k: (L[k][t0:t1].contiguous() if k in ("a", "g", "u", "r", "r_next") else L[k]) for k in L}
        dims = hna.make_dims(t1 - t0, ap.dims.hidden, ap.dims.H, ap.dims.G, ap.dims.d, ap.dims.I,
                             ap.dims.dtype)
        ws = hna.affinity_up(dims, part["a"], part["g"], part["u"], part["r"], part["r_next"],
                             ap.M, grp)
        hna.affinity_add(dims, part["a"], part["r"], ap.M, grp, ws)
        hna.finalize_up(dims, ap.wd_sq, ws, 1.0 / 1500, accumulate=(i > 0), S_fo=ap.S_fo,
                        S_add=ap.S_add, c_down=ap.c_down)
    torch.cuda.synchronize()
    for key, t in (("S_fo", ap.S_fo), ("S_add", ap.S_add), ("c_down", ap.c_down)):
        assert max_rel(f64(t), full[key]) < 1e-5, key


def test_zero_tokens(hna):
    L = dev(synth.make_config_layer(0, T=8))
    ap = hna.pass_for_layer(L)
    ap.fold(L)
    dims = hna.make_dims(0, ap.dims.hidden, ap.dims.H, ap.dims.G, ap.dims.d, ap.dims.I, ap.dims.dtype)
    ws = hna.affinity_up(dims, L["a"], L["g"], L["u"], L["r"], L["r_next"], ap.M,
                         L["group_of_head"].tolist())
    hna.affinity_add(dims, L["a"], L["r"], ap.M, L["group_of_head"].tolist(), ws)
    S_fo, S_add, c = hna.finalize_up(dims, ap.wd_sq, ws, 1.0)
    torch.cuda.synchronize()
    assert torch.count_nonzero(S_fo) == 0 and torch.count_nonzero(S_add) == 0
    assert torch.count_nonzero(c) == 0


# ------------------------------------------- full sizes, sampled outputs
@pytest.mark.parametrize("config,groups,neurons", [
    (1, [3], list(range(5, 3072, 193)) + [3071]),
    (2, [6], list(range(11, 4096, 257)) + [4095]),
    (4, [1], list(range(3, 14336, 1433)) + [14335]),
])
def test_full_size_sampled_entries(hna, config, groups, neurons):
    """At the benchmark's full token counts and launch configuration, sampled
    (group, neuron) entries agree with the oracle run on just those entries."""
    print(f"config {config}: generating on the GPU", flush=True)
    L = synth.make_config_layer(config, device="cuda")
    torch.cuda.synchronize()
    got = run(hna, L)
    print(f"config {config}: oracle on {len(groups)} group(s) x {len(neurons)} neurons", flush=True)
    check_sampled(got, sub_oracle(L, groups, neurons), groups, neurons)
    del L
    torch.cuda.empty_cache()
