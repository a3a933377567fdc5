"""Pins of the float64 oracle against things other than itself.

None of these tests retypes the oracle's formulas.  They check it against
  * a genuine forward pass of the synthetic layer with one head's piece
    removed (ablation, r held fixed), for the per-head piece p_h and ADD;
  * central finite differences of the neuron output silu(g) u under that
    removal, for the first-order damage of eq. (5);
  * the logistic function's textbook derivative and special values;
  * an independent Gram-matrix closed form of ADD;
  * the down edge's own forward pass (the next layer's q/k/v projections of a
    residual with one neuron's write removed);
  * invariants the definition implies: group sums, permutation equivariance
    (the paper's layout symmetry), scaling, token replication, chunking.
Source: "Affinity-Aware Sharding for Delayed Tensor Parallelism", section 3,
paragraphs "The layout as a free variable" and "Affinity scores", eq. (5).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def tiny(T=37, hidden=10, H=4, G=2, d=3, I=5, sigma=0.5, seed=7, resid=True):
    """A float64 synthetic layer; hidden != H*d on purpose (10 vs 12)."""
    sh = synth.LayerShape("pin", T, hidden, H, G, d, I, "f64", sigma)
    L = synth.make_layer(sh, seed, return_resid=resid)
    return {k: (v.numpy() if isinstance(v, torch.Tensor) else v) for k, v in L.items()}


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def forward_pre(L, x):
    """Gate/up pre-activations of the layer for residual x (r from the layer)."""
    y = L["gamma"][None, :] * x / L["r"][:, None]
    return y @ L["W_gate"].T, y @ L["W_up"].T


def head_write(L, h):
    """Head h's write into the residual, a_h W_o^(h)T (columns h*d..h*d+d-1)."""
    d = L["a"].shape[2]
    return L["a"][:, h, :] @ L["W_o"][:, h * d:(h + 1) * d].T


def run_up(L, grp=None, G=None, **kw):
    grp = L["group_of_head"] if grp is None else grp
    return oracle.affinity_up(L["a"], L["g"], L["u"], L["r"], L["gamma"], L["W_o"],
                              L["W_gate"], L["W_up"], L["W_down"], grp, G=G, **kw)


# ---------------------------------------------------------------- generator sanity
def test_generator_consistent_forward():
    L = tiny()
    g, u = forward_pre(L, L["x"])
    np.testing.assert_allclose(g, L["g"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(u, L["u"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(L["r"], np.sqrt((L["x"] ** 2).mean(1)), rtol=1e-14)


# ---------------------------------------------------------------- p_h and ADD
def test_head_pieces_sum_to_normalised_input():
    """sum_h p_h + (rest) equals the normalised FFN input (paper section 3)."""
    L = tiny()
    H = L["a"].shape[1]
    total = sum(oracle.head_piece(L["a"][:, h, :], L["r"], L["gamma"], L["W_o"], h)
                for h in range(H))
    rest = L["gamma"][None, :] * (L["x"] - sum(head_write(L, h) for h in range(H))) / L["r"][:, None]
    y = L["gamma"][None, :] * L["x"] / L["r"][:, None]
    np.testing.assert_allclose(total + rest, y, rtol=0, atol=1e-12)


def test_add_score_by_head_ablation():
    """ADD = mean squared change of the pre-activations when head h's write is
    removed from the residual with r held fixed, summed over the group's heads."""
    L = tiny()
    H = L["a"].shape[1]
    grp = L["group_of_head"]
    g0, u0 = forward_pre(L, L["x"])
    want = np.zeros((int(grp.max()) + 1, L["g"].shape[1]))
    for h in range(H):
        g1, u1 = forward_pre(L, L["x"] - head_write(L, h))
        want[grp[h]] += ((g0 - g1) ** 2 + (u0 - u1) ** 2).mean(0)
    _, S_add = run_up(L)
    np.testing.assert_allclose(S_add, want, rtol=1e-11, atol=0)


# ---------------------------------------------------------------- eq. (5)
def silu_fwd(z):
    return z / (1.0 + np.exp(-z))


@pytest.mark.parametrize("seed", [3, 11])
def test_first_order_damage_matches_finite_difference(seed):
    """Delta_thk is minus the derivative of the neuron output silu(g_k) u_k along
    the removal of head h's piece (r fixed); checked by a central difference."""
    L = tiny(T=9, seed=seed)
    D = oracle.first_order_damage(L["a"], L["g"], L["u"], L["r"], L["gamma"],
                                  L["W_o"], L["W_gate"], L["W_up"])
    eps = 1e-5
    H = L["a"].shape[1]
    for h in range(H):
        w = head_write(L, h)
        gp, up = forward_pre(L, L["x"] - eps * w)
        gm, um = forward_pre(L, L["x"] + eps * w)
        fd = (silu_fwd(gm) * um - silu_fwd(gp) * up) / (2 * eps)
        np.testing.assert_allclose(D[:, h, :], fd, rtol=2e-7, atol=1e-9)


def test_fo_score_from_finite_differences():
    """S_fo assembled from finite-difference damages: the group sum of the mean
    squared central difference, times ||w^d_k||^2."""
    L = tiny(T=23, H=4, G=2, seed=5)
    grp = L["group_of_head"]
    eps = 1e-5
    want = np.zeros((2, L["g"].shape[1]))
    for h in range(4):
        w = head_write(L, h)
        gp, up = forward_pre(L, L["x"] - eps * w)
        gm, um = forward_pre(L, L["x"] + eps * w)
        fd = (silu_fwd(gm) * um - silu_fwd(gp) * up) / (2 * eps)
        want[grp[h]] += (fd ** 2).mean(0)
    want *= (L["W_down"] ** 2).sum(0)[None, :]
    S_fo, _ = run_up(L)
    np.testing.assert_allclose(S_fo, want, rtol=1e-6)


def test_silu_parts_textbook():
    z = np.linspace(-30, 30, 601)
    sig, silu, dsilu = oracle.silu_parts(z)
    np.testing.assert_allclose(sig, 1.0 / (1.0 + np.exp(-z)), rtol=1e-13, atol=1e-300)
    h = 1e-6
    fd = (silu_fwd(z + h) - silu_fwd(z - h)) / (2 * h)
    np.testing.assert_allclose(dsilu, fd, rtol=1e-7, atol=1e-9)
    s0, l0, d0 = oracle.silu_parts(np.array([0.0]))
    assert s0[0] == 0.5 and l0[0] == 0.0 and d0[0] == 0.5
    _, lbig, dbig = oracle.silu_parts(np.array([60.0]))
    assert abs(lbig[0] - 60.0) < 1e-12 and abs(dbig[0] - 1.0) < 1e-12


def test_special_operating_points_relate_fo_to_add():
    """At g = 0, u = 1: Delta = p.w^g / 2.  At g = 60, u = 0: Delta = 60 p.w^u.
    Hence 4 S_fo(g=0,u=1) + S_fo(g=60,u=0)/3600 = ||w^d||^2 S_add."""
    L = tiny()
    wd2 = (L["W_down"] ** 2).sum(0)
    L0 = dict(L, g=np.zeros_like(L["g"]), u=np.ones_like(L["u"]))
    L1 = dict(L, g=np.full_like(L["g"], 60.0), u=np.zeros_like(L["u"]))
    fo0, add0 = run_up(L0)
    fo1, add1 = run_up(L1)
    np.testing.assert_allclose(4 * fo0 + fo1 / 3600.0, wd2[None, :] * add0, rtol=1e-12)
    # ADD does not depend on the operating point.
    np.testing.assert_array_equal(add0, add1)
    # g = 0 and u = 0 together kill the first-order damage entirely.
    fz, _ = run_up(dict(L, g=np.zeros_like(L["g"]), u=np.zeros_like(L["u"])))
    assert np.all(fz == 0.0)


# ---------------------------------------------------------------- closed form
def test_add_matches_gram_closed_form():
    """S_add[h,k] = m_g^T Sigma_h m_g + m_u^T Sigma_h m_u with
    m = W_o^(h)T (gamma * w_k) and Sigma_h = mean_t a_t a_t^T / r_t^2."""
    L = tiny(T=200, H=6, G=3, d=4, hidden=9, I=7)
    a, r, gam = L["a"], L["r"], L["gamma"]
    T, H, d = a.shape
    ident = np.arange(H)
    _, S_add = run_up(L, grp=ident, G=H)
    for h in range(H):
        ah = a[:, h, :] / r[:, None]
        Sig = np.cov(ah.T, bias=True, aweights=None) + np.outer(ah.mean(0), ah.mean(0))
        Woh = L["W_o"][:, h * d:(h + 1) * d]
        mg = Woh.T @ (gam[:, None] * L["W_gate"].T)      # [d, I]
        mu = Woh.T @ (gam[:, None] * L["W_up"].T)
        want = np.einsum("ik,ij,jk->k", mg, Sig, mg) + np.einsum("ik,ij,jk->k", mu, Sig, mu)
        np.testing.assert_allclose(S_add[h], want, rtol=1e-11)


# ---------------------------------------------------------------- invariants
def test_group_rows_are_sums_of_head_rows():
    L = tiny(H=6, G=3)
    fo_h, add_h = run_up(L, grp=np.arange(6), G=6)
    for grp in ([0, 0, 1, 1, 2, 2], [2, 0, 1, 0, 2, 1]):
        fo_g, add_g = run_up(L, grp=np.array(grp), G=3)
        for gg in range(3):
            hs = [h for h in range(6) if grp[h] == gg]
            np.testing.assert_allclose(fo_g[gg], fo_h[hs].sum(0), rtol=1e-13)
            np.testing.assert_allclose(add_g[gg], add_h[hs].sum(0), rtol=1e-13)


def test_neuron_permutation_permutes_columns():
    """The paper's layout symmetry: permuting gate/up rows, down columns (and so
    g, u columns) permutes the scores' neuron axis."""
    L = tiny(I=9)
    perm = np.random.default_rng(1).permutation(9)
    P = dict(L, W_gate=L["W_gate"][perm], W_up=L["W_up"][perm],
             W_down=L["W_down"][:, perm], g=L["g"][:, perm], u=L["u"][:, perm])
    fo, add = run_up(L)
    fo_p, add_p = run_up(P)
    np.testing.assert_allclose(fo_p, fo[:, perm], rtol=1e-13)
    np.testing.assert_allclose(add_p, add[:, perm], rtol=1e-13)


def test_group_permutation_permutes_rows():
    """Moving KV groups with their query heads (a's heads, W_o's column blocks and
    the group map) permutes the scores' group axis."""
    L = tiny(H=6, G=3)
    d = L["a"].shape[2]
    gperm = np.array([2, 0, 1])                     # new group j is old group gperm[j]
    grp = L["group_of_head"]
    heads = [h for j in range(3) for h in range(6) if grp[h] == gperm[j]]
    cols = np.concatenate([np.arange(h * d, (h + 1) * d) for h in heads])
    P = dict(L, a=L["a"][:, heads, :], W_o=L["W_o"][:, cols])
    fo, add = run_up(L)
    fo_p, add_p = run_up(P, grp=np.array([0, 0, 1, 1, 2, 2]), G=3)
    np.testing.assert_allclose(fo_p, fo[gperm], rtol=1e-13)
    np.testing.assert_allclose(add_p, add[gperm], rtol=1e-13)


def test_down_column_scaling():
    L = tiny()
    c = np.array([1.0, 3.0, 0.5, 2.0, 1.0])
    fo, add = run_up(L)
    fo2, add2 = run_up(dict(L, W_down=L["W_down"] * c[None, :]))
    np.testing.assert_allclose(fo2, fo * c[None, :] ** 2, rtol=1e-13)
    np.testing.assert_allclose(add2, add, rtol=1e-14)


def test_head_scaling_quadratic():
    L = tiny(H=4, G=4)
    a2 = L["a"].copy()
    a2[:, 2, :] *= 3.0
    fo, add = run_up(L, G=4, grp=np.arange(4))
    fo2, add2 = run_up(dict(L, a=a2), G=4, grp=np.arange(4))
    np.testing.assert_allclose(fo2[2], 9 * fo[2], rtol=1e-13)
    np.testing.assert_allclose(add2[2], 9 * add[2], rtol=1e-13)
    np.testing.assert_allclose(fo2[[0, 1, 3]], fo[[0, 1, 3]], rtol=1e-14)


def test_token_replication_and_chunking():
    """E_t is a mean: duplicating the token set changes nothing; chunking over
    tokens only changes summation order."""
    L = tiny(T=40)
    fo, add = run_up(L)
    D = {k: (np.concatenate([v, v]) if k in ("a", "g", "u", "r") else v) for k, v in L.items()}
    fo2, add2 = run_up(D)
    np.testing.assert_allclose(fo2, fo, rtol=1e-13)
    np.testing.assert_allclose(add2, add, rtol=1e-13)
    fo3, add3 = run_up(L, token_chunk=7)
    np.testing.assert_allclose(fo3, fo, rtol=1e-13)
    np.testing.assert_allclose(add3, add, rtol=1e-13)
    assert np.all(fo >= 0) and np.all(add >= 0)


def test_restricted_rows_and_columns_match_full():
    L = tiny(H=6, G=3, I=11)
    fo, add = run_up(L)
    ks, gs = [10, 0, 4], [2, 0]
    fo_s, add_s = run_up(L, groups=gs, neurons=ks)
    np.testing.assert_allclose(fo_s, fo[np.ix_(gs, ks)], rtol=1e-13)
    np.testing.assert_allclose(add_s, add[np.ix_(gs, ks)], rtol=1e-13)


# ---------------------------------------------------------------- down edge
def test_down_edge_by_neuron_ablation():
    """S_down[k,g] = mean over tokens of the squared change of the next layer's
    q/k/v projections of group g when neuron k's write alpha_k w^d_k is removed
    from the residual (next-layer rms r' held fixed)."""
    L = tiny(H=4, G=2, d=3, hidden=10, I=6)
    H, G, d = 4, 2, 3
    grp_n = L["group_of_head_next"]
    xn, rn, gn = L["x_next"], L["r_next"], L["gamma_next"]
    alpha = silu_fwd(L["g"]) * L["u"]

    def qkv(x):
        y = gn[None, :] * x / rn[:, None]
        return y @ L["W_q"].T, y @ L["W_k"].T, y @ L["W_v"].T

    q0, k0, v0 = qkv(xn)
    I = L["g"].shape[1]
    want = np.zeros((I, G))
    for k in range(I):
        q1, k1, v1 = qkv(xn - alpha[:, k:k + 1] * L["W_down"][:, k][None, :])
        for gp in range(G):
            qh = [h for h in range(H) if grp_n[h] == gp]
            dq = np.concatenate([q0[:, h * d:(h + 1) * d] - q1[:, h * d:(h + 1) * d] for h in qh], 1)
            dk = k0[:, gp * d:(gp + 1) * d] - k1[:, gp * d:(gp + 1) * d]
            dv = v0[:, gp * d:(gp + 1) * d] - v1[:, gp * d:(gp + 1) * d]
            want[k, gp] = ((dq ** 2).sum(1) + (dk ** 2).sum(1) + (dv ** 2).sum(1)).mean()
    c = oracle.down_moment(L["g"], L["u"], L["r_next"])
    n = oracle.down_weight_norms(L["W_q"], L["W_k"], L["W_v"], gn, L["W_down"], grp_n, G_next=G)
    np.testing.assert_allclose(oracle.affinity_down(c, n), want, rtol=1e-10)


def test_down_norms_sum_to_full_projection_norm():
    L = tiny(H=6, G=3, d=2, hidden=8, I=5)
    grp_n = np.array([1, 0, 2, 1, 0, 2])
    n = oracle.down_weight_norms(L["W_q"], L["W_k"], L["W_v"], L["gamma_next"],
                                 L["W_down"], grp_n, G_next=3)
    W_all = np.concatenate([L["W_q"], L["W_k"], L["W_v"]])
    full = np.linalg.norm(W_all @ (L["gamma_next"][:, None] * L["W_down"]), axis=0) ** 2
    np.testing.assert_allclose(n.sum(0), full, rtol=1e-12)


def test_down_restricted_columns_match_full():
    L = tiny(H=4, G=2, I=9)
    ks = [8, 1, 3]
    c = oracle.down_moment(L["g"], L["u"], L["r_next"])
    n = oracle.down_weight_norms(L["W_q"], L["W_k"], L["W_v"], L["gamma_next"], L["W_down"],
                                 L["group_of_head_next"], G_next=2)
    c_s = oracle.down_moment(L["g"], L["u"], L["r_next"], neurons=ks)
    n_s = oracle.down_weight_norms(L["W_q"], L["W_k"], L["W_v"], L["gamma_next"], L["W_down"],
                                   L["group_of_head_next"], G_next=2, neurons=ks)
    np.testing.assert_allclose(c_s, c[ks], rtol=1e-14)
    np.testing.assert_allclose(n_s, n[:, ks], rtol=1e-13)


def test_down_moment_chunking():
    L = tiny(T=50)
    c1 = oracle.down_moment(L["g"], L["u"], L["r_next"], token_chunk=7)
    c2 = oracle.down_moment(L["g"], L["u"], L["r_next"])
    np.testing.assert_allclose(c1, c2, rtol=1e-13)


def test_layer_bundle_on_bf16_layer():
    """The full bundle runs on a bf16-stored layer (values converted exactly)."""
    sh = synth.LayerShape("pin-bf16", 33, 16, 4, 2, 8, 12, "bf16", 0.5)
    L = synth.make_layer(sh, 5)
    out = oracle.affinity_layer(L)
    assert out["S_fo"].shape == (2, 12) and out["S_down"].shape == (12, 2)
    assert np.all(np.isfinite(out["S_fo"])) and np.all(out["S_down"] >= 0)
