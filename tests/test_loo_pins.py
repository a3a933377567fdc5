"""Pins of the leave-one-out oracle (section 3, "Affinity scores") to facts
outside its own code."""
import math

import numpy as np
import pytest

import oracle
import synth


def small_layer(seed=3, T=96, scale_a=1.0):
    sh = synth.LayerShape("loo-pin", T, 48, 4, 2, 16, 40, "f64", 0.5)
    L = synth.make_layer(sh, seed, with_next=False, with_x=True)
    return {k: (v.numpy() if hasattr(v, "numpy") else v) for k, v in L.items()}


def test_hand_computed_example():
    # hidden = 2, one head of width 1, one token: x = (3, 4), the head writes
    # o = (1, 0); gamma = 1; w^g = (1, 0), w^u = (0, 1).  Without the head the
    # residual is (2, 4): rms sqrt(12.5) -> sqrt(10).
    a = np.array([[[1.0]]])
    x = np.array([[3.0, 4.0]])
    W_o = np.array([[1.0], [0.0]])
    gamma = np.ones(2)
    W_gate = np.array([[1.0, 0.0]])
    W_up = np.array([[0.0, 1.0]])
    S = oracle.loo_scores(a, x, gamma, W_o, W_gate, W_up, [0])
    dg = 3 / math.sqrt(12.5) - 2 / math.sqrt(10)
    du = 4 / math.sqrt(12.5) - 4 / math.sqrt(10)
    assert S.shape == (1, 1)
    assert abs(S[0, 0] - (dg * dg + du * du)) < 1e-15


def test_equals_add_when_the_rms_is_unchanged():
    # one head; per token the rest of the residual is projected so that
    # x . o = |o|^2 / 2, i.e. |x - o| = |x|: removing the head leaves the rms
    # unchanged, and the leave-one-out score is exactly ADD
    rng = np.random.default_rng(6)
    T, D, d, I = 64, 24, 8, 30
    a = rng.standard_normal((T, 1, d))
    W_o = rng.standard_normal((D, d)) / math.sqrt(d)
    gamma = 1 + 0.1 * rng.standard_normal(D)
    W_gate = rng.standard_normal((I, D)) / math.sqrt(D)
    W_up = rng.standard_normal((I, D)) / math.sqrt(D)
    o = a[:, 0, :] @ W_o.T
    rest = rng.standard_normal((T, D))
    oo = (o * o).sum(1)
    rest -= (((rest * o).sum(1) + oo / 2) / oo)[:, None] * o
    x = rest + o
    assert np.allclose(((x - o) ** 2).sum(1), (x * x).sum(1))
    r = np.sqrt((x * x).mean(1))
    y = gamma * x / r[:, None]
    g, u = y @ W_gate.T, y @ W_up.T
    S_loo = oracle.loo_scores(a, x, gamma, W_o, W_gate, W_up, [0])
    _, S_add = oracle.affinity_up(a, g, u, r, gamma, W_o, W_gate, W_up, np.ones((D, I)), [0], G=1)
    assert np.max(np.abs(S_loo - S_add)) <= 1e-12 * np.max(S_add)


def test_split_into_rescaled_preactivation_and_piece():
    # g - g^(-h) = g (1 - r / r^(-h)) + (p_h . w^g) r / r^(-h), with p_h the
    # head piece of affinity.py: an algebraic route independent of the ablation
    L = small_layer(seed=4)
    a, x, gamma = L["a"], L["x_in"], L["gamma"]
    T, H, d = a.shape
    r = np.sqrt((x * x).mean(1))
    y = gamma * x / r[:, None]
    g, u = y @ L["W_gate"].T, y @ L["W_up"].T
    ref = np.zeros((2, L["W_gate"].shape[0]))
    for h in range(H):
        o = a[:, h, :] @ L["W_o"][:, h * d:(h + 1) * d].T
        rm = np.sqrt(((x - o) ** 2).mean(1))
        rho = (r / rm)[:, None]
        p = oracle.head_piece(a[:, h, :], r, gamma, L["W_o"], h)
        dg = g * (1 - rho) + (p @ L["W_gate"].T) * rho
        du = u * (1 - rho) + (p @ L["W_up"].T) * rho
        ref[L["group_of_head"][h]] += (dg * dg + du * du).mean(0)
    S = oracle.loo_scores(a, x, gamma, L["W_o"], L["W_gate"], L["W_up"], L["group_of_head"])
    assert np.max(np.abs(S - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_zero_heads_groups_and_duplicates():
    L = small_layer(seed=5)
    a = L["a"].copy()
    a[:, 0:2, :] = 0.0                                  # both heads of group 0 vanish
    args = (L["x_in"], L["gamma"], L["W_o"], L["W_gate"], L["W_up"])
    S = oracle.loo_scores(a, *args, L["group_of_head"])
    assert np.all(S[0] == 0.0) and np.all(S[1] > 0)
    # a group's row is the sum of its heads' rows
    per_head = oracle.loo_scores(L["a"], *args, np.arange(4), G=4)
    grouped = oracle.loo_scores(L["a"], *args, L["group_of_head"])
    assert np.allclose(grouped, per_head[[0, 2]] + per_head[[1, 3]], rtol=1e-13, atol=0)
    # duplicating every token leaves the mean unchanged; chunking only reorders sums
    a2 = np.concatenate([L["a"], L["a"]])
    x2 = np.concatenate([L["x_in"], L["x_in"]])
    S2 = oracle.loo_scores(a2, x2, *args[1:], L["group_of_head"], token_chunk=37)
    assert np.allclose(S2, grouped, rtol=1e-12, atol=0)
