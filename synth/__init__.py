"""Seeded synthetic calibration layers.

This module only draws and derives *inputs*: the activations and weights a
dense pre-norm SwiGLU layer would hand to the affinity pass.  It holds none of
the affinity arithmetic (no per-head pieces, no first-order damage, no scores),
so both the float64 oracle and the HIP path can consume what it produces
without sharing any of the method's code.

Recipe (one layer; every draw comes from one seeded torch generator, in this
fixed order):

  s_h  ~ LogNormal(0, sigma_s)            per-head magnitude, [H]
  a    ~ N(0, 1) * s_h                    per-head attention outputs, [T, H, d]
  W_o  ~ N(0, 1/(H*d))                    output projection, [hidden, H*d]
  W_gate, W_up ~ N(0, 1/hidden)           [I, hidden]
  W_down ~ N(0, 1/I)                      [hidden, I]
  gamma = 1 + 0.1*N(0, 1)                 FFN pre-norm gain, [hidden]
  x0   ~ N(0, 1)                          residual before attention, [T, hidden]
  W_q ~ N(0, 1/hidden) [H*d, hidden], W_k, W_v ~ N(0, 1/hidden) [G*d, hidden]
  gamma_next = 1 + 0.1*N(0, 1)            next layer's attention pre-norm gain
  (optional, drawn last) massive-activation tokens: each token is picked
  with probability frac, and value is added to residual dimension dim of x0
  on the picked tokens (the delimiter-token spikes of roughly 7000 in one
  residual dimension described in section 5, "Where the affinity
  concentrates"; the rms of such a token is about value / sqrt(hidden))

Derived quantities (float64, from the values already rounded to the storage
dtype, so that they are consistent with what the kernels see):

  x  = x0 + sum_h a_h W_o^(h)T            residual entering the FFN pre-norm
  r  = sqrt(mean(x^2))                    (no epsilon)
  g  = (gamma * x / r) W_gate^T,  u = (gamma * x / r) W_up^T
  alpha = silu(g) * u                     SwiGLU activation
  r_next = rms(x + alpha W_down^T)        rms entering the next layer's norm

Storage: "f32" rounds every tensor to float32; "bf16" rounds a, g, u and all
weight matrices to bfloat16 (round to nearest even) while gamma, gamma_next,
r, r_next stay float32 (gamma values are made bf16-representable).  "f64"
keeps everything in float64 (used by the oracle's own pin tests).

Standard GQA grouping is used: head h belongs to KV group h // (H // G).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch

__all__ = ["LayerShape", "CONFIGS", "layer_shape", "make_layer", "layer_seed",
           "contiguous_layout", "random_balanced_layout", "make_scores",
           "default_group_map"]


@dataclasses.dataclass(frozen=True)
class LayerShape:
    name: str
    T: int
    hidden: int
    H: int
    G: int
    d: int
    I: int
    dtype: str          # "f32" | "bf16" | "f64"
    sigma_s: float      # log-normal sigma of the per-head scales
    layers: int = 1

    def with_tokens(self, T: int) -> "LayerShape":
        return dataclasses.replace(self, T=int(T))

    def with_dtype(self, dtype: str) -> "LayerShape":
        return dataclasses.replace(self, dtype=dtype)


# The five workloads: a tiny fp32 layer, a Qwen3-0.6B-shaped layer, a
# Danube3-500M-shaped layer, the 28-layer Qwen3-0.6B-shaped stack and a large
# 4096/14336 layer with heavy-tailed head magnitudes.
CONFIGS: Dict[int, LayerShape] = {
    0: LayerShape("tiny-fp32", 256, 64, 4, 2, 16, 128, "f32", 0.5),
    1: LayerShape("qwen3-0.6b-layer", 65536, 1024, 16, 8, 128, 3072, "bf16", 0.5),
    2: LayerShape("danube3-500m-layer", 65536, 1536, 16, 8, 96, 4096, "bf16", 0.5),
    3: LayerShape("qwen3-0.6b-28-layer-stack", 65536, 1024, 16, 8, 128, 3072, "bf16", 0.5,
                  layers=28),
    4: LayerShape("large-4096x14336-layer", 131072, 4096, 32, 8, 128, 14336, "bf16", 1.0),
}


def layer_shape(config: int) -> LayerShape:
    return CONFIGS[int(config)]


def layer_seed(config: int, layer: int = 0, salt: int = 0) -> int:
    """Deterministic 63-bit seed for (config, layer, salt)."""
    v = (int(config) * 1_000_003 + int(layer)) * 1_000_033 + int(salt)
    return (v * 0x9E3779B97F4A7C15) % (1 << 63)


def default_group_map(H: int, G: int) -> torch.Tensor:
    per = H // G
    return torch.arange(H, dtype=torch.int32) // per


_STORE = {"f32": torch.float32, "bf16": torch.bfloat16, "f64": torch.float64}


def _round(x: torch.Tensor, dtype: str) -> torch.Tensor:
    """Round a float64 tensor to the storage dtype and return it as float64."""
    if dtype == "f64":
        return x
    if dtype == "f32":
        return x.to(torch.float32).to(torch.float64)
    # bf16: round through float32 first (the pages' tensors live in fp32 before
    # the bf16 cast), then round-to-nearest-even to bf16.
    return x.to(torch.float32).to(torch.bfloat16).to(torch.float64)


def _randn(gen: torch.Generator, shape, device) -> torch.Tensor:
    return torch.randn(shape, generator=gen, dtype=torch.float64, device=device)


def make_layer(shape: LayerShape, seed: int, device="cpu", with_next: bool = True,
               token_chunk: int = 8192, return_resid: bool = False,
               with_x: bool = False,
               massive: Optional[tuple] = None) -> Dict[str, torch.Tensor]:
    """Draw one synthetic layer.

    Returns a dict of tensors on ``device``.  Matrices use the (out, in)
    row-major convention of a linear layer.  Stored tensors have the storage
    dtype; r, r_next, gamma, gamma_next are float32 (float64 when dtype is
    "f64"), group_of_head is int32 on the CPU.  With ``return_resid`` the
    float64 residuals x (entering the FFN norm) and x_next (entering the next
    layer's norm) are returned too, for forward-pass checks on small layers.
    With ``with_x`` the residual entering the FFN norm is returned as "x_in",
    rounded to float32 (float64 for "f64"): the input of the leave-one-out
    score, which renormalises the residual without a head.
    ``massive`` = (frac, dim, value) adds massive-activation tokens (see the
    module docstring); the draw comes after every other one, so the rest of
    the layer is the same as without it.
    """
    device = torch.device(device)
    T, D, H, G, d, I = shape.T, shape.hidden, shape.H, shape.G, shape.d, shape.I
    if H % G:
        raise ValueError("H must be a multiple of G")
    st = shape.dtype
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))

    s_h = torch.exp(shape.sigma_s * _randn(gen, (H,), device))
    a = _round(_randn(gen, (T, H, d), device) * s_h[None, :, None], st)
    W_o = _round(_randn(gen, (D, H * d), device) / math.sqrt(H * d), st)
    W_gate = _round(_randn(gen, (I, D), device) / math.sqrt(D), st)
    W_up = _round(_randn(gen, (I, D), device) / math.sqrt(D), st)
    W_down = _round(_randn(gen, (D, I), device) / math.sqrt(I), st)
    gamma = 1.0 + 0.1 * _randn(gen, (D,), device)
    gamma = _round(gamma, "bf16" if st == "bf16" else st)
    x0 = _round(_randn(gen, (T, D), device), "f32" if st != "f64" else "f64")
    nxt = {}
    if with_next:
        nxt["W_q"] = _round(_randn(gen, (H * d, D), device) / math.sqrt(D), st)
        nxt["W_k"] = _round(_randn(gen, (G * d, D), device) / math.sqrt(D), st)
        nxt["W_v"] = _round(_randn(gen, (G * d, D), device) / math.sqrt(D), st)
        gn = 1.0 + 0.1 * _randn(gen, (D,), device)
        nxt["gamma_next"] = _round(gn, "bf16" if st == "bf16" else st)
    if massive is not None:
        frac, mdim, mval = massive
        picked = torch.rand((T,), generator=gen, dtype=torch.float64, device=device) < frac
        x0[picked, int(mdim)] += float(mval)

    out_dt = _STORE[st]
    scal_dt = torch.float64 if st == "f64" else torch.float32
    g_out = torch.empty((T, I), dtype=out_dt, device=device)
    u_out = torch.empty((T, I), dtype=out_dt, device=device)
    r_out = torch.empty((T,), dtype=scal_dt, device=device)
    rn_out = torch.empty((T,), dtype=scal_dt, device=device) if with_next else None
    x_keep, xn_keep = [], []
    x_in = torch.empty((T, D), dtype=scal_dt, device=device) if with_x else None
    a_flat = a.reshape(T, H * d)
    for t0 in range(0, T, token_chunk):
        t1 = min(T, t0 + token_chunk)
        x = x0[t0:t1] + a_flat[t0:t1] @ W_o.T
        r = torch.sqrt((x * x).mean(dim=1))
        r_st = r.to(scal_dt).to(torch.float64)
        y = gamma[None, :] * x / r_st[:, None]
        g = _round(y @ W_gate.T, st)
        u = _round(y @ W_up.T, st)
        g_out[t0:t1] = g.to(out_dt)
        u_out[t0:t1] = u.to(out_dt)
        r_out[t0:t1] = r_st.to(scal_dt)
        if with_next:
            alpha = g * torch.sigmoid(g) * u
            xn = x + alpha @ W_down.T
            rn_out[t0:t1] = torch.sqrt((xn * xn).mean(dim=1)).to(scal_dt)
            if return_resid:
                xn_keep.append(xn)
        if return_resid:
            x_keep.append(x)
        if with_x:
            x_in[t0:t1] = x.to(scal_dt)
        del x, y, g, u

    layer = {
        "a": a.to(out_dt), "g": g_out, "u": u_out, "r": r_out,
        "gamma": gamma.to(scal_dt), "W_o": W_o.to(out_dt),
        "W_gate": W_gate.to(out_dt), "W_up": W_up.to(out_dt),
        "W_down": W_down.to(out_dt),
        "group_of_head": default_group_map(H, G),
    }
    if with_next:
        layer.update({
            "r_next": rn_out,
            "W_q": nxt["W_q"].to(out_dt), "W_k": nxt["W_k"].to(out_dt),
            "W_v": nxt["W_v"].to(out_dt), "gamma_next": nxt["gamma_next"].to(scal_dt),
            "group_of_head_next": default_group_map(H, G),
        })
    if with_x:
        layer["x_in"] = x_in
    if return_resid:
        layer["x"] = torch.cat(x_keep)
        if with_next:
            layer["x_next"] = torch.cat(xn_keep)
    return layer


def make_config_layer(config: int, layer: int = 0, T: Optional[int] = None,
                      device="cpu", dtype: Optional[str] = None,
                      with_next: bool = True, with_x: bool = False) -> Dict[str, torch.Tensor]:
    """Layer ``layer`` of workload ``config`` (optionally with T or dtype overridden)."""
    sh = layer_shape(config)
    if T is not None:
        sh = sh.with_tokens(T)
    if dtype is not None:
        sh = sh.with_dtype(dtype)
    return make_layer(sh, layer_seed(config, layer), device=device, with_next=with_next,
                      with_x=with_x)


# ---------------------------------------------------------------------------
# Layouts and score matrices for the layout objective
#
# A layout of an N-layer stack on L devices is, per layer i, a device for each
# KV group (heads[i][g]) and for each FFN neuron (neurons[i][k]).  Every layout
# here is balanced: G/L groups and I/L neurons per device.  "Contiguous" slices
# groups and neurons in storage order; a random layout is a uniform balanced
# permutation of the contiguous one, drawn independently per layer.  These are
# inputs of the objective, as the scores are; nothing here evaluates it.

def contiguous_layout(N: int, G: int, I: int, L: int):
    """(heads [N, G], neurons [N, I]) int32: device g // (G/L) and k // (I/L)."""
    if G % L or I % L:
        raise ValueError(f"G={G} and I={I} must be multiples of L={L}")
    heads = (torch.arange(G, dtype=torch.int32) // (G // L)).repeat(N, 1)
    neurons = (torch.arange(I, dtype=torch.int32) // (I // L)).repeat(N, 1)
    return heads, neurons


def random_balanced_layout(N: int, G: int, I: int, L: int, seed: int):
    """Uniform balanced layout: each layer permutes the contiguous assignment."""
    gen = torch.Generator().manual_seed(seed)
    h0, n0 = contiguous_layout(1, G, I, L)
    heads = torch.stack([h0[0][torch.randperm(G, generator=gen)] for _ in range(N)])
    neurons = torch.stack([n0[0][torch.randperm(I, generator=gen)] for _ in range(N)])
    return heads, neurons


def make_scores(N: int, G: int, I: int, seed: int, sigma: float = 1.0, zero_frac: float = 0.0):
    """Non-negative stand-ins for the affinity scores of an N-layer stack:
    S_up [N, G, I] and S_down [N-1, I, G], float32, log-normal entries with a
    per-(layer, group) scale (some groups matter more, as on the pages'
    figures), optionally with a fraction of exact zeros."""
    gen = torch.Generator().manual_seed(seed)
    gscale = torch.exp(sigma * torch.randn(N, G, 1, generator=gen, dtype=torch.float64))
    up = gscale * torch.exp(sigma * torch.randn(N, G, I, generator=gen, dtype=torch.float64))
    gs2 = torch.exp(sigma * torch.randn(max(N - 1, 0), 1, G, generator=gen, dtype=torch.float64))
    down = gs2 * torch.exp(sigma * torch.randn(max(N - 1, 0), I, G, generator=gen, dtype=torch.float64))
    if zero_frac > 0:
        up[torch.rand(up.shape, generator=gen, dtype=torch.float64) < zero_frac] = 0
        down[torch.rand(down.shape, generator=gen, dtype=torch.float64) < zero_frac] = 0
    return up.to(torch.float32), down.to(torch.float32)
