"""One layer's affinity pass through the C ABI, with buffers allocated once.

The pass follows section 3 ("Affinity scores") of "Affinity-Aware Sharding for
Delayed Tensor Parallelism": fold the up weights, take ||w^d_k||^2, run the
hot kernel over the calibration tokens (FO and the down-edge moment), the ADD
score through per-head Gram matrices, reduce the partial sums into S_fo and
S_add, then the down edge's weight norms and S_down.  Every step is a libhna
call on torch's current stream; this module only owns the buffers.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import torch

from . import _binding as B


class AffinityPass:
    def __init__(self, T: int, hidden: int, H: int, G: int, d: int, I: int, dtype: torch.dtype,
                 device="cuda", with_down: bool = True, H_next: Optional[int] = None,
                 G_next: Optional[int] = None, d_next: Optional[int] = None):
        dev = torch.device(device)
        code = B.HNA_BF16 if dtype == torch.bfloat16 else B.HNA_F32
        self.dims = B.make_dims(T, hidden, H, G, d, I, code)
        self.T = T
        self.device = dev
        u8 = dict(dtype=torch.uint8, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        L = B.lib()
        import ctypes
        self.M = torch.empty(B.folded_bytes(self.dims), **u8)
        self.fold_ws = torch.empty(max(16, L.hna_fold_workspace_bytes(ctypes.byref(self.dims))), **u8)
        self.up_ws = torch.empty(max(16, B.up_workspace_bytes(self.dims)), **u8)
        self.wd_sq = torch.empty(I, **f32)
        self.S_fo = torch.empty((G, I), **f32)
        self.S_add = torch.empty((G, I), **f32)
        self.c_down = torch.empty(I, **f32)
        self.with_down = with_down
        if with_down:
            Hn = H if H_next is None else H_next
            Gn = G if G_next is None else G_next
            dn = d if d_next is None else d_next
            self.ddims = B.hna_down_dims(hidden, I, Hn, Gn, dn, code)
            self.down_ws = torch.empty(max(16, B.down_workspace_bytes(self.ddims)), **u8)
            self.n_down = torch.empty((Gn, I), **f32)
            self.S_down = torch.empty((I, Gn), **f32)

    # -- individual steps -------------------------------------------------
    def fold(self, layer):
        B.fold_up_weights(self.dims, layer["W_o"], layer["gamma"], layer["W_gate"], layer["W_up"],
                          out=self.M, workspace=self.fold_ws)
        B.down_col_sqnorm(self.dims, layer["W_down"], out=self.wd_sq)

    def hot(self, layer, group_of_head: Sequence[int]):
        B.affinity_up(self.dims, layer["a"], layer["g"], layer["u"], layer["r"],
                      layer.get("r_next") if self.with_down else None, self.M, group_of_head,
                      workspace=self.up_ws)

    def add(self, layer, group_of_head: Sequence[int]):
        B.affinity_add(self.dims, layer["a"], layer["r"], self.M, group_of_head, self.up_ws)

    def finalize(self, scale: float, accumulate: bool = False):
        B.finalize_up(self.dims, self.wd_sq, self.up_ws, scale, accumulate=accumulate,
                      S_fo=self.S_fo, S_add=self.S_add,
                      c_down=self.c_down if self.with_down else None, want_c=self.with_down)

    def down(self, layer, group_of_head_next: Sequence[int]):
        B.down_weight_norms(self.ddims, layer["W_q"], layer["W_k"], layer["W_v"],
                            layer["gamma_next"], layer["W_down"], group_of_head_next,
                            out=self.n_down, workspace=self.down_ws)
        B.down_combine(self.c_down, self.n_down, out=self.S_down)

    def loo(self, layer, group_of_head: Sequence[int], scale: Optional[float] = None):
        """The exact leave-one-out score (needs layer["x_in"], and fold() first)."""
        if not hasattr(self, "S_loo"):
            import ctypes
            f32 = dict(dtype=torch.float32, device=self.device)
            self.S_loo = torch.empty((self.dims.G, self.dims.I), **f32)
            self.loo_ws = torch.empty(max(16, B.loo_workspace_bytes(self.dims)),
                                      dtype=torch.uint8, device=self.device)
        B.affinity_loo(self.dims, layer["a"], layer["g"], layer["u"], layer["x_in"],
                       layer["W_o"], layer["gamma"], layer["W_gate"], layer["W_up"], self.M,
                       group_of_head,
                       1.0 / max(self.T, 1) if scale is None else scale,
                       S_loo=self.S_loo, workspace=self.loo_ws)
        return self.S_loo

    # -- whole pass ---------------------------------------------------------
    def run(self, layer: Dict[str, torch.Tensor], scale: Optional[float] = None) -> Dict[str, torch.Tensor]:
        grp = [int(x) for x in layer["group_of_head"].tolist()]
        self.fold(layer)
        self.hot(layer, grp)
        self.add(layer, grp)
        self.finalize(1.0 / max(self.T, 1) if scale is None else scale)
        out = {"S_fo": self.S_fo, "S_add": self.S_add}
        if self.with_down:
            self.down(layer, [int(x) for x in layer["group_of_head_next"].tolist()])
            out.update({"c_down": self.c_down, "n_down": self.n_down, "S_down": self.S_down})
        return out


def pass_for_layer(layer: Dict[str, torch.Tensor], with_down: bool = True) -> AffinityPass:
    T, H, d = layer["a"].shape
    I, hidden = layer["W_gate"].shape
    G = int(max(layer["group_of_head"].tolist())) + 1
    kw = {}
    if with_down:
        kw = dict(H_next=layer["W_q"].shape[0] // d, G_next=layer["W_k"].shape[0] // d, d_next=d)
    return AffinityPass(T, hidden, H, G, d, I, layer["a"].dtype, device=layer["a"].device,
                        with_down=with_down and "W_q" in layer, **kw)


def affinity_layer(layer: Dict[str, torch.Tensor], with_down: bool = True) -> Dict[str, torch.Tensor]:
    """Run the whole pass on one layer dict (tensors on the GPU) and return the scores."""
    ap = pass_for_layer(layer, with_down=with_down)
    return ap.run(layer)


class StackPass:
    """The affinity pass over an N-layer stack (section 3, "Affinity scores").

    Per layer i: the weight fold, ||w^d||^2, the hot pass (FO sums and the
    down-edge token moment of layer i's neurons), ADD and the fixed-order
    reduction into S_fo[i], S_add[i].  Per adjacent pair (i, i+1): the down
    edge from layer i's neurons to layer i+1's KV groups, whose weight part
    uses layer i+1's attention projections W_q, W_k, W_v and pre-norm gain
    gamma'.  In a layer dict these sit under "W_q", "W_k", "W_v",
    "gamma_next" and "group_of_head_next" of layer i (the weights that follow
    layer i's FFN), with r_next the rms entering layer i+1's pre-norm.

    The weight-only work (fold, ||w^d||^2, down-edge weight norms) of every
    layer runs on a side stream that runs ahead of the token passes: layer
    i's token pass waits only for layer i's weights, so the weight GEMMs of
    later layers overlap the token passes of earlier ones.  Each layer owns
    its buffers; results are S_fo, S_add [N, G, I] and S_down [N-1, I, G']
    fp32 on the device.
    """

    def __init__(self, layers: Sequence[Dict[str, torch.Tensor]], overlap: bool = True):
        n = len(layers)
        if n < 1:
            raise ValueError("a stack needs at least one layer")
        self.n = n
        self.passes = [pass_for_layer(L, with_down=(i + 1 < n)) for i, L in enumerate(layers)]
        self.groups = [[int(x) for x in L["group_of_head"].tolist()] for L in layers]
        self.groups_next = [[int(x) for x in L["group_of_head_next"].tolist()] if i + 1 < n else None
                            for i, L in enumerate(layers)]
        T = self.passes[0].T
        if any(P.T != T for P in self.passes):
            raise ValueError("every layer of a stack sees the same calibration tokens")
        self.T = T
        self.overlap = overlap
        dev = self.passes[0].device
        self.side = torch.cuda.Stream(device=dev) if overlap else None
        self.ready = [torch.cuda.Event() for _ in range(n)] if overlap else None

    def _weights(self, i, L):
        P = self.passes[i]
        P.fold(L)
        if P.with_down:
            B.down_weight_norms(P.ddims, L["W_q"], L["W_k"], L["W_v"], L["gamma_next"],
                                L["W_down"], self.groups_next[i], out=P.n_down,
                                workspace=P.down_ws)

    def _tokens(self, i, L, scale):
        P = self.passes[i]
        P.hot(L, self.groups[i])
        P.add(L, self.groups[i])
        P.finalize(scale)
        if P.with_down:
            B.down_combine(P.c_down, P.n_down, out=P.S_down)

    def run(self, layers: Sequence[Dict[str, torch.Tensor]], scale: Optional[float] = None):
        """Enqueue the whole stack on torch's current stream (and the side
        stream); returns nothing, the scores stay in each layer's buffers."""
        if len(layers) != self.n:
            raise ValueError("layer count differs from the one the stack was built for")
        sc = 1.0 / max(self.T, 1) if scale is None else scale
        main = torch.cuda.current_stream()
        if self.overlap:
            self.side.wait_stream(main)          # inputs and buffers are ready on main
            with torch.cuda.stream(self.side):
                for i, L in enumerate(layers):
                    self._weights(i, L)
                    self.ready[i].record(self.side)
            for i, L in enumerate(layers):
                main.wait_event(self.ready[i])
                self._tokens(i, L, sc)
            main.wait_stream(self.side)           # nothing left running on the side
        else:
            for i, L in enumerate(layers):
                self._weights(i, L)
                self._tokens(i, L, sc)

    def scores(self):
        """(S_fo [N, G, I], S_add [N, G, I], S_down [N-1, I, G']) stacked copies."""
        S_fo = torch.stack([P.S_fo for P in self.passes])
        S_add = torch.stack([P.S_add for P in self.passes])
        S_down = (torch.stack([P.S_down for P in self.passes[:-1]]) if self.n > 1 else None)
        return S_fo, S_add, S_down
