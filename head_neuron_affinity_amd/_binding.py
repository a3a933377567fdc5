"""ctypes binding of libhna (include/hna.h).

Argument marshalling only: tensors become device pointers, the stream is
torch's current HIP stream, and output / workspace buffers are allocated with
torch.  Every step of the computation runs in the library's HIP kernels.
There is no fallback: if the library is missing or the call fails, an
exception is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# HNA_LIB_PATH selects another build of the same library (the sanitizer
# build of the host-validation test); the default is the in-tree libhna.so
LIB_PATH = os.environ.get("HNA_LIB_PATH") or os.path.join(_PKG, "libhna.so")

HNA_OK = 0
HNA_ERR_INVALID_ARG = -1
HNA_ERR_UNSUPPORTED = -2
HNA_ERR_ALIGNMENT = -3
HNA_ERR_WORKSPACE = -4
HNA_ERR_HIP = -5
HNA_F32 = 0
HNA_BF16 = 1
HNA_ACCUMULATE = 1
HNA_LAYOUT_OK = 0
HNA_LAYOUT_BAD_HEADS = 1
HNA_LAYOUT_SWAP_LIMIT = 2
HNA_LAYOUT_NO_MOVE = 3
HNA_LAYOUT_BAD_NEURONS = 4
DUAL_ITERS = 300

EXPORTED = [
    "hna_abi_version", "hna_status_string", "hna_last_error", "hna_folded_bytes",
    "hna_fold_workspace_bytes", "hna_fold_up_weights", "hna_down_col_sqnorm",
    "hna_up_workspace_bytes", "hna_affinity_up", "hna_affinity_add", "hna_finalize_up",
    "hna_down_workspace_bytes", "hna_down_weight_norms", "hna_down_combine", "hna_unit_mass",
    "hna_layout_objective", "hna_neuron_step", "hna_head_step",
    "hna_layout_search_workspace_bytes", "hna_layout_search", "hna_loo_workspace_bytes",
    "hna_affinity_loo", "hna_static_scratch_bytes", "hna_affinity_up_static",
    "hna_mfma_rate_probe",
]


class hna_dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("hidden", ctypes.c_int32), ("H", ctypes.c_int32),
                ("G", ctypes.c_int32), ("d", ctypes.c_int32), ("I", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


class hna_down_dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("I", ctypes.c_int32), ("H", ctypes.c_int32),
                ("G", ctypes.c_int32), ("d", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class HnaError(RuntimeError):
    def __init__(self, status: int, where: str, msg: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({msg})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libhna.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m head_neuron_affinity_amd.build_lib`")
    L = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, i64, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    dp = ctypes.POINTER(hna_dims)
    ddp = ctypes.POINTER(hna_down_dims)
    ip = ctypes.POINTER(ctypes.c_int32)
    sig = {
        "hna_abi_version": (ctypes.c_int, []),
        "hna_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "hna_last_error": (ctypes.c_char_p, []),
        "hna_folded_bytes": (sz, [dp]),
        "hna_fold_workspace_bytes": (sz, [dp]),
        "hna_fold_up_weights": (ctypes.c_int, [dp, vp, vp, vp, vp, vp, sz, vp, sz, vp]),
        "hna_down_col_sqnorm": (ctypes.c_int, [dp, vp, vp, vp]),
        "hna_up_workspace_bytes": (sz, [dp]),
        "hna_affinity_up": (ctypes.c_int, [dp, vp, vp, vp, vp, vp, vp, ip, vp, sz, vp]),
        "hna_affinity_add": (ctypes.c_int, [dp, vp, vp, vp, ip, vp, sz, vp]),
        "hna_finalize_up": (ctypes.c_int, [dp, vp, f32, ctypes.c_int, vp, sz, vp, vp, vp, vp]),
        "hna_down_workspace_bytes": (sz, [ddp]),
        "hna_down_weight_norms": (ctypes.c_int, [ddp, vp, vp, vp, vp, vp, ip, vp, vp, sz, vp]),
        "hna_down_combine": (ctypes.c_int, [i32, i32, vp, vp, vp, vp]),
        "hna_unit_mass": (ctypes.c_int, [vp, i64, i32, vp, vp]),
        "hna_layout_objective": (ctypes.c_int, [i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]),
        "hna_neuron_step": (ctypes.c_int, [i32, i32, i32, i32, vp, vp, vp, i32, i32, vp, vp, vp]),
        "hna_head_step": (ctypes.c_int, [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp]),
        "hna_layout_search_workspace_bytes": (sz, [i32, i32, i32]),
        "hna_loo_workspace_bytes": (sz, [dp]),
        "hna_static_scratch_bytes": (sz, []),
        "hna_affinity_up_static": (ctypes.c_int, [dp, vp, vp, vp, vp, vp, vp, vp, ip, f32,
                                                  ctypes.c_int, vp, vp, vp, vp]),
        "hna_affinity_loo": (ctypes.c_int, [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ip, f32, vp, vp,
                                            sz, vp]),
        "hna_mfma_rate_probe": (ctypes.c_int, [i32, i32, i32, vp, vp, vp]),
        "hna_layout_search": (ctypes.c_int, [i32, i32, i32, i32, vp, vp, i32, i32, i32, vp, vp, vp,
                                              ctypes.POINTER(ctypes.c_double), ip, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().hna_status_string(int(status)).decode()


def last_error() -> str:
    return lib().hna_last_error().decode()


def _check(status: int, where: str):
    if status != HNA_OK:
        raise HnaError(status, where, last_error())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return HNA_BF16
    if t.dtype == torch.float32:
        return HNA_F32
    raise TypeError(f"unsupported dtype {t.dtype}: bf16 or fp32 only")


def _map(group_of_head: Sequence[int]):
    arr = (ctypes.c_int32 * len(group_of_head))(*[int(x) for x in group_of_head])
    return arr


def make_dims(T: int, hidden: int, H: int, G: int, d: int, I: int, dtype: int) -> hna_dims:
    return hna_dims(int(T), int(hidden), int(H), int(G), int(d), int(I), int(dtype))


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must live on the GPU")
        if t is not None and not t.is_contiguous():
            raise ValueError("all tensors must be contiguous")


def _torch_dtype(dims) -> torch.dtype:
    return torch.bfloat16 if dims.dtype == HNA_BF16 else torch.float32


def _expect(t: Optional[torch.Tensor], name: str, shape, dtype: torch.dtype,
            tokens: bool = False):
    """Shape and dtype of an argument, checked before its pointer is handed
    over (the C ABI sees addresses only, so a short or mistyped tensor would
    otherwise be read past its end).  With `tokens` the leading (token) dim may
    be longer than the call's T: the call reads the first T rows."""
    if t is None:
        return
    want = tuple(int(x) for x in shape)
    got = tuple(t.shape)
    ok = (len(got) == len(want) and got[1:] == want[1:] and got[0] >= want[0]) if tokens \
        else got == want
    if not ok:
        raise ValueError(f"{name}: shape {got}, expected {want}"
                         + (" (leading dim at least)" if tokens else ""))
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")


def _expect_bytes(t: torch.Tensor, name: str, nbytes: int):
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{name}: {t.numel() * t.element_size()} bytes, needs {nbytes}")


def _up_inputs(dims: hna_dims, a=None, g=None, u=None, r=None, r_next=None, M=None):
    dt = _torch_dtype(dims)
    _expect(a, "a", (dims.T, dims.H, dims.d), dt, tokens=True)
    _expect(g, "g", (dims.T, dims.I), dt, tokens=True)
    _expect(u, "u", (dims.T, dims.I), dt, tokens=True)
    _expect(r, "r", (dims.T,), torch.float32, tokens=True)
    _expect(r_next, "r_next", (dims.T,), torch.float32, tokens=True)
    if M is not None:
        _expect_bytes(M, "M", folded_bytes(dims))


def _weights(dims: hna_dims, W_o=None, gamma=None, W_gate=None, W_up=None, W_down=None):
    dt = _torch_dtype(dims)
    _expect(W_o, "W_o", (dims.hidden, dims.H * dims.d), dt)
    _expect(gamma, "gamma", (dims.hidden,), torch.float32)
    _expect(W_gate, "W_gate", (dims.I, dims.hidden), dt)
    _expect(W_up, "W_up", (dims.I, dims.hidden), dt)
    _expect(W_down, "W_down", (dims.hidden, dims.I), dt)


# ------------------------------------------------------------------ calls
def folded_bytes(dims: hna_dims) -> int:
    n = lib().hna_folded_bytes(ctypes.byref(dims))
    if n == 0:
        _check(HNA_ERR_INVALID_ARG, "hna_folded_bytes")
    return n


def fold_up_weights(dims: hna_dims, W_o, gamma, W_gate, W_up, out: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """M_h = W_o^(h)T diag(gamma) [W_gate; W_up]^T in the kernel's layout (opaque bytes)."""
    _need_cuda(W_o, gamma, W_gate, W_up)
    _weights(dims, W_o=W_o, gamma=gamma, W_gate=W_gate, W_up=W_up)
    L = lib()
    nb = folded_bytes(dims)
    if out is None:
        out = torch.empty(nb, dtype=torch.uint8, device=W_o.device)
    wsb = L.hna_fold_workspace_bytes(ctypes.byref(dims))
    if workspace is None:
        workspace = torch.empty(max(wsb, 16), dtype=torch.uint8, device=W_o.device)
    _check(L.hna_fold_up_weights(ctypes.byref(dims), _ptr(W_o), _ptr(gamma), _ptr(W_gate),
                                 _ptr(W_up), _ptr(out), out.numel() * out.element_size(),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(W_o.device)), "hna_fold_up_weights")
    return out


def down_col_sqnorm(dims: hna_dims, W_down, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    _need_cuda(W_down)
    _weights(dims, W_down=W_down)
    if out is None:
        out = torch.empty(dims.I, dtype=torch.float32, device=W_down.device)
    _expect(out, "out", (dims.I,), torch.float32)
    _check(lib().hna_down_col_sqnorm(ctypes.byref(dims), _ptr(W_down), _ptr(out),
                                     _stream(W_down.device)), "hna_down_col_sqnorm")
    return out


def up_workspace_bytes(dims: hna_dims) -> int:
    return int(lib().hna_up_workspace_bytes(ctypes.byref(dims)))


def affinity_up(dims: hna_dims, a, g, u, r, r_next, M, group_of_head,
                workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The hot pass; returns the workspace holding the partial sums."""
    _need_cuda(a, g, u, r, r_next, M)
    _up_inputs(dims, a, g, u, r, r_next, M)
    L = lib()
    wsb = L.hna_up_workspace_bytes(ctypes.byref(dims))
    if workspace is None:
        workspace = torch.empty(max(wsb, 16), dtype=torch.uint8, device=a.device)
    _check(L.hna_affinity_up(ctypes.byref(dims), _ptr(a), _ptr(g), _ptr(u), _ptr(r), _ptr(r_next),
                             _ptr(M), _map(group_of_head), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(a.device)),
           "hna_affinity_up")
    return workspace


def affinity_add(dims: hna_dims, a, r, M, group_of_head, workspace: torch.Tensor) -> torch.Tensor:
    """The ADD score through per-head Gram matrices, into the same workspace."""
    _need_cuda(a, r, M, workspace)
    _up_inputs(dims, a=a, r=r, M=M)
    _check(lib().hna_affinity_add(ctypes.byref(dims), _ptr(a), _ptr(r), _ptr(M),
                                  _map(group_of_head), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(a.device)),
           "hna_affinity_add")
    return workspace


def finalize_up(dims: hna_dims, wd_sq, workspace, scale: float, accumulate: bool = False,
                S_fo=None, S_add=None, c_down=None, want_c: bool = True):
    _need_cuda(wd_sq, workspace)
    dev = wd_sq.device
    if S_fo is None:
        S_fo = torch.empty((dims.G, dims.I), dtype=torch.float32, device=dev)
    if S_add is None:
        S_add = torch.empty((dims.G, dims.I), dtype=torch.float32, device=dev)
    if c_down is None and want_c:
        c_down = torch.empty(dims.I, dtype=torch.float32, device=dev)
    _need_cuda(S_fo, S_add, c_down)
    _expect(wd_sq, "wd_sq", (dims.I,), torch.float32)
    _expect(S_fo, "S_fo", (dims.G, dims.I), torch.float32)
    _expect(S_add, "S_add", (dims.G, dims.I), torch.float32)
    _expect(c_down, "c_down", (dims.I,), torch.float32)
    _check(lib().hna_finalize_up(ctypes.byref(dims), _ptr(wd_sq), float(scale),
                                 HNA_ACCUMULATE if accumulate else 0, _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _ptr(S_fo),
                                 _ptr(S_add), _ptr(c_down), _stream(dev)), "hna_finalize_up")
    return S_fo, S_add, c_down


def down_workspace_bytes(ddims: hna_down_dims) -> int:
    return int(lib().hna_down_workspace_bytes(ctypes.byref(ddims)))


def down_weight_norms(ddims: hna_down_dims, W_q, W_k, W_v, gamma_next, W_down, group_of_head_next,
                      out=None, workspace=None) -> torch.Tensor:
    _need_cuda(W_q, W_k, W_v, gamma_next, W_down)
    dt = torch.bfloat16 if ddims.dtype == HNA_BF16 else torch.float32
    _expect(W_q, "W_q", (ddims.H * ddims.d, ddims.hidden), dt)
    _expect(W_k, "W_k", (ddims.G * ddims.d, ddims.hidden), dt)
    _expect(W_v, "W_v", (ddims.G * ddims.d, ddims.hidden), dt)
    _expect(gamma_next, "gamma_next", (ddims.hidden,), torch.float32)
    _expect(W_down, "W_down", (ddims.hidden, ddims.I), dt)
    L = lib()
    dev = W_q.device
    if out is None:
        out = torch.empty((ddims.G, ddims.I), dtype=torch.float32, device=dev)
    wsb = L.hna_down_workspace_bytes(ctypes.byref(ddims))
    if workspace is None:
        workspace = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    _check(L.hna_down_weight_norms(ctypes.byref(ddims), _ptr(W_q), _ptr(W_k), _ptr(W_v),
                                   _ptr(gamma_next), _ptr(W_down), _map(group_of_head_next),
                                   _ptr(out), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(dev)),
           "hna_down_weight_norms")
    return out


def down_combine(c_down, n, out=None) -> torch.Tensor:
    _need_cuda(c_down, n)
    G, I = n.shape
    _expect(c_down, "c_down", (I,), torch.float32)
    _expect(n, "n", (G, I), torch.float32)
    if out is None:
        out = torch.empty((I, G), dtype=torch.float32, device=n.device)
    _check(lib().hna_down_combine(int(I), int(G), _ptr(c_down), _ptr(n), _ptr(out),
                                  _stream(n.device)), "hna_down_combine")
    return out


# ------------------------------------------------------- layout objective
def mfma_rate_probe(seed: torch.Tensor, n_workgroups: int, iters: int,
                    out: Optional[torch.Tensor] = None, shape: int = 0) -> torch.Tensor:
    """Run the matrix-core rate probe (hna_mfma_rate_probe; shape 0: 32x32x16
    MFMAs, 1: 16x16x32): `seed` holds n_workgroups * 256 * 128 bytes of bf16
    operands; returns the per-thread checksums (fp32, n_workgroups * 256)."""
    _need_cuda(seed)
    n = int(n_workgroups) * 256
    if seed.numel() * seed.element_size() < n * 128:
        raise ValueError(f"seed: {seed.numel() * seed.element_size()} bytes, needs {n * 128}")
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=seed.device)
    _expect(out, "out", (n,), torch.float32)
    _check(lib().hna_mfma_rate_probe(int(n_workgroups), int(iters), int(shape), _ptr(seed),
                                     _ptr(out), _stream(seed.device)), "hna_mfma_rate_probe")
    return out


def unit_mass(S: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Each matrix S[m] (fp32, last two dims) divided by its own sum; 0 if the sum is 0."""
    _need_cuda(S)
    if S.dtype != torch.float32 or S.dim() < 2:
        raise ValueError("S must be an fp32 tensor of at least 2 dims")
    if out is None:
        out = torch.empty_like(S)
    count = S.shape[-1] * S.shape[-2]
    n_mat = S.numel() // count if count else 0
    _check(lib().hna_unit_mass(_ptr(S), int(count), int(n_mat), _ptr(out), _stream(S.device)),
           "hna_unit_mass")
    return out


def layout_objective(S_up: torch.Tensor, S_down: Optional[torch.Tensor], head_device: torch.Tensor,
                     neuron_device: torch.Tensor, frac_up: Optional[torch.Tensor] = None,
                     frac_down: Optional[torch.Tensor] = None, J: Optional[torch.Tensor] = None):
    """J of eq. (6) with the per-matrix co-located fractions (fp64 device tensors).

    S_up [N, G, I], S_down [N-1, I, G] fp32; head_device [N, G], neuron_device [N, I] int32.
    Returns (J [1], frac_up [N], frac_down [N-1]).
    """
    _need_cuda(S_up, S_down, head_device, neuron_device)
    N, G, I = S_up.shape
    if S_up.dtype != torch.float32 or (S_down is not None and S_down.dtype != torch.float32):
        raise ValueError("scores must be fp32")
    if head_device.dtype != torch.int32 or neuron_device.dtype != torch.int32:
        raise ValueError("device maps must be int32")
    if tuple(head_device.shape) != (N, G) or tuple(neuron_device.shape) != (N, I):
        raise ValueError("device maps must be [N, G] and [N, I]")
    if N > 1 and (S_down is None or tuple(S_down.shape) != (N - 1, I, G)):
        raise ValueError("S_down must be [N-1, I, G]")
    dev = S_up.device
    if frac_up is None:
        frac_up = torch.empty(N, dtype=torch.float64, device=dev)
    if frac_down is None:
        frac_down = torch.empty(max(N - 1, 1), dtype=torch.float64, device=dev)
    if J is None:
        J = torch.empty(1, dtype=torch.float64, device=dev)
    _check(lib().hna_layout_objective(int(N), int(G), int(I), _ptr(S_up),
                                      _ptr(S_down) if N > 1 else None, _ptr(head_device),
                                      _ptr(neuron_device), _ptr(frac_up),
                                      _ptr(frac_down) if N > 1 else None, _ptr(J),
                                      _stream(dev)), "hna_layout_objective")
    return J, frac_up, frac_down[:N - 1]


def neuron_step(S_up_hat: torch.Tensor, S_down_hat: Optional[torch.Tensor],
                head_device: torch.Tensor, L: int, iters: int = DUAL_ITERS,
                max_swaps: Optional[int] = None, neuron_device: Optional[torch.Tensor] = None,
                stats: Optional[torch.Tensor] = None):
    """Neuron step of the layout search for every layer (section 3, "Optimiser").

    S_up_hat [N, G, I], S_down_hat [N-1, I, G] fp32 unit-mass scores;
    head_device [N, G] int32 in [0, L).  Returns (neuron_device [N, I] int32,
    stats [N, 4] int32: status, excess after the dual ascent, moves, swaps).
    """
    _need_cuda(S_up_hat, S_down_hat, head_device)
    N, G, I = S_up_hat.shape
    if S_up_hat.dtype != torch.float32 or (S_down_hat is not None and S_down_hat.dtype != torch.float32):
        raise ValueError("scores must be fp32")
    if head_device.dtype != torch.int32 or tuple(head_device.shape) != (N, G):
        raise ValueError("head_device must be int32 [N, G]")
    if N > 1 and (S_down_hat is None or tuple(S_down_hat.shape) != (N - 1, I, G)):
        raise ValueError("S_down_hat must be [N-1, I, G]")
    dev = S_up_hat.device
    if max_swaps is None:
        max_swaps = 4 * I
    if neuron_device is None:
        neuron_device = torch.empty((N, I), dtype=torch.int32, device=dev)
    if stats is None:
        stats = torch.empty((N, 4), dtype=torch.int32, device=dev)
    _check(lib().hna_neuron_step(int(N), int(G), int(I), int(L), _ptr(S_up_hat),
                                 _ptr(S_down_hat) if N > 1 else None, _ptr(head_device),
                                 int(iters), int(max_swaps), _ptr(neuron_device), _ptr(stats),
                                 _stream(dev)), "hna_neuron_step")
    return neuron_device, stats


def head_step(S_up_hat: torch.Tensor, S_down_hat: Optional[torch.Tensor],
              neuron_device: torch.Tensor, L: int):
    """Head step of the layout search for every layer (section 3, "Optimiser").

    Returns (head_device [N, G] int32, score [N] fp64, status [N] int32)."""
    _need_cuda(S_up_hat, S_down_hat, neuron_device)
    N, G, I = S_up_hat.shape
    if neuron_device.dtype != torch.int32 or tuple(neuron_device.shape) != (N, I):
        raise ValueError("neuron_device must be int32 [N, I]")
    if N > 1 and (S_down_hat is None or tuple(S_down_hat.shape) != (N - 1, I, G)):
        raise ValueError("S_down_hat must be [N-1, I, G]")
    dev = S_up_hat.device
    heads = torch.empty((N, G), dtype=torch.int32, device=dev)
    score = torch.empty(N, dtype=torch.float64, device=dev)
    status = torch.empty(N, dtype=torch.int32, device=dev)
    _check(lib().hna_head_step(int(N), int(G), int(I), int(L), _ptr(S_up_hat),
                               _ptr(S_down_hat) if N > 1 else None, _ptr(neuron_device),
                               _ptr(heads), _ptr(score), _ptr(status), _stream(dev)),
           "hna_head_step")
    return heads, score, status


def layout_search(S_up_hat: torch.Tensor, S_down_hat: Optional[torch.Tensor], L: int,
                  head_device: Optional[torch.Tensor] = None, iters: int = DUAL_ITERS,
                  max_swaps: Optional[int] = None, max_sweeps: int = 16,
                  workspace: Optional[torch.Tensor] = None) -> dict:
    """Coordinate-ascent layout search (section 3, "Optimiser").

    head_device: starting [N, G] int32 map (default contiguous).  Returns a
    dict with heads [N, G], neurons [N, I], neuron_stats [N, 4] (device
    tensors), J_history (list of floats, one per sweep run) and sweeps."""
    _need_cuda(S_up_hat, S_down_hat)
    N, G, I = S_up_hat.shape
    dev = S_up_hat.device
    if head_device is None:
        head_device = (torch.arange(G, dtype=torch.int32, device=dev) // (G // L)).repeat(N, 1)
    else:
        head_device = head_device.clone()
    _need_cuda(head_device)
    if max_swaps is None:
        max_swaps = 4 * I
    L_ = lib()
    wsb = L_.hna_layout_search_workspace_bytes(int(N), int(G), int(I))
    if workspace is None:
        workspace = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    neurons = torch.empty((N, I), dtype=torch.int32, device=dev)
    stats = torch.empty((N, 4), dtype=torch.int32, device=dev)
    hist = (ctypes.c_double * max_sweeps)()
    n = ctypes.c_int32(0)
    _check(L_.hna_layout_search(int(N), int(G), int(I), int(L), _ptr(S_up_hat),
                                _ptr(S_down_hat) if N > 1 else None, int(iters), int(max_swaps),
                                int(max_sweeps), _ptr(head_device), _ptr(neurons), _ptr(stats),
                                hist, ctypes.byref(n), _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(dev)),
           "hna_layout_search")
    return {"heads": head_device, "neurons": neurons, "neuron_stats": stats,
            "J_history": [hist[i] for i in range(n.value)], "sweeps": n.value}


# -------------------------------------------------- exact leave-one-out score
def loo_workspace_bytes(dims: hna_dims) -> int:
    return int(lib().hna_loo_workspace_bytes(ctypes.byref(dims)))


def affinity_loo(dims: hna_dims, a, g, u, x, W_o, gamma, W_gate, W_up, M, group_of_head,
                 scale: float, S_loo: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """S_loo [G, I] fp32: the exact leave-one-out score (section 3, "Affinity scores")."""
    _need_cuda(a, g, u, x, W_o, gamma, W_gate, W_up, M)
    if x.dtype != torch.float32 or gamma.dtype != torch.float32:
        raise ValueError("x and gamma must be fp32")
    _up_inputs(dims, a=a, g=g, u=u, M=M)
    _weights(dims, W_o=W_o, gamma=gamma, W_gate=W_gate, W_up=W_up)
    _expect(x, "x", (dims.T, dims.hidden), torch.float32, tokens=True)
    L = lib()
    dev = M.device
    if S_loo is None:
        S_loo = torch.empty((dims.G, dims.I), dtype=torch.float32, device=dev)
    wsb = L.hna_loo_workspace_bytes(ctypes.byref(dims))
    if workspace is None:
        workspace = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
    _check(L.hna_affinity_loo(ctypes.byref(dims), _ptr(a), _ptr(g), _ptr(u), _ptr(x), _ptr(W_o),
                              _ptr(gamma), _ptr(W_gate), _ptr(W_up), _ptr(M),
                              _map(group_of_head), float(scale), _ptr(S_loo),
                              _ptr(workspace), workspace.numel() * workspace.element_size(),
                              _stream(dev)), "hna_affinity_loo")
    return S_loo


# ------------------------------------------------ allocation-free up pass
def static_scratch_bytes() -> int:
    return int(lib().hna_static_scratch_bytes())


def affinity_up_static(dims: hna_dims, a, g, u, r, r_next, M, wd_sq, group_of_head, scale: float,
                       S_fo: torch.Tensor, S_add: torch.Tensor, c_down: Optional[torch.Tensor] = None,
                       accumulate: bool = False):
    """hna_affinity_up + hna_affinity_add + hna_finalize_up in one call on the
    library's fixed scratch array: no workspace, and nothing is allocated
    here either (the caller passes every output)."""
    _need_cuda(a, g, u, r, r_next, M, wd_sq, S_fo, S_add, c_down)
    _up_inputs(dims, a, g, u, r, r_next, M)
    _expect(wd_sq, "wd_sq", (dims.I,), torch.float32)
    _expect(S_fo, "S_fo", (dims.G, dims.I), torch.float32)
    _expect(S_add, "S_add", (dims.G, dims.I), torch.float32)
    _expect(c_down, "c_down", (dims.I,), torch.float32)
    _check(lib().hna_affinity_up_static(ctypes.byref(dims), _ptr(a), _ptr(g), _ptr(u), _ptr(r),
                                        _ptr(r_next), _ptr(M), _ptr(wd_sq), _map(group_of_head),
                                        float(scale), HNA_ACCUMULATE if accumulate else 0,
                                        _ptr(S_fo), _ptr(S_add), _ptr(c_down), _stream(M.device)),
           "hna_affinity_up_static")
    return S_fo, S_add, c_down
