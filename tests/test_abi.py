"""The C ABI without a GPU: the library loads, exports every declared entry point,
and rejects bad arguments on the host before launching anything.

Every call below fails validation on purpose (fake, never-dereferenced device
addresses are used only where a check earlier in the argument list fires), so
no HIP kernel is launched.
"""
import ctypes
import os
import re
import subprocess
import threading

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hna.h")


def _lib():
    import head_neuron_affinity_amd as hna
    if not os.path.exists(hna.LIB_PATH):
        pytest.skip("libhna.so not built (python -m head_neuron_affinity_amd.build_lib)")
    return hna


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(hna_[a-z_]+)\s*\(", txt)))


def test_header_declares_expected_entry_points():
    hna = _lib()
    assert declared_functions() == sorted(hna.EXPORTED)


def test_library_exports_every_declared_symbol():
    hna = _lib()
    out = subprocess.run(["nm", "-D", "--defined-only", hna.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(hna_[a-z_]+)$", out, flags=re.M))
    missing = set(declared_functions()) - exported
    assert not missing, f"declared but not exported: {missing}"
    L = hna.lib()
    for name in declared_functions():
        assert getattr(L, name) is not None


def test_version_and_status_strings():
    hna = _lib()
    L = hna.lib()
    assert L.hna_abi_version() == 2
    assert hna.status_string(0) == "HNA_OK"
    assert hna.status_string(-4) == "HNA_ERR_WORKSPACE"
    assert hna.status_string(-99) == "HNA_ERR_UNKNOWN"


FAKE = 0x7F0000000000   # 16-byte aligned, never dereferenced
MIS = FAKE + 2          # misaligned


def dims(hna, T=256, hidden=64, H=4, G=2, d=16, I=128, dtype=1):
    return hna.make_dims(T, hidden, H, G, d, I, dtype)


def call_up(hna, dm, a=FAKE, g=FAKE, u=FAKE, r=FAKE, rn=None, M=FAKE, grp=(0, 0, 1, 1),
            ws=FAKE, wsb=1 << 40):
    L = hna.lib()
    arr = (ctypes.c_int32 * len(grp))(*grp) if grp is not None else None
    vp = ctypes.c_void_p
    return L.hna_affinity_up(ctypes.byref(dm), vp(a), vp(g), vp(u), vp(r), vp(rn) if rn else None,
                             vp(M), arr, vp(ws), wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(H=4, G=3), -1),          # H not a multiple of G
    (dict(d=20), -2),              # d not a multiple of 16
    (dict(d=144), -2),             # d > 128
    (dict(hidden=60), -2),         # hidden not a multiple of 8
    (dict(dtype=7), -1),           # unknown dtype
    (dict(I=0), -1),
    (dict(T=-1), -1),
    (dict(H=0), -1),
    (dict(H=256, G=2), -2),        # too many heads
    (dict(T=2**31), -2),           # tokens beyond the kernels' 32-bit tile counts
    (dict(T=2**31 - 1, I=1 << 22), -2),   # hot-kernel grid beyond 2^24 workgroups
    (dict(I=(1 << 22) + 1), -2),   # too many neurons
])
def test_bad_dims_rejected(kw, status):
    hna = _lib()
    rc = call_up(hna, dims(hna, **kw), grp=tuple([0] * max(1, kw.get("H", 4))))
    assert rc == status, hna.last_error()
    assert hna.last_error() != ""


def test_null_dims_pointer():
    hna = _lib()
    L = hna.lib()
    assert L.hna_affinity_up(None, None, None, None, None, None, None, None, None, 0, None) == -1
    assert "dims is NULL" in hna.last_error()


def test_bad_group_map():
    hna = _lib()
    assert call_up(hna, dims(hna), grp=(0, 0, 2, 1)) == -1
    assert "group_of_head[2]" in hna.last_error()
    assert call_up(hna, dims(hna), grp=(0, -1, 1, 1)) == -1
    assert call_up(hna, dims(hna), grp=None) == -1


def test_null_and_misaligned_pointers():
    hna = _lib()
    assert call_up(hna, dims(hna), a=0) == -1
    assert "a is NULL" in hna.last_error()
    assert call_up(hna, dims(hna), g=MIS) == -3
    assert "g is not 16-byte aligned" in hna.last_error()
    assert call_up(hna, dims(hna), M=0) == -1
    assert call_up(hna, dims(hna), rn=MIS) == -3


def test_workspace_too_small():
    hna = _lib()
    dm = dims(hna)
    need = hna.up_workspace_bytes(dm)
    assert need > 0
    assert call_up(hna, dm, wsb=need - 1) == -4
    assert "workspace" in hna.last_error()


def test_workspace_sizes_follow_geometry():
    hna = _lib()
    a256 = lambda x: (x + 255) // 256 * 256
    # Qwen3-0.6B-shaped layer: 512 token tiles of 128 -> 64 chunks of 8 tiles;
    # FO partial sums [64][G+1][I] fp32, then the Gram partials over 32 token
    # chunks [32][H][d][d], the reduced Gram matrices [H][d][d], ADD [G][I] and
    # the per-head ADD sums [H][I].
    dm = hna.make_dims(65536, 1024, 16, 8, 128, 3072, 1)
    assert hna.up_workspace_bytes(dm) == (64 * 9 * 3072 * 4 + 32 * 16 * 128 * 128 * 4
                                          + 16 * 128 * 128 * 4 + 8 * 3072 * 4 + 16 * 3072 * 4)
    assert hna.folded_bytes(dm) == 16 * 128 * 2 * 3072 * 2
    # ragged neuron count pads to 32; T = 1 is one chunk and one Gram chunk
    dm = hna.make_dims(1, 64, 4, 2, 16, 101, 0)
    assert hna.up_workspace_bytes(dm) == (a256(1 * 3 * 128 * 4) + a256(4 * 16 * 16 * 4)
                                          + a256(4 * 16 * 16 * 4) + a256(2 * 128 * 4)
                                          + a256(4 * 128 * 4))
    assert hna.folded_bytes(dm) == 4 * 16 * 2 * 128 * 4
    # gamma'-scaled W_down^T in the input dtype, then the segment partials
    # [H' + 2G'][I]
    dd = hna.hna_down_dims(1024, 3072, 16, 8, 128, 1)
    assert hna.down_workspace_bytes(dd) == 3072 * 1024 * 2 + 32 * 3072 * 4
    # fold: gamma-scaled W_o^T in the input dtype
    dm = hna.make_dims(65536, 1024, 16, 8, 128, 3072, 1)
    assert hna.lib().hna_fold_workspace_bytes(ctypes.byref(dm)) == 2048 * 1024 * 2
    dm = hna.make_dims(1, 64, 4, 2, 16, 101, 0)
    assert hna.lib().hna_fold_workspace_bytes(ctypes.byref(dm)) == a256(64 * 64 * 4)


def test_lds_limit_reported_unsupported():
    hna = _lib()
    # fp32, d = 128 and 64 KV groups need more than 160 KiB of LDS
    dm = hna.make_dims(256, 4096, 64, 64, 128, 128, 0)
    rc = call_up(hna, dm, grp=tuple(range(64)))
    assert rc == -2 and "LDS" in hna.last_error()


def test_affinity_add_validates():
    hna = _lib()
    L = hna.lib()
    vp = ctypes.c_void_p
    dm = dims(hna)
    grp = (ctypes.c_int32 * 4)(0, 0, 1, 1)
    need = hna.up_workspace_bytes(dm)
    assert L.hna_affinity_add(None, vp(FAKE), vp(FAKE), vp(FAKE), grp, vp(FAKE), need, None) == -1
    bad = (ctypes.c_int32 * 4)(0, 0, 1, 3)
    assert L.hna_affinity_add(ctypes.byref(dm), vp(FAKE), vp(FAKE), vp(FAKE), bad, vp(FAKE), need,
                              None) == -1
    assert "group_of_head[3]" in hna.last_error()
    assert L.hna_affinity_add(ctypes.byref(dm), None, vp(FAKE), vp(FAKE), grp, vp(FAKE), need,
                              None) == -1
    assert L.hna_affinity_add(ctypes.byref(dm), vp(FAKE), vp(MIS), vp(FAKE), grp, vp(FAKE), need,
                              None) == -3
    assert L.hna_affinity_add(ctypes.byref(dm), vp(FAKE), vp(FAKE), vp(FAKE), grp, vp(FAKE),
                              need - 1, None) == -4


def test_finalize_and_other_calls_validate():
    hna = _lib()
    L = hna.lib()
    vp = ctypes.c_void_p
    dm = dims(hna)
    assert L.hna_finalize_up(ctypes.byref(dm), vp(FAKE), 1.0, 2, vp(FAKE), 1 << 30, vp(FAKE),
                             vp(FAKE), None, None) == -1        # unknown flag
    assert L.hna_finalize_up(ctypes.byref(dm), None, 1.0, 0, vp(FAKE), 1 << 30, vp(FAKE),
                             vp(FAKE), None, None) == -1        # wd_sq NULL
    assert L.hna_fold_up_weights(ctypes.byref(dm), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE),
                                 vp(FAKE), 10, vp(FAKE), 1 << 30, None) == -4  # M too small
    assert L.hna_down_col_sqnorm(ctypes.byref(dims(hna, d=8)), vp(FAKE), vp(FAKE), None) == -2
    dd = hna.hna_down_dims(64, 128, 4, 2, 16, 1)
    grp = (ctypes.c_int32 * 4)(0, 1, 0, 5)
    assert L.hna_down_weight_norms(ctypes.byref(dd), vp(FAKE), vp(FAKE), vp(FAKE), vp(FAKE),
                                   vp(FAKE), grp, vp(FAKE), vp(FAKE), 1 << 30, None) == -1
    assert L.hna_down_combine(0, 2, vp(FAKE), vp(FAKE), vp(FAKE), None) == -1
    assert L.hna_down_combine(8, 2, vp(MIS), vp(FAKE), vp(FAKE), None) == -3


def test_objective_calls_validate():
    hna = _lib()
    L = hna.lib()
    vp = ctypes.c_void_p
    F = vp(FAKE)
    # no-op sizes succeed without touching the (NULL) pointers
    assert L.hna_unit_mass(None, 0, 5, None, None) == 0
    assert L.hna_unit_mass(None, 16, 0, None, None) == 0
    assert L.hna_unit_mass(F, -1, 1, F, None) == -1
    assert L.hna_unit_mass(F, 16, -1, F, None) == -1
    assert L.hna_unit_mass(None, 16, 2, F, None) == -1
    assert L.hna_unit_mass(F, 16, 2, vp(MIS), None) == -3
    assert "out" in hna.last_error()
    obj = L.hna_layout_objective
    assert obj(0, 8, 64, F, F, F, F, F, F, F, None) == -1
    assert obj(2, 0, 64, F, F, F, F, F, F, F, None) == -1
    assert obj(2, 8, -3, F, F, F, F, F, F, F, None) == -1
    assert obj(2, 1 << 16, 1 << 16, F, F, F, F, F, F, F, None) == -2   # G*I > 2^31
    assert obj(2049, 8, 64, F, F, F, F, F, F, F, None) == -2            # N > 2048
    assert obj(2, 8, 64, F, None, F, F, F, F, F, None) == -1           # S_down needed
    assert obj(2, 8, 64, F, F, F, F, F, None, F, None) == -1           # frac_down needed
    assert obj(2, 8, 64, F, F, vp(MIS), F, F, F, F, None) == -3
    assert "head_device" in hna.last_error()
    assert obj(2, 8, 64, F, F, F, F, F, F, None, None) == -1           # J
    # N == 1 needs neither S_down nor frac_down; a NULL S_up still fails first
    assert obj(1, 8, 64, None, None, F, F, F, None, F, None) == -1
    assert "S_up" in hna.last_error()


def test_neuron_step_validates():
    hna = _lib()
    L = hna.lib()
    F = ctypes.c_void_p(FAKE)
    ns = L.hna_neuron_step
    ok = dict(N=3, G=8, I=3072, L=4)

    def call(N=3, G=8, I=3072, Ld=4, up=F, down=F, heads=F, iters=300, ms=100, out=F, st=F):
        return ns(N, G, I, Ld, up, down, heads, iters, ms, out, st, None)

    assert call(N=0) == -1
    assert call(Ld=0) == -1
    assert call(G=6) == -1                 # G not a multiple of L
    assert call(I=3070) == -1              # I not a multiple of L
    assert call(iters=-1) == -1
    assert call(ms=-1) == -1
    assert call(Ld=16, G=16, I=1024) == -2  # more than 8 devices
    assert call(Ld=8, I=4096) == -2         # I*L > 16384: the gains do not fit in LDS
    assert call(I=20480) == -2
    assert call(G=256) == -2
    assert call(up=None) == -1
    assert call(down=None) == -1
    assert call(N=1, down=None, heads=ctypes.c_void_p(MIS)) == -3
    assert call(st=None) == -1 and "stats" in hna.last_error()
    assert ok


def test_head_step_and_search_validate():
    hna = _lib()
    L = hna.lib()
    F = ctypes.c_void_p(FAKE)
    hs = L.hna_head_step

    def head(N=3, G=8, I=3072, Ld=4, up=F, down=F, nu=F, out=F, sc=F, st=F):
        return hs(N, G, I, Ld, up, down, nu, out, sc, st, None)

    assert head(N=0) == -1
    assert head(G=6) == -1                  # G not a multiple of L
    assert head(G=32, Ld=4) == -2           # more than 16 groups
    assert head(G=16, Ld=4) == -2           # 63,063,000 partitions > 2^24
    assert head(Ld=16, G=16, I=1024) == -2  # more than 8 devices
    assert head(up=None) == -1
    assert head(down=None) == -1
    assert head(N=1, down=None, sc=ctypes.c_void_p(MIS)) == -3
    assert head(st=None) == -1
    assert L.hna_layout_search_workspace_bytes(0, 8, 64) == 0
    need = L.hna_layout_search_workspace_bytes(3, 8, 3072)
    assert need >= 3 * 8 * 4 + 3 * 3072 * 4 + 3 * 16
    hist = (ctypes.c_double * 4)()
    n = ctypes.c_int32(0)
    ls = L.hna_layout_search

    def search(N=3, G=8, I=3072, Ld=4, iters=300, ms=100, sweeps=4, h=hist, nn=ctypes.byref(n),
               ws=F, wsb=need):
        return ls(N, G, I, Ld, F, F, iters, ms, sweeps, F, F, F, h, nn, ws, wsb, None)

    assert search(sweeps=0) == -1
    assert search(iters=-1) == -1
    assert search(G=16) == -2
    assert search(Ld=8, I=4096) == -2       # the neuron step's LDS limit
    assert search(h=None) == -1
    assert search(nn=None) == -1
    assert search(ws=None) == -1
    assert search(wsb=need - 1) == -4


def test_loo_validates():
    hna = _lib()
    L = hna.lib()
    vp = ctypes.c_void_p
    F = vp(FAKE)
    dm = dims(hna)
    grp = (ctypes.c_int32 * dm.H)(*[h * dm.G // dm.H for h in range(dm.H)])
    need = L.hna_loo_workspace_bytes(ctypes.byref(dm))
    assert need > 0
    loo = L.hna_affinity_loo

    def call(d=dm, a=F, x=F, gamma=F, Wg=F, Wu=F, M=F, S=F, ws=F, wsb=need, g=grp):
        return loo(ctypes.byref(d), a, F, F, x, F, gamma, Wg, Wu, M, g, 1.0, S, ws, wsb, None)

    assert call(d=dims(hna, d=20)) == -2            # head dim not a multiple of 16
    assert call(d=dims(hna, T=4_000_001)) == -2     # past the token limit of one call
    assert call(M=None) == -1
    assert call(S=vp(MIS)) == -3
    assert call(wsb=need - 1) == -4
    assert call(x=None) == -1
    assert call(gamma=None) == -1
    assert call(Wg=None) == -1
    assert call(Wu=vp(MIS)) == -3
    bad = (ctypes.c_int32 * dm.H)(*([0] * (dm.H - 1) + [dm.G]))
    assert call(g=bad) == -1
    assert L.hna_loo_workspace_bytes(None) == 0


def test_mfma_rate_probe_validates():
    hna = _lib()
    L = hna.lib()
    vp = ctypes.c_void_p
    F = vp(FAKE)
    probe = L.hna_mfma_rate_probe
    assert probe(0, 10, 0, F, F, None) == -1            # no workgroups
    assert probe(65537, 10, 0, F, F, None) == -1        # past the grid limit
    assert probe(8, 0, 0, F, F, None) == -1             # no rounds
    assert "iters" in L.hna_last_error().decode()
    assert probe(8, 1_000_001, 1, F, F, None) == -1     # past the round limit
    assert probe(8, 10, 2, F, F, None) == -1            # no such MFMA shape
    assert "shape" in L.hna_last_error().decode()
    assert probe(8, 10, 0, None, F, None) == -1
    assert probe(8, 10, 1, F, vp(MIS), None) == -3
    assert "out" in L.hna_last_error().decode()


def test_error_text_is_thread_local():
    hna = _lib()
    call_up(hna, dims(hna, d=20))
    mine = hna.last_error()
    seen = []

    def other():
        seen.append(hna.last_error())

    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert mine and seen == [""]


def test_binding_checks_shapes_and_dtypes():
    """The binding checks every tensor's shape and dtype against the dims
    before handing its address to the library (no GPU needed: the checks run
    on tensor metadata)."""
    import torch
    hna = _lib()
    from head_neuron_affinity_amd import _binding as B
    dm = dims(hna, T=10, hidden=64, H=4, G=2, d=16, I=40, dtype=1)
    bf = torch.bfloat16
    B._up_inputs(dm, a=torch.empty(10, 4, 16, dtype=bf), g=torch.empty(10, 40, dtype=bf),
                 r=torch.empty(10))
    B._up_inputs(dm, a=torch.empty(12, 4, 16, dtype=bf))      # longer token buffer: first T rows
    with pytest.raises(ValueError, match="a: shape"):
        B._up_inputs(dm, a=torch.empty(9, 4, 16, dtype=bf))   # too few tokens
    with pytest.raises(ValueError, match="g: shape"):
        B._up_inputs(dm, g=torch.empty(10, 41, dtype=bf))
    with pytest.raises(ValueError, match="u: dtype"):
        B._up_inputs(dm, u=torch.empty(10, 40, dtype=torch.float32))
    with pytest.raises(ValueError, match="r: dtype"):
        B._up_inputs(dm, r=torch.empty(10, dtype=bf))
    with pytest.raises(ValueError, match="M:"):
        B._up_inputs(dm, M=torch.empty(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="W_o: shape"):
        B._weights(dm, W_o=torch.empty(64, 60, dtype=bf))
    with pytest.raises(ValueError, match="W_down: dtype"):
        B._weights(dm, W_down=torch.empty(64, 40, dtype=torch.float32))
