"""Benchmark of the affinity pass on one MI355X.

A step is one pass of the whole path over one batch of calibration tokens:
weight fold, ||w^d||^2, the hot kernel (eq. (5), FO and ADD sums and the
down-edge moment), the fixed-order reduction, the down-edge weight norms and
S_down.  Inputs (seeded synthetic layer of the requested workload) are resident
in HBM before the timed region starts.

Prints one JSON line.  `value` is calibration tokens/s of the whole step;
`roofline` describes the hot kernel (algorithmic MFMA FLOPs per launch over
its average duration measured with HIP events on the launch stream);
`cpu_baseline` is the float64 oracle timed on this host on a bounded token
sample of the same layer; `mfma_loop` is the matrix cores' sustained bf16
rate on random operands (hna_mfma_rate_probe), the second reference for the
hot kernel's MFMA rate besides the published peak.  Unless --no-legs is given,
the line also carries the other single-layer workloads (Danube3-500M-shaped
and the large 4096 x 14336 layer, and the benchmark layer with fp32 inputs
against the fp32 matrix peak) measured the same way, the 28-layer
Qwen3-0.6B-shaped stack end to end, the leave-one-out score and the
layout-search calls.
Progress lines go to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 (matrix)
PEAK_HBM_GBS = 8000.0
PEAK_FP64_TFLOPS = 78.6     # MI355X fp64 vector
METRIC = "calibration tokens/s for S↑-fo affinity (Qwen3-0.6B layer); % MFMA peak"
HOT_SRC = os.path.join(ROOT, "head_neuron_affinity_amd", "csrc", "k_affinity.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hot_kernel_traffic.json")


def hot_source_hash() -> str:
    with open(HOT_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for(workload: str):
    """HBM bytes per hot-kernel launch from committed rocprofv3 counters, if they
    were taken on the current kernel source for this workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(workload)
    if not ent or ent.get("source_sha256_16") != hot_source_hash():
        return None
    return ent.get("bytes_per_launch")


def cpu_baseline(layer_gpu):
    """Time the float64 oracle on the first 4096 tokens of the same layer (one
    token chunk of the oracle; its cost is linear in the token count)."""
    import torch
    import oracle
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        libs = [f"{i.get('internal_api', '?')} ({i.get('num_threads', '?')} threads)"
                for i in info if i.get("user_api") == "blas"]
        blas = ", ".join(libs) or blas
    except Exception:  # pragma: no cover
        threads = os.cpu_count()

    def sample(T):
        out = {}
        for k, v in layer_gpu.items():
            if k in ("a", "g", "u", "r", "r_next"):
                out[k] = v[:T].cpu()
            elif isinstance(v, torch.Tensor):
                out[k] = v.cpu()
            else:
                out[k] = v
        return out

    def run(T):
        s = sample(T)
        t = time.perf_counter()
        oracle.affinity_layer(s)
        return time.perf_counter() - t

    Tmax = layer_gpu["a"].shape[0]
    T1 = min(4096, Tmax)                    # one token chunk of the oracle
    dt = run(T1)
    return {"value": T1 / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {T1} of the {Tmax} tokens of the same synthetic layer, whole pass "
                      f"(S_fo, S_add, S_down) in float64 numpy, {dt:.1f} s",
            "blas": blas, "host_cpus": os.cpu_count()}


def copy_probe(mib: int):
    """A plain device copy of known size, for scaling HBM byte counters."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def objective_bench(hna, reps: int):
    """Layout objective J (eq. 6) over a 28-layer stack of score matrices
    (8 KV groups x 3072 neurons, the Qwen3-0.6B shape) on 4 devices: average
    duration of one hna_layout_objective call over `reps` calls, HIP events on
    the launch stream.  Algorithmic bytes: every score read once plus the
    device maps."""
    import torch
    import synth
    N, G, I, L = 28, 8, 3072, 4
    S_up, S_down = synth.make_scores(N, G, I, seed=11)
    heads, neurons = synth.random_balanced_layout(N, G, I, L, seed=11)
    S_up, S_down, heads, neurons = (t.cuda() for t in (S_up, S_down, heads, neurons))
    fu = torch.empty(N, dtype=torch.float64, device="cuda")
    fd = torch.empty(N - 1, dtype=torch.float64, device="cuda")
    J = torch.empty(1, dtype=torch.float64, device="cuda")
    for _ in range(3):
        hna.layout_objective(S_up, S_down, heads, neurons, fu, fd, J)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        hna.layout_objective(S_up, S_down, heads, neurons, fu, fd, J)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    nbytes = 4 * (N * G * I + (N - 1) * I * G) + 4 * (N * G + N * I)
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"workload": f"score stack N={N} G={G} I={I}, {L} devices", "us_per_call": us,
            "J": float(J.cpu()[0]),
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS, "traffic": None}}


def neuron_step_bench(hna, reps: int):
    """Neuron step of the layout search over the same 28-layer stack (unit-mass
    scores, contiguous head devices on 4 devices): average duration of one
    hna_neuron_step call (all layers, one workgroup each) over `reps` calls,
    HIP events on the launch stream."""
    import torch
    import synth
    N, G, I, L = 28, 8, 3072, 4
    S_up, S_down = synth.make_scores(N, G, I, seed=11)
    S_up, S_down = S_up.cuda(), S_down.cuda()
    up, down = hna.unit_mass(S_up), hna.unit_mass(S_down)
    heads, _ = synth.contiguous_layout(N, G, I, L)
    heads = heads.cuda()
    nu = torch.empty((N, I), dtype=torch.int32, device="cuda")
    st = torch.empty((N, 4), dtype=torch.int32, device="cuda")
    for _ in range(2):
        hna.neuron_step(up, down, heads, L, neuron_device=nu, stats=st)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        hna.neuron_step(up, down, heads, L, neuron_device=nu, stats=st)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    iters = hna.DUAL_ITERS
    # algorithmic fp64 work of the dual ascent: per iteration and neuron, L
    # subtractions M - lam and L - 1 comparisons
    flops = (iters + 1) * N * I * (2 * L - 1)
    tflops = flops / (us * 1e-6) / 1e12
    return {"workload": f"score stack N={N} G={G} I={I}, {L} devices, {iters} dual iterations",
            "us_per_call": us, "us_per_dual_iteration": us / (iters + 1),
            "stats_sum": [int(x) for x in st.sum(0).tolist()],
            "roofline": {"bound": "alu", "achieved": tflops, "peak": PEAK_FP64_TFLOPS,
                         "unit": "TFLOP/s", "frac": tflops / PEAK_FP64_TFLOPS, "traffic": None}}


def search_bench(hna, reps: int):
    """Head step and the whole layout search over the same 28-layer stack:
    average hna_head_step duration (HIP events, `reps` calls, neuron devices
    from one neuron step), and the wall time of hna_layout_search from the
    contiguous heads (it synchronises once per sweep)."""
    import torch
    import synth
    N, G, I, L = 28, 8, 3072, 4
    S_up, S_down = synth.make_scores(N, G, I, seed=11)
    up, down = hna.unit_mass(S_up.cuda()), hna.unit_mass(S_down.cuda())
    heads, _ = synth.contiguous_layout(N, G, I, L)
    heads = heads.cuda()
    nu, _ = hna.neuron_step(up, down, heads, L)
    for _ in range(2):
        hna.head_step(up, down, nu, L)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        hna.head_step(up, down, nu, L)
    e1.record(stream)
    torch.cuda.synchronize()
    head_us = e0.elapsed_time(e1) * 1e3 / reps
    hna.layout_search(up, down, L)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    res = hna.layout_search(up, down, L)
    torch.cuda.synchronize()
    search_ms = (time.perf_counter() - t0) * 1e3
    # head step bytes: the scores read once plus the neuron devices
    nbytes = 4 * (N * G * I + (N - 1) * I * G) + 4 * N * I
    gbs = nbytes / (head_us * 1e-6) / 1e9
    return {"workload": f"score stack N={N} G={G} I={I}, {L} devices, 2520 partitions per layer",
            "head_step_us": head_us, "search_ms": search_ms, "sweeps": res["sweeps"],
            "J_history": res["J_history"],
            "head_step_roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS,
                                   "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS, "traffic": None}}


def loo_bench(hna, layer, P, grp, reps: int):
    """The exact leave-one-out score on the benchmark layer (folded weights
    already in P.M): average hna_affinity_loo duration over `reps` calls, HIP
    events on the launch stream.  Algorithmic matrix work of the call's
    formulation: x W_o and R = ((alpha beta / r) a)^T x (4 T H d hidden), the
    moments a_h . Q_h a_h and the beta^2-weighted Gram matrices (4 T H d^2),
    Y = R diag(gamma) [W_gate; W_up]^T (4 H d hidden I), the quadratic forms
    (4 H d^2 I) and T1 (2 T H I)."""
    import torch
    T, H, d = layer["a"].shape
    I, D = layer["W_gate"].shape
    for _ in range(2):
        P.loo(layer, grp)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        P.loo(layer, grp)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = (4.0 * T * H * d * D + 4.0 * T * H * d * d + 4.0 * H * d * D * I
             + 4.0 * H * d * d * I + 2.0 * T * H * I)
    tf = flops / (ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if layer["a"].dtype == torch.bfloat16 else PEAK_FP32_TFLOPS
    return {"workload": f"same layer, T={T}", "ms_per_call": ms, "tokens_per_s": T / (ms * 1e-3),
            "roofline": {"bound": "mfma", "achieved": tf, "peak": peak, "unit": "TFLOP/s",
                         "frac": tf / peak, "traffic": None}}


def progress(msg: str):
    """One progress line on stderr (the JSON record alone goes to stdout)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def time_layer(hna, layer, steps: int, warmup: int):
    """Whole-pass step time (wall clock over `steps` steps, synchronised on both
    sides) and the hot kernel's average duration (HIP events on the launch
    stream around hna_affinity_up, which launches only that kernel) for one
    layer resident in HBM."""
    import torch
    P = hna.pass_for_layer(layer)
    grp = [int(x) for x in layer["group_of_head"].tolist()]
    grp_n = [int(x) for x in layer["group_of_head_next"].tolist()]
    T = layer["a"].shape[0]
    stream = torch.cuda.current_stream()

    def step(ev=None):
        P.fold(layer)
        if ev is not None:
            ev[0].record(stream)
        P.hot(layer, grp)
        if ev is not None:
            ev[1].record(stream)
        P.add(layer, grp)
        P.finalize(1.0 / T)
        P.down(layer, grp_n)

    for _ in range(warmup):
        step()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    hot_ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    return P, wall * 1e3 / steps, hot_ms


def mfma_loop_bench(hna, hot_tflops: float, n_wg: int = 512, rounds: int = 10000, reps: int = 5):
    """The matrix cores' sustained bf16 rate on this device: hna_mfma_rate_probe
    (back-to-back 32x32x16 MFMAs, four independent accumulators per wave, two
    waves per SIMD, random operands so that power and clock are those of real
    data; about as long as one hot-kernel launch), timed with HIP events on the
    launch stream.  The hot kernel's MFMA rate is also reported as a fraction
    of it."""
    import torch
    gen = torch.Generator(device="cuda").manual_seed(20260)
    seed = torch.randn(n_wg * 256 * 64, device="cuda", generator=gen).to(torch.bfloat16)
    out = torch.empty(n_wg * 256, dtype=torch.float32, device="cuda")
    for _ in range(2):
        hna.mfma_rate_probe(seed, n_wg, rounds, out=out)
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        hna.mfma_rate_probe(seed, n_wg, rounds, out=out)
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tf = n_wg * 4 * rounds * 4 * 32768 / (ms * 1e-3) / 1e12
    return {"achieved": tf, "unit": "TFLOP/s", "frac_of_published_peak": tf / PEAK_BF16_TFLOPS,
            "hot_kernel_frac_of_loop": hot_tflops / tf, "ms_per_call": ms,
            "workgroups": n_wg, "waves_per_simd": 2, "rounds": rounds, "operands": "random bf16"}


def layer_figures(shape, ms_step: float, hot_ms: float):
    """Throughput and the hot kernel's roofline for one layer workload."""
    T, H, d, I = shape.T, shape.H, shape.d, shape.I
    flops_hot = 4.0 * T * H * d * I                          # algorithmic, one launch
    peak = PEAK_BF16_TFLOPS if shape.dtype == "bf16" else PEAK_FP32_TFLOPS
    achieved = flops_hot / (hot_ms * 1e-3) / 1e12
    esz = 2 if shape.dtype == "bf16" else 4
    stream_bytes = T * (esz * (H * d + 2 * I) + 8)           # a, g, u, r, r_next read once
    return {
        "tokens_per_s": T / (ms_step * 1e-3),
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": traffic_for(f"{shape.name}:T={T}")},
        "hot_kernel_ms": hot_ms,
        "mfma_frac_whole_step": flops_hot / (ms_step * 1e-3) / 1e12 / peak,
        "hot_stream_gbs": stream_bytes / (hot_ms * 1e-3) / 1e9,
    }


def layer_leg(hna, config: int, steps: int, warmup: int, dtype=None):
    """Another single-layer workload, measured like the main line (optionally
    with another input dtype, named as a workload of its own)."""
    import dataclasses
    import torch
    import synth
    shape = synth.layer_shape(config)
    if dtype is not None and dtype != shape.dtype:
        shape = dataclasses.replace(shape.with_dtype(dtype), name=f"{shape.name}-{dtype}")
    layer = synth.make_config_layer(config, device="cuda", dtype=dtype)
    torch.cuda.synchronize()
    _, ms_step, hot_ms = time_layer(hna, layer, steps, warmup)
    rec = {"workload": shape.name, "T": shape.T, "hidden": shape.hidden, "H": shape.H,
           "G": shape.G, "d": shape.d, "I": shape.I, "ms_per_step": ms_step}
    rec.update(layer_figures(shape, ms_step, hot_ms))
    del layer
    torch.cuda.empty_cache()
    return rec


def stack_leg(hna, reps: int, warmup: int, T=None):
    """The 28-layer Qwen3-0.6B-shaped stack end to end: every layer resident in
    HBM, one pass = fold, hot kernel, ADD and reduction for each layer plus the
    down edge of each adjacent pair (head_neuron_affinity_amd.StackPass, the
    weight work on a side stream ahead of the token passes).  Average pass
    time over `reps` passes (HIP events on the main stream, which waits for
    the side stream at the end of each pass); the same without the side
    stream for comparison."""
    import torch
    import synth
    shape = synth.layer_shape(3)
    if T is not None:
        shape = shape.with_tokens(T)
    layers = [synth.make_config_layer(3, layer=i, T=T, device="cuda") for i in range(shape.layers)]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    out = {"workload": shape.name, "layers": shape.layers, "T": shape.T}
    for overlap in (True, False):
        stack = hna.StackPass(layers, overlap=overlap)
        for _ in range(warmup):
            stack.run(layers)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            stack.run(layers)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        key = "ms_per_pass" if overlap else "ms_per_pass_one_stream"
        out[key] = ms
        if overlap:
            flops = 4.0 * shape.T * shape.H * shape.d * shape.I * shape.layers
            out["tokens_per_s"] = shape.T / (ms * 1e-3)
            out["layer_tokens_per_s"] = shape.T * shape.layers / (ms * 1e-3)
            out["mfma_frac_whole_pass"] = flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS
        del stack
    del layers
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", type=int, default=1, choices=[0, 1, 2, 4],
                    help="single-layer workload of the main line")
    ap.add_argument("--tokens", type=int, default=None, help="override T (not for reported numbers)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-legs", action="store_true",
                    help="main line only (no stack, other layers, leave-one-out or layout legs)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run a plain copy of this many MiB (counter scaling runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the pass would shard over tokens with one all-reduce of the partial sums, "
              "which is not built here).", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import head_neuron_affinity_amd as hna

    torch.cuda.set_device(0)
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
    shape = synth.layer_shape(args.config)
    if args.tokens:
        shape = shape.with_tokens(args.tokens)
    L0 = synth.make_config_layer(args.config, T=args.tokens, device="cuda",
                                 with_x=not args.no_legs)
    torch.cuda.synchronize()
    progress(f"{shape.name}: inputs ready")
    P0, ms_step, hot_ms = time_layer(hna, L0, args.steps, args.warmup)
    progress(f"{shape.name}: {ms_step:.3f} ms per step, hot kernel {hot_ms:.3f} ms")
    fig = layer_figures(shape, ms_step, hot_ms)
    rec = {
        "metric": METRIC, "value": fig["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": shape.dtype, "data": "synthetic (seeded generator, inputs resident in HBM)",
        "config": {"workload": shape.name, "T": shape.T, "hidden": shape.hidden, "H": shape.H,
                   "G": shape.G, "d": shape.d, "I": shape.I, "layers": 1},
        "roofline": fig["roofline"],
        "hot_kernel_ms": fig["hot_kernel_ms"],
        "mfma_frac_whole_step": fig["mfma_frac_whole_step"],
        "hot_stream_gbs": fig["hot_stream_gbs"],
    }
    if shape.dtype == "bf16":
        rec["mfma_loop"] = mfma_loop_bench(hna, fig["roofline"]["achieved"])
        progress("matrix-core rate probe done")
    if not args.no_legs:
        grp = [int(x) for x in L0["group_of_head"].tolist()]
        rec["loo"] = loo_bench(hna, L0, P0, grp, 5)
        progress("leave-one-out done")
        rec["objective"] = objective_bench(hna, 200)
        rec["neuron_step"] = neuron_step_bench(hna, 20)
        rec["layout_search"] = search_bench(hna, 50)
        progress("layout search done")
        legs = {}
        for c in (2, 4):
            if c != args.config:
                legs[synth.layer_shape(c).name] = layer_leg(hna, c, 10, 2)
                progress(f"{synth.layer_shape(c).name} done")
        if shape.dtype == "bf16":
            # the fp32 instantiation of the same layer, against the fp32 matrix peak
            fp = layer_leg(hna, args.config, 5, 1, dtype="f32")
            legs[fp["workload"]] = fp
            progress(f"{fp['workload']} done")
        rec["other_layers"] = legs
        rec["stack"] = stack_leg(hna, 3, 1, T=args.tokens)
        progress("stack done")
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(L0)
        progress("cpu baseline done")
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
