"""Benchmark of the BitLinear W1.58A8 hot path on one MI355X.

Default workload (one step): the 2B-class decode GEMV set -- 30 layers x
{q, k, v, o, gate, up, down} = 210 BitLinear matrices held in HBM as 2-bit
packed ternary codes (521.0 MB), one token (M = 1) of fresh fp32
activations per matrix.  A step quantizes every activation vector per token
(absmax -> int8) and contracts it with its packed matrix, rescaling to fp32
(grouped launches: one activation-quantization kernel, one contraction
kernel for all 210 problems).  Weights are quantized and packed once, before
timing, like loading an inference-ready checkpoint.

Timing: each measured step first runs back to back for --settle seconds
(default 0.1, reported as clock_settle_s) so that the clock governor has
reached this load's sustained state, then --warmup untimed steps, then
exactly --steps timed steps between synchronizations.

Printed: one JSON line.  value = packed weight bytes per step / step time.
roofline = the contraction kernel's algorithmic bytes (packed weights + int8
activations + fp32 outputs) over its average duration (HIP events on the
launch stream; the median of 7 windows, with min and max), against 8 TB/s.
prefill = the same 210 matrices at M = 512 (int8 TOP/s against 5.0 POP/s
dense int8).  graph = the decode step captured once in a HIP graph and
replayed.  curves = latency of a full sweep over the 3B-class stack at M in
{1, 8, 64, 256} and the 70B-class stack (17 GB resident) at M in {1, 16,
176}; for 3B also the same stack chained as pre-norm blocks (residual adds,
norms, the gated squared-ReLU, a single-key attention; q|k|v and gate|up
each one launch) at M in {1, 8, 64, 256}, eager and as a replayed HIP
graph.  bt5 = the same 2B stack packed five codes per byte (BT5-T32, 1.6
bits per weight) at M in {1, 8, 16}, next to the 2-bit path at the same M.
cpu_baseline = the CPU oracle on the host's cores on a bounded sample of
the same workload (decode, and one prefill layer extrapolated).

Inputs are synthetic: weights ~ N(0, 0.02) drawn on the device per matrix,
activations ~ N(0, 1) (prefill: 1% of channels x20), seeded.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synth  # noqa: E402

METRIC = "BitLinear packed-weight GB/s at M=1 (HBM roofline %) + int8 TOPS at M=512"
HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0
KERNEL_SOURCES = ["ternary_weight_w1_amd/csrc/gemv_stream.hip", "ternary_weight_w1_amd/csrc/gemm_tile.hip",
                  "ternary_weight_w1_amd/csrc/mm_common.hpp", "ternary_weight_w1_amd/csrc/common.hpp",
                  "ternary_weight_w1_amd/csrc/gemv5.hip", "ternary_weight_w1_amd/csrc/bt5.hpp",
                  "ternary_weight_w1_amd/csrc/quant_row.hpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def build_stack(B, torch, model: str, layers: int, dev, bt5: bool = False):
    """Quantize and pack every matrix of the stack on the device (with
    bt5, also in the five-codes-per-byte format)."""
    spec = synth.MODELS[model]
    mats = []
    for layer in range(layers):
        for j, (name, K, N) in enumerate(spec["shapes"]):
            W = synth.weights_torch(N, K, spec["sigma"], synth.matrix_seed(layer, j), dev)
            T, g = B.quantize_weights(W)
            del W
            P = B.pack(T)
            P5 = B.pack5(T) if bt5 else None
            del T
            mats.append(dict(layer=layer, name=name, K=K, N=N, P=P, P5=P5, gamma=g))
    torch.cuda.synchronize()
    return mats


def make_plan(B, torch, mats, M, dev, outliers=0.0, seed0=7, fmt=0):
    probs = []
    for i, m in enumerate(mats):
        X = synth.activations_torch(M, m["K"], seed0 + i, dev, outlier_frac=outliers)
        Y = torch.empty((M, m["N"]), dtype=torch.float32, device=dev)
        probs.append(dict(X=X, P=m["P5"] if fmt else m["P"], gamma=m["gamma"], Y=Y, N=m["N"],
                          format=fmt))
    plan = B.GroupPlan(probs, device=dev)
    torch.cuda.synchronize()
    return plan, probs


def settle(torch, fn, seconds):
    """Run fn back to back (synchronizing every 20 calls) for about
    `seconds`, so that the clock governor reaches the sustained state of
    this load before anything is timed: the step's clock ramps for tens of
    milliseconds (the 2B decode step measures 88 us in its first 17 ms and
    82 us after)."""
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()


SETTLE_S = 0.0  # seconds of clock settling before each timed measurement (set from --settle)


def time_plan(torch, plan, steps, warmup, windows=7, settle_s=None):
    """Wall time per step over `steps` steps (quantize + contract), then the
    contraction kernel alone: `windows` event windows, each `steps`
    back-to-back launches between one pair of HIP events on the launch
    stream (torch's current stream), giving the average launch duration
    without per-launch event overhead.  Before the `warmup` steps the step
    runs for settle_s seconds (see settle).  Returns (ms per step, median
    kernel ms, {min, median, max} over the windows): the median keeps one
    window taken while the clock settles from deciding the figure."""
    settle(torch, lambda: (plan.quant_act(), plan.matmul()), SETTLE_S if settle_s is None else settle_s)
    for _ in range(warmup):
        plan.quant_act()
        plan.matmul()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        plan.quant_act()
        plan.matmul()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = []
    for _ in range(windows):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            plan.matmul()
        b.record()
        torch.cuda.synchronize()
        per.append(a.elapsed_time(b) / steps)
    per.sort()
    med = per[len(per) // 2]
    spread = {"min": round(per[0], 5), "median": round(med, 5), "max": round(per[-1], 5), "windows": windows,
              "launches_per_window": steps}
    return wall / steps * 1e3, med, spread


def time_graph(torch, plan, steps, warmup):
    """The same step captured once into a HIP graph (torch.cuda.CUDAGraph on
    a default-priority side stream) and replayed `steps` times: wall time
    per replay."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            plan.quant_act()
            plan.matmul()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.quant_act()
        plan.matmul()
    settle(torch, graph.replay, SETTLE_S)
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps * 1e3


def curve(B, torch, model, Ms, dev, steps, warmup):
    """Latency of one full sweep over a model's BitLinear stack at each token
    count M (quantize + contract every matrix, grouped launches); "3b" adds
    the chained stack, "3b-chained" runs only that."""
    chained_only = model == "3b-chained"
    if chained_only:
        model = "3b"
    spec = synth.MODELS[model]
    log(f"building {model} stack: {spec['layers']} layers")
    mats = build_stack(B, torch, model, spec["layers"], dev)
    packed = sum(m["N"] * m["K"] // 4 for m in mats)
    out = {"matrices": len(mats), "packed_bytes": packed, "points": []}
    for M in Ms:
        plan, probs = make_plan(B, torch, mats, M, dev)
        ms, kern, _ = time_plan(torch, plan, steps, warmup, windows=5)
        ops = sum(2 * M * m["N"] * m["K"] for m in mats)
        alg = packed + sum(M * B.q_stride(m["K"]) + 8 * M + 4 * M * m["N"] for m in mats)
        out["points"].append({"M": M, "ms_per_sweep": round(ms, 4), "contraction_ms": round(kern, 4),
                              "packed_GBps": round(packed / (ms * 1e-3) / 1e9, 1),
                              "TOPs": round(ops / (ms * 1e-3) / 1e12, 1),
                              "contraction_hbm_frac": round(alg / (kern * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                              "contraction_mfma_frac": round(ops / (kern * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4)})
        log(f"  {model} M={M}: {ms:.3f} ms per sweep")
        del plan, probs
    if chained_only:
        del out["points"]
    if model == "3b":
        log("timing the 3B stack chained as pre-norm blocks")
        out["chained"] = stack_curve(B, torch, mats, dev, [1, 8, 64, 256], steps, warmup)
    del mats
    torch.cuda.empty_cache()
    return out


def bt5_section(B, torch, mats, dev, Ms, steps, warmup, model):
    """The stack in BT5-T32 (five codes per byte) against the 2-bit path at
    each M: step time (quantize + contract) and the contraction kernel's
    average duration (HIP events), with the BT5 kernel's algorithmic bytes
    per launch (packed bytes + int8 activations + scales + fp32 outputs)."""
    packed5 = sum(B.packed5_bytes(m["N"], m["K"]) for m in mats)
    out = {"format": "BT5-T32, five codes per byte (1.6 bits per weight)", "packed_bytes": packed5,
           "points": []}
    for M in Ms:
        plan, probs = make_plan(B, torch, mats, M, dev, fmt=1)
        ms5, k5, spread5 = time_plan(torch, plan, steps, warmup)
        del plan, probs
        plan, probs = make_plan(B, torch, mats, M, dev)
        ms2, k2, _ = time_plan(torch, plan, steps, warmup)
        del plan, probs
        alg = packed5 + sum(M * B.q_stride5(m["K"]) + 8 * M + 4 * M * m["N"] for m in mats)
        gbs = alg / (k5 * 1e-3) / 1e9
        out["points"].append({
            "M": M, "ms_per_step": round(ms5, 5), "kernel_ms": round(k5, 5),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": alg,
                         "traffic": load_traffic(f"bt5_{model}_m{M}"), "kernel_ms_spread": spread5},
            "bl2_ms_per_step": round(ms2, 5), "bl2_kernel_ms": round(k2, 5),
            "kernel_speedup_vs_bl2": round(k2 / k5, 3)})
        log(f"  BT5 M={M}: kernel {k5 * 1e3:.1f} us (2-bit {k2 * 1e3:.1f} us)")
    torch.cuda.empty_cache()
    return out


def stack_inputs(torch, dim, n_layers, M, dev):
    """Seeded inputs of the chained stack: the first residual stream x0
    (M x dim) and the RMSNorm gains, per layer (attention, feed-forward)
    and final, drawn in (0.5, 1.5)."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    gains = [(torch.rand(dim, generator=gen, device=dev) + 0.5, torch.rand(dim, generator=gen, device=dev) + 0.5)
             for _ in range(n_layers)]
    g_fin = torch.rand(dim, generator=gen, device=dev) + 0.5
    return synth.activations_torch(M, dim, 21, dev), gains, g_fin


class ChainedStack:
    """The stack chained as pre-norm blocks for M tokens, each stage a
    library call on one stream: residual add + RMSNorm + int8 cast and q|k|v
    (one input, one call), the attention of the first decode position (a
    single key, so its output is v), the cast of v and o, residual add +
    RMSNorm + cast and gate|up, the gated squared-ReLU cast and down; then
    the final residual add + norm + cast.  Each cast + contraction pair is
    one bitlinear_cast_matmul_multi call: a single launch where the
    contraction's workgroups cast their own input (q|k|v and o at one
    token), two otherwise (`launches` counts them per step).  The
    residual stream alternates between two buffers (a call's X_out may not
    be its X).  Buffers and workspaces are allocated once (workspaces
    zero-filled once, as the multi-matrix calls require).  After step(), x
    holds the final residual stream and (Q, a, rs) its final norm's int8
    cast."""

    def __init__(self, B, torch, mats, dev, M, x0, gains, g_fin):
        import ctypes
        self.L = L = B.lib()
        self.B = B
        self.layers = layers = {}
        for m in mats:
            layers.setdefault(m["layer"], {})[m["name"]] = m
        self.M = M
        self.dim = dim = layers[0]["q"]["K"]
        self.ffn = ffn = layers[0]["gate"]["N"]
        self.x0, self.gains, self.g_fin = x0, gains, g_fin
        f32 = lambda n: torch.empty((M, n), dtype=torch.float32, device=dev)
        self.x, self.xb = f32(dim), f32(dim)
        self.q, self.k, self.v, self.o = f32(dim), f32(dim), f32(dim), f32(dim)
        self.gate, self.up, self.d = f32(ffn), f32(ffn), f32(dim)
        self.ldd = B.q_stride(dim)
        self.Q = torch.empty((M, self.ldd), dtype=torch.int8, device=dev)
        self.a = torch.empty(M, dtype=torch.float32, device=dev)
        self.rs = torch.empty(M, dtype=torch.int32, device=dev)
        self.P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None

        def warr(lay, names, outs):
            arr = (B.Weight * len(names))()
            for i, (nm, Y) in enumerate(zip(names, outs)):
                arr[i] = B.Weight(lay[nm]["P"].data_ptr(), lay[nm]["gamma"].data_ptr(), Y.data_ptr(), None,
                                  lay[nm]["N"], 0, 0)
            return arr
        self.sites = {i: dict(qkv=warr(lay, ("q", "k", "v"), (self.q, self.k, self.v)),
                              o=warr(lay, ("o",), (self.o,)),
                              gu=warr(lay, ("gate", "up"), (self.gate, self.up)),
                              down=warr(lay, ("down",), (self.d,)))
                      for i, lay in layers.items()}
        # the largest workspace over the modes a site is called in (q|k|v: the
        # norm at layer 0, the residual add + norm after)
        self.wss = {}
        for key, K, modes in (("qkv", dim, (B.CAST_RMSNORM, B.CAST_ADD_RMSNORM)), ("o", dim, (B.CAST_PLAIN,)),
                              ("gu", dim, (B.CAST_ADD_RMSNORM,)), ("down", ffn, (B.CAST_RELU2_GATE,))):
            arr = self.sites[0][key]
            wsb = max(L.bitlinear_cast_multi_workspace_bytes(md, arr, len(arr), M, K) for md in modes)
            self.wss[key] = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev)
        # kernels one step enqueues, as the library's policy decides them
        # (layer 0's q|k|v cast has no residual add), plus the final cast
        def n(key, K, md):
            return L.bitlinear_cast_multi_launches(md, self.sites[0][key], len(self.sites[0][key]), M, K)
        rest = n("o", dim, B.CAST_PLAIN) + n("gu", dim, B.CAST_ADD_RMSNORM) + n("down", ffn, B.CAST_RELU2_GATE)
        self.launches = (1 + n("qkv", dim, B.CAST_RMSNORM) + (len(layers) - 1) * n("qkv", dim, B.CAST_ADD_RMSNORM)
                         + len(layers) * rest)

    def _check(self, st):
        if st != 0:
            raise RuntimeError(self.L.bitlinear_last_error().decode())

    def step(self, s):
        """Enqueue one pass over every layer on the raw stream handle s."""
        L, P, B, M, dim, ffn = self.L, self.P, self.B, self.M, self.dim, self.ffn
        xa, xb = self.x, self.xb

        def call(key, site, mode, X, K, aux=None, R=None, X_out=None):
            arr = site[key]
            self._check(L.bitlinear_cast_matmul_multi(mode, P(X), P(aux), P(R), 1e-5, P(X_out), M, K, arr,
                                                      len(arr), P(self.wss[key]), self.wss[key].numel(), s))
        for i in sorted(self.layers):
            ga, gf = self.gains[i]
            site = self.sites[i]
            if i == 0:
                call("qkv", site, B.CAST_RMSNORM, self.x0, dim, aux=ga)
            else:
                call("qkv", site, B.CAST_ADD_RMSNORM, xa, dim, aux=ga, R=self.d, X_out=xb)
            call("o", site, B.CAST_PLAIN, self.v, dim)
            call("gu", site, B.CAST_ADD_RMSNORM, self.x0 if i == 0 else xb, dim, aux=gf, R=self.o, X_out=xa)
            call("down", site, B.CAST_RELU2_GATE, self.gate, ffn, aux=self.up)
        self._check(L.bitlinear_quant_act_add_rmsnorm(P(xa), P(self.d), M, dim, P(self.g_fin), 1e-5, P(xa),
                                                      P(self.Q), self.ldd, P(self.a), P(self.rs), s))


def stack_curve(B, torch, mats, dev, Ms, steps, warmup):
    """Latency of the stack chained as pre-norm blocks (ChainedStack), one
    decode (or prefill) step of M tokens through every layer, timed eagerly
    and as one HIP graph replayed."""
    import ctypes
    n_layers = len({m["layer"] for m in mats})
    dim = next(m["K"] for m in mats if m["name"] == "q")
    ffn = next(m["N"] for m in mats if m["name"] == "gate")
    out = {"layers": n_layers, "dim": dim, "ffn": ffn, "points": []}
    for M in Ms:
        chain = ChainedStack(B, torch, mats, dev, M, *stack_inputs(torch, dim, n_layers, M, dev))
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            s = ctypes.c_void_p(side.cuda_stream)
            settle(torch, lambda: chain.step(s), SETTLE_S)
            for _ in range(max(1, warmup)):
                chain.step(s)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                chain.step(s)
            torch.cuda.synchronize()
            eager = (time.perf_counter() - t0) / steps * 1e3
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=side):
                chain.step(s)
        torch.cuda.current_stream().wait_stream(side)
        settle(torch, graph.replay, SETTLE_S)
        for _ in range(max(1, warmup)):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            graph.replay()
        torch.cuda.synchronize()
        gms = (time.perf_counter() - t0) / steps * 1e3
        out["points"].append({"M": M, "launches_per_step": chain.launches, "eager_ms_per_step": round(eager, 4),
                              "graph_ms_per_step": round(gms, 4)})
        log(f"  stack M={M}: eager {eager:.3f} ms, graph {gms:.3f} ms per step")
        del graph, chain
    torch.cuda.empty_cache()
    return out


def layer_calls(B, torch, dev, M, reps=20, rounds=20):
    """Latency of each library call of one 3B-class decode layer at M tokens
    (the chained stack's calls, on synthetic weights): every call captured
    reps times back to back in a HIP graph, replayed rounds times; us per
    call.  cast_*: the activation casts; mm_*: the multi-matrix contractions
    on int8 input; cast_mm_*: the cast + contraction calls the chained stack
    makes (at one token a single launch where the contraction casts its own
    input)."""
    import ctypes
    L = B.lib()
    dim, ffn = 3200, 8640
    P = lambda t: ctypes.c_void_p(t.data_ptr()) if t is not None else None
    g = torch.Generator(device=dev).manual_seed(1)
    rnd = lambda *sh: torch.randn(*sh, device=dev, generator=g)
    gam = torch.full((1,), 0.01, device=dev)
    keep = []

    def weights(Ns, K):
        arr = (B.Weight * len(Ns))()
        for i, N in enumerate(Ns):
            Pk = B.pack(torch.randint(-1, 2, (N, K), dtype=torch.int8, device=dev, generator=g))
            Y = torch.empty((M, N), device=dev)
            keep.extend([Pk, Y])
            arr[i] = B.Weight(Pk.data_ptr(), gam.data_ptr(), Y.data_ptr(), None, N, 0, 0)
        return arr
    sites = {"qkv": ((dim,) * 3, dim), "o": ((dim,), dim), "gu": ((ffn, ffn), dim), "down": ((dim,), ffn)}
    W = {k: weights(Ns, K) for k, (Ns, K) in sites.items()}
    x, r = rnd(M, dim), rnd(M, dim)
    xo, gains = torch.empty_like(x), 1 + 0.1 * rnd(dim)
    gt, up = rnd(M, ffn), rnd(M, ffn)
    Qd = torch.zeros((M, B.q_stride(dim)), dtype=torch.int8, device=dev)
    Qf = torch.zeros((M, B.q_stride(ffn)), dtype=torch.int8, device=dev)
    a, rs = torch.ones(M, device=dev), torch.zeros(M, dtype=torch.int32, device=dev)
    ws = {}
    for k, (Ns, K) in sites.items():
        n = max([L.bitlinear_multi_workspace_bytes(W[k], len(Ns), M, K)] +
                [L.bitlinear_cast_multi_workspace_bytes(md, W[k], len(Ns), M, K) for md in range(4)])
        ws[k] = torch.zeros(max(n, 16), dtype=torch.uint8, device=dev)

    def chk(st):
        if st:
            raise RuntimeError(L.bitlinear_last_error().decode())

    def mm(k, Q, K):
        return lambda s: chk(L.bitlinear_matmul_multi(P(Q), Q.shape[1], P(a), P(rs), M, K, W[k], len(sites[k][0]),
                                                      P(ws[k]), ws[k].numel(), s))

    def cmm(k, mode, X, aux, R, Xo, K):
        return lambda s: chk(L.bitlinear_cast_matmul_multi(mode, P(X), P(aux), P(R), 1e-5, P(Xo), M, K, W[k],
                                                           len(sites[k][0]), P(ws[k]), ws[k].numel(), s))
    calls = {
        "cast_add_rmsnorm_3200": lambda s: chk(L.bitlinear_quant_act_add_rmsnorm(
            P(x), P(r), M, dim, P(gains), 1e-5, P(xo), P(Qd), Qd.shape[1], P(a), P(rs), s)),
        "cast_plain_3200": lambda s: chk(L.bitlinear_quant_act(P(x), M, dim, P(Qd), Qd.shape[1], P(a), P(rs), s)),
        "cast_relu2_gate_8640": lambda s: chk(L.bitlinear_quant_act_relu2_gate(
            P(gt), P(up), M, ffn, P(Qf), Qf.shape[1], P(a), P(rs), s)),
        "mm_qkv": mm("qkv", Qd, dim), "mm_o": mm("o", Qd, dim), "mm_gate_up": mm("gu", Qd, dim),
        "mm_down": mm("down", Qf, ffn),
        "cast_mm_qkv": cmm("qkv", B.CAST_ADD_RMSNORM, x, gains, r, xo, dim),
        "cast_mm_o": cmm("o", B.CAST_PLAIN, x, None, None, None, dim),
        "cast_mm_gate_up": cmm("gu", B.CAST_ADD_RMSNORM, x, gains, r, xo, dim),
        "cast_mm_down": cmm("down", B.CAST_RELU2_GATE, gt, up, None, None, ffn),
    }
    out = {}
    side = torch.cuda.Stream()
    for name, fn in calls.items():
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            s = ctypes.c_void_p(side.cuda_stream)
            for _ in range(3):
                fn(s)
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr, stream=side):
                for _ in range(reps):
                    fn(s)
        torch.cuda.current_stream().wait_stream(side)
        for _ in range(3):
            gr.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(rounds):
            gr.replay()
        e1.record()
        torch.cuda.synchronize()
        out[name] = round(e0.elapsed_time(e1) * 1e3 / (reps * rounds), 2)
        del gr
    del keep
    torch.cuda.empty_cache()
    return out


def measured_peaks(B, torch, dev, seconds: float = 0.6):
    """What this part sustains on the two roofline resources, from the
    library's calibration probes (include/bitlinear_probe.h):
    * HBM read: a plain 16-byte streaming read of a 2 GiB buffer (8x the
      256 MB last-level cache), best of 256 KiB, 1 MiB and 4 MiB per
      workgroup, 10 launches each;
    * int8 matrix rate: chains of v_mfma_i32_32x32x32_i8 with no memory
      traffic on every resident workgroup slot, launched back to back in
      bursts for about `seconds`; the median of the later bursts (the clock
      settles under sustained load).
    Each probe's checksum is verified before its rate is reported."""
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def xor_all(t):
        t = t.clone()
        n = t.numel()
        while n > 1:
            h = n // 2
            if n % 2:
                t[0] ^= t[n - 1]
            t[:h] ^= t[h:2 * h]
            n = h
        return int(t[0]) & 0xFFFFFFFF

    nbytes = 2 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(0x5A)
    buf[0] = 1
    # 2^29 words: one is 0x5A5A5A01, an odd number of others are 0x5A5A5A5A
    want = 0x5A5A5A01 ^ 0x5A5A5A5A
    best = None
    for chunk in (256 << 10, 1 << 20, 4 << 20):
        sink = torch.empty(B.probe_read_sink_words(nbytes, chunk), dtype=torch.int32, device=dev)
        for _ in range(2):
            B.probe_read(buf, chunk, sink)
        a, b = ev(), ev()
        a.record()
        for _ in range(10):
            B.probe_read(buf, chunk, sink)
        b.record()
        torch.cuda.synchronize()
        gbs = nbytes * 10 / (a.elapsed_time(b) * 1e-3) / 1e9
        if xor_all(sink) != want:
            raise RuntimeError("read probe checksum mismatch")
        if best is None or gbs > best[0]:
            best = (gbs, chunk)
    del buf, sink
    torch.cuda.empty_cache()
    blocks = B.probe_mfma_blocks()
    iters, burst = 4096, 10
    ops = blocks * 4 * iters * 4 * 65536
    sink = torch.empty(256 * blocks, dtype=torch.int32, device=dev)
    rates = []
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        a, b = ev(), ev()
        a.record()
        for _ in range(burst):
            B.probe_mfma(iters, 1, 1, blocks, sink)
        b.record()
        b.synchronize()
        rates.append(ops * burst / (a.elapsed_time(b) * 1e-3) / 1e12)
    if not bool((sink == 2048 * iters).all()):
        raise RuntimeError("matrix-instruction probe checksum mismatch")
    later = sorted(rates[len(rates) // 2:])
    tops = later[len(later) // 2]
    # the same chains on operands from memory, which toggle as many bits as a
    # real contraction: (a) this workload's own operands, int8 codes of the
    # prefill activations (N(0, 1), 1% of channels x20, cast by the library)
    # against ternary fields of N(0, 0.02) weights (quantized by the
    # library); (b) uniform random int8 against uniform random fields.  The
    # probe's clock counters give the shader clock each load sustains.
    def frags(T):  # [32 rows, 128 codes] -> four 64-lane x 16-byte fragments
        return T.reshape(32, 4, 2, 16).permute(1, 2, 0, 3).reshape(4, 64, 16)

    Xw = synth.activations_torch(32, 2560, 777, dev, outlier_frac=0.01)
    Qw = B.quant_act(Xw)[0][:, :128]
    Tw, _ = B.quantize_weights(synth.weights_torch(32, 2560, 0.02, 778, dev))
    workload_ops = torch.stack([frags(Qw), frags((Tw[:, :128] + 1).to(torch.int8))], 1)
    rng = np.random.default_rng(12345)
    uniform_ops = np.empty((4, 2, 64, 16), np.int8)
    uniform_ops[:, 0] = rng.integers(-127, 128, (4, 64, 16))
    uniform_ops[:, 1] = rng.integers(0, 3, (4, 64, 16))
    clocks = torch.empty(3 * blocks, dtype=torch.int64, device=dev)

    def data_probe(dops):
        drates, ghz = [], []
        t_end = time.perf_counter() + seconds / 2
        while time.perf_counter() < t_end:
            a, b = ev(), ev()
            a.record()
            for _ in range(burst - 1):
                B.probe_mfma_data(iters, dops, blocks, sink, clocks)
            c = ev()
            c.record()
            B.probe_mfma_data(iters, dops, blocks, sink, clocks)
            b.record()
            b.synchronize()
            drates.append(ops * burst / (a.elapsed_time(b) * 1e-3) / 1e12)
            ck = clocks.cpu().numpy().reshape(blocks, 3).astype(np.float64)
            # reference-counter rate: the span of all workgroups' loops over
            # the last launch's event time (the loops fill nearly all of it)
            ref_hz = (ck[:, 2].max() - ck[:, 1].min()) / (c.elapsed_time(b) * 1e-3)
            ghz.append(float(np.median(ck[:, 0] / (ck[:, 2] - ck[:, 1]))) * ref_hz / 1e9)
        o64 = dops.cpu().numpy().reshape(4, 2, 64, 16).astype(np.int64)
        per_set = int((o64[:, 0].reshape(4, 2, 32, 16).sum(2) * o64[:, 1].reshape(4, 2, 32, 16).sum(2)).sum())
        want = (4 * iters * per_set) % (1 << 32)
        per = sink.cpu().numpy().view(np.uint32).reshape(blocks, 256).astype(np.uint64).sum(1) % (1 << 32)
        if not bool((per == want).all()):
            raise RuntimeError("matrix-instruction data probe checksum mismatch")
        half = len(drates) // 2
        return (sorted(drates[half:])[len(drates[half:]) // 2], sorted(ghz[half:])[len(ghz[half:]) // 2],
                len(drates) - half)

    data_runs = {"workload": data_probe(workload_ops.reshape(-1).contiguous()),
                 "uniform": data_probe(torch.from_numpy(uniform_ops.reshape(-1)).to(dev))}
    # grid-wide barrier with one word exchanged per workgroup, one workgroup
    # per compute unit: (time of R rounds - time of 1 round) / (R - 1)
    cus = B.probe_compute_units()

    def barrier_ms(rounds):
        best = None
        for _ in range(5):
            state = torch.zeros(2 + 2 * cus, dtype=torch.int32, device=dev)
            a, b = ev(), ev()
            a.record()
            state, _ = B.probe_barrier(rounds, cus, state=state)
            b.record()
            b.synchronize()
            if int(state[1]) != 0 or int(state[0]) != rounds * cus:
                raise RuntimeError("barrier probe gave up or miscounted")
            best = a.elapsed_time(b) if best is None else min(best, a.elapsed_time(b))
        return best
    barrier_us = (barrier_ms(2001) - barrier_ms(1)) / 2000 * 1e3
    return {
        "hbm_read": {"value": round(best[0], 1), "unit": "GB/s",
                     "probe": f"16-byte non-temporal streaming read of 2 GiB, {best[1] >> 10} KiB per workgroup"},
        "grid_barrier": {"value": round(barrier_us, 3), "unit": "us",
                         "probe": f"device-scope store + wait + atomic arrival + polling, one word exchanged per "
                                  f"workgroup, {cus} workgroups (one per compute unit), best of 5 runs of 2001 "
                                  f"rounds less 1 round"},
        "int8_mfma": {"value": round(tops, 1), "unit": "TOP/s",
                      "probe": f"v_mfma_i32_32x32x32_i8 chains, {blocks} workgroups, no memory traffic, "
                               f"every operand byte 1, median of {len(later)} sustained bursts"},
        **{f"int8_mfma_{k}_operands": {
            "value": round(v[0], 1), "unit": "TOP/s", "clock_ghz": round(v[1], 3),
            "probe": f"the same chains on four sets of A and B fragments held in registers ("
                     + ("int8 codes of N(0,1) activations with 1% of channels x20 against ternary fields of "
                        "N(0,0.02) weights, both quantized by the library" if k == "workload" else
                        "uniform random int8 against uniform random ternary fields")
                     + f"), median of {v[2]} sustained bursts; clock = shader-clock count over reference-"
                       f"counter span of each workgroup's loop, the reference rate from the launch's event time"}
           for k, v in data_runs.items()},
    }


def load_traffic(name):
    """HBM traffic of the dominant kernel from the committed rocprofv3 PMC
    summary, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    e = d.get(name)
    if not e or e.get("kernel_source_sha") != kernel_source_sha():
        return None
    return e.get("hbm_bytes_per_launch")


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(model: str, seconds: float = 10.0, prefill_M: int = 512, prefill_seconds: float = 6.0):
    """The oracle, untuned, on the host's cores (its OpenMP loops split the
    independent outputs over OMP_NUM_THREADS threads, every core by
    default): unpack + activation quantization + triple-loop contraction +
    rescale, on layer 0 of the stack (7 matrices).  Decode (M = 1) is
    repeated until about `seconds` of wall time; the prefill leg (M =
    prefill_M, 1% outlier channels) runs the layer until about
    `prefill_seconds` and is extrapolated to the whole stack, labelled so."""
    import oracle as O
    spec = synth.MODELS[model]
    work = []
    for j, (name, K, N) in enumerate(spec["shapes"]):
        W = synth.weights_np(N, K, spec["sigma"], synth.matrix_seed(0, j))
        T, g = O.quantize_weights(W)
        work.append((K, N, O.pack(T), g))
        del W, T
    threads = O.threads()
    reps, t, nbytes = 0, 0.0, 0
    xs = [synth.activations_np(1, K, 7 + j) for j, (K, N, P, g) in enumerate(work)]
    while t < seconds:
        t0 = time.perf_counter()
        for X, (K, N, P, g) in zip(xs, work):
            O.forward_packed(X, P, g, N)
            nbytes += N * K // 4
        t += time.perf_counter() - t0
        reps += 1
    out = {"value": nbytes / t / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"layer 0 of the {model.upper()} stack (7 matrices, M=1) x {reps} passes, {t:.1f} s on "
                     f"{threads} threads: unpack + act quant + int32 triple loop + rescale",
           "cpu_model": _cpu_model(), "host_cpus": os.cpu_count()}
    if prefill_M:
        xs = [synth.activations_np(prefill_M, K, 70 + j, outlier_frac=0.01) for j, (K, N, P, g) in enumerate(work)]
        passes, tp = 0, 0.0
        while tp < prefill_seconds or passes == 0:
            t0 = time.perf_counter()
            for X, (K, N, P, g) in zip(xs, work):
                O.forward_packed(X, P, g, N)
            tp += time.perf_counter() - t0
            passes += 1
        ops = sum(2 * prefill_M * N * K for K, N, P, g in work) * passes
        per_layer = tp / passes
        out["prefill"] = {"M": prefill_M, "value": round(ops / tp / 1e12, 4), "unit": "TOP/s",
                          "layer_s": round(per_layer, 3),
                          "sweep_s_extrapolated": round(per_layer * spec["layers"], 2),
                          "sample": f"layer 0 (7 matrices) at M={prefill_M} x {passes} passes, {tp:.1f} s on "
                                    f"{threads} threads; the {spec['layers']}-layer sweep time is that layer's "
                                    f"time x {spec['layers']} (extrapolated)"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle", type=float, default=0.1,
                    help="seconds the step runs before the warm-up steps, so that the clock has settled")
    ap.add_argument("--model", default="2b", choices=sorted(synth.MODELS))
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--M", type=int, default=1)
    ap.add_argument("--prefill-M", type=int, default=512)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--curves", default="3b,70b",
                    help="comma list of latency-vs-M curves: 3b (M 1,8,64,256, and chained), 70b (M 1,16,176), "
                         "3b-chained (the chained 3B stack only); 'none' to skip")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-bt5", action="store_true", help="skip the five-codes-per-byte comparison")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak calibration probes")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a plain device copy of known size (PMC calibration)")
    ap.add_argument("--layer-calls", default=None,
                    help="comma list of token counts: print only the per-call latency of one 3B-class decode "
                         "layer's library calls at each (JSON line)")
    args = ap.parse_args()
    global SETTLE_S
    SETTLE_S = max(0.0, args.settle)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import ternary_weight_w1_amd as B
    B.lib()
    dev = torch.device("cuda:0")

    if args.copy_probe:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: 3 x {n} bytes")
        return

    if args.layer_calls:
        res = {f"M={M}": layer_calls(B, torch, dev, int(M)) for M in args.layer_calls.split(",")}
        print(json.dumps({"layer_calls_us": res, "workload": "one 3B-class decode layer (dim 3200, ffn 8640)"}),
              flush=True)
        return

    spec = synth.MODELS[args.model]
    layers = args.layers or spec["layers"]
    log(f"building {args.model} stack: {layers} layers")
    mats = build_stack(B, torch, args.model, layers, dev, bt5=not args.no_bt5)
    packed = sum(m["N"] * m["K"] // 4 for m in mats)
    assert packed == sum(B.packed_bytes(m["N"], m["K"]) for m in mats)

    M = args.M
    plan, probs = make_plan(B, torch, mats, M, dev)
    log(f"timing decode sweep: {len(mats)} matrices, M={M}, {packed / 1e6:.1f} MB packed")
    ms, kern_ms, spread = time_plan(torch, plan, args.steps, args.warmup)
    value = packed / (ms * 1e-3) / 1e9
    act_bytes = sum(M * B.q_stride(m["K"]) + 8 * M for m in mats)
    out_bytes = sum(4 * M * m["N"] for m in mats)
    alg_bytes = packed + act_bytes + out_bytes
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    gms = None if args.no_graph else time_graph(torch, plan, args.steps, args.warmup)
    traffic = load_traffic(f"stream_{args.model}_m{M}")
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle_s": args.settle,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic (seeded N(0,0.02) weights quantized+packed on device; N(0,1) activations)",
        "config": {"workload": f"{args.model.upper()}-class decode GEMV set: {layers} layers x "
                               f"q,k,v,o,gate,up,down BitLinear, M={M}, packed ternary resident in HBM",
                   "matrices": len(mats), "M": M, "packed_bytes": packed},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "stream contraction (grouped, one launch per step)" +
                               (f", BITLINEAR_DOT4_VARIANT={os.environ['BITLINEAR_DOT4_VARIANT']}"
                                if os.environ.get("BITLINEAR_DOT4_VARIANT") else ""),
                     "kernel_ms_mean": round(kern_ms, 5), "kernel_ms_spread": spread,
                     "bytes_per_launch": alg_bytes},
    }
    if gms is not None:
        result["graph"] = {"ms_per_step": round(gms, 5), "GBps": round(packed / (gms * 1e-3) / 1e9, 2),
                           "note": "the same step captured once in a HIP graph and replayed"}
    del plan, probs
    torch.cuda.empty_cache()

    if not args.no_prefill:
        PM = args.prefill_M
        plan, probs = make_plan(B, torch, mats, PM, dev, outliers=0.01)
        log(f"timing prefill sweep: M={PM}")
        steps = max(20, args.steps)
        pms, pkern, pspread = time_plan(torch, plan, steps, max(5, args.warmup))
        ops = sum(2 * PM * m["N"] * m["K"] for m in mats)
        result["prefill"] = {
            "M": PM, "ms_per_step": round(pms, 4), "value": round(ops / (pms * 1e-3) / 1e12, 2),
            "unit": "TOP/s",
            "roofline": {"bound": "mfma", "achieved": round(ops / (pkern * 1e-3) / 1e12, 2),
                         "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                         "frac": round(ops / (pkern * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
                         "traffic": load_traffic(f"tile_{args.model}_m{PM}"),
                         "kernel": "tile contraction (grouped)", "kernel_ms_mean": round(pkern, 4),
                         "kernel_ms_spread": pspread, "ops_per_launch": ops},
        }
        del plan, probs
        torch.cuda.empty_cache()

    if not args.no_bt5:
        log("timing BT5-T32 sweeps")
        result["bt5"] = bt5_section(B, torch, mats, dev, [1, 8, 16], args.steps, args.warmup, args.model)
        for m in mats:
            m["P5"] = None
        torch.cuda.empty_cache()

    if not args.no_peaks:
        log("measuring the sustained HBM-read and int8-matrix peaks")
        peaks = measured_peaks(B, torch, dev)
        result["measured_peaks"] = peaks
        hbm, mfma = peaks["hbm_read"]["value"], peaks["int8_mfma"]["value"]
        result["roofline"]["measured_peak"] = hbm
        result["roofline"]["frac_of_measured"] = round(result["roofline"]["achieved"] / hbm, 4)
        for pt in result.get("bt5", {}).get("points", []):
            pt["roofline"]["measured_peak"] = hbm
            pt["roofline"]["frac_of_measured"] = round(pt["roofline"]["achieved"] / hbm, 4)
        if "prefill" in result:
            pr = result["prefill"]["roofline"]
            pr["measured_peak"] = mfma
            pr["frac_of_measured"] = round(pr["achieved"] / mfma, 4)
            wl = peaks["int8_mfma_workload_operands"]["value"]
            pr["measured_peak_workload_operands"] = wl
            pr["frac_of_measured_workload_operands"] = round(pr["achieved"] / wl, 4)

    curves = [c for c in args.curves.split(",") if c and c != "none"]
    if curves:
        del mats
        torch.cuda.empty_cache()
        points = {"3b": [1, 8, 64, 256], "70b": [1, 16, 176], "3b-chained": []}
        result["curves"] = {c: curve(B, torch, c, points[c], dev, max(5, args.steps // 5),
                                     max(1, args.warmup // 2)) for c in curves}

    if not args.no_cpu:
        log("timing CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(args.model)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
