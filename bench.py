"""Benchmark of the BitLinear W1.58A8 hot path on one MI355X.

Default workload (one step): the 2B-class decode GEMV set -- 30 layers x
{q, k, v, o, gate, up, down} = 210 BitLinear matrices held in HBM as 2-bit
packed ternary codes (521.0 MB), one token (M = 1) of fresh fp32
activations per matrix.  A step quantizes every activation vector per token
(absmax -> int8) and contracts it with its packed matrix, rescaling to fp32
(grouped launches: one activation-quantization kernel, one contraction
kernel for all 210 problems).  Weights are quantized and packed once, before
timing, like loading an inference-ready checkpoint.

Printed: one JSON line.  value = packed weight bytes per step / step time.
roofline = the contraction kernel's algorithmic bytes (packed weights + int8
activations + fp32 outputs) over its average duration (HIP events on the
launch stream), against 8 TB/s.  prefill = the same 210 matrices at
M = 512 (int8 TOP/s against 5.0 POP/s dense int8).  graph = the decode
step captured once in a HIP graph and replayed.  curves = latency of a full
sweep over the 3B-class stack at M in {1, 8, 64, 256} (and, on request, the
70B-class stack at M in {1, 16, 176}); for 3B also the same stack chained as
pre-norm blocks (residual adds, norms, the gated squared-ReLU, a single-key
attention; q|k|v and gate|up each one launch) at M in {1, 8, 64}, eager and
as a replayed HIP graph.  bt5 = the same 2B stack packed
five codes per byte (BT5-T32, 1.6 bits per weight) at M in {1, 8, 16},
next to the 2-bit path at the same M.  cpu_baseline = the CPU oracle
(single thread) on a bounded sample of the same workload.

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
                  "ternary_weight_w1_amd/csrc/gemv5.hip", "ternary_weight_w1_amd/csrc/bt5.hpp"]


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


def time_plan(torch, plan, steps, warmup):
    """Wall time per step over `steps` steps (quantize + contract), then the
    contraction kernel alone: `steps` back-to-back launches between one pair
    of HIP events on the launch stream (torch's current stream), giving its
    average launch duration without per-launch event overhead."""
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
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        plan.matmul()
    b.record()
    torch.cuda.synchronize()
    return wall / steps * 1e3, a.elapsed_time(b) / steps


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
    count M (quantize + contract every matrix, grouped launches)."""
    spec = synth.MODELS[model]
    log(f"building {model} stack: {spec['layers']} layers")
    mats = build_stack(B, torch, model, spec["layers"], dev)
    packed = sum(m["N"] * m["K"] // 4 for m in mats)
    out = {"matrices": len(mats), "packed_bytes": packed, "points": []}
    for M in Ms:
        plan, probs = make_plan(B, torch, mats, M, dev)
        ms, kern = time_plan(torch, plan, steps, warmup)
        ops = sum(2 * M * m["N"] * m["K"] for m in mats)
        out["points"].append({"M": M, "ms_per_sweep": round(ms, 4), "contraction_ms": round(kern, 4),
                              "packed_GBps": round(packed / (ms * 1e-3) / 1e9, 1),
                              "TOPs": round(ops / (ms * 1e-3) / 1e12, 1)})
        log(f"  {model} M={M}: {ms:.3f} ms per sweep")
        del plan, probs
    if model == "3b":
        log("timing the 3B stack chained as pre-norm blocks")
        out["chained"] = stack_curve(B, torch, mats, dev, [1, 8, 64], steps, warmup)
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
        ms5, k5 = time_plan(torch, plan, steps, warmup)
        del plan, probs
        plan, probs = make_plan(B, torch, mats, M, dev)
        ms2, k2 = time_plan(torch, plan, steps, warmup)
        del plan, probs
        alg = packed5 + sum(M * B.q_stride5(m["K"]) + 8 * M + 4 * M * m["N"] for m in mats)
        gbs = alg / (k5 * 1e-3) / 1e9
        out["points"].append({
            "M": M, "ms_per_step": round(ms5, 5), "kernel_ms": round(k5, 5),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_launch": alg,
                         "traffic": load_traffic(f"bt5_{model}_m{M}")},
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
    library call on one stream: residual add + RMSNorm + int8 cast, q|k|v in
    one launch (one input), the attention of the first decode position (a
    single key, so its output is v), the cast of v, o, residual add + RMSNorm
    + cast, gate|up in one launch, the gated squared-ReLU cast, down; then
    the final residual add + norm + cast: 8 launches per layer.  Buffers and
    workspaces are allocated once (workspaces zero-filled once, as the
    multi-matrix call requires).  After step(), x holds the final residual
    stream and (Q, a, rs) its final norm's int8 cast."""

    def __init__(self, B, torch, mats, dev, M, x0, gains, g_fin):
        import ctypes
        self.L = L = B.lib()
        self.layers = layers = {}
        for m in mats:
            layers.setdefault(m["layer"], {})[m["name"]] = m
        self.M = M
        self.dim = dim = layers[0]["q"]["K"]
        self.ffn = ffn = layers[0]["gate"]["N"]
        self.x0, self.gains, self.g_fin = x0, gains, g_fin
        f32 = lambda n: torch.empty((M, n), dtype=torch.float32, device=dev)
        self.x, self.q, self.k, self.v, self.o = f32(dim), f32(dim), f32(dim), f32(dim), f32(dim)
        self.gate, self.up, self.d = f32(ffn), f32(ffn), f32(dim)
        self.ldd, self.ldf = B.q_stride(dim), B.q_stride(ffn)
        self.Q = torch.empty((M, self.ldd), dtype=torch.int8, device=dev)
        self.Qf = torch.empty((M, self.ldf), dtype=torch.int8, device=dev)
        self.a = torch.empty(M, dtype=torch.float32, device=dev)
        self.rs = torch.empty(M, dtype=torch.int32, device=dev)
        self.P = lambda t: ctypes.c_void_p(t.data_ptr())

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
        self.wss = {}
        for key, K in (("qkv", dim), ("o", dim), ("gu", dim), ("down", ffn)):
            arr = self.sites[0][key]
            wsb = L.bitlinear_multi_workspace_bytes(arr, len(arr), M, K)
            self.wss[key] = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=dev)

    def _check(self, st):
        if st != 0:
            raise RuntimeError(self.L.bitlinear_last_error().decode())

    def step(self, s):
        """Enqueue one pass over every layer on the raw stream handle s."""
        L, P, M, dim, ffn, ldd, ldf = self.L, self.P, self.M, self.dim, self.ffn, self.ldd, self.ldf
        x, a, rs, Q = self.x, self.a, self.rs, self.Q

        def multi(Qin, ld, K, key, site):
            arr = site[key]
            self._check(L.bitlinear_matmul_multi(P(Qin), ld, P(a), P(rs), M, K, arr, len(arr), P(self.wss[key]),
                                                 self.wss[key].numel(), s))
        for i in sorted(self.layers):
            ga, gf = self.gains[i]
            site = self.sites[i]
            if i == 0:
                self._check(L.bitlinear_quant_act_rmsnorm(P(self.x0), M, dim, P(ga), 1e-5, P(Q), ldd, P(a),
                                                          P(rs), s))
            else:
                self._check(L.bitlinear_quant_act_add_rmsnorm(P(x), P(self.d), M, dim, P(ga), 1e-5, P(x), P(Q),
                                                              ldd, P(a), P(rs), s))
            multi(Q, ldd, dim, "qkv", site)
            self._check(L.bitlinear_quant_act(P(self.v), M, dim, P(Q), ldd, P(a), P(rs), s))
            multi(Q, ldd, dim, "o", site)
            self._check(L.bitlinear_quant_act_add_rmsnorm(P(self.x0 if i == 0 else x), P(self.o), M, dim, P(gf),
                                                          1e-5, P(x), P(Q), ldd, P(a), P(rs), s))
            multi(Q, ldd, dim, "gu", site)
            self._check(L.bitlinear_quant_act_relu2_gate(P(self.gate), P(self.up), M, ffn, P(self.Qf), ldf, P(a),
                                                         P(rs), s))
            multi(self.Qf, ldf, ffn, "down", site)
        self._check(L.bitlinear_quant_act_add_rmsnorm(P(x), P(self.d), M, dim, P(self.g_fin), 1e-5, P(x), P(Q),
                                                      ldd, P(a), P(rs), s))


def stack_curve(B, torch, mats, dev, Ms, steps, warmup):
    """Latency of the stack chained as pre-norm blocks (ChainedStack), one
    decode (or prefill) step of M tokens through every layer, timed eagerly
    and as one HIP graph replayed."""
    import ctypes
    n_layers = len({m["layer"] for m in mats})
    dim = next(m["K"] for m in mats if m["name"] == "q")
    ffn = next(m["N"] for m in mats if m["name"] == "gate")
    out = {"layers": n_layers, "dim": dim, "ffn": ffn, "launches_per_step": 8 * n_layers + 1, "points": []}
    for M in Ms:
        chain = ChainedStack(B, torch, mats, dev, M, *stack_inputs(torch, dim, n_layers, M, dev))
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            s = ctypes.c_void_p(side.cuda_stream)
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
        for _ in range(max(1, warmup)):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            graph.replay()
        torch.cuda.synchronize()
        gms = (time.perf_counter() - t0) / steps * 1e3
        out["points"].append({"M": M, "eager_ms_per_step": round(eager, 4), "graph_ms_per_step": round(gms, 4)})
        log(f"  stack M={M}: eager {eager:.3f} ms, graph {gms:.3f} ms per step")
        del graph, chain
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
    return {
        "hbm_read": {"value": round(best[0], 1), "unit": "GB/s",
                     "probe": f"16-byte non-temporal streaming read of 2 GiB, {best[1] >> 10} KiB per workgroup"},
        "int8_mfma": {"value": round(tops, 1), "unit": "TOP/s",
                      "probe": f"v_mfma_i32_32x32x32_i8 chains, {blocks} workgroups, no memory traffic, "
                               f"median of {len(later)} sustained bursts"},
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


def cpu_baseline(model: str, seconds: float = 10.0):
    """The oracle, untuned, single thread: unpack + activation quantization +
    triple-loop contraction + rescale on one layer of the stack (7 matrices,
    M = 1), repeated until about `seconds` of CPU time."""
    import oracle as O
    spec = synth.MODELS[model]
    work = []
    for j, (name, K, N) in enumerate(spec["shapes"]):
        W = synth.weights_np(N, K, spec["sigma"], synth.matrix_seed(0, j))
        T, g = O.quantize_weights(W)
        work.append((synth.activations_np(1, K, 7 + j), O.pack(T), g, N, N * K // 4))
        del W, T
    reps, t, nbytes = 0, 0.0, 0
    while t < seconds:
        t0 = time.perf_counter()
        for X, P, g, N, b in work:
            O.forward_packed(X, P, g, N)
            nbytes += b
        t += time.perf_counter() - t0
        reps += 1
    return {"value": nbytes / t / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"layer 0 of the {model.upper()} stack (7 matrices, M=1) x {reps} passes, "
                      f"{t:.1f} s single-thread: unpack + act quant + int32 triple loop + rescale"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--model", default="2b", choices=sorted(synth.MODELS))
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--M", type=int, default=1)
    ap.add_argument("--prefill-M", type=int, default=512)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--curves", default="3b",
                    help="comma list of latency-vs-M curves to add: 3b (M 1,8,64,256), 70b (M 1,16,176); "
                         "'none' to skip")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-bt5", action="store_true", help="skip the five-codes-per-byte comparison")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak calibration probes")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a plain device copy of known size (PMC calibration)")
    args = ap.parse_args()

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

    spec = synth.MODELS[args.model]
    layers = args.layers or spec["layers"]
    log(f"building {args.model} stack: {layers} layers")
    mats = build_stack(B, torch, args.model, layers, dev, bt5=not args.no_bt5)
    packed = sum(m["N"] * m["K"] // 4 for m in mats)
    assert packed == sum(B.packed_bytes(m["N"], m["K"]) for m in mats)

    M = args.M
    plan, probs = make_plan(B, torch, mats, M, dev)
    log(f"timing decode sweep: {len(mats)} matrices, M={M}, {packed / 1e6:.1f} MB packed")
    ms, kern_ms = time_plan(torch, plan, args.steps, args.warmup)
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
                     "kernel_ms_mean": round(kern_ms, 5), "bytes_per_launch": alg_bytes},
    }
    if gms is not None:
        result["graph"] = {"ms_per_step": round(gms, 5), "GBps": round(packed / (gms * 1e-3) / 1e9, 2),
                           "note": "the same step captured once in a HIP graph and replayed"}
    del plan, probs
    torch.cuda.empty_cache()

    if not args.no_bt5:
        log("timing BT5-T32 sweeps")
        result["bt5"] = bt5_section(B, torch, mats, dev, [1, 8, 16], args.steps, args.warmup, args.model)
        for m in mats:
            m["P5"] = None
        torch.cuda.empty_cache()

    if not args.no_prefill:
        PM = args.prefill_M
        plan, probs = make_plan(B, torch, mats, PM, dev, outliers=0.01)
        log(f"timing prefill sweep: M={PM}")
        steps = max(3, args.steps // 5)
        pms, pkern = time_plan(torch, plan, steps, max(1, args.warmup // 2))
        ops = sum(2 * PM * m["N"] * m["K"] for m in mats)
        result["prefill"] = {
            "M": PM, "ms_per_step": round(pms, 4), "value": round(ops / (pms * 1e-3) / 1e12, 2),
            "unit": "TOP/s",
            "roofline": {"bound": "mfma", "achieved": round(ops / (pkern * 1e-3) / 1e12, 2),
                         "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                         "frac": round(ops / (pkern * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4),
                         "traffic": load_traffic(f"tile_{args.model}_m{PM}"),
                         "kernel": "tile contraction (grouped)", "kernel_ms_mean": round(pkern, 4),
                         "ops_per_launch": ops},
        }
        del plan, probs
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

    curves = [c for c in args.curves.split(",") if c and c != "none"]
    if curves:
        del mats
        torch.cuda.empty_cache()
        points = {"3b": [1, 8, 64, 256], "70b": [1, 16, 176]}
        result["curves"] = {c: curve(B, torch, c, points[c], dev, max(5, args.steps // 5),
                                     max(1, args.warmup // 2)) for c in curves}

    if not args.no_cpu:
        log("timing CPU oracle baseline")
        result["cpu_baseline"] = cpu_baseline(args.model)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
