"""Parity in the exact launch configurations bench.py times.

1. Whole stacks in one grouped plan, built by bench.make_plan and stepped as
   the benchmark steps them (grouped quantization, then the grouped
   contraction, no int32 side output): the 2B-class stack (30 layers x q, k,
   v, o, gate, up, down = 210 matrices) at the decode (M = 1), batched
   decode (M = 8, 16: the 2-bit sweeps of the BT5 comparison) and prefill
   (M = 512, 1% outlier channels) sizes and packed five codes per byte at
   M = 1, 8, 16; the 3B-class curve (182 matrices) at M = 1, 8, 64, 256; the
   70B-class curve (560 matrices, 17 GB packed) at M = 1, 16, 176.
2. The 3B-class stack chained as the benchmark chains it (bench.ChainedStack,
   all 26 layers at 1, 8, 64 and 256 tokens), checked at its end against
   the oracle's chain on up to 16 sampled tokens.

The oracle sees only the seeded inputs: for the sampled layers the fp32
weights drawn on the device are copied to the host and quantized and packed
by the oracle; the GPU must reproduce the packed bytes exactly given the
oracle's scale, and for 16 sampled output rows of each sampled matrix
(always including the last) every token's fp32 output must equal the
oracle's, bit for bit, and be within 1e-5 relative of the fp64 rescale.  The
other matrices run in the same launches with the GPU's own scales, as in the
benchmark."""
import numpy as np
import pytest
import torch

import bench
import oracle as O
import synth
from fp_exact import decided_or_skip

pytestmark = pytest.mark.gpu

ROWS = 16
# sampled layers per model (the oracle quantizes these); None = every layer
SAMPLED = {"2b": (0, 17, 29), "3b": None, "70b": (0, 79)}
_STACKS = {}


def host(t):
    return t.detach().cpu().numpy()


def gamma_dev(g):
    return torch.tensor([g], dtype=torch.float32, device="cuda")


def _stack(model):
    """The model's whole stack packed on the device as bench.build_stack packs
    it (also five codes per byte for 2B), the sampled layers from the
    oracle's codes and scales; cached for the module."""
    if model in _STACKS:
        return _STACKS[model]
    import ternary_weight_w1_amd as B
    spec = synth.MODELS[model]
    layers = SAMPLED[model]
    bt5 = model == "2b"
    mats, ref, codes = [], {}, {}
    for layer in range(spec["layers"]):
        sampled = layers is None or layer in layers
        for j, (name, K, N) in enumerate(spec["shapes"]):
            W = synth.weights_torch(N, K, spec["sigma"], synth.matrix_seed(layer, j), "cuda")
            if sampled:
                T, g = O.quantize_weights(host(W))
                Tg, gg = B.quantize_weights(W, gamma_in=gamma_dev(g))
            else:
                Tg, gg = B.quantize_weights(W)
            del W
            Pg = B.pack(Tg)
            P5g = B.pack5(Tg) if bt5 else None
            del Tg
            if sampled:
                P = O.pack(T)
                np.testing.assert_array_equal(host(Pg), P, err_msg=f"{model} packed bytes layer {layer} {name}")
                P5 = None
                if bt5:
                    P5 = O.pack5(T)
                    np.testing.assert_array_equal(host(P5g), P5, err_msg=f"{model} BT5 bytes layer {layer} {name}")
                ref[len(mats)] = (name, P, P5, g)
                if model == "3b":
                    codes[(layer, name)] = (T, np.float32(g))
                del T
            mats.append(dict(layer=layer, name=name, K=K, N=N, P=Pg, P5=P5g, gamma=gg))
    torch.cuda.synchronize()
    _STACKS[model] = (B, mats, ref, codes)
    return _STACKS[model]


@pytest.fixture(scope="module", autouse=True)
def _release_stacks():
    yield
    _STACKS.clear()
    torch.cuda.empty_cache()


def _check_sampled(mats, ref, probs, M, fmt, every=1):
    rng = np.random.default_rng(M + 1000 * fmt)
    for idx, (i, (name, P, P5, g)) in enumerate(sorted(ref.items())):
        if idx % every:
            continue
        N, K = mats[i]["N"], mats[i]["K"]
        Q, a, rs = O.quant_act(host(probs[i]["X"]))
        rows = np.sort(rng.choice(N, size=ROWS, replace=False))
        rows[-1] = N - 1
        if fmt:
            acc = O.matmul_packed5_rows(Q, P5, N, K, rows)
        else:
            acc = O.matmul_packed_rows(Q, P, N, K, rows)
        Y = host(probs[i]["Y"])[:, rows]
        what = f"matrix {i} ({name}, layer {mats[i]['layer']}) M={M} format={fmt}"
        np.testing.assert_array_equal(Y, O.epilogue(acc, g, a), err_msg=what)
        y64 = O.epilogue_f64(acc, g, a)
        nz = y64 != 0
        rel = np.abs(Y.astype(np.float64)[nz] - y64[nz]) / np.abs(y64[nz])
        assert rel.size == 0 or rel.max() <= 1e-5, what


@pytest.mark.parametrize("model,M,outliers", [("2b", 1, 0.0), ("2b", 8, 0.0), ("2b", 16, 0.0), ("2b", 512, 0.01),
                                              ("3b", 1, 0.0), ("3b", 8, 0.0),
                                              ("3b", 64, 0.0), ("3b", 256, 0.0), ("70b", 1, 0.0), ("70b", 16, 0.0),
                                              ("70b", 176, 0.0)])
def test_bench_launch_configuration_sampled(model, M, outliers):
    B, mats, ref, _ = _stack(model)
    print(f"bench configuration: {model}, {len(mats)} matrices, M={M}", flush=True)
    plan, probs = bench.make_plan(B, torch, mats, M, torch.device("cuda:0"), outliers=outliers)
    plan.quant_act()
    plan.matmul()
    torch.cuda.synchronize()
    # every layer of the 3B stack has oracle codes; check every fourth matrix
    _check_sampled(mats, ref, probs, M, 0, every=4 if model == "3b" else 1)
    del plan, probs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M", [1, 8, 16])
def test_bench_bt5_configuration_sampled(M):
    # the benchmark's five-codes-per-byte sweeps: the same 210 matrices in
    # BT5-T32, one grouped plan per token count
    B, mats, ref, _ = _stack("2b")
    print(f"bench BT5 configuration: 210 matrices, M={M}", flush=True)
    plan, probs = bench.make_plan(B, torch, mats, M, torch.device("cuda:0"), fmt=1)
    plan.quant_act()
    plan.matmul()
    torch.cuda.synchronize()
    _check_sampled(mats, ref, probs, M, 1)
    del plan, probs
    torch.cuda.empty_cache()


# ------------------------------------------- the chained 3B stack, full depth --

@pytest.mark.parametrize("M", [1, 8, 64, 256])
def test_bench_chained_3b_stack(M):
    # bench.py's chained stack (the latency curve it reports): 26 pre-norm
    # blocks, q|k|v and gate|up each in one multi-matrix launch, every
    # workspace reused by all 26 layers (at 64 and 256 tokens the tile
    # kernel's launches split K and reuse their arrival tickets layer after
    # layer).  Tokens never mix in this chain (the single-key attention
    # passes v through), so the oracle follows up to 16 sampled tokens
    # through all 26 layers; on those rows the final residual stream, its
    # final norm's int8 cast, and the last layer's q and k (the two outputs
    # of the timed q|k|v launch the chain itself does not consume) must
    # equal the oracle's bit for bit.
    import ctypes
    B, mats, _, codes = _stack("3b")
    n_layers = synth.MODELS["3b"]["layers"]
    print(f"chained 3B stack, {n_layers} layers, M={M}", flush=True)
    dim = next(m["K"] for m in mats if m["name"] == "q")
    x0, gains, g_fin = bench.stack_inputs(torch, dim, n_layers, M, torch.device("cuda:0"))
    chain = bench.ChainedStack(B, torch, mats, torch.device("cuda:0"), M, x0, gains, g_fin)
    chain.step(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    rows = np.arange(M) if M <= 16 else np.sort(np.random.default_rng(M).choice(M, 16, replace=False))
    if M > 16:
        rows[-1] = M - 1

    def lin(Q, a, layer, name):
        T, g = codes[(layer, name)]
        return O.epilogue(O.matmul(Q, T), g, a)

    xh = host(x0)[rows]
    x, d = xh, None
    for i in range(n_layers):
        ga, gf = host(gains[i][0]), host(gains[i][1])
        if i == 0:
            decided_or_skip(xh, 1e-5, "layer 0 attention norm")
            Q, a, rs, _, _ = O.rmsnorm_quant_act(xh, ga, 1e-5)
        else:
            Q, a, rs, x, _, _ = O.add_rmsnorm_quant_act(x, d, ga, 1e-5)
            decided_or_skip(x, 1e-5, f"layer {i} attention norm")
        if i == n_layers - 1:
            q_last, k_last = lin(Q, a, i, "q"), lin(Q, a, i, "k")
        v = lin(Q, a, i, "v")
        Qo, ao, _ = O.quant_act(v)
        o = lin(Qo, ao, i, "o")
        Qf, af, _, x, _, _ = O.add_rmsnorm_quant_act(xh if i == 0 else x, o, gf, 1e-5)
        decided_or_skip(x, 1e-5, f"layer {i} feed-forward norm")
        Qd, ad, _, _ = O.relu2_gate_quant_act(lin(Qf, af, i, "gate"), lin(Qf, af, i, "up"))
        d = lin(Qd, ad, i, "down")
    Qfin, afin, rsfin, xfin, _, _ = O.add_rmsnorm_quant_act(x, d, host(g_fin), 1e-5)
    decided_or_skip(xfin, 1e-5, "final norm")
    np.testing.assert_array_equal(host(chain.q)[rows], q_last, err_msg="last layer q")
    np.testing.assert_array_equal(host(chain.k)[rows], k_last, err_msg="last layer k")
    np.testing.assert_array_equal(host(chain.x)[rows], xfin, err_msg="final residual stream")
    np.testing.assert_array_equal(host(chain.Q)[rows, :dim], Qfin, err_msg="final int8 cast")
    np.testing.assert_array_equal(host(chain.a)[rows], afin, err_msg="final absmax")
    np.testing.assert_array_equal(host(chain.rs)[rows], rsfin, err_msg="final row sums")
    del chain
    torch.cuda.empty_cache()
