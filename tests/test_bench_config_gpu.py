"""Parity in the exact launch configurations bench.py times.

1. The whole 2B-class stack (30 layers x q, k, v, o, gate, up, down = 210
   matrices) in one grouped plan, built by bench.make_plan, stepped as the
   benchmark steps it (grouped quantization, then the grouped contraction,
   no int32 side output), at the decode (M = 1) and prefill (M = 512, 1%
   outlier channels) sizes, and packed five codes per byte at M = 1, 8, 16.
2. The 3B-class stack chained as the benchmark chains it (bench.ChainedStack,
   26 layers), checked at its end against the oracle's chain.

The oracle sees only the seeded inputs: for three sampled layers (21
matrices) the fp32 weights drawn on the device are copied to the host and
quantized and packed by the oracle; the GPU must reproduce the packed bytes
exactly given the oracle's scale, and for 16 sampled output rows of each of
those matrices (always including the last) every token's fp32 output must
equal the oracle's, bit for bit, and be within 1e-5 relative of the fp64
rescale.  The other 189 matrices run in the same launches with the GPU's
own scales, as in the benchmark."""
import numpy as np
import pytest
import torch

import bench
import oracle as O
import synth

pytestmark = pytest.mark.gpu

SAMPLED_LAYERS = (0, 17, 29)
ROWS = 16


def host(t):
    return t.detach().cpu().numpy()


def gamma_dev(g):
    return torch.tensor([g], dtype=torch.float32, device="cuda")


@pytest.fixture(scope="module")
def stack():
    import ternary_weight_w1_amd as B
    spec = synth.MODELS["2b"]
    mats, ref = [], {}
    for layer in range(spec["layers"]):
        for j, (name, K, N) in enumerate(spec["shapes"]):
            W = synth.weights_torch(N, K, spec["sigma"], synth.matrix_seed(layer, j), "cuda")
            sampled = layer in SAMPLED_LAYERS
            if sampled:
                T, g = O.quantize_weights(host(W))
                P, P5 = O.pack(T), O.pack5(T)
                del T
                Tg, gg = B.quantize_weights(W, gamma_in=gamma_dev(g))
            else:
                Tg, gg = B.quantize_weights(W)
            del W
            Pg, P5g = B.pack(Tg), B.pack5(Tg)
            del Tg
            if sampled:
                np.testing.assert_array_equal(host(Pg), P, err_msg=f"packed bytes layer {layer} {name}")
                np.testing.assert_array_equal(host(P5g), P5, err_msg=f"BT5 bytes layer {layer} {name}")
                ref[len(mats)] = (name, P, P5, g)
            mats.append(dict(layer=layer, name=name, K=K, N=N, P=Pg, P5=P5g, gamma=gg))
    torch.cuda.synchronize()
    assert len(mats) == 210
    return B, mats, ref


def _check_sampled(mats, ref, probs, M, fmt):
    rng = np.random.default_rng(M + 1000 * fmt)
    for i, (name, P, P5, g) in ref.items():
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


@pytest.mark.parametrize("M,outliers", [(1, 0.0), (512, 0.01)])
def test_bench_launch_configuration_sampled(stack, M, outliers):
    B, mats, ref = stack
    print(f"bench configuration: 210 matrices, M={M}", flush=True)
    plan, probs = bench.make_plan(B, torch, mats, M, torch.device("cuda:0"), outliers=outliers)
    plan.quant_act()
    plan.matmul()
    torch.cuda.synchronize()
    _check_sampled(mats, ref, probs, M, 0)
    del plan, probs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M", [1, 8, 16])
def test_bench_bt5_configuration_sampled(stack, M):
    # the benchmark's five-codes-per-byte sweeps: the same 210 matrices in
    # BT5-T32, one grouped plan per token count
    B, mats, ref = stack
    print(f"bench BT5 configuration: 210 matrices, M={M}", flush=True)
    plan, probs = bench.make_plan(B, torch, mats, M, torch.device("cuda:0"), fmt=1)
    plan.quant_act()
    plan.matmul()
    torch.cuda.synchronize()
    _check_sampled(mats, ref, probs, M, 1)
    del plan, probs
    torch.cuda.empty_cache()


# ------------------------------------------- the chained 3B stack, full depth --

@pytest.fixture(scope="module")
def stack_3b():
    """Every 3B-class matrix (26 layers) quantized by the oracle from the
    seeded device-drawn weights; the GPU packs the same codes (bytes checked)
    and the oracle keeps its codes for the reference chain."""
    import ternary_weight_w1_amd as B
    spec = synth.MODELS["3b"]
    mats, codes = [], {}
    for layer in range(spec["layers"]):
        for j, (name, K, N) in enumerate(spec["shapes"]):
            W = synth.weights_torch(N, K, spec["sigma"], synth.matrix_seed(layer, j), "cuda")
            T, g = O.quantize_weights(host(W))
            Tg, gg = B.quantize_weights(W, gamma_in=gamma_dev(g))
            del W
            Pg = B.pack(Tg)
            del Tg
            np.testing.assert_array_equal(host(Pg), O.pack(T), err_msg=f"packed bytes layer {layer} {name}")
            codes[(layer, name)] = (T, np.float32(g))
            mats.append(dict(layer=layer, name=name, K=K, N=N, P=Pg, P5=None, gamma=gg))
    torch.cuda.synchronize()
    return B, mats, codes, spec["layers"]


@pytest.mark.parametrize("M", [1, 8])
def test_bench_chained_3b_stack(stack_3b, M):
    # bench.py's chained stack (the latency curve it reports): 26 pre-norm
    # blocks, q|k|v and gate|up each in one multi-matrix launch, every
    # workspace reused by all 26 layers; the final residual stream and its
    # final norm's int8 cast must equal the oracle's chain bit for bit.
    import ctypes
    B, mats, codes, n_layers = stack_3b
    print(f"chained 3B stack, {n_layers} layers, M={M}", flush=True)
    dim = next(m["K"] for m in mats if m["name"] == "q")
    x0, gains, g_fin = bench.stack_inputs(torch, dim, n_layers, M, torch.device("cuda:0"))
    chain = bench.ChainedStack(B, torch, mats, torch.device("cuda:0"), M, x0, gains, g_fin)
    chain.step(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()

    def lin(Q, a, layer, name):
        T, g = codes[(layer, name)]
        return O.epilogue(O.matmul(Q, T), g, a)

    xh = host(x0)
    x, d = xh, None
    for i in range(n_layers):
        ga, gf = host(gains[i][0]), host(gains[i][1])
        if i == 0:
            Q, a, rs, _, _ = O.rmsnorm_quant_act(xh, ga, 1e-5)
        else:
            Q, a, rs, x, _, _ = O.add_rmsnorm_quant_act(x, d, ga, 1e-5)
        v = lin(Q, a, i, "v")
        Qo, ao, _ = O.quant_act(v)
        o = lin(Qo, ao, i, "o")
        Qf, af, _, x, _, _ = O.add_rmsnorm_quant_act(xh if i == 0 else x, o, gf, 1e-5)
        Qd, ad, _, _ = O.relu2_gate_quant_act(lin(Qf, af, i, "gate"), lin(Qf, af, i, "up"))
        d = lin(Qd, ad, i, "down")
    Qfin, afin, rsfin, xfin, _, _ = O.add_rmsnorm_quant_act(x, d, host(g_fin), 1e-5)
    np.testing.assert_array_equal(host(chain.x), xfin, err_msg="final residual stream")
    np.testing.assert_array_equal(host(chain.Q)[:, :dim], Qfin, err_msg="final int8 cast")
    np.testing.assert_array_equal(host(chain.a), afin, err_msg="final absmax")
    np.testing.assert_array_equal(host(chain.rs), rsfin, err_msg="final row sums")
    del chain
    torch.cuda.empty_cache()
