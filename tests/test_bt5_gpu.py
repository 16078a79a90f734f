"""Parity of the BT5-T32 path (five ternary codes per byte) with the CPU
oracle, through the C ABI.

Bar: packed bytes and decoded codes bit-exact; int32 accumulators bit-exact;
fp32 outputs equal to the oracle's fp32 rescale of the same accumulators
(and within 1e-5 relative of its fp64 rescale).  Every expected value comes
from the oracle on the same seeded inputs.

Format: BitNet b1.58 2B4T video transcript (yousumm.com), "Transcription"
(the ~0.4 GB footprint of the 2B model read as five codes per byte).
"""
import itertools
import sys

import numpy as np
import pytest
import torch

import oracle as O
import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def B():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import ternary_weight_w1_amd as B
    B.lib()
    return B


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def gamma_dev(g):
    return dev(np.array([g], np.float32))


def check_outputs(Y, acc, ref_acc, gamma, absmax, what=""):
    np.testing.assert_array_equal(acc, ref_acc, err_msg=f"acc {what}")
    y64 = O.epilogue_f64(ref_acc, gamma, absmax)
    nz = y64 != 0
    rel = np.abs(Y.astype(np.float64)[nz] - y64[nz]) / np.abs(y64[nz])
    assert rel.size == 0 or rel.max() <= 1e-5, f"Y rel err {rel.max()} {what}"
    np.testing.assert_array_equal(Y, O.epilogue(ref_acc, gamma, absmax), err_msg=f"Y {what}")


def padded_q(Q, K, ldq):
    Qp = np.zeros((Q.shape[0], ldq), np.int8)
    Qp[:, :K] = Q
    return Qp


# ------------------------------------------------------------------ packing --

@pytest.mark.parametrize("N,K", [(1, 1), (3, 17), (32, 160), (33, 161), (70, 333), (200, 2560),
                                 (64, 6912), (1000, 37)])
def test_pack5_parity(B, N, K):
    say("pack5", N, K)
    T = synth.random_ternary(N, K, seed=N * 5 + K)
    P = O.pack5(T)
    Pg = B.pack5(dev(T))
    np.testing.assert_array_equal(host(Pg), P)
    np.testing.assert_array_equal(host(B.unpack5(Pg, N, K)), T)


def test_pack5_golden_single_codes(B, golden_dir):
    say("pack5 golden")
    import os
    rows = [ln.split() for ln in open(os.path.join(golden_dir, "bt5_t32_fixtures.txt"))
            if ln.startswith("single")]
    assert len(rows) == 7
    for _, N, K, n, k, code, idx, val in rows:
        N, K, n, k, code, idx = map(int, (N, K, n, k, code, idx))
        T = np.zeros((N, K), np.int8)
        T[n, k] = code
        want = np.full(O.packed5_bytes(N, K), 0x80, np.uint8)
        want[idx] = int(val, 16)
        np.testing.assert_array_equal(host(B.pack5(dev(T))), want)


def test_unpack5_every_byte_value(B):
    # all 243 five-code combinations, in every digit position of a 16-byte
    # slot: the kernel's multiply-and-select planes against the oracle's
    # base-3 division
    say("unpack5 all bytes")
    combos = np.array(list(itertools.product((-1, 0, 1), repeat=5)), np.int8)
    N, K = 32, 160 * 8
    T = np.zeros((N, K), np.int8)
    j = 0
    for n in range(N):
        for u in range(8):
            for g in range(2):
                for p in range(16):
                    for i in range(5):
                        T[n, 160 * u + 32 * i + 16 * g + p] = combos[j % 243][i]
                    j += 1
    P = O.pack5(T)
    assert len(np.unique(P)) == 243
    np.testing.assert_array_equal(host(B.unpack5(dev(P), N, K)), T)


# -------------------------------------------------------------- contraction --

MM5_CASES = [
    # (M, N, K): one token, small batches, more than 16 tokens (several token
    # groups), ragged N (32-row tiles) and K (160-code units) throughout
    (1, 32, 160), (1, 100, 200), (1, 257, 640), (1, 640, 2560), (1, 37, 7),
    (2, 64, 64), (5, 100, 333), (16, 257, 640), (17, 640, 2560), (32, 130, 1000),
    (40, 100, 200), (3, 2560, 6912),
]


@pytest.mark.parametrize("M,N,K", MM5_CASES)
def test_matmul5_parity(B, M, N, K):
    say("matmul5", M, N, K)
    T = synth.random_ternary(N, K, seed=M + 3 * N + 7 * K + 1)
    X = synth.activations_np(M, K, seed=M * 17 + K, outlier_frac=0.01)
    Q, a, rs = O.quant_act(X)
    g = 0.0123
    ref = O.matmul(Q, T)
    ldq = B.q_stride5(K)
    Y, acc = B.matmul5(dev(padded_q(Q, K, ldq)), dev(a), dev(rs), dev(O.pack5(T)), gamma_dev(g),
                       N, K, with_acc=True)
    check_outputs(host(Y), host(acc), ref, g, a, f"M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(1, 32, 8192), (5, 64, 8192), (1, 200, 4000), (3, 40, 131072),
                                   (20, 64, 8192)])
def test_matmul5_split_k(B, M, N, K):
    # few row tiles and a long K: K is split over workgroups and the last
    # to arrive adds the partial sums
    say("matmul5 split-K", M, N, K)
    assert B.workspace_bytes(B.WS_MATMUL5, M, N, K) > 0
    T = synth.random_ternary(N, K, seed=N + K)
    Q = synth.random_int8(M, K, seed=M + K)
    rs = Q.astype(np.int64).sum(axis=1).astype(np.int32)
    a = np.linspace(0.5, 3.0, M).astype(np.float32)
    ref = O.matmul(Q, T)
    ldq = B.q_stride5(K) + 32  # a wider stride than needed
    for rep in range(2):       # the arrival counters are clean for the next call
        Y, acc = B.matmul5(dev(padded_q(Q, K, ldq)), dev(a), dev(rs), dev(O.pack5(T)),
                           gamma_dev(0.02), N, K, with_acc=True)
        check_outputs(host(Y), host(acc), ref, 0.02, a, f"split rep {rep}")


def test_matmul5_extreme_values(B):
    # |acc| at its largest: every code +1 against +127 (and -1 against -127)
    say("matmul5 extremes")
    M, N, K = 2, 64, 6912
    T = np.ones((N, K), np.int8)
    T[1::2] = -1
    Q = np.full((M, K), 127, np.int8)
    Q[1] = -127
    rs = Q.astype(np.int64).sum(axis=1).astype(np.int32)
    a = np.ones(M, np.float32)
    ref = O.matmul(Q, T)
    assert abs(ref).max() == 127 * K
    Y, acc = B.matmul5(dev(padded_q(Q, K, B.q_stride5(K))), dev(a), dev(rs), dev(O.pack5(T)),
                       gamma_dev(1.0), N, K, with_acc=True)
    check_outputs(host(Y), host(acc), ref, 1.0, a, "extremes")


@pytest.mark.parametrize("M,N,K", [(1, 640, 2560), (4, 100, 200), (16, 257, 640), (33, 300, 700),
                                   (1, 64, 8192)])
def test_forward5_parity(B, M, N, K):
    say("forward5", M, N, K)
    W = synth.weights_np(N, K, 0.02, seed=N * 3 + K)
    T, g = O.quantize_weights(W)
    X = synth.activations_np(M, K, seed=M + N, outlier_frac=0.01)
    ref = O.forward(X, T, g)
    Tg, _ = B.quantize_weights(dev(W), gamma_in=gamma_dev(g))
    P5 = B.pack5(Tg)
    np.testing.assert_array_equal(host(P5), O.pack5(T))
    Y, acc = B.forward5(dev(X), P5, gamma_dev(g), N, with_acc=True)
    check_outputs(host(Y), host(acc), ref["acc"], g, ref["absmax"], f"M={M} N={N} K={K}")
    # same result through the 2-bit format
    Y2, acc2 = B.forward(dev(X), B.pack(Tg), gamma_dev(g), N, with_acc=True)
    np.testing.assert_array_equal(host(acc2), host(acc))
    np.testing.assert_array_equal(host(Y2), host(Y))


# ------------------------------------------------------------------- groups --

def _group_problems(B, specs, seed0):
    probs, refs = [], []
    for i, (M, N, K, fmt) in enumerate(specs):
        T = synth.random_ternary(N, K, seed=seed0 + i)
        X = synth.activations_np(M, K, seed=seed0 + 100 + i, outlier_frac=0.01)
        g = np.float32(0.01 * (i + 1))
        refs.append((O.forward(X, T, g), g))
        P = O.pack5(T) if fmt == 1 else O.pack(T)
        probs.append(dict(X=dev(X), P=dev(P), gamma=gamma_dev(g), format=fmt,
                          Y=torch.empty((M, N), dtype=torch.float32, device="cuda"),
                          acc=torch.empty((M, N), dtype=torch.int32, device="cuda"), N=N))
    return probs, refs


def test_group_bt5_and_mixed_formats(B):
    say("group BT5 + BL2")
    specs = [(1, 640, 2560, 1), (1, 100, 200, 0), (4, 257, 640, 1), (40, 300, 700, 0),
             (17, 64, 8192, 1), (1, 32, 160, 1), (33, 100, 333, 1)]
    probs, refs = _group_problems(B, specs, 900)
    plan = B.GroupPlan(probs)
    plan.forward()
    first = [(host(p["Y"]).copy(), host(p["acc"]).copy()) for p in probs]
    for (Y, acc), (ref, g) in zip(first, refs):
        check_outputs(Y, acc, ref["acc"], float(g), ref["absmax"], "group")
    plan.quant_act()
    plan.matmul()
    for p, (Y, acc) in zip(probs, first):
        np.testing.assert_array_equal(host(p["Y"]), Y)
        np.testing.assert_array_equal(host(p["acc"]), acc)


def test_group_bt5_graph_replay(B):
    # The grouped BT5 step (quantize, then contract) captured once in a HIP
    # graph: every replay -- with eager library work and synchronizations
    # between replays -- matches the eager result and the oracle bit for bit.
    # The mix has a split-K problem (arrival tickets re-armed on every replay).
    say("group BT5 graph replay")
    specs = [(1, 640, 2560, 1), (1, 64, 8192, 1), (5, 2560, 640, 1)]
    probs, refs = _group_problems(B, specs, 950)
    plan = B.GroupPlan(probs)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        plan.quant_act()
        plan.matmul()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = [(host(p["Y"]).copy(), host(p["acc"]).copy()) for p in probs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        plan.quant_act()
        plan.matmul()
    Xo = dev(synth.activations_np(7, 300, seed=998))
    for rep in range(3):
        for p in probs:
            p["Y"].fill_(-1.0)
            p["acc"].fill_(-1)
        B.quant_act(Xo)  # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for p, (Y, acc), (ref, g) in zip(probs, eager, refs):
            np.testing.assert_array_equal(host(p["Y"]), Y, err_msg=f"replay {rep}")
            np.testing.assert_array_equal(host(p["acc"]), acc, err_msg=f"replay {rep}")
            check_outputs(host(p["Y"]), host(p["acc"]), ref["acc"], float(g), ref["absmax"],
                          f"graph replay {rep}")


# ------------------------------------------------ full model shapes, sampled --

def _bt5_layer(B, shapes, M, sigma, seed_layer):
    """One layer of model-shaped BitLinears in BT5-T32 through the grouped
    forward (the launch configuration the benchmark times); the oracle reads
    48 sampled rows straight from its own packed bytes."""
    rng = np.random.default_rng(seed_layer)
    probs, refs = [], []
    for j, (name, K, N) in enumerate(shapes):
        W = synth.weights_np(N, K, sigma, seed=synth.matrix_seed(seed_layer, j))
        T, g = O.quantize_weights(W)
        P = O.pack5(T)
        del T
        Tg, _ = B.quantize_weights(dev(W), gamma_in=gamma_dev(g))
        del W
        Pg = B.pack5(Tg)
        del Tg
        np.testing.assert_array_equal(host(Pg), P, err_msg=name)
        X = synth.activations_np(M, K, seed=11 + j)
        Q, a, rs = O.quant_act(X)
        rows = np.sort(rng.choice(N, size=48, replace=False))
        rows[-1] = N - 1
        refs.append((name, rows, O.matmul_packed5_rows(Q, P, N, K, rows), g, a))
        probs.append(dict(X=dev(X), P=Pg, gamma=gamma_dev(g), format=1,
                          Y=torch.empty((M, N), dtype=torch.float32, device="cuda"),
                          acc=torch.empty((M, N), dtype=torch.int32, device="cuda"), N=N))
    plan = B.GroupPlan(probs)
    plan.forward()
    for p, (name, rows, ref_acc, g, a) in zip(probs, refs):
        check_outputs(host(p["Y"])[:, rows], host(p["acc"])[:, rows], ref_acc, g, a, f"{name} M={M}")


@pytest.mark.parametrize("M", [1, 8])
def test_2b_layer_bt5_sampled(B, M):
    say("2B layer BT5", M)
    _bt5_layer(B, synth.SHAPES_2B, M, 0.02, 0)


def test_70b_layer_bt5_sampled(B):
    say("70B layer BT5", 1)
    shapes = [s for s in synth.SHAPES_70B if s[0] in ("q", "k", "down")]
    _bt5_layer(B, shapes, 1, 0.01, 2)
