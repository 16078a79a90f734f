"""bitlinear_forward_noalloc (the forward that allocates nothing: its
workspace is the library's own device array) against bitlinear_forward with
a caller workspace, through the C ABI: int32 accumulators and fp32 outputs
bit for bit, and both against the oracle.  Two calls in a row, the second
smaller, then the first size again: the array keeps the last call's
contents, so the split-K arrival counters must come back to zero."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import synth

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def test_noalloc_matches_forward_on_consecutive_calls():
    import ternary_weight_w1_amd as B
    L = B.lib()
    g = np.float32(0.021)
    gd = torch.tensor([g], dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    # a tile-kernel case whose K is split in two (partial sums and counters in
    # the array), a smaller one-token case whose K is split on the streaming
    # kernel, and the first case again
    cases = [(96, 640, 2560), (1, 300, 1000), (96, 640, 2560)]
    for M, N, K in cases:
        say("forward_noalloc", M, N, K)
        need = B.workspace_bytes(B.WS_FORWARD, M, N, K)
        assert 0 < need <= B.noalloc_scratch_bytes()
        T = synth.random_ternary(N, K, seed=M + N + K)
        X = synth.activations_np(M, K, seed=M + 2 * K, outlier_frac=0.01)
        P = torch.from_numpy(O.pack(T)).cuda()
        Xd = torch.from_numpy(X).cuda()
        Y_ref, acc_ref = B.forward(Xd, P, gd, N, with_acc=True)
        Y = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        acc = torch.full((M, N), -7, dtype=torch.int32, device="cuda")
        st = L.bitlinear_forward_noalloc(Xd.data_ptr(), M, K, P.data_ptr(), gd.data_ptr(), N, Y.data_ptr(),
                                         acc.data_ptr(), stream)
        assert st == 0, L.bitlinear_last_error().decode()
        torch.cuda.synchronize()
        assert torch.equal(acc, acc_ref), (M, N, K)
        assert torch.equal(Y, Y_ref), (M, N, K)
        ref = O.forward(X, T, g)
        np.testing.assert_array_equal(acc.cpu().numpy(), ref["acc"])
        np.testing.assert_array_equal(Y.cpu().numpy(), ref["Y"])
    # the binding's wrapper (marshalling only) gives the same
    Y2 = B.forward_noalloc(Xd, P, gd, N)
    torch.cuda.synchronize()
    assert torch.equal(Y2, Y_ref)


def test_noalloc_rejects_sizes_beyond_the_array():
    import ternary_weight_w1_amd as B
    L = B.lib()
    M, N, K = 4096, 2560, 2560
    assert B.workspace_bytes(B.WS_FORWARD, M, N, K) > B.noalloc_scratch_bytes()
    X = torch.zeros((M, K), dtype=torch.float32, device="cuda")
    P = torch.zeros(B.packed_bytes(N, K), dtype=torch.uint8, device="cuda")
    gd = torch.ones(1, dtype=torch.float32, device="cuda")
    Y = torch.full((M, N), 3.0, dtype=torch.float32, device="cuda")
    st = L.bitlinear_forward_noalloc(X.data_ptr(), M, K, P.data_ptr(), gd.data_ptr(), N, Y.data_ptr(), None,
                                     torch.cuda.current_stream().cuda_stream)
    assert st == -4 and b"scratch" in L.bitlinear_last_error()
    torch.cuda.synchronize()
    assert bool((Y == 3.0).all())  # nothing was enqueued
