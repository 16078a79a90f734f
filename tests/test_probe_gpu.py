"""The calibration probes behind the measured roofline denominators
(include/bitlinear_probe.h): each must really do its work, which their
checksums show against closed forms computed on the host."""
import numpy as np
import pytest
import torch

import ternary_weight_w1_amd as B

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,chunk", [(16, 4096), (4096, 4096), (3 * (1 << 20) + 48, 65536),
                                          ((1 << 20) + 4096, 1 << 20)])
def test_probe_read_xor_matches_host(nbytes, chunk):
    print(f"probe_read nbytes={nbytes} chunk={chunk}", flush=True)
    g = torch.Generator().manual_seed(nbytes)
    host = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g)
    buf = host.to("cuda")
    sink = B.probe_read(buf, chunk)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    assert got.size == B.probe_read_sink_words(nbytes, chunk)
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert int(np.bitwise_xor.reduce(got)) == int(want)
    # each chunk's 256 threads together fold exactly that chunk
    words = host.numpy().view(np.uint32)
    per = chunk // 4
    for c in range(got.size // 256):
        assert int(np.bitwise_xor.reduce(got[256 * c:256 * (c + 1)])) == \
            int(np.bitwise_xor.reduce(words[per * c:per * (c + 1)]))


@pytest.mark.parametrize("iters,a,b,blocks", [(1, 1, 1, 1), (7, 3, -5, 5), (60, -128, 127, 3),
                                             (4096, 1, 1, 2)])
def test_probe_mfma_closed_form(iters, a, b, blocks):
    print(f"probe_mfma iters={iters} a={a} b={b} blocks={blocks}", flush=True)
    sink = B.probe_mfma(iters, a, b, blocks, device="cuda")
    torch.cuda.synchronize()
    assert sink.numel() == 256 * blocks
    assert bool((sink == 2048 * a * b * iters).all())


def probe_operands(seed):
    """Four (A, B) fragment sets: A random int8 in [-127, 127], B random
    ternary fields {0, 1, 2}, as the contraction kernels feed them."""
    rng = np.random.default_rng(seed)
    ops = np.empty((4, 2, 64, 16), np.int8)
    ops[:, 0] = rng.integers(-127, 128, (4, 64, 16))
    ops[:, 1] = rng.integers(0, 3, (4, 64, 16))
    return ops


@pytest.mark.parametrize("iters,blocks", [(1, 1), (9, 3), (2048, 2)])
def test_probe_mfma_data_checksum(iters, blocks):
    # byte i of A lane l meets byte i of B lane l' exactly when the lanes
    # hold the same K half (l // 32 == l' // 32): the sum over all outputs
    # of A B is sum_k colsum_A[k] rowsum_B[k]
    print(f"probe_mfma_data iters={iters} blocks={blocks}", flush=True)
    ops = probe_operands(iters)
    sink, clocks = B.probe_mfma_data(iters, torch.from_numpy(ops.reshape(-1)).to("cuda"), blocks)
    torch.cuda.synchronize()
    o = ops.astype(np.int64)
    per_set = (o[:, 0].reshape(4, 2, 32, 16).sum(2) * o[:, 1].reshape(4, 2, 32, 16).sum(2)).sum()
    want = (4 * iters * per_set) % (1 << 32)
    per = sink.cpu().numpy().view(np.uint32).reshape(blocks, 256).astype(np.uint64).sum(1) % (1 << 32)
    assert (per == want).all()
    ck = clocks.cpu().numpy().reshape(blocks, 3)
    assert (ck[:, 0] > 0).all() and (ck[:, 2] >= ck[:, 1]).all()


def test_probe_mfma_blocks_fill_the_device():
    n = B.probe_mfma_blocks()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert n >= cus and n % cus == 0


@pytest.mark.parametrize("rounds,blocks", [(1, 1), (5, 3), (64, 256), (1000, 256)])
def test_probe_barrier_exchange(rounds, blocks):
    # every barrier completes (no give-up), the counter ends at rounds x
    # blocks, and every workgroup saw every other workgroup's word of every
    # round: its sum is the closed form
    cus = B.probe_compute_units()
    blocks = min(blocks, cus)
    print(f"probe_barrier rounds={rounds} blocks={blocks}", flush=True)
    state, sink = B.probe_barrier(rounds, blocks, spin_limit=1 << 20)
    torch.cuda.synchronize()
    st = state.cpu().numpy().view(np.uint32)
    assert int(st[1]) == 0, "a workgroup gave up waiting"
    assert int(st[0]) == rounds * blocks
    want = sum(r * blocks + i for r in range(rounds) for i in range(blocks)) % (1 << 32)
    per = sink.cpu().numpy().view(np.uint32).reshape(blocks, 256).astype(np.uint64).sum(1) % (1 << 32)
    assert (per == want).all()
