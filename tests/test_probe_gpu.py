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


def test_probe_mfma_blocks_fill_the_device():
    n = B.probe_mfma_blocks()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert n >= cus and n % cus == 0
