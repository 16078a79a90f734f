"""C-ABI checks that need no GPU: the library loads, exports every function
include/bitlinear.h and include/bitlinear_probe.h declare, sizes its buffers
as documented, and rejects
bad arguments before touching the HIP runtime (nothing is enqueued, so these
calls never reach a device)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

import ternary_weight_w1_amd as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("bitlinear.h", "bitlinear_probe.h")]

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH),
                                reason="libbitlinear.so not built (run __graft_entry__.build())")

FAKE = 1 << 40  # a 16-byte aligned address that is never dereferenced


def _declared():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(bitlinear_\w+)\s*\(", src))
    return sorted(names)


def test_every_header_is_checked():
    inc = sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))
    assert inc == sorted(os.path.basename(h) for h in HEADERS)


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) == 41, names
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (bitlinear_\w+)", out))
    assert set(names) <= exported, set(names) - exported
    L = B.lib()
    for n in names:
        assert hasattr(L, n)


def test_no_oracle_in_product():
    # the product library never links or names the oracle
    out = subprocess.run(["nm", "-D", B.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in out
    ldd = subprocess.run(["ldd", B.LIB_PATH], capture_output=True, text=True).stdout
    assert "oracle" not in ldd


def test_version_and_strings():
    L = B.lib()
    assert L.bitlinear_abi_version() == 2
    for st in range(-6, 1):
        assert L.bitlinear_strerror(st)
    assert L.bitlinear_strerror(-99) == b"unknown status"


@pytest.mark.parametrize("N,K", [(1, 1), (64, 64), (65, 129), (2560, 2560), (6912, 2560),
                                 (28672, 8192)])
def test_packed_bytes_matches_oracle(N, K):
    import oracle
    assert B.packed_bytes(N, K) == oracle.packed_bytes(N, K)


def test_size_helpers_reject_bad_sizes():
    assert B.packed_bytes(0, 64) == 0
    assert B.packed_bytes(64, 131073) == 0
    assert B.q_stride(100) == 128 and B.q_stride(128) == 128 and B.q_stride(0) == 0
    smax = ctypes.c_size_t(-1).value
    assert B.workspace_bytes(B.WS_FORWARD, 0, 64, 64) == smax
    assert B.workspace_bytes(99, 1, 64, 64) == smax
    # forward workspace holds at least Q, absmax and the row sums
    assert B.workspace_bytes(B.WS_FORWARD, 4, 256, 256) >= 4 * 256 + 8
    # a matmul without K splits needs no workspace: the tile kernel on enough
    # work items (M = 2048: 32 x 40 = 1280, the split target is 1024) ...
    assert B.workspace_bytes(B.WS_MATMUL, 2048, 10240, 2560) == 0
    # ... while 80 items (M = 512, N = 2560) split K in two: 64 KiB of int32
    # partials per item and split, one 4-byte ticket per item (256-aligned)
    assert B.workspace_bytes(B.WS_MATMUL, 512, 2560, 2560) == 2 * 80 * 65536 + 512


def _st(f, *args):
    L = B.lib()
    st = getattr(L, f)(*args)
    return st, L.bitlinear_last_error().decode()


def test_quantize_weights_validation():
    st, msg = _st("bitlinear_quantize_weights", None, 4, 4, None, FAKE, FAKE, FAKE, 1 << 20, None)
    assert st == -1 and "required" in msg
    assert _st("bitlinear_quantize_weights", FAKE, 0, 4, None, FAKE, FAKE, FAKE, 1 << 20, None)[0] == -2
    assert _st("bitlinear_quantize_weights", FAKE, 4, 131073, None, FAKE, FAKE, FAKE, 1 << 20, None)[0] == -2
    assert _st("bitlinear_quantize_weights", FAKE + 4, 4, 4, None, FAKE, FAKE, FAKE, 1 << 20, None)[0] == -3
    assert _st("bitlinear_quantize_weights", FAKE, 4, 4, None, FAKE, FAKE, None, 0, None)[0] == -4
    assert _st("bitlinear_quantize_weights", FAKE, 4, 4, None, FAKE, FAKE, FAKE, 4, None)[0] == -4


def test_pack_quant_matmul_forward_validation():
    assert _st("bitlinear_pack", None, 4, 4, FAKE, None)[0] == -1
    assert _st("bitlinear_pack", FAKE, 4, -1, FAKE, None)[0] == -2
    assert _st("bitlinear_pack", FAKE, 4, 4, FAKE + 8, None)[0] == -3
    assert _st("bitlinear_unpack", FAKE, 4, 4, None, None)[0] == -1
    assert _st("bitlinear_quant_act", FAKE, 2, 100, FAKE, 96, FAKE, FAKE, None)[0] == -2  # ldq < K
    assert _st("bitlinear_quant_act", FAKE, 2, 100, FAKE, 104, FAKE, FAKE, None)[0] == -2  # ldq % 16
    assert _st("bitlinear_quant_act", FAKE, 0, 100, FAKE, 112, FAKE, FAKE, None)[0] == -2
    assert _st("bitlinear_quant_act", FAKE, 2, 100, FAKE + 1, 112, FAKE, FAKE, None)[0] == -3
    # RMSNorm + cast: same checks, plus eps and the gain alignment
    L = B.lib()
    q = L.bitlinear_quant_act_rmsnorm
    assert q(None, 2, 100, None, 1e-5, FAKE, 112, FAKE, FAKE, None) == -1
    assert q(FAKE, 2, 100, None, 1e-5, FAKE, 96, FAKE, FAKE, None) == -2
    assert q(FAKE, 2, 100, None, -1.0, FAKE, 112, FAKE, FAKE, None) == -6
    assert q(FAKE, 2, 100, None, float("nan"), FAKE, 112, FAKE, FAKE, None) == -6
    assert q(FAKE, 2, 100, FAKE + 2, 1e-5, FAKE, 112, FAKE, FAKE, None) == -3
    # residual add + RMSNorm + cast: the sum may be written over X or R only
    ad = L.bitlinear_quant_act_add_rmsnorm
    assert ad(FAKE, None, 2, 100, None, 1e-5, FAKE, FAKE, 112, FAKE, FAKE, None) == -1
    assert ad(FAKE, FAKE + 4096, 2, 100, None, 1e-5, FAKE + 8192, FAKE + 12288, 104, FAKE, FAKE, None) == -2
    assert ad(FAKE, FAKE + 4096, 2, 100, None, -1.0, FAKE + 8192, FAKE + 12288, 112, FAKE, FAKE, None) == -6
    assert ad(FAKE, FAKE + 4096, 2, 100, None, 1e-5, FAKE + 8200, FAKE + 12288, 112, FAKE, FAKE, None) == -3
    assert ad(FAKE, FAKE + 4096, 2, 100, None, 1e-5, FAKE + 16, FAKE + 12288, 112, FAKE, FAKE, None) == -6
    assert ad(FAKE, FAKE + 4096, 2, 100, None, 1e-5, FAKE + 8192, FAKE + 8192, 112, FAKE, FAKE, None) == -6
    # gated squared-ReLU + cast
    r = L.bitlinear_quant_act_relu2_gate
    assert r(FAKE, None, 2, 100, FAKE, 112, FAKE, FAKE, None) == -1
    assert r(FAKE, FAKE, 2, 0, FAKE, 112, FAKE, FAKE, None) == -2
    assert r(FAKE, FAKE, 2, 100, FAKE, 104, FAKE, FAKE, None) == -2
    assert r(FAKE, FAKE + 4, 2, 100, FAKE, 112, FAKE, FAKE, None) == -3
    # matmul: ldq must cover K rounded up to 64, and stay within 2^26
    assert _st("bitlinear_matmul", FAKE, 112, FAKE, FAKE, 2, 100, FAKE, FAKE, 64, FAKE, None,
               None, 0, None)[0] == -2
    assert _st("bitlinear_matmul", FAKE, (1 << 26) + 16, FAKE, FAKE, 2, 100, FAKE, FAKE, 64, FAKE, None,
               None, 0, None)[0] == -2
    assert _st("bitlinear_matmul", None, 128, FAKE, FAKE, 2, 100, FAKE, FAKE, 64, FAKE, None,
               None, 0, None)[0] == -1
    # forward needs a workspace
    assert _st("bitlinear_forward", FAKE, 1, 64, FAKE, FAKE, 64, FAKE, None, None, 0, None)[0] == -4
    assert _st("bitlinear_forward", FAKE, 1, 64, FAKE, FAKE, 64, FAKE + 4, None, FAKE, 1 << 20,
               None)[0] == -3
    # one token, one row tile: a wide workgroup (8 waves x 12 units) covers
    # K = 6144 without a split and needs no workspace; longer K is split
    assert B.workspace_bytes(B.WS_MATMUL, 1, 64, 6144) == 0
    assert B.workspace_bytes(B.WS_MATMUL, 1, 64, 6145) > 0
    # 2..16 tokens: a split holds at most what 64 KiB of staged activations
    # take (80 bytes per token per unit): 50 units at 16 tokens; at 8 tokens
    # the 96 units eight waves hold
    assert B.workspace_bytes(B.WS_MATMUL, 16, 64, 3200) == 0
    assert B.workspace_bytes(B.WS_MATMUL, 16, 64, 3264) > 0
    assert B.workspace_bytes(B.WS_MATMUL, 8, 64, 96 * 64) == 0
    assert B.workspace_bytes(B.WS_MATMUL, 8, 64, 97 * 64) > 0
    need = B.workspace_bytes(B.WS_MATMUL, 1, 64, 16384)
    assert need > 0
    assert _st("bitlinear_matmul", FAKE, 16384, FAKE, FAKE, 1, 16384, FAKE, FAKE, 64, FAKE, None,
               FAKE, need - 1, None)[0] == -4


def _problems(specs, fmt=0):
    arr = (B.Problem * len(specs))()
    for i, (M, N, K) in enumerate(specs):
        arr[i] = B.Problem(FAKE, FAKE, FAKE, FAKE, None, M, N, K, fmt, 0)
    return arr


def test_group_plan_table_on_host():
    L = B.lib()
    specs = [(1, 2560, 2560), (1, 640, 2560), (1, 6912, 2560), (1, 2560, 6912)]
    arr = _problems(specs)
    tb = L.bitlinear_group_table_bytes(arr, len(specs))
    wsb = L.bitlinear_group_workspace_bytes(arr, len(specs))
    assert tb > 0 and wsb > 0
    host = np.zeros(tb, np.uint8)
    st = L.bitlinear_group_plan(arr, len(specs), FAKE, wsb, host.ctypes.data, tb)
    assert st == 0, L.bitlinear_last_error()
    hdr = np.frombuffer(host[:48].tobytes(), np.int32)
    assert hdr[0] == np.int32(np.uint32(0xB17E0002).astype(np.int32))
    assert hdr[1] == 4            # problems
    assert hdr[2] == 4            # tokens quantized by the quantization kernel
    items = sum((N + 63) // 64 for _, N, _ in specs)
    assert hdr[3] >= items        # streaming work items (K splits may add more)
    assert hdr[4] == 0            # no tile-kernel items at M = 1
    # workspace too small -> rejected, nothing written
    host2 = np.zeros(tb, np.uint8)
    assert L.bitlinear_group_plan(arr, len(specs), FAKE, wsb - 1, host2.ctypes.data, tb) == -4
    assert not host2.any()
    # a bad problem anywhere rejects the whole plan
    bad = _problems(specs + [(1, 0, 64)])
    assert L.bitlinear_group_table_bytes(bad, 5) == 0
    assert L.bitlinear_group_plan(bad, 5, FAKE, wsb, host.ctypes.data, tb) == -2


def _plan_tables(specs):
    """Host plan table of `specs`: (header ints, header offsets, problem
    fields by name, map entries of each kernel as (problem, local) pairs)."""
    L = B.lib()
    arr = _problems(specs)
    tb = L.bitlinear_group_table_bytes(arr, len(specs))
    wsb = L.bitlinear_group_workspace_bytes(arr, len(specs))
    host = np.zeros(tb, np.uint8)
    assert L.bitlinear_group_plan(arr, len(specs), FAKE, wsb, host.ctypes.data, tb) == 0, L.bitlinear_last_error()
    hdr = np.frombuffer(host[:48].tobytes(), np.int32)
    off = np.frombuffer(host[48:104].tobytes(), np.int64)  # ws_bytes, probs, tok, stream, tile, bt5, total
    # Problem: ten pointers and ldq (88 bytes), then int32 fields from M on
    names = ["M", "N", "K", "KU", "NT", "ks", "upsplit", "kind", "mtile", "qtiled", "mt", "ntt"]
    size = 160
    probs = []
    for i in range(len(specs)):
        f = np.frombuffer(host[off[1] + i * size + 88: off[1] + i * size + 88 + 4 * len(names)].tobytes(), np.int32)
        probs.append(dict(zip(names, (int(v) for v in f))))
    maps = {}
    for key, n, o in (("stream", hdr[3], off[3]), ("tile", hdr[4], off[4])):
        maps[key] = np.frombuffer(host[o: o + 8 * n].tobytes(), np.uint32).reshape(-1, 2)
    return hdr, off, probs, maps


def _slices(entries):
    """The eight XCD slices of a map: workgroup b runs on XCD b % 8 and takes
    logical item (b % 8) * per + b / 8, so slice x is entries x, x + 8, ..."""
    return [entries[x::8] for x in range(8)]


def test_group_plan_item_order():
    # streaming items run longest first within each XCD slice (a slice must
    # not end on its long down projections); the tile kernel keeps problem
    # order, so consecutive items share activation and weight tiles
    specs = [(1, 2560, 2560), (1, 2560, 6912), (1, 6912, 2560), (1, 2560, 2560), (1, 640, 13824)] * 3
    _, _, probs, maps = _plan_tables(specs)
    st = maps["stream"]
    assert all(p["kind"] == 0 for p in probs) and len(st) > 0 and len(st) % 8 == 0

    def units(e):
        p = probs[e[0]]
        split = int(e[1]) % p["ks"]
        return min(p["KU"], (split + 1) * p["upsplit"]) - split * p["upsplit"]
    lengths = set()
    for sl in _slices(st):
        u = [units(e) for e in sl if e[0] != 0xFFFFFFFF]
        lengths |= set(u)
        assert u == sorted(u, reverse=True), u
        idle = [e[0] == 0xFFFFFFFF for e in sl]
        assert idle == sorted(idle)  # idle entries only at a slice's end
    assert len(lengths) > 1  # the case mixes item lengths
    # every item of every problem appears exactly once
    seen = sorted((int(a), int(b)) for a, b in st if a != 0xFFFFFFFF)
    want = sorted((i, j) for i, p in enumerate(probs) if p["kind"] == 0
                  for j in range((p["ntt"] if p["ntt"] > 0 else p["NT"]) * p["ks"]))
    assert seen == want

    tspecs = [(512, 2560, 2560), (512, 6912, 2560), (512, 2560, 6912)] * 2
    _, _, tprobs, tmaps = _plan_tables(tspecs)
    tl = tmaps["tile"]
    assert all(p["kind"] == 1 for p in tprobs) and len(tl) > 0 and len(tl) % 8 == 0
    per = len(tl) // 8
    logical = [tl[8 * j + x] for x in range(8) for j in range(per)]
    order = [(int(a), int(b)) for a, b in logical if a != 0xFFFFFFFF]
    assert order == sorted(order)  # problem order, then local item order


def test_group_plan_single_token_quantization():
    # 16 single-token problems with 64 row tiles each (no K split): every
    # token goes to the quantization kernel and the dot4 kernel reads LDS-
    # staged activations (3); a 2-token problem switches the streaming kernel to the two-slot dot4
    # token-loop kernel (6), whose LDS holds 64 bytes per unit for one-token
    # problems and 128 for two-token ones; a 5-token problem switches it to
    # the MFMA stream with activations staged in LDS (80 bytes per token per
    # unit, one tile per wave; 11, held to four waves per SIMD, while four
    # workgroups' staging fits a compute unit's LDS, else 10)
    L = B.lib()
    specs = [(1, 4096, 256)] * 16
    arr = _problems(specs)
    tb = L.bitlinear_group_table_bytes(arr, 16)
    host = np.zeros(tb, np.uint8)
    wsb = L.bitlinear_group_workspace_bytes(arr, 16)
    assert L.bitlinear_group_plan(arr, 16, FAKE, wsb, host.ctypes.data, tb) == 0
    hdr = np.frombuffer(host[:48].tobytes(), np.int32)
    assert hdr[3] == 16 * 64
    assert (hdr[2], hdr[7]) == (16, 3)
    arr2 = _problems(specs + [(2, 64, 64)])
    tb2 = L.bitlinear_group_table_bytes(arr2, 17)
    host2 = np.zeros(tb2, np.uint8)
    wsb2 = L.bitlinear_group_workspace_bytes(arr2, 17)
    assert L.bitlinear_group_plan(arr2, 17, FAKE, wsb2, host2.ctypes.data, tb2) == 0
    hdr2 = np.frombuffer(host2[:48].tobytes(), np.int32)
    assert hdr2[2] == 18 and hdr2[7] == 6
    assert hdr2[9] == max(64 * 4, 128 * 1)  # K = 256: 4 units; K = 64: 1 unit
    arr3 = _problems(specs + [(5, 64, 64)])
    tb3 = L.bitlinear_group_table_bytes(arr3, 17)
    host3 = np.zeros(tb3, np.uint8)
    wsb3 = L.bitlinear_group_workspace_bytes(arr3, 17)
    assert L.bitlinear_group_plan(arr3, 17, FAKE, wsb3, host3.ctypes.data, tb3) == 0
    hdr3 = np.frombuffer(host3[:48].tobytes(), np.int32)
    assert hdr3[2] == 21 and hdr3[7] == 11 and hdr3[9] == max(80 * 1 * 4, 80 * 5 * 1)
    # a one-token problem whose K range (1250 units) would need more than
    # 64 KiB of staged activations is split in two (625 units, 40000 bytes),
    # so a 2-token launch still takes the token loop (6)
    arr4 = _problems(specs + [(1, 64, 80000), (2, 64, 64)])
    tb4 = L.bitlinear_group_table_bytes(arr4, 18)
    host4 = np.zeros(tb4, np.uint8)
    wsb4 = L.bitlinear_group_workspace_bytes(arr4, 18)
    assert L.bitlinear_group_plan(arr4, 18, FAKE, wsb4, host4.ctypes.data, tb4) == 0
    hdr4 = np.frombuffer(host4[:48].tobytes(), np.int32)
    assert hdr4[7] == 6 and hdr4[9] == 64 * 625
    # a launch whose eight-tile groups fill the split target keeps two tiles
    # per wave (1) above 16 tokens: 130 problems of 64 tiles at M = 17; at
    # M = 5 the staged-activation stream takes one tile per wave (11)
    arr5 = _problems([(5, 4096, 256)] * 130)
    tb5 = L.bitlinear_group_table_bytes(arr5, 130)
    host5 = np.zeros(tb5, np.uint8)
    wsb5 = L.bitlinear_group_workspace_bytes(arr5, 130)
    assert L.bitlinear_group_plan(arr5, 130, FAKE, wsb5, host5.ctypes.data, tb5) == 0
    hdr5 = np.frombuffer(host5[:48].tobytes(), np.int32)
    assert hdr5[7] == 11 and hdr5[3] == 130 * 16
    # 16 tokens over K = 2560 stage 40 units x 16 x 80 = 51200 bytes per
    # workgroup (120 problems of 10 tile groups: enough work items that K is
    # not split): more than a quarter of the LDS, so three waves per SIMD (10)
    arr7 = _problems([(16, 2560, 2560)] * 120)
    tb7 = L.bitlinear_group_table_bytes(arr7, 120)
    host7 = np.zeros(tb7, np.uint8)
    wsb7 = L.bitlinear_group_workspace_bytes(arr7, 120)
    assert L.bitlinear_group_plan(arr7, 120, FAKE, wsb7, host7.ctypes.data, tb7) == 0
    hdr7 = np.frombuffer(host7[:48].tobytes(), np.int32)
    assert hdr7[7] == 10 and hdr7[9] == 80 * 16 * 40
    # the same at 8 tokens stages 25600 bytes: four per compute unit fit (11)
    arr8 = _problems([(8, 2560, 2560)] * 120)
    tb8 = L.bitlinear_group_table_bytes(arr8, 120)
    host8 = np.zeros(tb8, np.uint8)
    wsb8 = L.bitlinear_group_workspace_bytes(arr8, 120)
    assert L.bitlinear_group_plan(arr8, 120, FAKE, wsb8, host8.ctypes.data, tb8) == 0
    hdr8 = np.frombuffer(host8[:48].tobytes(), np.int32)
    assert hdr8[7] == 11 and hdr8[9] == 80 * 8 * 40
    arr6 = _problems([(17, 4096, 256)] * 130)
    tb6 = L.bitlinear_group_table_bytes(arr6, 130)
    host6 = np.zeros(tb6, np.uint8)
    wsb6 = L.bitlinear_group_workspace_bytes(arr6, 130)
    assert L.bitlinear_group_plan(arr6, 130, FAKE, wsb6, host6.ctypes.data, tb6) == 0
    hdr6 = np.frombuffer(host6[:48].tobytes(), np.int32)
    assert hdr6[7] == 1 and hdr6[3] == 130 * 8


def test_group_calls_reject_foreign_tables():
    L = B.lib()
    junk = np.zeros(256, np.uint8)
    assert L.bitlinear_group_forward(junk.ctypes.data, FAKE, None) == -6
    assert L.bitlinear_group_matmul(None, FAKE, None) == -1


# ----------------------------------------------------- BT5-T32 (five per byte) --

@pytest.mark.parametrize("N,K", [(1, 1), (32, 160), (33, 161), (2560, 2560), (2560, 6912),
                                 (28672, 8192)])
def test_packed5_bytes_matches_oracle(N, K):
    import oracle
    assert B.packed5_bytes(N, K) == oracle.packed5_bytes(N, K)


def test_bt5_size_helpers():
    assert B.packed5_bytes(0, 160) == 0 and B.packed5_bytes(32, 131073) == 0
    assert B.q_stride5(100) == 160 and B.q_stride5(161) == 320 and B.q_stride5(0) == 0
    smax = ctypes.c_size_t(-1).value
    assert B.workspace_bytes(B.WS_FORWARD5, 0, 64, 64) == smax
    assert B.workspace_bytes(6, 1, 64, 64) == smax
    # forward5 holds Q at stride q_stride5(K), absmax and row sums
    assert B.workspace_bytes(B.WS_FORWARD5, 4, 256, 256) >= 4 * 320 + 8
    # many row tiles: no K split, no matmul5 workspace; one tile, long K: split
    assert B.workspace_bytes(B.WS_MATMUL5, 1, 6912 * 40, 2560) == 0
    assert B.workspace_bytes(B.WS_MATMUL5, 1, 32, 8192) > 0


def test_bt5_validation():
    assert _st("bitlinear_pack5", None, 4, 4, FAKE, None)[0] == -1
    assert _st("bitlinear_pack5", FAKE, 4, 0, FAKE, None)[0] == -2
    assert _st("bitlinear_pack5", FAKE, 4, 4, FAKE + 8, None)[0] == -3
    assert _st("bitlinear_unpack5", FAKE, 4, 4, None, None)[0] == -1
    # matmul5: ldq must cover K rounded up to 160 (128 does not for K = 100)
    assert _st("bitlinear_matmul5", FAKE, 128, FAKE, FAKE, 2, 100, FAKE, FAKE, 64, FAKE, None,
               None, 0, None)[0] == -2
    assert _st("bitlinear_matmul5", FAKE, 168, FAKE, FAKE, 2, 100, FAKE, FAKE, 64, FAKE, None,
               None, 0, None)[0] == -2  # not a multiple of 16
    assert _st("bitlinear_matmul5", FAKE, 1 << 27, FAKE, FAKE, 2, 100, FAKE, FAKE, 64, FAKE,
               None, None, 0, None)[0] == -2
    assert _st("bitlinear_matmul5", None, 160, FAKE, FAKE, 2, 100, FAKE, FAKE, 64, FAKE, None,
               None, 0, None)[0] == -1
    assert _st("bitlinear_matmul5", FAKE, 160, FAKE, FAKE, 2, 100, FAKE + 4, FAKE, 64, FAKE,
               None, None, 0, None)[0] == -3
    need = B.workspace_bytes(B.WS_MATMUL5, 1, 32, 8192)
    assert _st("bitlinear_matmul5", FAKE, 8320, FAKE, FAKE, 1, 8192, FAKE, FAKE, 32, FAKE, None,
               FAKE, need - 1, None)[0] == -4
    assert _st("bitlinear_forward5", FAKE, 1, 64, FAKE, FAKE, 64, FAKE, None, None, 0, None)[0] == -4
    assert _st("bitlinear_forward5", FAKE, 1, 64, FAKE, FAKE, 0, FAKE, None, FAKE, 1 << 20,
               None)[0] == -2


def test_group_plan_bt5_items():
    # BT5 problems go to the BT5 kernel's own item map: (four 32-row tiles,
    # 16 tokens, K split) per item
    L = B.lib()
    specs = [(1, 2560, 2560), (1, 640, 2560), (1, 6912, 2560), (1, 2560, 6912)] * 30
    arr = _problems(specs, fmt=1)
    tb = L.bitlinear_group_table_bytes(arr, len(specs))
    wsb = L.bitlinear_group_workspace_bytes(arr, len(specs))
    host = np.zeros(tb, np.uint8)
    assert L.bitlinear_group_plan(arr, len(specs), FAKE, max(wsb, 16), host.ctypes.data, tb) == 0
    hdr = np.frombuffer(host[:48].tobytes(), np.int32)
    items = sum(((N + 31) // 32 + 3) // 4 for _, N, _ in specs)
    assert hdr[3] == 0 and hdr[4] == 0          # no 2-bit work
    assert hdr[10] >= items and hdr[10] % 8 == 0  # BT5 items, padded for the XCD order
    assert hdr[2] == len(specs)                  # every token quantized by the separate kernel
    # unknown format or a nonzero reserved field rejects the plan
    assert L.bitlinear_group_table_bytes(_problems([(1, 64, 64)], fmt=2), 1) == 0
    bad = _problems([(1, 64, 64)], fmt=1)
    bad[0].reserved = 1
    assert L.bitlinear_group_table_bytes(bad, 1) == 0


def _weights(Ns, fmt=0):
    arr = (B.Weight * len(Ns))()
    for i, N in enumerate(Ns):
        arr[i] = B.Weight(FAKE, FAKE, FAKE, None, N, fmt, 0)
    return arr


def test_matmul_multi_validation():
    L = B.lib()
    w = _weights([640, 640, 2560])
    smax = ctypes.c_size_t(-1).value
    assert L.bitlinear_multi_workspace_bytes(w, 3, 1, 2560) != smax
    assert L.bitlinear_multi_workspace_bytes(w, 0, 1, 2560) == smax
    assert L.bitlinear_multi_workspace_bytes(_weights([64] * 5), 5, 1, 64) == smax
    # one long-K small-N matrix splits K beyond what one wide workgroup
    # covers: counters and partials need workspace
    assert L.bitlinear_multi_workspace_bytes(_weights([64]), 1, 1, 6144) == 0
    assert L.bitlinear_multi_workspace_bytes(_weights([64]), 1, 1, 8192) > 0
    mm = L.bitlinear_matmul_multi
    assert mm(None, 2560, FAKE, FAKE, 1, 2560, w, 3, None, 0, None) == -1
    assert mm(FAKE, 2496, FAKE, FAKE, 1, 2560, w, 3, None, 0, None) == -2      # ldq < K
    assert mm(FAKE, 2560, FAKE, FAKE, 1, 2560, w, 5, None, 0, None) == -2      # count
    mixed = _weights([640, 640])
    mixed[1].format = 1
    assert mm(FAKE, 2560, FAKE, FAKE, 1, 2560, mixed, 2, None, 0, None) == -6
    bt5 = _weights([640], fmt=1)
    assert mm(FAKE, 2560, FAKE, FAKE, 1, 2561, bt5, 1, None, 0, None) == -2   # BT5 needs ldq >= 2720 (160-code units)
    need = L.bitlinear_multi_workspace_bytes(_weights([64]), 1, 1, 16384)
    assert mm(FAKE, 16384, FAKE, FAKE, 1, 16384, _weights([64]), 1, FAKE, need - 1, None) == -4


def test_cast_matmul_multi_validation():
    # every rejection happens on the host, before anything is enqueued
    L = B.lib()
    smax = ctypes.c_size_t(-1).value
    w = _weights([3200, 3200, 3200])
    # one token, 150 row tiles: the contraction casts its own input (no
    # workspace beyond the multi-matrix one); eight tokens cast into the
    # workspace first (Q, absmax and row sums on top)
    assert L.bitlinear_cast_multi_workspace_bytes(3, w, 3, 1, 3200) == L.bitlinear_multi_workspace_bytes(w, 3, 1, 3200)
    assert (L.bitlinear_cast_multi_workspace_bytes(3, w, 3, 8, 3200)
            >= L.bitlinear_multi_workspace_bytes(w, 3, 8, 3200) + 8 * 3200 + 64)
    # gate|up (270 row tiles) and the down projection after the gated
    # squared ReLU (more input bytes than weight bytes per workgroup) cast in
    # a launch of their own
    gu, down = _weights([8640, 8640]), _weights([3200])
    assert L.bitlinear_cast_multi_workspace_bytes(3, gu, 2, 1, 3200) > L.bitlinear_multi_workspace_bytes(gu, 2, 1, 3200)
    assert L.bitlinear_cast_multi_workspace_bytes(2, down, 1, 1, 8640) > L.bitlinear_multi_workspace_bytes(down, 1, 1, 8640)
    assert L.bitlinear_cast_multi_workspace_bytes(0, w, 0, 1, 3200) == smax
    assert L.bitlinear_cast_multi_workspace_bytes(4, w, 3, 1, 3200) == smax
    # the launch count follows the same rule
    n = L.bitlinear_cast_multi_launches
    assert (n(3, w, 3, 1, 3200), n(0, _weights([3200]), 1, 1, 3200), n(3, w, 3, 8, 3200)) == (1, 1, 2)
    assert (n(3, gu, 2, 1, 3200), n(2, down, 1, 1, 8640)) == (2, 2)
    assert (n(0, w, 0, 1, 3200), n(4, w, 3, 1, 3200), n(0, w, 3, 0, 3200)) == (-1, -1, -1)
    cm = L.bitlinear_cast_matmul_multi
    X, R, Xo = FAKE, FAKE + (1 << 20), FAKE + (2 << 20)
    assert cm(4, X, None, None, 0.0, None, 1, 3200, w, 3, None, 0, None) == -6            # mode
    assert cm(-1, X, None, None, 0.0, None, 1, 3200, w, 3, None, 0, None) == -6
    assert cm(0, None, None, None, 0.0, None, 1, 3200, w, 3, None, 0, None) == -1         # X
    assert cm(2, X, None, None, 0.0, None, 1, 3200, w, 3, None, 0, None) == -1            # gate needs U
    assert cm(3, X, None, None, 1e-5, Xo, 1, 3200, w, 3, None, 0, None) == -1             # add needs R
    assert cm(3, X, None, R, 1e-5, None, 1, 3200, w, 3, None, 0, None) == -1              # and X_out
    assert cm(1, X, None, None, -1.0, None, 1, 3200, w, 3, None, 0, None) == -6           # eps
    assert cm(1, X, None, None, float("nan"), None, 1, 3200, w, 3, None, 0, None) == -6
    assert cm(0, X + 4, None, None, 0.0, None, 1, 3200, w, 3, None, 0, None) == -3        # alignment
    assert cm(2, X, X + 8, None, 0.0, None, 1, 3200, w, 3, None, 0, None) == -3
    assert cm(3, X, None, R, 1e-5, X, 1, 3200, w, 3, None, 0, None) == -6                 # X_out = X
    assert cm(3, X, None, R, 1e-5, R + 16, 1, 3200, w, 3, None, 0, None) == -6            # overlaps R
    assert cm(0, X, None, None, 0.0, None, 0, 3200, w, 3, None, 0, None) == -2            # M
    assert cm(0, X, None, None, 0.0, None, 1, 3200, w, 5, None, 0, None) == -2            # count
    need = L.bitlinear_cast_multi_workspace_bytes(0, w, 3, 8, 3200)
    assert cm(0, X, None, None, 0.0, None, 8, 3200, w, 3, FAKE, need - 1, None) == -4     # workspace


# ---- calibration probes (include/bitlinear_probe.h): validation only


def test_probe_read_sink_words():
    L = B.lib()
    assert L.bitlinear_probe_read_sink_words(1 << 20, 65536) == 16 * 256
    assert L.bitlinear_probe_read_sink_words((1 << 20) + 16, 65536) == 17 * 256
    assert L.bitlinear_probe_read_sink_words(16, 4096) == 256
    for nbytes, chunk in [(0, 4096), (-16, 4096), (24, 4096), (4096, 0), (4096, 2048), (4096, 6000)]:
        assert L.bitlinear_probe_read_sink_words(nbytes, chunk) == 0, (nbytes, chunk)


def test_probe_read_rejects_bad_arguments():
    L = B.lib()
    assert L.bitlinear_probe_read(None, 4096, 4096, FAKE, None) == -1
    assert L.bitlinear_probe_read(FAKE, 4096, 4096, None, None) == -1
    assert L.bitlinear_probe_read(FAKE + 8, 4096, 4096, FAKE, None) == -3
    assert L.bitlinear_probe_read(FAKE, 4100, 4096, FAKE, None) == -2
    assert L.bitlinear_probe_read(FAKE, 4096, 1000, FAKE, None) == -2
    assert L.bitlinear_probe_read(FAKE, 0, 4096, FAKE, None) == -2


def test_probe_barrier_rejects_bad_arguments():
    L = B.lib()
    assert L.bitlinear_probe_barrier(10, 4, 100, None, FAKE, None) == -1
    assert L.bitlinear_probe_barrier(10, 4, 100, FAKE, None, None) == -1
    assert L.bitlinear_probe_barrier(10, 4, 100, FAKE + 2, FAKE, None) == -3
    assert L.bitlinear_probe_barrier(0, 4, 100, FAKE, FAKE, None) == -2
    assert L.bitlinear_probe_barrier(10, 4, 0, FAKE, FAKE, None) == -6


def test_probe_mfma_rejects_bad_arguments():
    L = B.lib()
    assert L.bitlinear_probe_mfma(10, 1, 1, 1, None, None) == -1
    assert L.bitlinear_probe_mfma(10, 128, 1, 1, FAKE, None) == -6
    assert L.bitlinear_probe_mfma(10, 1, -129, 1, FAKE, None) == -6
    assert L.bitlinear_probe_mfma(0, 1, 1, 1, FAKE, None) == -2
    assert L.bitlinear_probe_mfma(10, 1, 1, 0, FAKE, None) == -2
    # 2048 |a b| iters must stay below 2^31: 2048 * 127 * 128 * 65 = 2,164,260,864
    assert L.bitlinear_probe_mfma(65, 127, -128, 1, FAKE, None) == -2
    assert L.bitlinear_probe_mfma((1 << 20), 1, 1, 1, FAKE, None) == -2
    assert L.bitlinear_probe_mfma_blocks(None) == -1


def test_probe_mfma_data_rejects_bad_arguments():
    L = B.lib()
    assert L.bitlinear_probe_mfma_data(10, None, 1, FAKE, FAKE, None) == -1
    assert L.bitlinear_probe_mfma_data(10, FAKE, 1, None, FAKE, None) == -1
    assert L.bitlinear_probe_mfma_data(10, FAKE, 1, FAKE, None, None) == -1
    assert L.bitlinear_probe_mfma_data(10, FAKE + 4, 1, FAKE, FAKE, None) == -3
    assert L.bitlinear_probe_mfma_data(10, FAKE, 1, FAKE, FAKE + 4, None) == -3
    assert L.bitlinear_probe_mfma_data(0, FAKE, 1, FAKE, FAKE, None) == -2
    assert L.bitlinear_probe_mfma_data(10, FAKE, 0, FAKE, FAKE, None) == -2



def test_group_plan_tile_split():
    # tile-kernel problems (M > 32) in a launch with 7 work items, short of
    # the 1024-workgroup split target and at most 32 items: K splits up to
    # four ways keeping at least 16 units each -- 40 units in two (3 items ->
    # 6), 63 units in three (4 items -> 12): 18 items, padded to whole XCD
    # slices of 8 -- and the workspace holds 64 KiB of partials per item and
    # split; with enough items (1040) nothing splits
    L = B.lib()
    specs = [(64, 640, 2560), (100, 300, 4000)]
    arr = _problems(specs)
    tb = L.bitlinear_group_table_bytes(arr, 2)
    host = np.zeros(tb, np.uint8)
    wsb = L.bitlinear_group_workspace_bytes(arr, 2)
    assert L.bitlinear_group_plan(arr, 2, FAKE, wsb, host.ctypes.data, tb) == 0
    hdr = np.frombuffer(host[:48].tobytes(), np.int32)
    assert hdr[4] == 24
    assert wsb >= (3 * 2 + 4 * 3) * 65536
    big = _problems([(64, 4096 * 4, 2560)] * 65)  # 65 x 64 items of 256 rows
    tb2 = L.bitlinear_group_table_bytes(big, 65)
    host2 = np.zeros(tb2, np.uint8)
    wsb2 = L.bitlinear_group_workspace_bytes(big, 65)
    assert L.bitlinear_group_plan(big, 65, FAKE, wsb2, host2.ctypes.data, tb2) == 0
    hdr2 = np.frombuffer(host2[:48].tobytes(), np.int32)
    assert hdr2[4] == 65 * 64


def test_noalloc_forward_rejects_before_touching_the_device():
    # the no-allocation forward validates first: bad pointers and sizes whose
    # workspace exceeds the library's 16 MiB scratch array are refused before
    # any HIP call (FAKE addresses are never dereferenced)
    L = B.lib()
    assert L.bitlinear_noalloc_scratch_bytes() == 16 << 20
    assert L.bitlinear_forward_noalloc(None, 1, 64, FAKE, FAKE, 64, FAKE, None, None) == -1
    assert L.bitlinear_forward_noalloc(FAKE, 0, 64, FAKE, FAKE, 64, FAKE, None, None) == -2
    assert L.bitlinear_forward_noalloc(FAKE + 4, 1, 64, FAKE, FAKE, 64, FAKE, None, None) == -3
    M, N, K = 4096, 2560, 2560
    assert L.bitlinear_workspace_bytes(3, M, N, K) > 16 << 20
    assert L.bitlinear_forward_noalloc(FAKE, M, K, FAKE, FAKE, N, FAKE, None, None) == -4
    assert b"scratch" in L.bitlinear_last_error()
