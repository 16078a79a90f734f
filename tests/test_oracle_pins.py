"""Pins of the CPU oracle to things other than itself (closed forms, hand-
derived fixtures, library routines, brute force, statistics with known
expectations).  CPU only.

Pages cited (title, section):
  [AN] anthology note-168 on arXiv 2402.17764 (dmarx.github.io)
  [YT] BitNet b1.58 2B4T video transcript (yousumm.com), "Transcription"
  [PI] "BitNet: Microsoft's AI Revolution Shows Why Precision May be
       Overrated" (promptinjection.net)
"""
import math
import os
import subprocess
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import synth
from fp_exact import fl32, fp32_margin, inv_rms_exact, rint_half_even, rms_fp64_error_bound

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


# ---------------------------------------------------------------- helpers --

def _golden(name):
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


def _frac_round_half_even(x: Fraction) -> int:
    fl = math.floor(x)
    rem = x - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def _exact_ternary(w: float, gamma: float) -> int:
    """Nearest of {-1, 0, +1} to w/gamma in exact arithmetic, ties to 0."""
    r = Fraction(w) / Fraction(gamma)
    best = None
    for v in (0, 1, -1):  # 0 first: it wins every tie it takes part in
        d = abs(r - v)
        if best is None or d < best[0]:
            best = (d, v)
    return best[1]


# ------------------------------------------------------- P-A closed forms --

def test_bits_per_weight_is_log2_3():
    # [YT] prints 1.58496 bits per weight; [AN] "What it does" prints 1.58.
    # Three equiprobable codes carry -sum p log2 p = log2 3 bits.
    h = -sum((1 / 3) * math.log2(1 / 3) for _ in range(3))
    assert round(h, 5) == 1.58496
    assert round(h, 2) == 1.58


@pytest.mark.parametrize("N,K", [(64, 64), (256, 256), (2560, 2560), (640, 2560), (2560, 6912)])
def test_packed_size_is_two_bits_per_weight(N, K):
    # Four codes per byte ([YT]); with N and K multiples of 64 there is no
    # padding, so the buffer is exactly N*K/4 bytes = 2 bits per weight.
    assert O.packed_bytes(N, K) * 8 == 2 * N * K
    assert abs(2 / math.log2(3) - 1.2619) < 1e-4  # storage overhead vs log2 3


def test_packed_size_of_2b_stack():
    # A 2B-class model's BitLinear weights (30 layers of q,k,v,o,gate,up,down)
    # hold 2.084e9 weights: 0.521 GB at 2 bits, 0.413 GB at log2(3) bits --
    # the ~0.4 GB the pages quote ([YT]; [PI] "3. Benchmarks") is the log2(3)
    # figure, which a 2-bit layout cannot reach.
    n_weights = 30 * sum(K * N for _, K, N in synth.SHAPES_2B)
    assert n_weights == 2_084_044_800
    total = 30 * sum(O.packed_bytes(N, K) for _, K, N in synth.SHAPES_2B)
    assert total == n_weights // 4 == 521_011_200
    assert abs(n_weights * math.log2(3) / 8 / 1e9 - 0.4129) < 1e-3


def test_padding_rounds_up_to_64():
    assert O.packed_bytes(1, 1) == 1024
    assert O.packed_bytes(65, 64) == 2048
    assert O.packed_bytes(130, 200) == 3 * 4 * 1024
    assert O.packed_bytes(0, 64) == 0


# ------------------------------------------------- P-B format and invariants --

def test_pack_golden_single_codes():
    rows = [ln.split() for ln in _golden("bl2_t64_fixtures.txt") if ln.startswith("single")]
    assert len(rows) == 7
    for _, N, K, n, k, code, byte_idx, byte_hex in rows:
        N, K, n, k, code, byte_idx = map(int, (N, K, n, k, code, byte_idx))
        T = np.zeros((N, K), np.int8)
        T[n, k] = code
        P = O.pack(T)
        expect = np.full(O.packed_bytes(N, K), 0x55, np.uint8)
        expect[byte_idx] = int(byte_hex, 16)
        np.testing.assert_array_equal(P, expect)
        T2, bad = O.unpack(P, N, K)
        assert bad == 0
        np.testing.assert_array_equal(T2, T)


def test_pack_golden_word():
    rows = [ln.split() for ln in _golden("bl2_t64_fixtures.txt") if ln.startswith("word")]
    assert len(rows) == 1
    _, N, K, n, codes, first, bytes_hex = rows[0]
    N, K, n, first = map(int, (N, K, n, first))
    codes = [int(c) for c in codes.split(",")]
    T = np.zeros((N, K), np.int8)
    T[n, :16] = codes
    P = O.pack(T)
    want = [int(b, 16) for b in bytes_hex.split(",")]
    assert list(P[first:first + 4]) == want
    word = int.from_bytes(bytes(P[first:first + 4]), "little")
    # each plane j of the word yields the fields of codes 4j..4j+3 in byte order
    for j in range(4):
        plane = (word >> (2 * j)) & 0x03030303
        fields = [(plane >> (8 * b)) & 0xFF for b in range(4)]
        assert fields == [c + 1 for c in codes[4 * j:4 * j + 4]]


def test_zero_matrix_packs_to_0x55():
    P = O.pack(np.zeros((100, 130), np.int8))
    assert P.size == O.packed_bytes(100, 130)
    assert np.all(P == 0x55)


@pytest.mark.parametrize("N,K", [(1, 1), (3, 17), (64, 64), (65, 129), (130, 200), (200, 640)])
def test_pack_roundtrip_and_fields(N, K):
    T = synth.random_ternary(N, K, seed=N * 1000 + K)
    P = O.pack(T)
    fields = np.stack([(P >> s) & 3 for s in (0, 2, 4, 6)])
    assert not np.any(fields == 3)  # 0b11 is never written
    T2, bad = O.unpack(P, N, K)
    assert bad == 0
    np.testing.assert_array_equal(T2, T)
    # number of nonzero fields == number of nonzero codes (zero survives)
    assert int(np.sum(fields != 1)) == int(np.count_nonzero(T))


def test_unpack_reports_malformed_fields():
    P = O.pack(np.zeros((64, 64), np.int8))
    P[7] = 0xFF  # four fields of value 3
    _, bad = O.unpack(P, 64, 64)
    assert bad == 4
    P = O.pack(np.zeros((3, 10), np.int8))
    P[-1] = 0x00  # padding region no longer zero codes
    _, bad = O.unpack(P, 3, 10)
    assert bad == 4


# ------------------------------------------- BT5-T32 (five codes per byte) --

def _bt5_value(codes):
    """Stored byte of five codes, digit 0 most significant (the format's
    definition, evaluated with exact rationals)."""
    b = 0
    for c in codes:
        b = 3 * b + (c + 1)
    return math.ceil(Fraction(256 * b, 243))


def test_bt5_golden_bytes():
    rows = [ln.split() for ln in _golden("bt5_t32_fixtures.txt") if ln.startswith("byte")]
    assert len(rows) == 7
    for _, codes, value in rows:
        codes = [int(c) for c in codes.split(",")]
        T = np.zeros((1, 160), np.int8)
        for i, c in enumerate(codes):
            T[0, 32 * i] = c  # digit i of byte 0 (g = 0, p = 0)
        P = O.pack5(T)
        assert P[0] == int(value, 16)
        assert _bt5_value(codes) == int(value, 16)


def test_bt5_golden_single_codes():
    rows = [ln.split() for ln in _golden("bt5_t32_fixtures.txt") if ln.startswith("single")]
    assert len(rows) == 7
    for _, N, K, n, k, code, byte_idx, byte_hex in rows:
        N, K, n, k, code, byte_idx = map(int, (N, K, n, k, code, byte_idx))
        T = np.zeros((N, K), np.int8)
        T[n, k] = code
        P = O.pack5(T)
        expect = np.full(O.packed5_bytes(N, K), 0x80, np.uint8)
        expect[byte_idx] = int(byte_hex, 16)
        np.testing.assert_array_equal(P, expect)
        T2, bad = O.unpack5(P, N, K)
        assert bad == 0
        np.testing.assert_array_equal(T2, T)


def test_bt5_all_243_byte_values():
    # every five-code combination: distinct stored bytes, increasing with the
    # base-3 value b, and b = floor(243 s / 256) recovers it
    import itertools
    seen = []
    for b, codes in enumerate(itertools.product((-1, 0, 1), repeat=5)):
        s = _bt5_value(codes)
        assert 0 <= s <= 255
        assert (243 * s) // 256 == b
        seen.append(s)
    assert seen == sorted(seen) and len(set(seen)) == 243
    # the same through the oracle, 243 combinations in the 16 x 2 bytes x 8 rows
    T = np.zeros((8, 160), np.int8)
    combos = list(itertools.product((-1, 0, 1), repeat=5))
    for j, codes in enumerate(combos):
        n, g, pp = j // 32, (j % 32) // 16, j % 16
        for i, c in enumerate(codes):
            T[n, 32 * i + 16 * g + pp] = c
    P = O.pack5(T)
    got = [P[16 * (j // 32 + 32 * ((j % 32) // 16)) + j % 16] for j in range(243)]
    assert got == seen


def test_bt5_prefix_digits_by_multiply_shift():
    # The format's reason for storing ceil(256 b / 243): floor(s * 3^j / 256)
    # is the integer formed by the top j base-3 digits of b, exactly, for
    # every byte and j = 0..5 (243 < 256 keeps the rounding error below one
    # digit).
    for b in range(243):
        s = math.ceil(Fraction(256 * b, 243))
        for j in range(6):
            assert (s * 3 ** j) >> 8 == b // 3 ** (5 - j)


def test_bt5_size_is_1_6_bits_and_2b_stack_is_0_4_gb():
    # 32 | N and 160 | K: no padding, 8 bits per 5 codes
    for N, K in ((32, 160), (2560, 2560), (6912, 2560)):
        assert O.packed5_bytes(N, K) * 8 * 5 == 8 * N * K
    # [YT] "Transcription": about 0.4 GB for the 2B model; the 6912-wide down
    # projection pads K to 7040
    total = 30 * sum(O.packed5_bytes(N, K) for _, K, N in synth.SHAPES_2B)
    assert total == 418_775_040
    assert 0.40 < total / 1e9 < 0.42


@pytest.mark.parametrize("N,K", [(1, 1), (32, 160), (33, 161), (37, 333), (64, 320), (70, 2560)])
def test_bt5_roundtrip(N, K):
    T = synth.random_ternary(N, K, seed=N * 7 + K)
    P = O.pack5(T)
    assert P.size == O.packed5_bytes(N, K)
    T2, bad = O.unpack5(P, N, K)
    assert bad == 0
    np.testing.assert_array_equal(T2, T)
    # only the 243 images occur
    allowed = {math.ceil(Fraction(256 * b, 243)) for b in range(243)}
    assert set(np.unique(P).tolist()) <= allowed


def test_bt5_unpack_reports_malformed():
    P = O.pack5(np.zeros((32, 160), np.int8))
    P[3] = 1  # no five codes map to 1 (b = 0 -> 0, b = 1 -> 2)
    _, bad = O.unpack5(P, 32, 160)
    assert bad == 1
    P = O.pack5(np.zeros((3, 10), np.int8))
    P[-1] = 0xFF  # a padding byte holding five +1 codes
    _, bad = O.unpack5(P, 3, 10)
    assert bad == 5


@pytest.mark.parametrize("M,N,K", [(1, 33, 161), (3, 40, 480), (5, 64, 1000)])
def test_bt5_packed_rows_matmul(M, N, K):
    T = synth.random_ternary(N, K, seed=M + 3 * N + K)
    Q = synth.random_int8(M, K, seed=M * N + 1)
    P = O.pack5(T)
    rows = np.array([0, N // 2, N - 1], np.int64)
    got = O.matmul_packed5_rows(Q, P, N, K, rows)
    want = Q.astype(np.int64) @ T[rows].astype(np.int64).T  # numpy integer product
    np.testing.assert_array_equal(got, want)


def test_bt5_prefix_plane_identity():
    # The contraction over one byte's five codes written with the prefix
    # integers H_j = floor(s 3^j / 256) (j = 1..5) and the digits d_i = code_i
    # + 1: sum_i d_i q_i = sum_{j=1..3} H_j (q_{j-1} - 3 q_j) + H_4 q_3
    # + (H_5 - 3 H_4) q_4.  Checked for every byte against random activations.
    rng = np.random.default_rng(5)
    import itertools
    for codes in itertools.product((-1, 0, 1), repeat=5):
        s = _bt5_value(codes)
        H = [(s * 3 ** j) >> 8 for j in range(6)]
        d = [c + 1 for c in codes]
        for q in rng.integers(-127, 128, size=(4, 5)):
            lhs = sum(d[i] * int(q[i]) for i in range(5))
            rhs = sum(H[j] * (int(q[j - 1]) - 3 * int(q[j])) for j in (1, 2, 3))
            rhs += H[4] * int(q[3]) + (H[5] - 3 * H[4]) * int(q[4])
            assert lhs == rhs
            assert 0 <= H[5] - 3 * H[4] <= 2 and max(H[1:5]) <= 80


def test_ternary_codes_only_in_set():
    # [AN] "What it does": weights in {-1, 0, +1}; zero is a real state.
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((300, 200)) * rng.choice([1e-3, 1.0, 50.0], (300, 1))).astype(np.float32)
    T, g = O.quantize_weights(W)
    assert set(np.unique(T)).issubset({-1, 0, 1})
    assert np.any(T == 0) and np.any(T == 1) and np.any(T == -1)


# ------------------------------------------------- quantizer fixtures/ties --

def test_weight_quantizer_golden_ties():
    rows = {ln.split()[1]: ln.split()[2:] for ln in _golden("quant_fixtures.txt")
            if ln.startswith("weights")}
    W = np.array([float(v) for v in rows["W"]], np.float32).reshape(4, 4)
    gamma = O.absmean_scale(W)
    assert gamma == float(rows["gamma"][0])
    T = O.ternarize(W, gamma)
    np.testing.assert_array_equal(T.ravel(), np.array([int(v) for v in rows["T"]], np.int8))


def test_weight_quantizer_is_nearest_code_with_ties_to_zero():
    # exact-arithmetic argmin over {-1,0,1}, ties to 0, on random values and
    # on constructed exact ties |w| = gamma/2 and |w| = 3*gamma/2
    rng = np.random.default_rng(11)
    gammas = np.float32(2.0) ** rng.integers(-12, 3, 64).astype(np.float32)
    for g in gammas:
        g = float(g)
        ws = list(rng.standard_normal(40).astype(np.float32) * np.float32(g))
        ws += [g / 2, -g / 2, 1.5 * g, -1.5 * g, g, -g, 0.0, -0.0, 3 * g, -3 * g]
        W = np.array(ws, np.float32).reshape(1, -1)
        T = O.ternarize(W, g)
        want = [_exact_ternary(float(w), g) for w in W.ravel()]
        assert list(T.ravel()) == want


def test_absmean_scale_matches_exact_mean():
    # gamma = mean |W| in exact arithmetic, rounded once to fp32
    rng = np.random.default_rng(3)
    for shape in [(4, 4), (7, 13), (64, 96)]:
        W = (rng.standard_normal(shape) * 0.02).astype(np.float32)
        exact = sum(Fraction(float(abs(w))) for w in W.ravel()) / W.size
        want = np.float32(float(exact))
        got = O.absmean_scale(W)
        # the fp64 running sum may differ from the exact mean in the last
        # fp64 bits; after rounding to fp32 the two agree to 1 ulp
        assert abs(got - float(want)) <= float(np.spacing(want))
        assert abs(got - float(exact)) / float(exact) < 1e-6
    assert O.absmean_scale(np.zeros((3, 5), np.float32)) == np.float32(1e-5)


def test_activation_quantizer_golden():
    acts = [ln for ln in _golden("quant_fixtures.txt") if ln.startswith("act ")]
    assert len(acts) == 4
    for ln in acts:
        x, q, tail = ln[4:].split("|")
        X = np.array([float(v) for v in x.split()], np.float32).reshape(1, -1)
        Q, a, rs = O.quant_act(X)
        assert list(Q.ravel()) == [int(v) for v in q.split()]
        amax, rsum = tail.split()
        assert a[0] == np.float32(float(amax))
        assert rs[0] == int(rsum)


def test_activation_quantizer_exact_rounding_power_of_two_scales():
    # with a = 127 * 2^e the multiplier 127/a = 2^-e is exact, so x*s is
    # exact and q must be the half-to-even rounding of the exact product
    rng = np.random.default_rng(17)
    for e in range(-6, 7):
        a = 127.0 * 2.0 ** e
        x = (rng.integers(-254, 255, 200) / 2.0 * 2.0 ** e).astype(np.float32)
        x[0] = a
        X = x.reshape(1, -1)
        Q, am, rs = O.quant_act(X)
        assert am[0] == np.float32(a)
        want = [max(-127, min(127, _frac_round_half_even(Fraction(float(v)) / Fraction(2.0 ** e))))
                for v in x]
        assert list(Q.ravel()) == want
        assert rs[0] == sum(want)


def test_epilogue_golden():
    for ln in (ln for ln in _golden("quant_fixtures.txt") if ln.startswith("epi ")):
        head, acc, y = ln[4:].split("|")
        gamma, amax = (float(v) for v in head.split())
        acc = np.array([int(v) for v in acc.split()], np.int32).reshape(1, -1)
        Y = O.epilogue(acc, gamma, np.array([amax], np.float32))
        np.testing.assert_array_equal(Y.ravel(), np.array([float(v) for v in y.split()], np.float32))


def test_activation_scale_order_fixture_discriminates():
    # R3 fixes the order s = fl(127/a), then q = rint(fl(x*s)); the pages fix
    # none.  The fixture row a = 19/16, x = a/2 makes the exact product the
    # tie 63.5: derived here in exact rationals with fp32 rounding modelled,
    # the stated order gives 63, both other orders 64.  A consistent swap of
    # the order in the oracle (and the kernels) fails this pin.
    line = [ln for ln in _golden("quant_fixtures.txt") if ln.startswith("act 1.1875")][0]
    x, q, _ = line[4:].split("|")
    xs = [Fraction(float(v)) for v in x.split()]
    a = max(abs(v) for v in xs)
    s = fl32(Fraction(127) / a)
    stated = [max(-127, min(127, rint_half_even(fl32(v * s)))) for v in xs]
    mul_first = [rint_half_even(fl32(fl32(v * 127) / a)) for v in xs]
    div_scale = [rint_half_even(fl32(v / fl32(a / 127))) for v in xs]
    assert stated == [int(v) for v in q.split()]
    assert stated[1] == 63 and mul_first[1] == 64 and div_scale[1] == 64
    assert stated[2] == -63 and mul_first[2] == -64 and div_scale[2] == -64
    Q, am, rs = O.quant_act(np.array([[float(v) for v in x.split()]], np.float32))
    assert list(Q.ravel()) == stated and rs[0] == sum(stated)


def test_epilogue_scale_order_fixture_discriminates():
    # R4 fixes c = fl(fl(gamma*a)/127), y = fl(float(acc)*c).  The fixture's
    # gamma = 3/256, a = 69/64 round the other two orders one ulp lower.
    line = [ln for ln in _golden("quant_fixtures.txt") if ln.startswith("epi 0.01171875")][0]
    head, acc, y = line[4:].split("|")
    g, a = (Fraction(float(v)) for v in head.split())
    accs = [int(v) for v in acc.split()]
    c = fl32(fl32(g * a) / 127)
    c_alt1 = fl32(g * fl32(a / 127))
    c_alt2 = fl32(fl32(g / 127) * a)
    assert c != c_alt1 and c != c_alt2
    stated = [fl32(v * c) for v in accs]
    assert stated == [Fraction(float(v)) for v in y.split()]
    assert all(fl32(v * c_alt1) != t for v, t in zip(accs, stated))
    Y = O.epilogue(np.array([accs], np.int32), float(g), np.array([float(a)], np.float32))
    assert [Fraction(float(v)) for v in Y.ravel()] == stated


# ------------------------------------------ P-C identity and library check --

@pytest.mark.parametrize("M,N,K", [(1, 7, 5), (4, 256, 256), (9, 65, 130)])
def test_matmul_identity_and_library(M, N, K):
    T = synth.random_ternary(N, K, seed=M + N + K)
    Q = synth.random_int8(M, K, seed=M * N)
    acc = O.matmul(Q, T)
    # [AN]: with ternary weights the product is additions and subtractions
    np.testing.assert_array_equal(acc, O.matmul_addsub(Q, T))
    # library routine, int64 so nothing can wrap
    np.testing.assert_array_equal(acc, Q.astype(np.int64) @ T.astype(np.int64).T)
    # straight from the packed buffer, every row
    P = O.pack(T)
    np.testing.assert_array_equal(O.matmul_packed_rows(Q, P, N, K, np.arange(N)), acc)


def test_matmul_catches_transposed_operand():
    # a non-symmetric case where Q @ T.T and Q @ T differ
    T = np.array([[1, 0], [0, 0]], np.int8)
    Q = np.array([[0, 5]], np.int8)
    acc = O.matmul(Q, T)
    assert acc.tolist() == [[0, 0]]
    T = np.array([[0, 1], [0, 0]], np.int8)
    assert O.matmul(Q, T).tolist() == [[5, 0]]


# ---------------------------------------------------- P-D brute force 4x4 --

def test_bruteforce_all_ternary_4x4_small_block():
    # all 81 ternary 1x4 rows against a set of int8 rows, in Python
    import itertools
    Q = np.array([[127, -127, 0, 1], [-1, 2, -3, 4], [100, -50, 25, -12]], np.int8)
    rows = np.array(list(itertools.product((-1, 0, 1), repeat=4)), np.int8)
    acc = O.matmul(Q, rows)
    for m in range(3):
        for n in range(81):
            assert acc[m, n] == sum(int(Q[m, k]) * int(rows[n, k]) for k in range(4))


@pytest.mark.slow
def test_bruteforce_all_3pow16_ternary_4x4(tmp_path):
    # every one of the 3^16 ternary 4x4 matrices, in C (about 20 s)
    O.lib()
    exe = tmp_path / "bruteforce_4x4"
    src = os.path.join(ROOT, "tests", "csrc", "bruteforce_4x4.c")
    odir = os.path.join(ROOT, "oracle")
    subprocess.run(["gcc", "-O2", "-o", str(exe), src, f"-L{odir}", "-loracle",
                    f"-Wl,-rpath,{odir}"], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout
    assert out.strip() == "ok 43046721"


# ------------------------------------------------------- P-E fixed points --

def test_fixed_points():
    rng = np.random.default_rng(23)
    # quantize(g0 * T) == T for a ternary T with at least one nonzero
    T = synth.random_ternary(37, 91, seed=4)
    for g0 in (0.02, 1.0, 3.5):
        W = (T.astype(np.float32) * np.float32(g0))
        T2, g = O.quantize_weights(W)
        np.testing.assert_array_equal(T2, T)
        assert g <= np.float32(g0) * (1 + 1e-6)
    # integer rows with max |x| = 127 quantize to themselves
    X = rng.integers(-127, 128, (5, 64)).astype(np.float32)
    X[:, 3] = 127
    Q, a, rs = O.quant_act(X)
    np.testing.assert_array_equal(Q, X.astype(np.int8))
    assert np.all(a == 127) and np.all(rs == X.sum(1))
    # T = I gives acc = Q; all +1 gives rowsum; all -1 gives -rowsum
    Qi = synth.random_int8(3, 50, seed=9)
    np.testing.assert_array_equal(O.matmul(Qi, np.eye(50, dtype=np.int8)), Qi.astype(np.int32))
    rsum = Qi.astype(np.int32).sum(1)
    np.testing.assert_array_equal(O.matmul(Qi, np.ones((4, 50), np.int8)), np.repeat(rsum[:, None], 4, 1))
    np.testing.assert_array_equal(O.matmul(Qi, -np.ones((4, 50), np.int8)), -np.repeat(rsum[:, None], 4, 1))


def test_all_zero_token_and_matrix():
    X = np.zeros((2, 64), np.float32)
    X[1] = 0.5
    W = np.zeros((8, 64), np.float32)
    T, g = O.quantize_weights(W)
    assert g == np.float32(1e-5) and not T.any()
    out = O.forward(X, T, g)
    assert out["absmax"][0] == np.float32(1e-5)
    assert not out["Q"][0].any() and not out["Y"].any()


# ------------------------------------------------ P-F / P-G statistics ------

def _p_zero_gaussian():
    # w ~ N(0, s^2): gamma = E|w| = s sqrt(2/pi); t = 0 iff |w| <= gamma/2
    return math.erf(0.5 * math.sqrt(2 / math.pi) / math.sqrt(2))


def test_zero_fraction_closed_form_config1():
    p0 = _p_zero_gaussian()
    assert abs(p0 - 0.31006) < 1e-5  # "about one-third zeros"
    W, _ = synth.config1()
    T, g = O.quantize_weights(W)
    n = T.size
    sd = math.sqrt(p0 * (1 - p0) / n)
    frac0 = np.mean(T == 0)
    assert abs(frac0 - p0) < 5 * sd
    # the +1 and -1 halves are symmetric
    assert abs(np.mean(T == 1) - np.mean(T == -1)) < 5 * math.sqrt(0.5 / n)


@pytest.mark.slow
def test_zero_fraction_closed_form_2560():
    p0 = _p_zero_gaussian()
    W = synth.weights_np(2560, 2560, 0.02, seed=1000)
    T, g = O.quantize_weights(W)
    sd = math.sqrt(p0 * (1 - p0) / T.size)
    assert abs(np.mean(T == 0) - p0) < 5 * sd
    assert abs(g - 0.02 * math.sqrt(2 / math.pi)) / g < 2e-3


def test_output_cosine_closed_form():
    # weight-level correlation of t with w for Gaussian w:
    # 2 phi(a) / sqrt(1 - p0) with a = sqrt(2/pi)/2  (= 0.8871)
    a = 0.5 * math.sqrt(2 / math.pi)
    rho = 2 * math.exp(-a * a / 2) / math.sqrt(2 * math.pi) / math.sqrt(1 - _p_zero_gaussian())
    assert abs(rho - 0.8871) < 1e-4
    W = synth.weights_np(1024, 1024, 0.02, seed=77)
    X = synth.activations_np(16, 1024, seed=78)
    T, g = O.quantize_weights(W)
    Y = O.forward(X, T, g)["Y"].astype(np.float64)
    Yr = X.astype(np.float64) @ W.astype(np.float64).T
    cos = np.sum(Y * Yr) / math.sqrt(np.sum(Y * Y) * np.sum(Yr * Yr))
    assert abs(cos - rho) < 0.03
    # the scale is pinned too, not only the direction.  Regressing the real
    # output on the quantized one gives E[t w] / (gamma E[t^2])
    # = 2 phi(a) / (sqrt(2/pi) (1 - p0)) = 1.3385 for Gaussian w: absmean is
    # not the least-squares scale, and a lost or doubled factor shows here.
    gain_cf = 2 * math.exp(-a * a / 2) / math.sqrt(2 * math.pi) / (
        math.sqrt(2 / math.pi) * (1 - _p_zero_gaussian()))
    assert abs(gain_cf - 1.3385) < 1e-3
    gain = np.sum(Y * Yr) / np.sum(Y * Y)
    assert abs(gain - gain_cf) < 0.03


# ---------------------------------------------------- P-H bounds -------------

def test_bounds_and_fp64_reference():
    W, X = synth.config1()
    T, g = O.quantize_weights(W)
    out = O.forward(X, T, g)
    K = X.shape[1]
    assert np.all(np.abs(out["acc"]) <= 127 * K)
    y, y64 = out["Y"].astype(np.float64), out["Y64"]
    nz = y64 != 0
    assert np.all(np.abs(y[nz] - y64[nz]) <= 1e-5 * np.abs(y64[nz]))
    assert np.all(y[~nz] == 0)
    # and acc == 0 gives exactly 0
    assert np.all(out["Y"][out["acc"] == 0] == 0)


# ------------------------------------------------ P-I per-token outliers -----

def test_outlier_channels_raise_only_their_token_scale():
    K = 2560
    X = synth.activations_np(64, K, seed=5, outlier_frac=0.01)
    Xc = synth.activations_np(64, K, seed=5)
    Q, a, _ = O.quant_act(X)
    Qc, ac, _ = O.quant_act(Xc)
    ch = synth.outlier_channels(K, 5)
    assert ch.size == 26
    assert np.all(a > 4 * ac)           # the scale follows the outliers
    assert 30 < np.median(a) < 60       # ~20 x the max of ~26 |N(0,1)| draws
    # zero fraction of ordinary channels per token is 2 Phi(a/254) - 1
    mask = np.ones(K, bool)
    mask[ch] = False
    z = np.mean(Q[:, mask] == 0, axis=1)
    expect = np.array([math.erf((float(t) / 254) / math.sqrt(2)) for t in a])
    sd = np.sqrt(expect * (1 - expect) / mask.sum())
    assert np.all(np.abs(z - expect) < 5 * sd + 1e-3)
    assert 0.10 < float(np.mean(z)) < 0.20
    # one token's outlier scale does not touch another's: token-wise scales
    X2 = Xc.copy()
    X2[0, 0] = 1000.0
    Q2, a2, _ = O.quant_act(X2)
    np.testing.assert_array_equal(Q2[1:], Qc[1:])
    np.testing.assert_array_equal(a2[1:], ac[1:])


# ------------------------------------------ RMSNorm + int8 cast (NEXT-1) --

def _rms_fixtures():
    rows = []
    for line in _golden("rmsnorm_fixtures.txt"):
        if not line.strip() or line.startswith("#"):
            continue
        head, x, q, rs = [f.strip() for f in line.split("|")]
        K, eps, g = head.split()
        g = None if g == "1" else np.array([float(v) for v in g.split(",")], np.float32)
        rows.append((int(K), float(eps), g, np.array([float(v) for v in x.split(",")], np.float32),
                     np.array([int(v) for v in q.split(",")]), int(rs)))
    return rows


def test_rmsnorm_golden_fixtures():
    # hand-derived worked examples (tests/golden/rmsnorm_fixtures.txt)
    for K, eps, g, x, q, rs in _rms_fixtures():
        Q, a, r, Xn, inv = O.rmsnorm_quant_act(x[None, :], g, eps)
        np.testing.assert_array_equal(Q[0], q)
        assert r[0] == rs


def test_rmsnorm_matches_float64_definition():
    # x_hat against the definition evaluated in float64 (three fp32 roundings
    # separate them: inv, x*inv, *g), and the codes against the plain int8
    # cast of the oracle's own x_hat (the composition the reading states)
    rng = np.random.default_rng(11)
    for M, K, eps in [(3, 37, 1e-5), (4, 1000, 1e-5), (2, 4096, 1e-6), (2, 300, 10.0)]:
        X = (rng.standard_normal((M, K)) * rng.uniform(0.1, 10)).astype(np.float32)
        g = rng.standard_normal(K).astype(np.float32)
        Q, a, rs, Xn, inv = O.rmsnorm_quant_act(X, g, eps)
        x64 = X.astype(np.float64)
        want = x64 / np.sqrt((x64 * x64).mean(axis=1, keepdims=True) + eps) * g.astype(np.float64)
        rel = np.abs(Xn - want) / np.maximum(np.abs(want), 1e-30)
        assert rel.max() <= 4e-7, rel.max()
        inv64 = 1.0 / np.sqrt((x64 * x64).mean(axis=1) + eps)
        assert np.all(np.abs(inv - inv64) / inv64 <= 6e-8)
        Q2, a2, rs2 = O.quant_act(Xn)
        np.testing.assert_array_equal(Q, Q2)
        np.testing.assert_array_equal(a, a2)
        np.testing.assert_array_equal(rs, rs2)


def test_fp32_margin_helper():
    # the switch points of fp32 rounding around 1 are 1 - 2^-25 and 1 + 2^-24
    assert fp32_margin(Fraction(1)) == 2.0 ** -25
    assert fp32_margin(Fraction(1) + Fraction(1, 2 ** 24)) == 0.0
    assert fl32(Fraction(1) + Fraction(1, 2 ** 24)) == 1  # the tie goes to even
    assert inv_rms_exact([4.0], 0.0) == Fraction(1, 4)
    assert inv_rms_exact([3.0, 4.0], 0.0) ** 2 <= Fraction(2, 25) < (inv_rms_exact([3.0, 4.0], 0.0)
                                                                    + Fraction(1, 2 ** 100)) ** 2


def test_rmsnorm_factor_is_correctly_rounded_when_decided():
    # R13 computes inv in fp64 and rounds it to fp32 once.  Whenever the
    # exact factor sits farther from an fp32 switch point than fp64 can err,
    # any correct fp64 order -- the oracle's sequential sum, the kernel's
    # tree -- must give fl32(exact), which pins the oracle's factor to the
    # definition itself (a sum in fp32, eps outside the root, or a missing
    # 1/K fail here).  Rows too close to call are counted, not compared.
    rng = np.random.default_rng(23)
    checked = undecided = 0
    for K, eps in [(3, 1e-5), (37, 1e-5), (1000, 0.0), (4096, 1e-6), (300, 10.0)]:
        X = (rng.standard_normal((40, K)) * rng.uniform(0.01, 100)).astype(np.float32)
        _, _, _, _, inv = O.rmsnorm_quant_act(X, None, eps)
        bound = rms_fp64_error_bound(K) + 2.0 ** -60
        for m in range(X.shape[0]):
            exact = inv_rms_exact(X[m], eps)
            if fp32_margin(exact) <= bound:
                undecided += 1
                continue
            assert Fraction(float(inv[m])) == fl32(exact), (K, m)
            checked += 1
    assert checked >= 195 and undecided <= 5


def test_rmsnorm_power_of_two_invariance():
    # with eps = 0 RMSNorm is scale-free, and scaling x by 2^j is exact in
    # floating point at every step: identical x_hat and codes, inv scaled by
    # 2^-j exactly; scaling g by 2 doubles x_hat exactly and keeps the codes
    rng = np.random.default_rng(12)
    X = rng.standard_normal((6, 777)).astype(np.float32)
    g = rng.uniform(-2, 2, 777).astype(np.float32)
    Q, a, rs, Xn, inv = O.rmsnorm_quant_act(X, g, 0.0)
    for j in (-3, 5):
        Qj, aj, rsj, Xnj, invj = O.rmsnorm_quant_act(X * np.float32(2.0 ** j), g, 0.0)
        np.testing.assert_array_equal(Qj, Q)
        np.testing.assert_array_equal(Xnj, Xn)
        np.testing.assert_array_equal(invj, inv * np.float32(2.0 ** -j))
    Q2, a2, rs2, Xn2, _ = O.rmsnorm_quant_act(X, g * np.float32(2), 0.0)
    np.testing.assert_array_equal(Q2, Q)
    np.testing.assert_array_equal(Xn2, Xn * 2)
    np.testing.assert_array_equal(a2, a * 2)


def test_add_rmsnorm_residual_sum_and_reductions():
    # R17: the residual sum is one fp32 addition per element (numpy's IEEE
    # float32 add is the reference), and the cast is then exactly the RMSNorm
    # cast of that sum; R = 0 reduces to the plain RMSNorm cast, R = -X to an
    # all-zero row, and the hand fixture (3, 4) arrives as (1, 2) + (2, 2)
    rng = np.random.default_rng(17)
    for M, K in [(1, 5), (3, 37), (4, 2560)]:
        X = rng.standard_normal((M, K)).astype(np.float32) * 3
        R = rng.standard_normal((M, K)).astype(np.float32)
        g = (rng.random(K) + 0.5).astype(np.float32)
        Q, a, rs, S, Xn, inv = O.add_rmsnorm_quant_act(X, R, g, 1e-5)
        np.testing.assert_array_equal(S, np.add(X, R, dtype=np.float32))
        Q2, a2, rs2, Xn2, inv2 = O.rmsnorm_quant_act(np.add(X, R, dtype=np.float32), g, 1e-5)
        np.testing.assert_array_equal(Q, Q2)
        np.testing.assert_array_equal(a, a2)
        np.testing.assert_array_equal(rs, rs2)
        Q0, a0, rs0, S0, _, _ = O.add_rmsnorm_quant_act(X, np.zeros_like(X), g, 1e-5)
        Q1, a1, rs1, _, _ = O.rmsnorm_quant_act(X, g, 1e-5)
        np.testing.assert_array_equal(S0, X)
        np.testing.assert_array_equal(Q0, Q1)
        Qz, az, rsz, Sz, _, _ = O.add_rmsnorm_quant_act(X, -X, None, 1e-5)
        assert not Sz.any() and not Qz.any() and not rsz.any()
    Q, a, rs, S, _, _ = O.add_rmsnorm_quant_act(np.array([[1.0, 2.0]], np.float32),
                                                np.array([[2.0, 2.0]], np.float32), None, 0.0)
    assert S.tolist() == [[3.0, 4.0]] and Q[0].tolist() == [95, 127] and rs[0] == 222


def test_rmsnorm_special_cases():
    # no gain == unit gain; a zero row stays zero (inv = 1/sqrt(eps), codes 0,
    # absmax at its floor); a constant row normalizes to +-1 -> +-127
    rng = np.random.default_rng(13)
    X = rng.standard_normal((3, 64)).astype(np.float32)
    A = O.rmsnorm_quant_act(X, None, 1e-5)
    B = O.rmsnorm_quant_act(X, np.ones(64, np.float32), 1e-5)
    for u, v in zip(A, B):
        np.testing.assert_array_equal(u, v)
    Z = np.zeros((1, 64), np.float32)
    Q, a, rs, Xn, inv = O.rmsnorm_quant_act(Z, None, 1e-4)
    assert not Q.any() and a[0] == np.float32(1e-5) and rs[0] == 0
    assert inv[0] == np.float32(100.0)
    C = np.full((1, 64), -0.25, np.float32)
    C[0, 1::2] = 0.25
    Q, a, rs, Xn, inv = O.rmsnorm_quant_act(C, None, 0.0)
    np.testing.assert_array_equal(np.abs(Q), 127)
    assert rs[0] == 0


# ------------------------------- gated squared-ReLU + int8 cast (NEXT-2) --

def test_relu2_gate_hand_values():
    # h = relu(g)^2 * u by hand: g = (-2, 0, 0.5, 3), u = (5, 5, -4, 2)
    #   -> h = (0, 0, -1, 18); a = 18; q = rint(h * 127/18) = (0, 0, -7, 127)
    #   (-127/18 = -7.0555... -> -7); rowsum 120
    G = np.array([[-2, 0, 0.5, 3]], np.float32)
    U = np.array([[5, 5, -4, 2]], np.float32)
    Q, a, rs, H = O.relu2_gate_quant_act(G, U)
    np.testing.assert_array_equal(H[0], [0, 0, -1, 18])
    np.testing.assert_array_equal(Q[0], [0, 0, -7, 127])
    assert a[0] == 18 and rs[0] == 120


def test_relu2_gate_matches_float64_definition():
    # h against the definition in float64 (two fp32 roundings apart), and the
    # codes against the plain int8 cast of the oracle's own h
    rng = np.random.default_rng(21)
    for M, N in [(3, 37), (4, 6912), (2, 1000)]:
        G = (rng.standard_normal((M, N)) * 3).astype(np.float32)
        U = rng.standard_normal((M, N)).astype(np.float32)
        Q, a, rs, H = O.relu2_gate_quant_act(G, U)
        want = np.maximum(G.astype(np.float64), 0) ** 2 * U.astype(np.float64)
        nz = want != 0
        assert np.all(H[~nz] == 0)
        rel = np.abs(H[nz] - want[nz]) / np.abs(want[nz])
        assert rel.max() <= 2.5e-7, rel.max()
        Q2, a2, rs2 = O.quant_act(H)
        np.testing.assert_array_equal(Q, Q2)
        np.testing.assert_array_equal(rs, rs2)


def test_relu2_gate_special_cases():
    # gate <= 0 everywhere -> zero codes, absmax at its floor; gate = 1 -> the
    # plain cast of u; negating u negates h and the codes exactly
    rng = np.random.default_rng(22)
    U = rng.standard_normal((3, 500)).astype(np.float32)
    Q, a, rs, H = O.relu2_gate_quant_act(-np.abs(U), U)
    assert not Q.any() and np.all(a == np.float32(1e-5))
    Q, a, rs, H = O.relu2_gate_quant_act(np.ones_like(U), U)
    Q2, a2, rs2 = O.quant_act(U)
    np.testing.assert_array_equal(Q, Q2)
    np.testing.assert_array_equal(a, a2)
    G = rng.standard_normal((3, 500)).astype(np.float32)
    Qa, aa, rsa, Ha = O.relu2_gate_quant_act(G, U)
    Qb, ab, rsb, Hb = O.relu2_gate_quant_act(G, -U)
    np.testing.assert_array_equal(Qb, -Qa)
    np.testing.assert_array_equal(ab, aa)
    np.testing.assert_array_equal(rsb, -rsa)


def test_oracle_results_do_not_depend_on_thread_count(tmp_path):
    # the OpenMP pragmas only split independent outputs across threads: the
    # same inputs give the same bytes with one thread as with four (sizes
    # above the pragmas' thresholds, so every parallel loop runs parallel)
    import sys
    script = (
        "import numpy as np, sys; sys.path.insert(0, %r)\n"
        "import oracle as O, synth\n"
        "T = synth.random_ternary(1030, 1100, seed=5); X = synth.activations_np(1000, 1100, seed=6)\n"
        "Q, a, rs = O.quant_act(X); P = O.pack(T); T2, bad = O.unpack(P, 1030, 1100); assert bad == 0\n"
        "acc = O.matmul(Q[:9], T2); Y, _ = O.forward_packed(X[:9], P, 0.02, 1030)\n"
        "rows = np.array([0, 64, 1029]); ap = O.matmul_packed_rows(Q, P, 1030, 1100, rows)\n"
        "np.savez(sys.argv[1], Q=Q, a=a, rs=rs, T2=T2, acc=acc, Y=Y, ap=ap, n=O.threads())\n" % ROOT)
    outs = []
    for threads in ("1", "4"):
        f = tmp_path / f"t{threads}.npz"
        env = dict(os.environ, OMP_NUM_THREADS=threads)
        subprocess.run([sys.executable, "-c", script, str(f)], env=env, check=True)
        outs.append(np.load(f))
    assert int(outs[0]["n"]) == 1 and int(outs[1]["n"]) == 4
    for key in ("Q", "a", "rs", "T2", "acc", "Y", "ap"):
        np.testing.assert_array_equal(outs[0][key], outs[1][key], err_msg=key)
