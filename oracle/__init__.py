"""numpy front end of the CPU oracle (oracle.c) -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark
may import this package.  It loads liboracle.so (built by oracle/build.py with
gcc) through ctypes and hands it numpy arrays.  It shares nothing with the HIP
library and never imports it.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_vp = ctypes.c_void_p


def lib():
    """Load liboracle.so, compiling it first if it is not there."""
    global _lib
    if _lib is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        L.oracle_absmean_scale.restype = _f32
        L.oracle_absmean_scale.argtypes = [_vp, _i64, _i64]
        L.oracle_ternarize.restype = None
        L.oracle_ternarize.argtypes = [_vp, _i64, _i64, _f32, _vp]
        L.oracle_packed_bytes.restype = _i64
        L.oracle_packed_bytes.argtypes = [_i64, _i64]
        L.oracle_pack.restype = None
        L.oracle_pack.argtypes = [_vp, _i64, _i64, _vp]
        L.oracle_unpack.restype = _i64
        L.oracle_unpack.argtypes = [_vp, _i64, _i64, _vp]
        L.oracle_packed5_bytes.restype = _i64
        L.oracle_packed5_bytes.argtypes = [_i64, _i64]
        L.oracle_pack5.restype = None
        L.oracle_pack5.argtypes = [_vp, _i64, _i64, _vp]
        L.oracle_unpack5.restype = _i64
        L.oracle_unpack5.argtypes = [_vp, _i64, _i64, _vp]
        L.oracle_matmul_packed5_rows.restype = None
        L.oracle_matmul_packed5_rows.argtypes = [_vp, _vp, _i64, _i64, _i64, _vp, _i64, _vp]
        L.oracle_quant_act.restype = None
        L.oracle_quant_act.argtypes = [_vp, _i64, _i64, _vp, _vp, _vp]
        L.oracle_relu2_gate_quant_act.restype = None
        L.oracle_relu2_gate_quant_act.argtypes = [_vp, _vp, _i64, _i64, _vp, _vp, _vp, _vp]
        L.oracle_rmsnorm_quant_act.restype = None
        L.oracle_rmsnorm_quant_act.argtypes = [_vp, _i64, _i64, _vp, _f32, _vp, _vp, _vp, _vp, _vp]
        L.oracle_add_rmsnorm_quant_act.restype = None
        L.oracle_add_rmsnorm_quant_act.argtypes = [_vp, _vp, _i64, _i64, _vp, _f32, _vp, _vp, _vp, _vp, _vp, _vp]
        for name in ("oracle_matmul", "oracle_matmul_addsub"):
            f = getattr(L, name)
            f.restype = None
            f.argtypes = [_vp, _vp, _i64, _i64, _i64, _vp]
        L.oracle_matmul_packed_rows.restype = None
        L.oracle_matmul_packed_rows.argtypes = [_vp, _vp, _i64, _i64, _i64, _vp, _i64, _vp]
        L.oracle_epilogue.restype = None
        L.oracle_epilogue.argtypes = [_vp, _i64, _i64, _f32, _vp, _vp]
        L.oracle_epilogue_f64.restype = None
        L.oracle_epilogue_f64.argtypes = [_vp, _i64, _i64, _f32, _vp, _vp]
        L.oracle_threads.restype = ctypes.c_int
        L.oracle_threads.argtypes = []
        L.oracle_forward_packed.restype = _i64
        L.oracle_forward_packed.argtypes = [_vp, _i64, _i64, _vp, _f32, _i64, _vp,
                                            _vp, _vp, _vp, _vp, _vp]
        _lib = L
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def absmean_scale(W):
    """fp32 per-tensor absmean scale of an N x K fp32 matrix."""
    W = _c(W, np.float32)
    N, K = W.shape
    return float(np.float32(lib().oracle_absmean_scale(_p(W), N, K)))


def ternarize(W, gamma):
    W = _c(W, np.float32)
    N, K = W.shape
    T = np.empty((N, K), np.int8)
    lib().oracle_ternarize(_p(W), N, K, float(np.float32(gamma)), _p(T))
    return T


def quantize_weights(W, gamma_in=None):
    """(T, gamma): ternary codes and the fp32 scale used to make them."""
    gamma = absmean_scale(W) if gamma_in is None else float(np.float32(gamma_in))
    return ternarize(W, gamma), gamma


def packed_bytes(N, K):
    return int(lib().oracle_packed_bytes(N, K))


def pack(T):
    T = _c(T, np.int8)
    N, K = T.shape
    P = np.empty(packed_bytes(N, K), np.uint8)
    lib().oracle_pack(_p(T), N, K, _p(P))
    return P


def unpack(P, N, K):
    """(T, bad): decoded N x K codes and the count of malformed fields."""
    P = _c(P, np.uint8)
    if P.size != packed_bytes(N, K):
        raise ValueError("packed buffer has the wrong size")
    T = np.empty((N, K), np.int8)
    bad = lib().oracle_unpack(_p(P), N, K, _p(T))
    return T, int(bad)


def packed5_bytes(N, K):
    return int(lib().oracle_packed5_bytes(N, K))


def pack5(T):
    """BT5-T32 bytes of the N x K codes T (five codes per byte, base 3)."""
    T = _c(T, np.int8)
    N, K = T.shape
    P = np.empty(packed5_bytes(N, K), np.uint8)
    lib().oracle_pack5(_p(T), N, K, _p(P))
    return P


def unpack5(P, N, K):
    """(T, bad): decoded N x K codes and the count of malformed bytes/padding."""
    P = _c(P, np.uint8)
    if P.size != packed5_bytes(N, K):
        raise ValueError("packed buffer has the wrong size")
    T = np.empty((N, K), np.int8)
    bad = lib().oracle_unpack5(_p(P), N, K, _p(T))
    return T, int(bad)


def matmul_packed5_rows(Q, P, N, K, rows):
    """acc[:, i] for output row rows[i], read straight from a BT5-T32 buffer."""
    Q = _c(Q, np.int8)
    P = _c(P, np.uint8)
    rows = _c(rows, np.int64)
    M = Q.shape[0]
    assert Q.shape[1] == K and P.size == packed5_bytes(N, K)
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < N)
    acc = np.empty((M, rows.size), np.int32)
    lib().oracle_matmul_packed5_rows(_p(Q), _p(P), M, N, K, _p(rows), rows.size, _p(acc))
    return acc


def quant_act(X):
    """(Q int8 M x K, absmax fp32 [M], rowsum int32 [M])."""
    X = _c(X, np.float32)
    M, K = X.shape
    Q = np.empty((M, K), np.int8)
    a = np.empty(M, np.float32)
    rs = np.empty(M, np.int32)
    lib().oracle_quant_act(_p(X), M, K, _p(Q), _p(a), _p(rs))
    return Q, a, rs


def rmsnorm_quant_act(X, g=None, eps=1e-5):
    """RMSNorm (gain g, all ones when None) then the absmax int8 cast:
    (Q int8 M x K, absmax fp32 [M], rowsum int32 [M], Xn fp32 M x K,
    inv fp32 [M])."""
    X = _c(X, np.float32)
    M, K = X.shape
    gp = None if g is None else _c(g, np.float32)
    Q = np.empty((M, K), np.int8)
    a = np.empty(M, np.float32)
    rs = np.empty(M, np.int32)
    Xn = np.empty((M, K), np.float32)
    inv = np.empty(M, np.float32)
    lib().oracle_rmsnorm_quant_act(_p(X), M, K, None if gp is None else _p(gp), eps, _p(Xn),
                                   _p(inv), _p(Q), _p(a), _p(rs))
    return Q, a, rs, Xn, inv


def add_rmsnorm_quant_act(X, R, g=None, eps=1e-5):
    """S = X + R (fp32), then rmsnorm_quant_act on S:
    (Q, absmax, rowsum, S, Xn, inv)."""
    X = _c(X, np.float32)
    R = _c(R, np.float32)
    M, K = X.shape
    assert R.shape == X.shape
    gp = None if g is None else _c(g, np.float32)
    Q = np.empty((M, K), np.int8)
    a = np.empty(M, np.float32)
    rs = np.empty(M, np.int32)
    S = np.empty((M, K), np.float32)
    Xn = np.empty((M, K), np.float32)
    inv = np.empty(M, np.float32)
    lib().oracle_add_rmsnorm_quant_act(_p(X), _p(R), M, K, None if gp is None else _p(gp), eps, _p(S),
                                       _p(Xn), _p(inv), _p(Q), _p(a), _p(rs))
    return Q, a, rs, S, Xn, inv


def relu2_gate_quant_act(G, U):
    """Gated squared-ReLU h = relu(G)^2 * U, then the absmax int8 cast:
    (Q int8 M x N, absmax fp32 [M], rowsum int32 [M], H fp32 M x N)."""
    G = _c(G, np.float32)
    U = _c(U, np.float32)
    assert G.shape == U.shape
    M, N = G.shape
    Q = np.empty((M, N), np.int8)
    a = np.empty(M, np.float32)
    rs = np.empty(M, np.int32)
    H = np.empty((M, N), np.float32)
    lib().oracle_relu2_gate_quant_act(_p(G), _p(U), M, N, _p(H), _p(Q), _p(a), _p(rs))
    return Q, a, rs, H


def matmul(Q, T):
    Q = _c(Q, np.int8)
    T = _c(T, np.int8)
    M, K = Q.shape
    N = T.shape[0]
    assert T.shape[1] == K
    acc = np.empty((M, N), np.int32)
    lib().oracle_matmul(_p(Q), _p(T), M, N, K, _p(acc))
    return acc


def matmul_addsub(Q, T):
    Q = _c(Q, np.int8)
    T = _c(T, np.int8)
    M, K = Q.shape
    N = T.shape[0]
    assert T.shape[1] == K
    acc = np.empty((M, N), np.int32)
    lib().oracle_matmul_addsub(_p(Q), _p(T), M, N, K, _p(acc))
    return acc


def matmul_packed_rows(Q, P, N, K, rows):
    """acc[:, i] for output row rows[i], read straight from the packed buffer."""
    Q = _c(Q, np.int8)
    P = _c(P, np.uint8)
    rows = _c(rows, np.int64)
    M = Q.shape[0]
    assert Q.shape[1] == K and P.size == packed_bytes(N, K)
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < N)
    acc = np.empty((M, rows.size), np.int32)
    lib().oracle_matmul_packed_rows(_p(Q), _p(P), M, N, K, _p(rows), rows.size, _p(acc))
    return acc


def epilogue(acc, gamma, absmax):
    acc = _c(acc, np.int32)
    absmax = _c(absmax, np.float32)
    M, N = acc.shape
    Y = np.empty((M, N), np.float32)
    lib().oracle_epilogue(_p(acc), M, N, float(np.float32(gamma)), _p(absmax), _p(Y))
    return Y


def epilogue_f64(acc, gamma, absmax):
    acc = _c(acc, np.int32)
    absmax = _c(absmax, np.float32)
    M, N = acc.shape
    Y = np.empty((M, N), np.float64)
    lib().oracle_epilogue_f64(_p(acc), M, N, float(np.float32(gamma)), _p(absmax), _p(Y))
    return Y


def forward(X, T, gamma):
    """Whole layer from fp32 X and ternary codes: dict of every intermediate."""
    Q, a, rs = quant_act(X)
    acc = matmul(Q, T)
    Y = epilogue(acc, gamma, a)
    return {"Q": Q, "absmax": a, "rowsum": rs, "acc": acc, "Y": Y,
            "Y64": epilogue_f64(acc, gamma, a)}


def threads() -> int:
    """Threads the oracle's OpenMP loops use (OMP_NUM_THREADS, else every
    core)."""
    return int(lib().oracle_threads())


def forward_packed(X, P, gamma, N):
    """Whole layer from fp32 X and the packed buffer (unpack, quantize,
    contract, rescale) -- the form the CPU baseline times."""
    X = _c(X, np.float32)
    P = _c(P, np.uint8)
    M, K = X.shape
    Y = np.empty((M, N), np.float32)
    Q = np.empty((M, K), np.int8)
    a = np.empty(M, np.float32)
    rs = np.empty(M, np.int32)
    T = np.empty((N, K), np.int8)
    acc = np.empty((M, N), np.int32)
    bad = lib().oracle_forward_packed(_p(X), M, K, _p(P), float(np.float32(gamma)), N,
                                      _p(Y), _p(Q), _p(a), _p(rs), _p(T), _p(acc))
    if bad:
        raise ValueError(f"packed buffer holds {bad} malformed fields")
    return Y, acc
