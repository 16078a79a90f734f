"""Python binding of libbitlinear.so (include/bitlinear.h), the gfx950 HIP
BitLinear W1.58A8 library.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  torch supplies device memory and the current stream.  There is no
fallback: if the shared library is missing, importing works but the first
call raises.

Functions carry the C names without the ``bitlinear_`` prefix:
quantize_weights, pack, unpack, quant_act, matmul, forward, their BT5-T32
(five codes per byte) twins pack5, unpack5, matmul5, forward5, plus the
grouped forward (GroupPlan).
"""
from __future__ import annotations

import ctypes
import functools
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbitlinear.so")

OK = 0
WS_QUANTIZE_WEIGHTS = 1
WS_MATMUL = 2
WS_FORWARD = 3
WS_MATMUL5 = 4
WS_FORWARD5 = 5
FORMAT_BL2 = 0
FORMAT_BT5 = 1
CAST_PLAIN = 0
CAST_RMSNORM = 1
CAST_RELU2_GATE = 2
CAST_ADD_RMSNORM = 3

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_int = ctypes.c_int


class Weight(ctypes.Structure):
    """ctypes mirror of struct bitlinear_weight."""
    _fields_ = [("P", _vp), ("gamma", _vp), ("Y", _vp), ("acc", _vp), ("N", _i64),
                ("format", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class Problem(ctypes.Structure):
    """ctypes mirror of struct bitlinear_problem."""
    _fields_ = [("X", _vp), ("P", _vp), ("gamma", _vp), ("Y", _vp), ("acc", _vp),
                ("M", _i64), ("N", _i64), ("K", _i64), ("format", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded libbitlinear.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python ternary_weight_w1_amd/build.py` (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "bitlinear_abi_version": (_int, []),
            "bitlinear_strerror": (ctypes.c_char_p, [_int]),
            "bitlinear_last_error": (ctypes.c_char_p, []),
            "bitlinear_packed_bytes": (_sz, [_i64, _i64]),
            "bitlinear_q_stride": (_i64, [_i64]),
            "bitlinear_packed5_bytes": (_sz, [_i64, _i64]),
            "bitlinear_q_stride5": (_i64, [_i64]),
            "bitlinear_pack5": (_int, [_vp, _i64, _i64, _vp, _vp]),
            "bitlinear_unpack5": (_int, [_vp, _i64, _i64, _vp, _vp]),
            "bitlinear_matmul5": (_int, [_vp, _i64, _vp, _vp, _i64, _i64, _vp, _vp, _i64, _vp, _vp,
                                         _vp, _sz, _vp]),
            "bitlinear_forward5": (_int, [_vp, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
            "bitlinear_workspace_bytes": (_sz, [_int, _i64, _i64, _i64]),
            "bitlinear_quantize_weights": (_int, [_vp, _i64, _i64, _vp, _vp, _vp, _vp, _sz, _vp]),
            "bitlinear_pack": (_int, [_vp, _i64, _i64, _vp, _vp]),
            "bitlinear_unpack": (_int, [_vp, _i64, _i64, _vp, _vp]),
            "bitlinear_quant_act": (_int, [_vp, _i64, _i64, _vp, _i64, _vp, _vp, _vp]),
            "bitlinear_quant_act_rmsnorm": (_int, [_vp, _i64, _i64, _vp, ctypes.c_float, _vp, _i64, _vp,
                                                   _vp, _vp]),
            "bitlinear_quant_act_relu2_gate": (_int, [_vp, _vp, _i64, _i64, _vp, _i64, _vp, _vp, _vp]),
            "bitlinear_quant_act_add_rmsnorm": (_int, [_vp, _vp, _i64, _i64, _vp, ctypes.c_float, _vp, _vp,
                                                       _i64, _vp, _vp, _vp]),
            "bitlinear_matmul": (_int, [_vp, _i64, _vp, _vp, _i64, _i64, _vp, _vp, _i64, _vp, _vp,
                                        _vp, _sz, _vp]),
            "bitlinear_forward": (_int, [_vp, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _vp, _sz, _vp]),
            "bitlinear_forward_noalloc": (_int, [_vp, _i64, _i64, _vp, _vp, _i64, _vp, _vp, _vp]),
            "bitlinear_noalloc_scratch_bytes": (_sz, []),
            "bitlinear_multi_workspace_bytes": (_sz, [ctypes.POINTER(Weight), _int, _i64, _i64]),
            "bitlinear_matmul_multi": (_int, [_vp, _i64, _vp, _vp, _i64, _i64, ctypes.POINTER(Weight), _int,
                                              _vp, _sz, _vp]),
            "bitlinear_cast_multi_workspace_bytes": (_sz, [_int, ctypes.POINTER(Weight), _int, _i64, _i64]),
            "bitlinear_cast_multi_launches": (_int, [_int, ctypes.POINTER(Weight), _int, _i64, _i64]),
            "bitlinear_cast_matmul_multi": (_int, [_int, _vp, _vp, _vp, ctypes.c_float, _vp, _i64, _i64,
                                                   ctypes.POINTER(Weight), _int, _vp, _sz, _vp]),
            "bitlinear_group_table_bytes": (_sz, [ctypes.POINTER(Problem), _int]),
            "bitlinear_group_workspace_bytes": (_sz, [ctypes.POINTER(Problem), _int]),
            "bitlinear_group_plan": (_int, [ctypes.POINTER(Problem), _int, _vp, _sz, _vp, _sz]),
            "bitlinear_group_quant_act": (_int, [_vp, _vp, _vp]),
            "bitlinear_group_matmul": (_int, [_vp, _vp, _vp]),
            "bitlinear_group_forward": (_int, [_vp, _vp, _vp]),
            "bitlinear_probe_read_sink_words": (_i64, [_i64, _i64]),
            "bitlinear_probe_read": (_int, [_vp, _i64, _i64, _vp, _vp]),
            "bitlinear_probe_mfma": (_int, [_i64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _vp, _vp]),
            "bitlinear_probe_mfma_data": (_int, [_i64, _vp, ctypes.c_int32, _vp, _vp, _vp]),
            "bitlinear_probe_mfma_blocks": (_int, [ctypes.POINTER(ctypes.c_int32)]),
            "bitlinear_probe_barrier": (_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _vp, _vp, _vp]),
            "bitlinear_probe_compute_units": (_int, [ctypes.POINTER(ctypes.c_int32)]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int, what: str):
    if status != OK:
        L = lib()
        raise RuntimeError(f"{what}: {L.bitlinear_strerror(status).decode()} "
                           f"({L.bitlinear_last_error().decode()})")


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _torch_stream(stream):
    """The torch stream object a call enqueues on: the current stream for
    None, the object itself, or an ExternalStream around a raw hipStream_t."""
    if stream is None:
        return torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream))


def _on_stream(fn):
    """Run a call with its launch stream current, so that the outputs and
    temporary workspaces it allocates belong to that stream in torch's
    caching allocator: their memory is not handed to other streams' work
    while the library's kernels may still use it."""
    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kw):
        s = _torch_stream(stream)
        with torch.cuda.stream(s):
            return fn(*args, stream=s, **kw)
    return wrapper


def _ptr(t):
    return None if t is None else t.data_ptr()


def _dev_tensor(t, dtype, name):
    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == dtype and t.is_contiguous()):
        raise TypeError(f"{name} must be a contiguous {dtype} CUDA tensor")
    return t


def packed_bytes(N: int, K: int) -> int:
    return int(lib().bitlinear_packed_bytes(N, K))


def q_stride(K: int) -> int:
    return int(lib().bitlinear_q_stride(K))


def workspace_bytes(op: int, M: int, N: int, K: int) -> int:
    return int(lib().bitlinear_workspace_bytes(op, M, N, K))


def _workspace(nbytes, device):
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


@_on_stream
def quantize_weights(W, gamma_in=None, stream=None):
    """(T int8 N x K, gamma fp32 [1]) for fp32 N x K weights."""
    _dev_tensor(W, torch.float32, "W")
    N, K = W.shape
    T = torch.empty((N, K), dtype=torch.int8, device=W.device)
    gamma = torch.empty(1, dtype=torch.float32, device=W.device)
    ws = _workspace(workspace_bytes(WS_QUANTIZE_WEIGHTS, 0, N, K), W.device)
    _check(lib().bitlinear_quantize_weights(_ptr(W), N, K, _ptr(gamma_in), _ptr(T), _ptr(gamma),
                                            _ptr(ws), 0 if ws is None else ws.numel(),
                                            _stream(stream)), "quantize_weights")
    return T, gamma


@_on_stream
def pack(T, stream=None):
    """BL2-T64 packed bytes (uint8, packed_bytes(N, K)) of int8 codes."""
    _dev_tensor(T, torch.int8, "T")
    N, K = T.shape
    P = torch.empty(packed_bytes(N, K), dtype=torch.uint8, device=T.device)
    _check(lib().bitlinear_pack(_ptr(T), N, K, _ptr(P), _stream(stream)), "pack")
    return P


@_on_stream
def unpack(P, N: int, K: int, stream=None):
    _dev_tensor(P, torch.uint8, "P")
    T = torch.empty((N, K), dtype=torch.int8, device=P.device)
    _check(lib().bitlinear_unpack(_ptr(P), N, K, _ptr(T), _stream(stream)), "unpack")
    return T


@_on_stream
def quant_act(X, ldq: int | None = None, stream=None):
    """(Q int8 M x ldq, absmax fp32 [M], rowsum int32 [M]); ldq defaults to
    q_stride(K), the stride the matmul call accepts."""
    _dev_tensor(X, torch.float32, "X")
    M, K = X.shape
    ldq = q_stride(K) if ldq is None else ldq
    Q = torch.empty((M, ldq), dtype=torch.int8, device=X.device)
    a = torch.empty(M, dtype=torch.float32, device=X.device)
    rs = torch.empty(M, dtype=torch.int32, device=X.device)
    _check(lib().bitlinear_quant_act(_ptr(X), M, K, _ptr(Q), ldq, _ptr(a), _ptr(rs),
                                     _stream(stream)), "quant_act")
    return Q, a, rs


@_on_stream
def quant_act_rmsnorm(X, norm_weight=None, eps: float = 1e-5, ldq: int | None = None, stream=None):
    """RMSNorm (gain norm_weight, all ones when None) then the absmax int8
    cast: (Q int8 M x ldq, absmax fp32 [M] of the normalized rows, rowsum
    int32 [M])."""
    _dev_tensor(X, torch.float32, "X")
    if norm_weight is not None:
        _dev_tensor(norm_weight, torch.float32, "norm_weight")
    M, K = X.shape
    ldq = q_stride(K) if ldq is None else ldq
    Q = torch.empty((M, ldq), dtype=torch.int8, device=X.device)
    a = torch.empty(M, dtype=torch.float32, device=X.device)
    rs = torch.empty(M, dtype=torch.int32, device=X.device)
    _check(lib().bitlinear_quant_act_rmsnorm(_ptr(X), M, K, _ptr(norm_weight), float(eps), _ptr(Q), ldq,
                                             _ptr(a), _ptr(rs), _stream(stream)), "quant_act_rmsnorm")
    return Q, a, rs


@_on_stream
def quant_act_add_rmsnorm(X, R, norm_weight=None, eps: float = 1e-5, out=None, ldq: int | None = None,
                          stream=None):
    """(Q, absmax, rowsum, Xsum): Xsum = X + R (written to `out`, which may
    be X or R for an in-place update), then the RMSNorm int8 cast of Xsum."""
    _dev_tensor(X, torch.float32, "X")
    _dev_tensor(R, torch.float32, "R")
    if norm_weight is not None:
        _dev_tensor(norm_weight, torch.float32, "norm_weight")
    M, K = X.shape
    if R.shape != X.shape:
        raise ValueError("R must have the shape of X")
    ldq = q_stride(K) if ldq is None else ldq
    Xs = torch.empty_like(X) if out is None else _dev_tensor(out, torch.float32, "out")
    Q = torch.empty((M, ldq), dtype=torch.int8, device=X.device)
    a = torch.empty(M, dtype=torch.float32, device=X.device)
    rs = torch.empty(M, dtype=torch.int32, device=X.device)
    _check(lib().bitlinear_quant_act_add_rmsnorm(_ptr(X), _ptr(R), M, K, _ptr(norm_weight), float(eps), _ptr(Xs),
                                                 _ptr(Q), ldq, _ptr(a), _ptr(rs), _stream(stream)),
           "quant_act_add_rmsnorm")
    return Q, a, rs, Xs


@_on_stream
def quant_act_relu2_gate(G, U, ldq: int | None = None, stream=None):
    """Gated squared-ReLU H = relu(G)^2 * U of the gate and up projections'
    outputs (M x N fp32 each), then the absmax int8 cast: (Q int8 M x ldq,
    absmax fp32 [M] of H, rowsum int32 [M])."""
    _dev_tensor(G, torch.float32, "G")
    _dev_tensor(U, torch.float32, "U")
    if G.shape != U.shape:
        raise ValueError("G and U must have the same shape")
    M, N = G.shape
    ldq = q_stride(N) if ldq is None else ldq
    Q = torch.empty((M, ldq), dtype=torch.int8, device=G.device)
    a = torch.empty(M, dtype=torch.float32, device=G.device)
    rs = torch.empty(M, dtype=torch.int32, device=G.device)
    _check(lib().bitlinear_quant_act_relu2_gate(_ptr(G), _ptr(U), M, N, _ptr(Q), ldq, _ptr(a), _ptr(rs),
                                                _stream(stream)), "quant_act_relu2_gate")
    return Q, a, rs


@_on_stream
def matmul(Q, absmax, rowsum, P, gamma, N: int, K: int, with_acc: bool = False, stream=None):
    """Y (and acc) from already-quantized activations Q (M rows, stride
    Q.shape[1] >= q_stride(K), zero beyond K)."""
    _dev_tensor(Q, torch.int8, "Q")
    _dev_tensor(absmax, torch.float32, "absmax")
    _dev_tensor(rowsum, torch.int32, "rowsum")
    _dev_tensor(P, torch.uint8, "P")
    _dev_tensor(gamma, torch.float32, "gamma")
    M, ldq = Q.shape
    Y = torch.empty((M, N), dtype=torch.float32, device=Q.device)
    acc = torch.empty((M, N), dtype=torch.int32, device=Q.device) if with_acc else None
    ws = _workspace(workspace_bytes(WS_MATMUL, M, N, K), Q.device)
    _check(lib().bitlinear_matmul(_ptr(Q), ldq, _ptr(absmax), _ptr(rowsum), M, K, _ptr(P),
                                  _ptr(gamma), N, _ptr(Y), _ptr(acc), _ptr(ws),
                                  0 if ws is None else ws.numel(), _stream(stream)), "matmul")
    return (Y, acc) if with_acc else Y


@_on_stream
def forward(X, P, gamma, N: int, with_acc: bool = False, ws=None, out=None, stream=None):
    """BitLinear forward: Y = rescale(ternary(P) x int8(X)), M x N fp32."""
    _dev_tensor(X, torch.float32, "X")
    _dev_tensor(P, torch.uint8, "P")
    _dev_tensor(gamma, torch.float32, "gamma")
    M, K = X.shape
    Y = torch.empty((M, N), dtype=torch.float32, device=X.device) if out is None else out
    acc = torch.empty((M, N), dtype=torch.int32, device=X.device) if with_acc else None
    if ws is None:
        ws = _workspace(workspace_bytes(WS_FORWARD, M, N, K), X.device)
    _check(lib().bitlinear_forward(_ptr(X), M, K, _ptr(P), _ptr(gamma), N, _ptr(Y), _ptr(acc),
                                   _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)),
           "forward")
    return (Y, acc) if with_acc else Y


@_on_stream
def forward_noalloc(X, P, gamma, N: int, with_acc: bool = False, out=None, acc=None, stream=None):
    """BitLinear forward in the library's own scratch array (no workspace):
    bit-identical to forward().  Calls on one GPU share that array and must
    not overlap."""
    _dev_tensor(X, torch.float32, "X")
    _dev_tensor(P, torch.uint8, "P")
    _dev_tensor(gamma, torch.float32, "gamma")
    M, K = X.shape
    Y = torch.empty((M, N), dtype=torch.float32, device=X.device) if out is None else out
    if with_acc and acc is None:
        acc = torch.empty((M, N), dtype=torch.int32, device=X.device)
    _check(lib().bitlinear_forward_noalloc(_ptr(X), M, K, _ptr(P), _ptr(gamma), N, _ptr(Y), _ptr(acc),
                                           _stream(stream)), "forward_noalloc")
    return (Y, acc) if with_acc else Y


def noalloc_scratch_bytes() -> int:
    return int(lib().bitlinear_noalloc_scratch_bytes())


def packed5_bytes(N: int, K: int) -> int:
    return int(lib().bitlinear_packed5_bytes(N, K))


def q_stride5(K: int) -> int:
    return int(lib().bitlinear_q_stride5(K))


@_on_stream
def pack5(T, stream=None):
    """BT5-T32 bytes (five codes per byte) of the N x K int8 codes T."""
    _dev_tensor(T, torch.int8, "T")
    N, K = T.shape
    P = torch.empty(packed5_bytes(N, K), dtype=torch.uint8, device=T.device)
    _check(lib().bitlinear_pack5(_ptr(T), N, K, _ptr(P), _stream(stream)), "pack5")
    return P


@_on_stream
def unpack5(P, N: int, K: int, stream=None):
    _dev_tensor(P, torch.uint8, "P")
    T = torch.empty((N, K), dtype=torch.int8, device=P.device)
    _check(lib().bitlinear_unpack5(_ptr(P), N, K, _ptr(T), _stream(stream)), "unpack5")
    return T


@_on_stream
def matmul5(Q, absmax, rowsum, P, gamma, N: int, K: int, with_acc: bool = False, stream=None):
    """matmul over BT5-T32 weights; Q rows have stride Q.shape[1] >=
    q_stride5(K) and are zero beyond K."""
    _dev_tensor(Q, torch.int8, "Q")
    _dev_tensor(absmax, torch.float32, "absmax")
    _dev_tensor(rowsum, torch.int32, "rowsum")
    _dev_tensor(P, torch.uint8, "P")
    _dev_tensor(gamma, torch.float32, "gamma")
    M, ldq = Q.shape
    Y = torch.empty((M, N), dtype=torch.float32, device=Q.device)
    acc = torch.empty((M, N), dtype=torch.int32, device=Q.device) if with_acc else None
    ws = _workspace(workspace_bytes(WS_MATMUL5, M, N, K), Q.device)
    _check(lib().bitlinear_matmul5(_ptr(Q), ldq, _ptr(absmax), _ptr(rowsum), M, K, _ptr(P),
                                   _ptr(gamma), N, _ptr(Y), _ptr(acc), _ptr(ws),
                                   0 if ws is None else ws.numel(), _stream(stream)), "matmul5")
    return (Y, acc) if with_acc else Y


@_on_stream
def forward5(X, P, gamma, N: int, with_acc: bool = False, ws=None, out=None, stream=None):
    """BitLinear forward over BT5-T32 weights."""
    _dev_tensor(X, torch.float32, "X")
    _dev_tensor(P, torch.uint8, "P")
    _dev_tensor(gamma, torch.float32, "gamma")
    M, K = X.shape
    Y = torch.empty((M, N), dtype=torch.float32, device=X.device) if out is None else out
    acc = torch.empty((M, N), dtype=torch.int32, device=X.device) if with_acc else None
    if ws is None:
        ws = _workspace(workspace_bytes(WS_FORWARD5, M, N, K), X.device)
    _check(lib().bitlinear_forward5(_ptr(X), M, K, _ptr(P), _ptr(gamma), N, _ptr(Y), _ptr(acc),
                                    _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)),
           "forward5")
    return (Y, acc) if with_acc else Y


def probe_read_sink_words(nbytes: int, chunk_bytes: int) -> int:
    return int(lib().bitlinear_probe_read_sink_words(nbytes, chunk_bytes))


@_on_stream
def probe_read(buf, chunk_bytes: int, sink=None, stream=None):
    """Streaming-read calibration probe over the bytes of a contiguous CUDA
    tensor; returns the uint32 sink (XOR of all sink words = XOR of all
    32-bit words of the buffer)."""
    if not (isinstance(buf, torch.Tensor) and buf.is_cuda and buf.is_contiguous()):
        raise TypeError("buf must be a contiguous CUDA tensor")
    nbytes = buf.numel() * buf.element_size()
    words = probe_read_sink_words(nbytes, chunk_bytes)
    if sink is None:
        sink = torch.empty(max(words, 1), dtype=torch.int32, device=buf.device)
    _check(lib().bitlinear_probe_read(buf.data_ptr(), nbytes, chunk_bytes, sink.data_ptr(), _stream(stream)),
           "probe_read")
    return sink


def probe_mfma_blocks() -> int:
    n = ctypes.c_int32(0)
    _check(lib().bitlinear_probe_mfma_blocks(ctypes.byref(n)), "probe_mfma_blocks")
    return int(n.value)


@_on_stream
def probe_mfma(iters: int, a: int, b: int, blocks: int, sink=None, device=None, stream=None):
    """Int8 matrix-instruction calibration probe: blocks*4*iters*4*65536
    int8 operations; every sink entry becomes 2048*a*b*iters."""
    if sink is None:
        sink = torch.empty(256 * blocks, dtype=torch.int32, device=device or "cuda")
    _check(lib().bitlinear_probe_mfma(iters, a, b, blocks, sink.data_ptr(), _stream(stream)), "probe_mfma")
    return sink


@_on_stream
def probe_mfma_data(iters: int, operands, blocks: int, sink=None, clocks=None, device=None, stream=None):
    """Int8 matrix-instruction probe on operands from memory (an int8 CUDA
    tensor of 8192 bytes: four (A, B) fragment sets of 64 lanes x 16
    bytes): blocks*4*iters*4*65536 int8 operations.  Returns (sink, clocks):
    int32[256*blocks] accumulator sums and int64[3*blocks]: per workgroup
    the shader-clock count over its loop and the reference counter at the
    loop's start and end."""
    _dev_tensor(operands, torch.int8, "operands")
    if operands.numel() != 8192:
        raise ValueError("operands must hold 4 x 2 x 64 x 16 bytes")
    dev = operands.device
    if sink is None:
        sink = torch.empty(256 * blocks, dtype=torch.int32, device=dev)
    if clocks is None:
        clocks = torch.empty(3 * blocks, dtype=torch.int64, device=dev)
    _check(lib().bitlinear_probe_mfma_data(iters, operands.data_ptr(), blocks, sink.data_ptr(), clocks.data_ptr(),
                                           _stream(stream)), "probe_mfma_data")
    return sink, clocks


def probe_compute_units() -> int:
    n = ctypes.c_int32(0)
    _check(lib().bitlinear_probe_compute_units(ctypes.byref(n)), "probe_compute_units")
    return int(n.value)


@_on_stream
def probe_barrier(rounds: int, blocks: int, spin_limit: int = 1 << 20, state=None, sink=None, device=None,
                  stream=None):
    """Grid-barrier calibration probe: `rounds` barriers among `blocks`
    workgroups with a word exchanged per workgroup per barrier; returns
    (state, sink).  state[0] ends at rounds * blocks, state[1] counts
    give-ups; each workgroup's 256 sink words add up to the sum over rounds r
    and workgroups i of r * blocks + i (mod 2^32)."""
    device = device or "cuda"
    if state is None:
        state = torch.zeros(2 + 2 * blocks, dtype=torch.int32, device=device)
    if sink is None:
        sink = torch.empty(256 * blocks, dtype=torch.int32, device=device)
    _check(lib().bitlinear_probe_barrier(rounds, blocks, spin_limit, state.data_ptr(), sink.data_ptr(),
                                         _stream(stream)), "probe_barrier")
    return state, sink


class MultiMatmul:
    """Several weight matrices that read the same int8 activations (q|k|v,
    gate|up), contracted in one launch.  weights: sequence of dicts with P,
    gamma (CUDA tensors), N and optionally format.  The object owns a
    zero-filled workspace for its sizes (reused call after call)."""

    def __init__(self, weights, M: int, K: int, device=None):
        L = lib()
        n = len(weights)
        self.arr = (Weight * n)()
        self.M, self.K, self.count = M, K, n
        self.Ns = [int(w["N"]) for w in weights]
        self.fmt = int(weights[0].get("format", FORMAT_BL2))
        self._keep = []
        device = device or weights[0]["P"].device
        for i, w in enumerate(weights):
            _dev_tensor(w["P"], torch.uint8, "P")
            _dev_tensor(w["gamma"], torch.float32, "gamma")
            self.arr[i] = Weight(w["P"].data_ptr(), w["gamma"].data_ptr(), None, None, self.Ns[i],
                                 int(w.get("format", FORMAT_BL2)), 0)
            self._keep.append(w)
        wsb = L.bitlinear_multi_workspace_bytes(self.arr, n, M, K)
        if wsb == ctypes.c_size_t(-1).value:
            _check(-2, "multi_workspace_bytes")
        self.ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=device)

    @_on_stream
    def __call__(self, Q, absmax, rowsum, outs=None, accs=None, stream=None):
        """Y_i (M x N_i fp32) for every weight; outs/accs: optional tensors."""
        _dev_tensor(Q, torch.int8, "Q")
        M, ldq = Q.shape
        if M != self.M:
            raise ValueError("Q has the wrong number of rows")
        outs = outs or [torch.empty((M, N), dtype=torch.float32, device=Q.device) for N in self.Ns]
        for i in range(self.count):
            self.arr[i].Y = outs[i].data_ptr()
            self.arr[i].acc = None if accs is None else accs[i].data_ptr()
        _check(lib().bitlinear_matmul_multi(_ptr(Q), ldq, _ptr(absmax), _ptr(rowsum), M, self.K, self.arr,
                                            self.count, _ptr(self.ws), self.ws.numel(), _stream(stream)),
               "matmul_multi")
        return outs


class CastMultiMatmul(MultiMatmul):
    """An activation cast (mode CAST_PLAIN, CAST_RMSNORM, CAST_RELU2_GATE or
    CAST_ADD_RMSNORM) and the weight matrices that read its int8 codes, in
    one call (bitlinear_cast_matmul_multi); weights as MultiMatmul.  The
    object owns a zero-filled workspace for its mode and sizes."""

    def __init__(self, mode, weights, M: int, K: int, device=None):
        super().__init__(weights, M, K, device)
        self.mode = int(mode)
        wsb = lib().bitlinear_cast_multi_workspace_bytes(self.mode, self.arr, self.count, M, K)
        if wsb == ctypes.c_size_t(-1).value:
            _check(-2, "cast_multi_workspace_bytes")
        self.ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device=self.ws.device)

    @_on_stream
    def __call__(self, X, aux=None, R=None, eps=0.0, X_out=None, outs=None, accs=None, stream=None):
        """Y_i (M x N_i fp32) for every weight of the cast of X (aux: norm
        gains or the up projection's output; R, X_out: the residual sum)."""
        _dev_tensor(X, torch.float32, "X")
        if tuple(X.shape) != (self.M, self.K):
            raise ValueError("X must be M x K")
        outs = outs or [torch.empty((self.M, N), dtype=torch.float32, device=X.device) for N in self.Ns]
        for i in range(self.count):
            self.arr[i].Y = outs[i].data_ptr()
            self.arr[i].acc = None if accs is None else accs[i].data_ptr()
        _check(lib().bitlinear_cast_matmul_multi(self.mode, _ptr(X), _ptr(aux), _ptr(R), float(eps), _ptr(X_out),
                                                 self.M, self.K, self.arr, self.count, _ptr(self.ws),
                                                 self.ws.numel(), _stream(stream)),
               "cast_matmul_multi")
        return outs


class GroupPlan:
    """A grouped forward over independent BitLinear problems.

    problems: sequence of dicts with keys X, P, gamma, Y (torch CUDA
    tensors), N, and optionally acc and format (FORMAT_BL2, the default, or
    FORMAT_BT5 for pack5 weights).  M and K come from X.  The plan binds
    these tensors and its own workspace; run it with forward() (both stages)
    or quant_act() then matmul().
    """

    def __init__(self, problems, device=None):
        L = lib()
        n = len(problems)
        arr = (Problem * n)()
        keep = []
        for i, p in enumerate(problems):
            X, P, g, Y = p["X"], p["P"], p["gamma"], p["Y"]
            acc = p.get("acc")
            _dev_tensor(X, torch.float32, "X")
            _dev_tensor(P, torch.uint8, "P")
            _dev_tensor(g, torch.float32, "gamma")
            _dev_tensor(Y, torch.float32, "Y")
            M, K = X.shape
            arr[i] = Problem(X.data_ptr(), P.data_ptr(), g.data_ptr(), Y.data_ptr(),
                             _ptr(acc), M, int(p["N"]), K, int(p.get("format", FORMAT_BL2)), 0)
            keep.append((X, P, g, Y, acc))
        device = device or problems[0]["X"].device
        ws_bytes = L.bitlinear_group_workspace_bytes(arr, n)
        tb = L.bitlinear_group_table_bytes(arr, n)
        if tb == 0:
            _check(-2, "group_table_bytes")
        self.ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=device)
        self.table_host = torch.empty(tb, dtype=torch.uint8)
        _check(L.bitlinear_group_plan(arr, n, self.ws.data_ptr(), self.ws.numel(),
                                      self.table_host.data_ptr(), tb), "group_plan")
        self.table_dev = self.table_host.to(device)
        self._keep = keep
        self.count = n

    def quant_act(self, stream=None):
        _check(lib().bitlinear_group_quant_act(self.table_host.data_ptr(), self.table_dev.data_ptr(),
                                               _stream(stream)), "group_quant_act")

    def matmul(self, stream=None):
        _check(lib().bitlinear_group_matmul(self.table_host.data_ptr(), self.table_dev.data_ptr(),
                                            _stream(stream)), "group_matmul")

    def forward(self, stream=None):
        _check(lib().bitlinear_group_forward(self.table_host.data_ptr(), self.table_dev.data_ptr(),
                                             _stream(stream)), "group_forward")
