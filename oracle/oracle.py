"""CPU oracle of the ternary BitLinear forward path -- numpy wrapper.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by
the benchmark's CPU-baseline leg, never by the product package.  The oracle
and the HIP library share no code; this module never imports
``ternary_bit_linear_amd``.

The arithmetic lives in ``oracle.c`` (plain loops, fp32 where the method's
integer decisions are taken, fp64 for the final rescale).  This wrapper
builds it with gcc when no build is present and marshals numpy arrays.

Sources: huggingface/transformers PR #38087 "Add optional RMSNorm support to
BitNet quantization (config + layers)" (RMSNorm before quantisation, eps
1e-6, use_rms_norm; the BitNetMLP excerpt of the review thread for the FFN
block); eejd/cpp-bitnet PR #7 "fix: I2_S ARM kernel layout + squared-ReLU
FFN" (I2_S layout, code offset, per-tensor scale, trailer, K % 128; squared
ReLU as the 2B4T FFN activation).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OK = 0
ERR_SHAPE = 2
ERR_NOT_TERNARY = 4


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so (gcc, no fp contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math",
               "-fopenmp", "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        build()  # compiles only when the library is missing or older than oracle.c
        L = ctypes.CDLL(_LIB)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        L.oracle_packed_bytes.restype = i64
        L.oracle_packed_bytes.argtypes = [i64, i64]
        L.oracle_pack_i2s.restype = ctypes.c_int
        L.oracle_pack_i2s.argtypes = [p, i64, i64, p, p]
        L.oracle_unpack_i2s.restype = ctypes.c_int
        L.oracle_unpack_i2s.argtypes = [p, i64, i64, p]
        L.oracle_code_at.restype = ctypes.c_int
        L.oracle_code_at.argtypes = [p, i64, i64, i64]
        L.oracle_read_scale.restype = ctypes.c_float
        L.oracle_read_scale.argtypes = [p, i64, i64]
        L.oracle_sumsq.restype = ctypes.c_float
        L.oracle_sumsq.argtypes = [p, i64]
        L.oracle_rmsnorm.restype = ctypes.c_int
        L.oracle_rmsnorm.argtypes = [p, p, ctypes.c_float, i64, i64, p]
        L.oracle_act_quant.restype = ctypes.c_int
        L.oracle_act_quant.argtypes = [p, p, ctypes.c_float, i64, i64, p, p, p, p]
        L.oracle_matmul_i2s.restype = ctypes.c_int
        L.oracle_matmul_i2s.argtypes = [p, p, p, i64, i64, i64, p]
        L.oracle_rescale.restype = ctypes.c_int
        L.oracle_rescale.argtypes = [p, p, ctypes.c_float, i64, i64, p]
        L.oracle_rescale_f32.restype = ctypes.c_int
        L.oracle_rescale_f32.argtypes = [p, p, ctypes.c_float, i64, i64, p]
        f = ctypes.c_float
        L.oracle_bf16_to_f32.restype = ctypes.c_int
        L.oracle_bf16_to_f32.argtypes = [p, i64, p]
        L.oracle_f32_to_bf16.restype = ctypes.c_int
        L.oracle_f32_to_bf16.argtypes = [p, i64, p]
        L.oracle_relu2_mul.restype = ctypes.c_int
        L.oracle_relu2_mul.argtypes = [p, p, i64, p]
        L.oracle_ffn.restype = ctypes.c_int
        L.oracle_ffn.argtypes = [p, p, f, i64, i64, i64, p, f, p, f, p, f, p, p, p, p, p]
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


class OracleError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: oracle status {status}")
        self.status = status


def packed_bytes(N: int, K: int) -> int:
    return int(lib().oracle_packed_bytes(N, K))


def pack_i2s(w: np.ndarray) -> tuple[np.ndarray, float]:
    """fp32 W[N][K] (ternary x scale) -> (uint8[N*K/4 + 32], scale)."""
    w = _f32(w)
    N, K = w.shape
    out = np.zeros(max(packed_bytes(N, K), 1), dtype=np.uint8)
    sc = np.zeros(1, dtype=np.float32)
    st = lib().oracle_pack_i2s(_ptr(w), N, K, _ptr(out), _ptr(sc))
    if st != OK:
        raise OracleError(st, "pack_i2s")
    return out, float(sc[0])


def unpack_i2s(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    w = np.empty((N, K), dtype=np.float32)
    st = lib().oracle_unpack_i2s(_ptr(packed), N, K, _ptr(w))
    if st != OK:
        raise OracleError(st, "unpack_i2s")
    return w


def code_at(packed: np.ndarray, K: int, n: int, k: int) -> int:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    return int(lib().oracle_code_at(_ptr(packed), K, n, k))


def read_scale(packed: np.ndarray, N: int, K: int) -> float:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    return float(lib().oracle_read_scale(_ptr(packed), N, K))


def sumsq(v: np.ndarray) -> np.float32:
    """Sum of squares of one row in the pinned O256 order."""
    v = _f32(v).ravel()
    return np.float32(lib().oracle_sumsq(_ptr(v), v.size))


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    x = _f32(np.atleast_2d(x))
    gamma = _f32(gamma)
    M, K = x.shape
    xn = np.empty_like(x)
    st = lib().oracle_rmsnorm(_ptr(x), _ptr(gamma), ctypes.c_float(eps), M, K, _ptr(xn))
    if st != OK:
        raise OracleError(st, "rmsnorm")
    return xn


def act_quant(x: np.ndarray, gamma, eps: float = 1e-6):
    """-> (q int8[M][K], inv fp32[M], qsum int32[M]).  gamma None: the layer
    without RMSNorm (x is quantised as it is)."""
    x = _f32(np.atleast_2d(x))
    gamma = None if gamma is None else _f32(gamma)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.int8)
    inv = np.empty(M, dtype=np.float32)
    qsum = np.empty(M, dtype=np.int32)
    xn = np.empty((M, K), dtype=np.float32)
    gp = ctypes.c_void_p(None) if gamma is None else _ptr(gamma)
    st = lib().oracle_act_quant(_ptr(x), gp, ctypes.c_float(eps), M, K,
                                _ptr(q), _ptr(inv), _ptr(qsum), _ptr(xn))
    if st != OK:
        raise OracleError(st, "act_quant")
    return q, inv, qsum


def matmul_i2s(q: np.ndarray, qsum: np.ndarray, packed: np.ndarray, N: int) -> np.ndarray:
    """-> acc int32[M][N] = sum_k code(n,k) q[m,k] - qsum[m]."""
    q = np.ascontiguousarray(np.atleast_2d(q), dtype=np.int8)
    qsum = np.ascontiguousarray(qsum, dtype=np.int32)
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    M, K = q.shape
    acc = np.empty((M, N), dtype=np.int32)
    st = lib().oracle_matmul_i2s(_ptr(q), _ptr(qsum), _ptr(packed), M, K, N, _ptr(acc))
    if st != OK:
        raise OracleError(st, "matmul_i2s")
    return acc


def rescale(acc: np.ndarray, inv: np.ndarray, w_scale: float) -> np.ndarray:
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    inv = _f32(inv)
    M, N = acc.shape
    y = np.empty((M, N), dtype=np.float64)
    st = lib().oracle_rescale(_ptr(acc), _ptr(inv), ctypes.c_float(w_scale), M, N, _ptr(y))
    if st != OK:
        raise OracleError(st, "rescale")
    return y


def forward(x: np.ndarray, packed: np.ndarray, w_scale: float, gamma,
            eps: float, N: int) -> np.ndarray:
    """Whole forward; returns fp64 y[M][N].  gamma None: no RMSNorm."""
    q, inv, qsum = act_quant(x, gamma, eps)
    acc = matmul_i2s(q, qsum, packed, N)
    return rescale(acc, inv, w_scale)


def rescale_f32(acc: np.ndarray, inv: np.ndarray, w_scale: float) -> np.ndarray:
    """fp32 BitLinear output (float)acc * (w_scale / inv[m])."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    inv = _f32(inv)
    M, N = acc.shape
    y = np.empty((M, N), dtype=np.float32)
    st = lib().oracle_rescale_f32(_ptr(acc), _ptr(inv), ctypes.c_float(w_scale), M, N, _ptr(y))
    if st != OK:
        raise OracleError(st, "rescale_f32")
    return y


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> fp32, exact."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float32)
    lib().oracle_bf16_to_f32(_ptr(bits), bits.size, _ptr(out))
    return out


def f32_to_bf16(v: np.ndarray) -> np.ndarray:
    """fp32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    v = _f32(v)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_f32_to_bf16(_ptr(v), v.size, _ptr(out))
    return out


def to_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Activations of the given I/O type to fp32 (exact for every type)."""
    if dtype == "f32":
        return _f32(x)
    if dtype == "bf16":
        return bf16_to_f32(x)
    if dtype == "f16":
        return np.asarray(x, np.float16).astype(np.float32)
    raise ValueError(dtype)


def from_f32(y: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 outputs rounded to the I/O type (nearest, ties to even): bf16 as
    uint16 bit patterns, f16 by numpy's IEEE conversion."""
    if dtype == "f32":
        return _f32(y)
    if dtype == "bf16":
        return f32_to_bf16(y)
    if dtype == "f16":
        with np.errstate(over="ignore"):  # beyond 65504 rounds to inf, as IEEE says
            return _f32(y).astype(np.float16)
    raise ValueError(dtype)


def forward_io(x: np.ndarray, x_dtype: str, packed: np.ndarray, w_scale: float, gamma,
               eps: float, N: int, y_dtype: str) -> np.ndarray:
    """Forward with half-precision activation I/O: x of x_dtype (bf16 as
    uint16 bits) is widened exactly to fp32, the fp32 path runs as in
    forward(), and the fp32 output (float)acc * (w_scale / inv) is rounded
    to y_dtype."""
    xf = to_f32(np.atleast_2d(x), x_dtype)
    q, inv, qsum = act_quant(xf, gamma, eps)
    acc = matmul_i2s(q, qsum, packed, N)
    return from_f32(rescale_f32(acc, inv, w_scale), y_dtype)


def dequant_i2s(packed: np.ndarray, N: int, K: int, dtype: str) -> np.ndarray:
    """The to_float direction in a dense type: unpack (code - 1) * scale in
    fp32, then round to dtype (bf16 as uint16 bit patterns)."""
    return from_f32(unpack_i2s(packed, N, K), dtype)


def relu2_mul(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """a = (max(g, 0)^2) * u in fp32 (the FFN block's gate)."""
    g, u = _f32(g), _f32(u)
    a = np.empty_like(g)
    st = lib().oracle_relu2_mul(_ptr(g), _ptr(u), g.size, _ptr(a))
    if st != OK:
        raise OracleError(st, "relu2_mul")
    return a


def ffn(x: np.ndarray, gamma_in, eps: float, gate, up, down, gamma_sub):
    """BitNet FFN block y = down(sub_norm(relu(g)^2 * u)), g / u = gate / up(x).
    gate, up, down: (packed, scale) pairs, packed from [F][H], [F][H], [H][F].
    gamma_in [H] / gamma_sub [F], or None for no RMSNorm.
    Returns (y fp64 [M][H], g, u, a fp32 [M][F])."""
    x = _f32(np.atleast_2d(x))
    M, H = x.shape
    (pg, sg), (pu, su), (pd, sd) = gate, up, down
    pg, pu, pd = (np.ascontiguousarray(p, dtype=np.uint8) for p in (pg, pu, pd))
    F = (pg.size - 32) * 4 // H
    gi = None if gamma_in is None else _f32(gamma_in)
    gs = None if gamma_sub is None else _f32(gamma_sub)
    g = np.empty((M, F), np.float32)
    u = np.empty((M, F), np.float32)
    a = np.empty((M, F), np.float32)
    y = np.empty((M, H), np.float64)
    null = ctypes.c_void_p(None)
    st = lib().oracle_ffn(_ptr(x), null if gi is None else _ptr(gi), ctypes.c_float(eps), M, H, F,
                          _ptr(pg), ctypes.c_float(sg), _ptr(pu), ctypes.c_float(su),
                          _ptr(pd), ctypes.c_float(sd), null if gs is None else _ptr(gs),
                          _ptr(g), _ptr(u), _ptr(a), _ptr(y))
    if st != OK:
        raise OracleError(st, "ffn")
    return y, g, u, a


def packed_rows(packed: np.ndarray, K: int, rows) -> np.ndarray:
    """Packed bytes of the selected weight rows (rows are contiguous K/4-byte
    runs when K % 128 == 0), with a zero trailer, for sampled checks."""
    rows = np.asarray(rows, dtype=np.int64)
    rb = K // 4
    idx = (rows[:, None] * rb + np.arange(rb)[None, :]).ravel()
    out = np.zeros(rows.size * rb + 32, dtype=np.uint8)
    out[: rows.size * rb] = np.asarray(packed)[idx]
    return out
