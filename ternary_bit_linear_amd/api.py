"""Python binding of ``libbitlinear.so`` (the C ABI in ``include/bitlinear.h``).

Argument marshalling only: every step of the BitLinear path runs in the HIP
kernels behind the C ABI.  PyTorch provides device memory (tensors are
allocated here and their pointers passed down) and the stream
(``torch.cuda.current_stream()``).  There is no fallback: if the library is
missing, loading it raises.

Functions mirror the C entry points: :func:`pack_i2s`, :func:`unpack_i2s`,
:func:`read_scale`, :func:`forward`, :func:`forward_batch`,
:func:`ffn_forward`, :func:`act_quant`, :func:`matmul_i2s`.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbitlinear.so")

OK, ERR_INVALID_ARG, ERR_SHAPE, ERR_ALIGN, ERR_NOT_TERNARY, ERR_WORKSPACE, ERR_HIP = range(7)
PATH_AUTO, PATH_GEMV, PATH_GEMM = 0, 1, 2

# Every symbol the header declares, with (restype, argtypes).
_i64, _p, _f, _i, _sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_int, ctypes.c_size_t


class Launch(ctypes.Structure):
    """bl_launch: path (bl_path), fuse (-1/0/1), variant (0 = auto)."""
    _fields_ = [("path", ctypes.c_int32), ("fuse", ctypes.c_int32),
                ("variant", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class ForwardDesc(ctypes.Structure):
    """bl_forward_desc: the arguments of one bitlinear_forward."""
    _fields_ = [("x", ctypes.c_void_p), ("packed_w", ctypes.c_void_p),
                ("w_scale", ctypes.c_float), ("gamma", ctypes.c_void_p),
                ("eps", ctypes.c_float), ("M", ctypes.c_int64), ("K", ctypes.c_int64),
                ("N", ctypes.c_int64), ("y", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t)]


class FfnDesc(ctypes.Structure):
    """bl_ffn_desc: the arguments of one bitlinear_ffn_forward."""
    _fields_ = [("x", ctypes.c_void_p), ("gamma_in", ctypes.c_void_p),
                ("packed_gate", ctypes.c_void_p), ("s_gate", ctypes.c_float),
                ("packed_up", ctypes.c_void_p), ("s_up", ctypes.c_float),
                ("packed_down", ctypes.c_void_p), ("s_down", ctypes.c_float),
                ("gamma_sub", ctypes.c_void_p), ("eps", ctypes.c_float),
                ("M", ctypes.c_int64), ("H", ctypes.c_int64), ("F", ctypes.c_int64),
                ("y", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t)]


class IoDesc(ctypes.Structure):
    """bl_forward_io_desc: the arguments of one bitlinear_forward_io."""
    _fields_ = [("x", ctypes.c_void_p), ("x_dtype", ctypes.c_int), ("packed_w", ctypes.c_void_p),
                ("w_scale", ctypes.c_float), ("gamma", ctypes.c_void_p), ("eps", ctypes.c_float),
                ("M", ctypes.c_int64), ("K", ctypes.c_int64), ("N", ctypes.c_int64),
                ("y", ctypes.c_void_p), ("y_dtype", ctypes.c_int), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t)]


SIGNATURES = {
    "bitlinear_status_string": (ctypes.c_char_p, [_i]),
    "bitlinear_abi_version": (_i, []),
    "bitlinear_num_variants": (_i, [_i]),
    "bitlinear_packed_bytes": (_sz, [_i64, _i64]),
    "bitlinear_workspace_bytes": (_sz, [_i64, _i64]),
    "bitlinear_pack_i2s": (_i, [_p, _i64, _i64, _p, _p, _p]),
    "bitlinear_unpack_i2s": (_i, [_p, _i64, _i64, _p, _p]),
    "bitlinear_read_scale": (_i, [_p, _i64, _i64, _p, _p]),
    "bitlinear_forward": (_i, [_p, _p, _f, _p, _f, _i64, _i64, _i64, _p, _p, _sz, _p]),
    "bitlinear_forward_ex": (_i, [_p, _p, _f, _p, _f, _i64, _i64, _i64, _p, _p, _sz,
                                  ctypes.POINTER(Launch), _p]),
    "bitlinear_forward_noalloc": (_i, [_p, _p, _f, _p, _f, _i64, _i64, _i64, _p, _p]),
    "bitlinear_probe_read_sink_words": (_sz, [_sz]),
    "bitlinear_probe_read": (_i, [_p, _sz, _p, _sz, _p]),
    "bitlinear_probe_mfma": (_i, [_i64, _i64, _p, _sz, _p]),
    "bitlinear_forward_batch": (_i, [ctypes.POINTER(ForwardDesc), _i, ctypes.POINTER(Launch), _p]),
    "bitlinear_act_quant": (_i, [_p, _p, _f, _i64, _i64, _p, _p, _p, _p]),
    "bitlinear_ffn_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "bitlinear_io_workspace_bytes": (_sz, [_i64, _i64, _i64]),
    "bitlinear_dequant_i2s": (_i, [_p, _i64, _i64, _p, _i, _p]),
    "bitlinear_forward_io": (_i, [_p, _i, _p, _f, _p, _f, _i64, _i64, _i64, _p, _i, _p, _sz, _p]),
    "bitlinear_forward_io_batch": (_i, [ctypes.POINTER(IoDesc), _i, _p]),
    "bitlinear_ffn_forward": (_i, [ctypes.POINTER(FfnDesc), _p]),
    "bitlinear_fp32_ops": (_i, [_i, _p, _p, _f, _i64, _p, _p]),
    "bitlinear_matmul_i2s": (_i, [_p, _p, _p, _i64, _i64, _i64, _p, _p]),
    "bitlinear_matmul_i2s_ex": (_i, [_p, _p, _p, _i64, _i64, _i64, _p,
                                     ctypes.POINTER(Launch), _p]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it was not built)."""
    global _lib
    if _lib is None:
        # PyTorch ships its own HIP runtime; importing it first makes the
        # library bind to that same runtime (its device pointers and streams),
        # instead of loading a second one from the system ROCm.
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m ternary_bit_linear_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class BitLinearError(RuntimeError):
    def __init__(self, status: int, what: str):
        msg = lib().bitlinear_status_string(status).decode()
        super().__init__(f"{what}: {msg}")
        self.status = status


def _check(status: int, what: str) -> None:
    if status != OK:
        raise BitLinearError(status, what)


def _torch():
    import torch
    return torch


def _stream():
    return ctypes.c_void_p(_torch().cuda.current_stream().cuda_stream)


def _dev(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _gamma(g):
    """gamma tensor, or None for the layer without RMSNorm (NULL pointer)."""
    torch = _torch()
    return ctypes.c_void_p(None) if g is None else _dev(g, torch.float32, "gamma")


def _launch(path, fuse, variant):
    if path == PATH_AUTO and fuse == -1 and variant == 0:
        return None
    return ctypes.byref(Launch(path, fuse, variant, 0))


def packed_bytes(N: int, K: int) -> int:
    return int(lib().bitlinear_packed_bytes(N, K))


def workspace_bytes(M: int, K: int) -> int:
    return int(lib().bitlinear_workspace_bytes(M, K))


def num_variants(path: int) -> int:
    return int(lib().bitlinear_num_variants(path))


def pack_i2s(w):
    """fp32 W[N][K] (ternary x scale, on the GPU) -> (uint8 packed tensor of
    N*K/4 + 32 bytes, scale).  Synchronous."""
    torch = _torch()
    N, K = w.shape
    nb = packed_bytes(N, K)
    if nb == 0:
        raise BitLinearError(ERR_SHAPE, "pack_i2s")
    packed = torch.empty(nb, dtype=torch.uint8, device=w.device)
    sc = ctypes.c_float(0.0)
    _check(lib().bitlinear_pack_i2s(_dev(w, torch.float32, "w"), N, K,
                                    ctypes.c_void_p(packed.data_ptr()),
                                    ctypes.byref(sc), _stream()), "pack_i2s")
    return packed, sc.value


def unpack_i2s(packed, N: int, K: int):
    torch = _torch()
    w = torch.empty((N, K), dtype=torch.float32, device=packed.device)
    _check(lib().bitlinear_unpack_i2s(_dev(packed, torch.uint8, "packed"), N, K,
                                      ctypes.c_void_p(w.data_ptr()), _stream()), "unpack_i2s")
    return w


def read_scale(packed, N: int, K: int) -> float:
    torch = _torch()
    v = ctypes.c_float(0.0)
    _check(lib().bitlinear_read_scale(_dev(packed, torch.uint8, "packed"), N, K,
                                      ctypes.byref(v), _stream()), "read_scale")
    return v.value


def act_quant(x, gamma, eps: float = 1e-6):
    """-> (q int8 [M][K], inv fp32 [M], qsum int32 [M]); gamma None: no RMSNorm."""
    torch = _torch()
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    inv = torch.empty(M, dtype=torch.float32, device=x.device)
    qsum = torch.empty(M, dtype=torch.int32, device=x.device)
    _check(lib().bitlinear_act_quant(_dev(x, torch.float32, "x"), _gamma(gamma),
                                     eps, M, K, ctypes.c_void_p(q.data_ptr()),
                                     ctypes.c_void_p(inv.data_ptr()),
                                     ctypes.c_void_p(qsum.data_ptr()), _stream()), "act_quant")
    return q, inv, qsum


FP_SQRT, FP_DIV, FP_RMS_SCALE, FP_QUANT_SCALE = range(4)


def fp32_ops(op: int, a, b=None, eps: float = 0.0):
    """Elementwise device fp32 arithmetic of the normalisation and
    quantisation scales (bl_fp_op): sqrtf(a), a / b, 1 / sqrtf(a / b + eps)
    with b = K, or 127 / max(a, 1e-5).  -> fp32 tensor like a."""
    torch = _torch()
    out = torch.empty_like(a)
    bp = ctypes.c_void_p(None) if b is None else _dev(b, torch.float32, "b")
    _check(lib().bitlinear_fp32_ops(op, _dev(a, torch.float32, "a"), bp, eps, a.numel(),
                                    ctypes.c_void_p(out.data_ptr()), _stream()), "fp32_ops")
    return out


def matmul_i2s(q, qsum, packed, N: int, path: int = PATH_AUTO, variant: int = 0):
    """-> acc int32 [M][N] = sum_k code(n,k) q[m,k] - qsum[m]."""
    torch = _torch()
    M, K = q.shape
    acc = torch.empty((M, N), dtype=torch.int32, device=q.device)
    _check(lib().bitlinear_matmul_i2s_ex(_dev(q, torch.int8, "q"), _dev(qsum, torch.int32, "qsum"),
                                         _dev(packed, torch.uint8, "packed"), M, K, N,
                                         ctypes.c_void_p(acc.data_ptr()),
                                         _launch(path, -1, variant), _stream()), "matmul_i2s")
    return acc


def new_workspace(M: int, K: int, device="cuda"):
    torch = _torch()
    return torch.empty(workspace_bytes(M, K), dtype=torch.uint8, device=device)


def forward(x, packed, w_scale: float, gamma, eps: float = 1e-6, N: int | None = None,
            out=None, workspace=None, path: int = PATH_AUTO, fuse: int = -1, variant: int = 0):
    """y = BitLinear(x) with I2_S weights; x fp32 [M][K] -> y fp32 [M][N].
    gamma None: the layer without RMSNorm (x is quantised as it is)."""
    torch = _torch()
    M, K = x.shape
    if N is None:
        N = (packed.numel() - 32) * 4 // K
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = new_workspace(M, K, x.device)
    _check(lib().bitlinear_forward_ex(
        _dev(x, torch.float32, "x"), _dev(packed, torch.uint8, "packed"), w_scale,
        _gamma(gamma), eps, M, K, N, _dev(out, torch.float32, "out"),
        _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
        _launch(path, fuse, variant), _stream()), "forward")
    return out


NOALLOC_SCRATCH_BYTES = (16 << 20) + (64 << 10)  # BITLINEAR_NOALLOC_SCRATCH_BYTES


def forward_noalloc(x, packed, w_scale: float, gamma, eps: float, out):
    """forward() through the allocation-free entry point: q / inv / qsum go
    to the library's per-device scratch array; `out` (fp32 [M][N]) must be
    preallocated.  Calls that overlap on one device race."""
    torch = _torch()
    M, K = x.shape
    N = out.shape[1]
    _check(lib().bitlinear_forward_noalloc(
        _dev(x, torch.float32, "x"), _dev(packed, torch.uint8, "packed"), w_scale,
        _gamma(gamma), eps, M, K, N, _dev(out, torch.float32, "out"), _stream()),
        "forward_noalloc")
    return out


def probe_read(src, sink=None):
    """Calibration probe: one launch reading every byte of `src` (a device
    tensor).  Returns the sink tensor (so a caller can reuse it)."""
    torch = _torch()
    nb = src.numel() * src.element_size()
    words = int(lib().bitlinear_probe_read_sink_words(nb))
    if sink is None:
        sink = torch.empty(max(words, 1), dtype=torch.int32, device=src.device)
    _check(lib().bitlinear_probe_read(ctypes.c_void_p(src.data_ptr()), nb,
                                      ctypes.c_void_p(sink.data_ptr()), sink.numel(), _stream()),
           "probe_read")
    return sink


def probe_mfma(iters: int, workgroups: int, sink=None):
    """Calibration probe: back-to-back int8 32x32x32 MFMAs (4 per round per
    wave, 65536 int ops each) in `workgroups` workgroups of 256 threads."""
    torch = _torch()
    if sink is None:
        sink = torch.empty(workgroups * 256, dtype=torch.int32, device="cuda")
    _check(lib().bitlinear_probe_mfma(iters, workgroups, ctypes.c_void_p(sink.data_ptr()),
                                      sink.numel(), _stream()), "probe_mfma")
    return sink


def forward_batch(items, path: int = PATH_AUTO, fuse: int = -1, variant: int = 0):
    """Several independent forwards in as few launches as possible.
    items: sequence of (x, packed, w_scale, gamma, eps, out, workspace) with
    out fp32 [M][N] preallocated; bit-identical to forward() per item."""
    torch = _torch()
    arr = (ForwardDesc * len(items))()
    for i, (x, packed, w_scale, gamma, eps, out, ws) in enumerate(items):
        M, K = x.shape
        N = out.shape[1]
        arr[i] = ForwardDesc(_dev(x, torch.float32, "x"), _dev(packed, torch.uint8, "packed"),
                             w_scale, _gamma(gamma), eps, M, K, N,
                             _dev(out, torch.float32, "out"), _dev(ws, torch.uint8, "workspace"),
                             ws.numel())
    _check(lib().bitlinear_forward_batch(arr, len(items), _launch(path, fuse, variant), _stream()),
           "forward_batch")


def workspace_views(workspace, M: int, K: int):
    """(q, inv, qsum) views of a forward workspace (for inspection)."""
    torch = _torch()
    a = lambda v: (v + 255) // 256 * 256  # noqa: E731
    q = workspace[: M * K].view(torch.int8).view(M, K)
    o = a(M * K)
    inv = workspace[o: o + 4 * M].view(torch.float32)
    o += a(4 * M)
    qsum = workspace[o: o + 4 * M].view(torch.int32)
    return q, inv, qsum


def ffn_workspace_bytes(M: int, H: int, F: int) -> int:
    return int(lib().bitlinear_ffn_workspace_bytes(M, H, F))


def ffn_forward(x, gamma_in, eps: float, gate, up, down, gamma_sub, out=None, workspace=None):
    """BitNet FFN block y = down(sub_norm(relu(g)^2 * u)), g / u = gate / up(x).
    gate, up, down: (packed, scale) pairs (packed from [F][H], [F][H], [H][F]);
    gamma_in [H] / gamma_sub [F] or None (no RMSNorm).  x fp32 [M][H] -> y fp32 [M][H]."""
    torch = _torch()
    M, H = x.shape
    (pg, sg), (pu, su), (pd, sd) = gate, up, down
    F = (pg.numel() - 32) * 4 // H
    if out is None:
        out = torch.empty((M, H), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(ffn_workspace_bytes(M, H, F), dtype=torch.uint8, device=x.device)
    d = FfnDesc(_dev(x, torch.float32, "x"), _gamma(gamma_in), _dev(pg, torch.uint8, "gate"), sg,
                _dev(pu, torch.uint8, "up"), su, _dev(pd, torch.uint8, "down"), sd,
                _gamma(gamma_sub), eps, M, H, F, _dev(out, torch.float32, "out"),
                _dev(workspace, torch.uint8, "workspace"), workspace.numel())
    _check(lib().bitlinear_ffn_forward(ctypes.byref(d), _stream()), "ffn_forward")
    return out


def ffn_workspace_views(workspace, M: int, F: int):
    """(g, u) fp32 [M][F] views of an FFN workspace after the call."""
    torch = _torch()
    gb = (4 * M * F + 255) // 256 * 256
    g = workspace[: 4 * M * F].view(torch.float32).view(M, F)
    u = workspace[gb: gb + 4 * M * F].view(torch.float32).view(M, F)
    return g, u


DTYPES = {"f32": 0, "bf16": 1, "f16": 2}


def _io_dtype(t):
    torch = _torch()
    m = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}
    if t not in m:
        raise TypeError(f"unsupported activation type {t}")
    return m[t]


def forward_io(x, packed, w_scale: float, gamma, eps: float = 1e-6, N: int | None = None,
               y_dtype=None, out=None, workspace=None):
    """forward() with x and y in float32 / bfloat16 / float16 (x's dtype is
    read from the tensor; y_dtype defaults to x's)."""
    torch = _torch()
    M, K = x.shape
    if N is None:
        N = (packed.numel() - 32) * 4 // K
    if out is None:
        out = torch.empty((M, N), dtype=y_dtype or x.dtype, device=x.device)
    if workspace is None:
        workspace = torch.empty(int(lib().bitlinear_io_workspace_bytes(M, K, N)),
                                dtype=torch.uint8, device=x.device)
    if not (x.is_cuda and x.is_contiguous() and out.is_cuda and out.is_contiguous()):
        raise ValueError("x and out must be contiguous HIP tensors")
    _check(lib().bitlinear_forward_io(
        ctypes.c_void_p(x.data_ptr()), _io_dtype(x.dtype), _dev(packed, torch.uint8, "packed"),
        w_scale, _gamma(gamma), eps, M, K, N, ctypes.c_void_p(out.data_ptr()),
        _io_dtype(out.dtype), _dev(workspace, torch.uint8, "workspace"), workspace.numel(),
        _stream()), "forward_io")
    return out


def io_workspace(M: int, K: int, N: int, device="cuda"):
    torch = _torch()
    return torch.empty(int(lib().bitlinear_io_workspace_bytes(M, K, N)), dtype=torch.uint8,
                       device=device)


def forward_io_batch(items):
    """Several typed forwards: items of (x, packed, w_scale, gamma, eps, out,
    workspace) with x / out float32, bfloat16 or float16 tensors; per item
    bit-identical to forward_io()."""
    torch = _torch()
    arr = (IoDesc * len(items))()
    for i, (x, packed, w_scale, gamma, eps, out, ws) in enumerate(items):
        M, K = x.shape
        N = out.shape[1]
        if not (x.is_cuda and x.is_contiguous() and out.is_cuda and out.is_contiguous()):
            raise ValueError("x and out must be contiguous HIP tensors")
        arr[i] = IoDesc(x.data_ptr(), _io_dtype(x.dtype), _dev(packed, torch.uint8, "packed"),
                        w_scale, _gamma(gamma), eps, M, K, N, out.data_ptr(), _io_dtype(out.dtype),
                        _dev(ws, torch.uint8, "workspace"), ws.numel())
    _check(lib().bitlinear_forward_io_batch(arr, len(items), _stream()), "forward_io_batch")


def dequant_i2s(packed, N: int, K: int, dtype=None):
    """Dense W [N][K] = (code - 1) * scale in float32 / bfloat16 / float16."""
    torch = _torch()
    dtype = dtype or torch.float32
    w = torch.empty((N, K), dtype=dtype, device=packed.device)
    _check(lib().bitlinear_dequant_i2s(_dev(packed, torch.uint8, "packed"), N, K,
                                       ctypes.c_void_p(w.data_ptr()), _io_dtype(dtype), _stream()),
           "dequant_i2s")
    return w
