"""The C-ABI library loads, exports every symbol the header declares, and
rejects bad arguments on the host before touching the GPU (no device is
needed: every call below fails validation, so nothing is enqueued)."""
import ctypes
import os
import re

import pytest

from ternary_bit_linear_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitlinear.h")

F = ctypes.c_void_p
A = 0x10000  # a 16-byte aligned fake device address (never dereferenced)
MIS = 0x10004  # a misaligned one


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bitlinear_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(api.LIB_PATH):
        pytest.fail("libbitlinear.so is not built (run __graft_entry__.build())")
    return api.lib()


def test_exports_every_declared_symbol(L):
    names = header_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(api.SIGNATURES), "binding signatures cover the header"


def test_version_and_strings(L):
    assert L.bitlinear_abi_version() == 1
    for st in range(7):
        s = L.bitlinear_status_string(st)
        assert s and s.decode().startswith("BL_")
    assert L.bitlinear_status_string(99) == b"unknown bitlinear status"
    assert L.bitlinear_num_variants(api.PATH_GEMV) >= 2
    assert L.bitlinear_num_variants(api.PATH_GEMM) >= 2
    assert L.bitlinear_num_variants(0) == 0


@pytest.mark.parametrize("N,K,expect", [(1, 128, 64), (640, 2560, 409632), (8192, 28672, 58720288),
                                        (1, 100, 0), (0, 128, 0), (3, 0, 0), (-1, 128, 0)])
def test_packed_bytes(L, N, K, expect):
    assert L.bitlinear_packed_bytes(N, K) == expect


def test_workspace_bytes(L):
    assert L.bitlinear_workspace_bytes(1, 256) == 256 + 256 + 256
    assert L.bitlinear_workspace_bytes(512, 2560) == 512 * 2560 + 2048 + 2048
    assert L.bitlinear_workspace_bytes(0, 256) == 0


def fwd(L, x=A, p=A, s=0.02, g=A, eps=1e-6, M=1, K=256, N=256, y=A, ws=A, wsb=1 << 20, launch=None):
    return L.bitlinear_forward_ex(F(x), F(p), s, F(g), eps, M, K, N, F(y), F(ws), wsb, launch, None)


@pytest.mark.parametrize("M,K,N", [(0, 256, 4), (1, 100, 4), (1, 256, 0), (1, 64, 4),
                                   (-3, 256, 4), (1, 1 << 41, 4), (1, (1 << 22) + 128, 4)])
def test_forward_shape_errors(L, M, K, N):
    assert fwd(L, M=M, K=K, N=N) == api.ERR_SHAPE


@pytest.mark.parametrize("which", ["x", "p", "y", "ws"])
def test_forward_null(L, which):
    assert fwd(L, **{which: 0}) == api.ERR_INVALID_ARG


@pytest.mark.parametrize("eps", [1e-6, 0.0, float("nan")])
def test_forward_null_gamma_is_the_layer_without_norm(L, eps):
    """gamma NULL selects the layer without RMSNorm and eps is then not
    validated: the call gets past both checks to the alignment check (a
    misaligned y stops it there, before anything is enqueued)."""
    assert fwd(L, g=0, eps=eps, y=MIS) == api.ERR_ALIGN


@pytest.mark.parametrize("which", ["x", "p", "g", "y", "ws"])
def test_forward_align(L, which):
    assert fwd(L, **{which: MIS}) == api.ERR_ALIGN


@pytest.mark.parametrize("eps", [0.0, -1e-6, float("inf"), float("nan")])
def test_forward_eps(L, eps):
    assert fwd(L, eps=eps) == api.ERR_INVALID_ARG


def test_forward_workspace(L):
    need = L.bitlinear_workspace_bytes(4, 256)
    assert fwd(L, M=4, wsb=need - 1) == api.ERR_WORKSPACE


@pytest.mark.parametrize("launch", [(3, -1, 0, 0), (0, 2, 0, 0), (1, -1, 99, 0), (0, -1, 1, 0),
                                    (1, -1, 0, 7), (2, 1, 0, 0), (1, -1, -1, 0)])
def test_forward_bad_launch(L, launch):
    lp = ctypes.byref(api.Launch(*launch))
    assert fwd(L, launch=lp) == api.ERR_INVALID_ARG


@pytest.mark.parametrize("path,M", [(api.PATH_GEMV, 1048561), (api.PATH_GEMM, 2097121)])
def test_grid_row_limits(L, path, M):
    """M past the launch grid of a route is a shape error, not a failed launch."""
    lp = ctypes.byref(api.Launch(path, 0, 0, 0))
    assert fwd(L, M=M, K=128, N=4, wsb=1 << 40, launch=lp) == api.ERR_SHAPE


def test_fused_needs_small_m(L):
    lp = ctypes.byref(api.Launch(api.PATH_GEMV, 1, 0, 0))
    assert fwd(L, M=8, wsb=1 << 20, launch=lp) == api.ERR_INVALID_ARG


def test_pack_errors(L):
    assert L.bitlinear_pack_i2s(F(A), 4, 100, F(A), None, None) == api.ERR_SHAPE
    assert L.bitlinear_pack_i2s(F(0), 4, 128, F(A), None, None) == api.ERR_INVALID_ARG
    assert L.bitlinear_pack_i2s(F(A), 4, 128, F(0), None, None) == api.ERR_INVALID_ARG
    assert L.bitlinear_pack_i2s(F(MIS), 4, 128, F(A), None, None) == api.ERR_ALIGN
    assert L.bitlinear_unpack_i2s(F(A), 4, 96, F(A), None) == api.ERR_SHAPE
    assert L.bitlinear_unpack_i2s(F(A), 4, 128, F(MIS), None) == api.ERR_ALIGN
    out = ctypes.c_float()
    assert L.bitlinear_read_scale(F(A), 0, 128, ctypes.byref(out), None) == api.ERR_SHAPE
    assert L.bitlinear_read_scale(F(A), 2, 128, None, None) == api.ERR_INVALID_ARG


def test_stage_errors(L):
    aq = L.bitlinear_act_quant
    assert aq(F(A), F(A), 1e-6, 2, 200, F(A), F(A), F(A), None) == api.ERR_SHAPE
    assert aq(F(0), F(A), 1e-6, 2, 256, F(A), F(A), F(A), None) == api.ERR_INVALID_ARG
    # gamma NULL (no RMSNorm) with eps 0 passes validation up to the alignment check
    assert aq(F(A), F(0), 0.0, 2, 256, F(MIS), F(A), F(A), None) == api.ERR_ALIGN
    assert aq(F(A), F(A), 0.0, 2, 256, F(A), F(A), F(A), None) == api.ERR_INVALID_ARG
    assert aq(F(A), F(A), 1e-6, 2, 256, F(MIS), F(A), F(A), None) == api.ERR_ALIGN
    mm = L.bitlinear_matmul_i2s_ex
    assert mm(F(A), F(A), F(A), 2, 130, 4, F(A), None, None) == api.ERR_SHAPE
    assert mm(F(A), F(0), F(A), 2, 256, 4, F(A), None, None) == api.ERR_INVALID_ARG
    fused = ctypes.byref(api.Launch(api.PATH_GEMV, 1, 0, 0))
    assert mm(F(A), F(A), F(A), 2, 256, 4, F(A), fused, None) == api.ERR_INVALID_ARG
    assert L.bitlinear_matmul_i2s(F(MIS), F(A), F(A), 2, 256, 4, F(A), None) == api.ERR_ALIGN


def test_product_never_imports_oracle():
    """The product package must not reach the oracle (test infrastructure)."""
    pkg = os.path.join(ROOT, "ternary_bit_linear_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"\boracle\b", text.lower()) or f == "workloads.py", f


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(api, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(api, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        api.lib()


def _desc(M=1, K=256, N=16, x=A, p=A, g=A, y=A, ws=A, wsb=1 << 20, eps=1e-6):
    return api.ForwardDesc(x, p, 0.02, g, eps, M, K, N, y, ws, wsb)


def test_forward_batch_validation(L):
    fb = L.bitlinear_forward_batch
    one = (api.ForwardDesc * 1)(_desc())
    assert fb(None, 1, None, None) == api.ERR_INVALID_ARG
    assert fb(one, 0, None, None) == api.ERR_INVALID_ARG
    many = (api.ForwardDesc * 65)(*[_desc() for _ in range(65)])
    assert fb(many, 65, None, None) == api.ERR_INVALID_ARG
    # one bad descriptor anywhere fails the whole call before any launch
    for bad, code in [(_desc(K=100), api.ERR_SHAPE), (_desc(x=0), api.ERR_INVALID_ARG),
                      (_desc(y=MIS), api.ERR_ALIGN), (_desc(wsb=10), api.ERR_WORKSPACE),
                      (_desc(eps=0.0), api.ERR_INVALID_ARG)]:
        arr = (api.ForwardDesc * 3)(_desc(), _desc(M=2, K=512), bad)
        assert fb(arr, 3, None, None) == code
    lp = ctypes.byref(api.Launch(api.PATH_GEMM, 1, 0, 0))
    assert fb(one, 1, lp, None) == api.ERR_INVALID_ARG


def _ffn(x=A, gi=A, pg=A, pu=A, pd=A, gs=A, eps=1e-6, M=1, H=256, F=512, y=A, ws=A,
         wsb=1 << 24, sg=0.02, su=0.02, sd=0.02):
    return api.FfnDesc(x, gi, pg, sg, pu, su, pd, sd, gs, eps, M, H, F, y, ws, wsb)


def test_ffn_workspace_bytes(L):
    al = lambda v: (v + 255) // 256 * 256  # noqa: E731
    M, H, F = 4, 256, 640
    expect = 2 * al(4 * M * F) + 2 * al(L.bitlinear_workspace_bytes(M, H)) + \
        al(L.bitlinear_workspace_bytes(M, F))
    assert L.bitlinear_ffn_workspace_bytes(M, H, F) == expect
    # rows longer than 8192 also hold a = relu(g)^2 * u
    F = 9216
    expect = 3 * al(4 * M * F) + 2 * al(L.bitlinear_workspace_bytes(M, H)) + \
        al(L.bitlinear_workspace_bytes(M, F))
    assert L.bitlinear_ffn_workspace_bytes(M, H, F) == expect
    assert L.bitlinear_ffn_workspace_bytes(0, H, F) == 0
    assert L.bitlinear_ffn_workspace_bytes(M, 100, F) == 0
    assert L.bitlinear_ffn_workspace_bytes(M, H, 100) == 0


@pytest.mark.parametrize("kw,code", [
    ({"M": 0}, api.ERR_SHAPE), ({"H": 200}, api.ERR_SHAPE), ({"F": 130}, api.ERR_SHAPE),
    ({"x": 0}, api.ERR_INVALID_ARG), ({"pg": 0}, api.ERR_INVALID_ARG),
    ({"pu": 0}, api.ERR_INVALID_ARG), ({"pd": 0}, api.ERR_INVALID_ARG),
    ({"y": 0}, api.ERR_INVALID_ARG), ({"ws": 0}, api.ERR_INVALID_ARG),
    ({"eps": 0.0}, api.ERR_INVALID_ARG), ({"eps": float("nan")}, api.ERR_INVALID_ARG),
    ({"sd": float("inf")}, api.ERR_INVALID_ARG),
    ({"x": MIS}, api.ERR_ALIGN), ({"gi": MIS}, api.ERR_ALIGN), ({"gs": MIS}, api.ERR_ALIGN),
    ({"pd": MIS}, api.ERR_ALIGN), ({"y": MIS}, api.ERR_ALIGN), ({"ws": MIS}, api.ERR_ALIGN),
    ({"wsb": 1000}, api.ERR_WORKSPACE),
    # no RMSNorm anywhere: eps is not checked, the call reaches the alignment check
    ({"gi": 0, "gs": 0, "eps": 0.0, "y": MIS}, api.ERR_ALIGN)])
def test_ffn_validation(L, kw, code):
    d = _ffn(**kw)
    assert L.bitlinear_ffn_forward(ctypes.byref(d), None) == code
    assert L.bitlinear_ffn_forward(None, None) == api.ERR_INVALID_ARG


def test_io_workspace_bytes(L):
    al = lambda v: (v + 255) // 256 * 256  # noqa: E731
    assert L.bitlinear_io_workspace_bytes(3, 256, 77) == al(L.bitlinear_workspace_bytes(3, 256)) + al(4 * 3 * 77)
    assert L.bitlinear_io_workspace_bytes(0, 256, 4) == 0
    assert L.bitlinear_io_workspace_bytes(2, 100, 4) == 0


def fio(L, x=A, xd=1, p=A, s=0.02, g=A, eps=1e-6, M=1, K=256, N=256, y=A, yd=1, ws=A,
        wsb=1 << 20):
    return L.bitlinear_forward_io(F(x), xd, F(p), s, F(g), eps, M, K, N, F(y), yd, F(ws), wsb, None)


@pytest.mark.parametrize("kw,code", [
    ({"M": 0}, api.ERR_SHAPE), ({"K": 100}, api.ERR_SHAPE), ({"N": 0}, api.ERR_SHAPE),
    ({"x": 0}, api.ERR_INVALID_ARG), ({"p": 0}, api.ERR_INVALID_ARG),
    ({"y": 0}, api.ERR_INVALID_ARG), ({"ws": 0}, api.ERR_INVALID_ARG),
    ({"xd": 3}, api.ERR_INVALID_ARG), ({"yd": -1}, api.ERR_INVALID_ARG),
    ({"eps": 0.0}, api.ERR_INVALID_ARG), ({"s": float("nan")}, api.ERR_INVALID_ARG),
    ({"x": MIS}, api.ERR_ALIGN), ({"y": MIS}, api.ERR_ALIGN), ({"g": MIS}, api.ERR_ALIGN),
    ({"wsb": 100}, api.ERR_WORKSPACE),
    ({"g": 0, "eps": 0.0, "y": MIS}, api.ERR_ALIGN)])
def test_forward_io_validation(L, kw, code):
    assert fio(L, **kw) == code


def test_forward_io_batch_validation(L):
    fb = L.bitlinear_forward_io_batch
    good = api.IoDesc(A, 1, A, 0.02, A, 1e-6, 1, 256, 16, A, 1, A, 1 << 20)
    bad = api.IoDesc(A, 7, A, 0.02, A, 1e-6, 1, 256, 16, A, 1, A, 1 << 20)
    assert fb(None, 1, None) == api.ERR_INVALID_ARG
    assert fb((api.IoDesc * 1)(good), 0, None) == api.ERR_INVALID_ARG
    assert fb((api.IoDesc * 65)(*[good] * 65), 65, None) == api.ERR_INVALID_ARG
    # one bad descriptor fails the whole call before anything is enqueued
    assert fb((api.IoDesc * 3)(good, good, bad), 3, None) == api.ERR_INVALID_ARG
    mis = api.IoDesc(A, 1, A, 0.02, A, 1e-6, 1, 256, 16, MIS, 1, A, 1 << 20)
    assert fb((api.IoDesc * 2)(good, mis), 2, None) == api.ERR_ALIGN


def test_dequant_validation(L):
    dq = L.bitlinear_dequant_i2s
    assert dq(F(A), 4, 100, F(A), 1, None) == api.ERR_SHAPE
    assert dq(F(0), 4, 128, F(A), 1, None) == api.ERR_INVALID_ARG
    assert dq(F(A), 4, 128, F(0), 1, None) == api.ERR_INVALID_ARG
    assert dq(F(A), 4, 128, F(A), 5, None) == api.ERR_INVALID_ARG
    assert dq(F(A), 4, 128, F(MIS), 2, None) == api.ERR_ALIGN


def test_fp32_ops_validation(L):
    fo = L.bitlinear_fp32_ops
    assert fo(0, F(A), F(0), 0.0, 0, F(A), None) == api.ERR_SHAPE
    assert fo(4, F(A), F(A), 0.0, 8, F(A), None) == api.ERR_INVALID_ARG
    assert fo(-1, F(A), F(A), 0.0, 8, F(A), None) == api.ERR_INVALID_ARG
    assert fo(0, F(0), F(0), 0.0, 8, F(A), None) == api.ERR_INVALID_ARG
    assert fo(3, F(A), F(0), 0.0, 8, F(0), None) == api.ERR_INVALID_ARG
    assert fo(1, F(A), F(0), 0.0, 8, F(A), None) == api.ERR_INVALID_ARG  # division needs b
    assert fo(2, F(A), F(0), 1e-6, 8, F(A), None) == api.ERR_INVALID_ARG
    assert fo(2, F(A), F(A), float("inf"), 8, F(A), None) == api.ERR_INVALID_ARG


def test_forward_noalloc_validation(L):
    """Host-side checks of the allocation-free forward run before the scratch
    array is looked up (no device is touched here)."""
    fn = L.bitlinear_forward_noalloc
    assert api.NOALLOC_SCRATCH_BYTES == (16 << 20) + (64 << 10)

    def call(x=A, p=A, s=0.02, g=A, eps=1e-6, M=1, K=256, N=256, y=A):
        return fn(F(x), F(p), s, F(g), eps, M, K, N, F(y), None)
    assert call(M=0) == api.ERR_SHAPE
    assert call(K=100) == api.ERR_SHAPE
    assert call(x=0) == api.ERR_INVALID_ARG
    assert call(y=0) == api.ERR_INVALID_ARG
    assert call(eps=0.0) == api.ERR_INVALID_ARG
    assert call(s=float("inf")) == api.ERR_INVALID_ARG
    assert call(y=MIS) == api.ERR_ALIGN
    # beyond the scratch array: 16 MiB of q plus inv / qsum
    assert call(M=2048, K=8192 + 128) == api.ERR_WORKSPACE
    assert call(M=(16 << 20) // 128 + 1, K=128) == api.ERR_WORKSPACE


def test_probe_validation(L):
    assert L.bitlinear_probe_read_sink_words(0) == 0
    assert L.bitlinear_probe_read_sink_words(100) == 0
    assert L.bitlinear_probe_read_sink_words(32768) == 1
    assert L.bitlinear_probe_read_sink_words(32768 + 16) == 2
    pr = L.bitlinear_probe_read
    assert pr(F(A), 100, F(A), 10, None) == api.ERR_SHAPE
    assert pr(F(0), 1 << 20, F(A), 1 << 10, None) == api.ERR_INVALID_ARG
    assert pr(F(A), 1 << 20, F(A), 31, None) == api.ERR_INVALID_ARG  # needs 32 words
    assert pr(F(MIS), 1 << 20, F(A), 32, None) == api.ERR_ALIGN
    pm = L.bitlinear_probe_mfma
    assert pm(0, 4, F(A), 1024, None) == api.ERR_SHAPE
    assert pm(10, 0, F(A), 1024, None) == api.ERR_SHAPE
    assert pm(10, 4, F(A), 1023, None) == api.ERR_INVALID_ARG
    assert pm(10, 4, F(0), 1024, None) == api.ERR_INVALID_ARG
