"""The allocation-free forward (bitlinear_forward_noalloc, for callers that
cannot allocate device memory) against bitlinear_forward: the same bits,
and the oracle's values within 1e-5, on consecutive calls whose sizes
shrink, so each call runs over the scratch contents the previous one left.
"""
import sys

import numpy as np
import pytest

from ternary_bit_linear_amd import workloads as wl

pytestmark = pytest.mark.gpu


def announce(*a):
    print("[gpu-case]", *a, file=sys.__stderr__, flush=True)


@pytest.fixture(scope="module")
def torch():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return torch


@pytest.fixture(scope="module")
def bl(torch):
    from ternary_bit_linear_amd import api
    api.lib()
    return api


def case(seed, M, K, N, norm=True):
    x = wl.activations(seed, M, K, 0.01)
    w, _ = wl.ternary(seed + 1, N, K, 0.4, 0.015)
    g = wl.gamma(seed + 2, K, "u0.8-1.2") if norm else None
    return x, w, g


def test_forward_noalloc_matches_forward(torch, bl, orc):
    # largest block the scratch array holds (M * K = 16 MiB, prefill tile
    # route), then smaller ones: few tokens, one token (fused decode), a
    # long row, one token without RMSNorm
    shapes = [(2048, 8192, 64, True), (64, 2560, 640, True), (4, 1024, 77, True),
              (1, 2560, 300, True), (2, 28672, 48, True), (1, 6912, 130, False)]
    for i, (M, K, N, norm) in enumerate(shapes):
        announce("forward_noalloc", M, K, N, norm)
        x, w, g = case(1700 + 10 * i, M, K, N, norm)
        packed, s = orc.pack_i2s(w)
        X = torch.from_numpy(x).cuda()
        P = torch.from_numpy(packed).cuda()
        G = None if g is None else torch.from_numpy(g).cuda()
        y_na = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        bl.forward_noalloc(X, P, s, G, 1e-6, y_na)
        torch.cuda.synchronize()
        y_ref = bl.forward(X, P, s, G, 1e-6, N)
        torch.cuda.synchronize()
        a, b = y_na.cpu().numpy(), y_ref.cpu().numpy()
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (M, K, N)
        y64 = orc.forward(x, packed, s, g, 1e-6, N)
        assert np.all(np.isfinite(a))
        zero = y64 == 0
        assert np.all(a[zero] == 0)
        assert np.all(np.abs(a - y64) <= 1e-5 * np.abs(y64)), (M, K, N)


def test_forward_noalloc_rejects_beyond_scratch(torch, bl):
    M, K, N = 2048, 8192 + 128, 16
    x = torch.zeros((M, K), dtype=torch.float32, device="cuda")
    P = torch.zeros(N * K // 4 + 32, dtype=torch.uint8, device="cuda")
    y = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    with pytest.raises(bl.BitLinearError) as e:
        bl.forward_noalloc(x, P, 1.0, None, 1e-6, y)
    assert e.value.status == bl.ERR_WORKSPACE
