"""Pins of the oracle's half-precision activation I/O (bf16 / fp16 x and y).

Page: huggingface/transformers PR #38087 "Add optional RMSNorm support to
BitNet quantization (config + layers)" (the layer's activations; the page
fixes no storage type).  Reading: x is widened exactly to fp32, the fp32
path runs unchanged, and y is rounded to the output type to nearest with
ties to even.  The checks use values whose roundings are derived by hand.
"""
import numpy as np
import pytest

from ternary_bit_linear_amd import workloads as wl


def bits(f):
    return int(np.float32(f).view(np.uint32))


def test_bf16_widening_is_the_high_half(orc):
    b = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x4049, 0x7F80, 0x0001], np.uint16)
    f = orc.bf16_to_f32(b)
    assert [int(v) for v in f.view(np.uint32)] == [int(x) << 16 for x in b]
    assert f[0] == 1.0 and f[1] == -1.0 and f[4] == np.float32(3.140625)
    assert np.isinf(f[5]) and f[6] == np.float32(2.0 ** -133)


def test_bf16_rounding_hand_values(orc):
    """bf16 keeps 7 fraction bits: at 1.0 the spacing is 2^-7."""
    cases = [
        (1.0, 0x3F80),
        (1 + 2.0 ** -8, 0x3F80),               # tie between 1 and 1 + 2^-7: even (1)
        (1 + 3 * 2.0 ** -8, 0x3F82),           # tie between 1 + 2^-7 and 1 + 2^-6: even
        (1 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),  # just above the tie: up
        (1 + 2.0 ** -8 - 2.0 ** -20, 0x3F80),  # just below: down
        (-(1 + 3 * 2.0 ** -8), 0xBF82),        # sign symmetric
        (3.4e38, 0x7F80),                      # past the largest finite bf16: inf
        (0.0, 0x0000),
    ]
    got = orc.f32_to_bf16(np.array([c for c, _ in cases], np.float32))
    assert [int(g) for g in got] == [e for _, e in cases]
    nan = orc.f32_to_bf16(np.array([np.float32("nan")]))[0]
    assert (int(nan) & 0x7F80) == 0x7F80 and (int(nan) & 0x007F) != 0


def test_bf16_round_trip_and_order(orc):
    """Every finite bf16 value survives widening and rounding unchanged, and
    rounding keeps the order of the inputs (monotone)."""
    b = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    assert np.array_equal(orc.f32_to_bf16(orc.bf16_to_f32(b)), b)
    rng = np.random.default_rng(4)
    v = np.sort(rng.standard_normal(5000).astype(np.float32))
    r = orc.bf16_to_f32(orc.f32_to_bf16(v))
    assert np.all(np.diff(r) >= 0)
    assert np.all(np.abs(r - v) <= 2.0 ** -8 * np.abs(v))


def test_f16_rounding_hand_values(orc):
    """fp16 keeps 10 fraction bits: 1 + 2^-11 ties to 1, 1 + 3 * 2^-11 to
    1 + 2^-9; 65520 rounds to inf."""
    y = orc.from_f32(np.array([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 65520.0, 65504.0],
                              np.float32), "f16")
    assert y.dtype == np.float16
    assert y[0] == 1.0 and y[1] == np.float16(1 + 2.0 ** -9)
    assert np.isinf(y[2]) and y[3] == 65504.0


@pytest.mark.parametrize("xd,yd", [("bf16", "bf16"), ("f16", "f16"), ("bf16", "f32"),
                                   ("f32", "bf16")])
def test_forward_io_is_the_f32_path_on_widened_inputs(orc, xd, yd):
    """x of a half type gives exactly the codes of its fp32 widening, and y
    is the fp32 output rounded once: checked against values built by hand
    from the widening (x = small integers / 64, exact in every type) and a
    power-of-two identity weight, where y = s * x exactly."""
    K = 128
    m = (np.arange(2 * K).reshape(2, K) % 255 - 127).astype(np.float32)
    m[:, 0] = -127.0  # amax 127: inv = 1, q = m
    xf = m / np.float32(64.0)
    x = orc.from_f32(xf, xd)
    assert np.array_equal(orc.to_f32(x, xd), xf)
    packed, s = orc.pack_i2s(np.eye(K, dtype=np.float32) * np.float32(0.5))
    y = orc.forward_io(x, xd, packed, s, None, 1e-6, K, yd)
    # no norm: q = m, inv = 127 / (127/64) = 64, y = m * (0.5 / 64) = xf / 2
    assert np.array_equal(orc.to_f32(y, yd), xf / np.float32(2.0))


def test_forward_io_with_norm_matches_rounded_f32(orc):
    """With RMSNorm: the output is the fp32 BitLinear output of the widened
    input, rounded; the rounding moves it by at most half a unit in the
    last place of the output type (relative 2^-8 for bf16)."""
    M, K, N = 3, 256, 96
    xf = wl.activations(31, M, K)
    x = orc.from_f32(xf, "bf16")
    w, _ = wl.ternary(32, N, K, 1 / 3, 0.02)
    g = wl.gamma(33, K, "u0.8-1.2")
    packed, s = orc.pack_i2s(w)
    y = orc.to_f32(orc.forward_io(x, "bf16", packed, s, g, 1e-6, N, "bf16"), "bf16")
    y64 = orc.forward(orc.to_f32(x, "bf16"), packed, s, g, 1e-6, N)
    assert np.all(np.abs(y - y64) <= 2.0 ** -8 * np.abs(y64) * (1 + 1e-5))


def test_dequant_hand_values(orc):
    """(code - 1) * s rounded once: s = 0.1 (fp32 0x3DCCCCCD) is 0x3DCD in
    bf16 (dropped half 0xCCCD > 0x8000 rounds up) and 0x2E66 in fp16."""
    t = np.array([[1, 0, -1, 1] * 32, [0, -1, 0, 1] * 32], np.float32)
    w = t * np.float32(0.1)
    packed, s = orc.pack_i2s(w)
    assert s == np.float32(0.1)
    b = orc.dequant_i2s(packed, 2, 128, "bf16")
    expect_b = np.where(t > 0, 0x3DCD, np.where(t < 0, 0xBDCD, 0)).astype(np.uint16)
    assert np.array_equal(b, expect_b)
    h = orc.dequant_i2s(packed, 2, 128, "f16").view(np.uint16)
    expect_h = np.where(t > 0, 0x2E66, np.where(t < 0, 0xAE66, 0)).astype(np.uint16)
    assert np.array_equal(h, expect_h)
    f = orc.dequant_i2s(packed, 2, 128, "f32")
    assert np.array_equal(f, w)
