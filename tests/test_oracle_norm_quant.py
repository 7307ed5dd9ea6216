"""Pins of the oracle's RMSNorm + per-token int8 quantisation.

Pages: huggingface/transformers PR #38087 "Add optional RMSNorm support to
BitNet quantization (config + layers)", "What does this PR do?" (RMSNorm on
the activations before quantisation, rms_norm_eps default 1e-6); eejd/
cpp-bitnet PR #7 NEON-kernel commit (int8 activations and their sum).

The pages give no formula; the closed forms and fp64 checks below pin the
textbook RMSNorm x / sqrt(mean(x^2) + eps) * gamma and the symmetric absmax
int8 quantisation q = round(xn * 127 / amax).
"""
import numpy as np
import pytest

U = 2.0 ** -24  # fp32 unit roundoff


def rms64(x, g, eps):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * np.asarray(g, np.float64)


def test_sumsq_exact_on_integers(orc):
    """Small integers: every partial sum is exact, so any order gives the
    true sum of squares."""
    rng = np.random.default_rng(0)
    for K in (128, 256, 2560, 6912):
        v = rng.integers(-8, 9, K).astype(np.float32)
        assert orc.sumsq(v) == np.float32(np.sum(v.astype(np.int64) ** 2))


def test_sumsq_pinned_order(orc):
    """Hand-derived values that only the pinned O256 order gives: 256 fmaf
    chains (chain (k/4) % 256, increasing k), a halving tree inside each
    group of 64 chains, then (g0 + g1) + (g2 + g3).  Ties round to even at
    2^24, where the fp32 spacing is 2."""
    # fmaf within a chain, in increasing k: 2^-24 first, then a^2 fused
    v = np.zeros(128, np.float32)
    v[0], v[1] = 2.0 ** -12, 1 + 2.0 ** -12
    assert orc.sumsq(v) == np.float32(1 + 2.0 ** -11 + 2.0 ** -23)
    # reversed order inside the chain loses the 2^-24 terms
    v[0], v[1] = 1 + 2.0 ** -12, 2.0 ** -12
    assert orc.sumsq(v) == np.float32(1 + 2.0 ** -11)
    # two ones in chain 0 next to 2^24 are absorbed one by one
    v = np.zeros(128, np.float32)
    v[0], v[1], v[2] = 4096, 1, 1
    assert orc.sumsq(v) == np.float32(2.0 ** 24)
    # ones in chains 1 and 3 meet in the tree before reaching chain 0
    v = np.zeros(128, np.float32)
    v[0], v[4], v[12] = 4096, 1, 1
    assert orc.sumsq(v) == np.float32(2.0 ** 24 + 2)
    # elements 256 and 257 are chain 64 (second group): they are summed
    # first and survive (a 64-chain order would put them in chain 0)
    v = np.zeros(512, np.float32)
    v[0], v[256], v[257] = 4096, 1, 1
    assert orc.sumsq(v) == np.float32(2.0 ** 24 + 2)
    # element 1024 is chain 0 again (chains wrap every 1024 elements)
    v = np.zeros(2048, np.float32)
    v[0], v[1024], v[1025] = 4096, 1, 1
    assert orc.sumsq(v) == np.float32(2.0 ** 24)
    # groups 2 and 3 are added to each other before group 0:
    # (g0 + g1) + (g2 + g3) = 2^24 + 2, while a left-to-right sum gives 2^24
    v = np.zeros(1024, np.float32)
    v[0], v[512], v[768] = 4096, 1, 1
    assert orc.sumsq(v) == np.float32(2.0 ** 24 + 2)


@pytest.mark.parametrize("a", [1.0, -3.0, 0.001, 1e-4, 250.0])
@pytest.mark.parametrize("K", [128, 2560, 6912])
def test_rmsnorm_constant_row(orc, a, K):
    """x = a * ones: xn_k = gamma_k * a / sqrt(a^2 + eps) (closed form)."""
    g = np.linspace(0.8, 1.2, K).astype(np.float32)
    x = np.full((1, K), a, np.float32)
    xn = orc.rmsnorm(x, g, 1e-6)[0].astype(np.float64)
    ref = g.astype(np.float64) * a / np.sqrt(a * a + 1e-6)
    assert np.all(np.abs(xn - ref) <= (K / 256 + 10) * U * np.abs(ref))


@pytest.mark.parametrize("K", [128, 256, 8192])
def test_rmsnorm_one_hot(orc, K):
    """x = a e_j: xn_j = gamma_j a / sqrt(a^2/K + eps), all other entries 0."""
    a, j = 2.5, K // 3
    x = np.zeros((1, K), np.float32)
    x[0, j] = a
    g = np.full(K, 1.1, np.float32)
    xn = orc.rmsnorm(x, g, 1e-6)[0]
    ref = 1.1 * a / np.sqrt(a * a / K + 1e-6)
    assert abs(xn[j] - ref) <= 8 * U * ref
    assert np.count_nonzero(xn) == 1


def test_rmsnorm_zero_row(orc):
    xn = orc.rmsnorm(np.zeros((1, 256), np.float32), np.ones(256, np.float32), 1e-6)
    assert np.all(xn == 0)


@pytest.mark.parametrize("K", [256, 2560, 6912, 8192])
def test_rmsnorm_vs_fp64(orc, K):
    """Random rows over a range of magnitudes (including rows whose mean
    square is comparable to eps, where dropping eps would show) against the
    fp64 textbook formula, within the fp32 error bound of the pinned order:
    K/256 FMA steps per chain + 8 tree levels for the sum, half of that
    through the square root, plus a few roundings."""
    rng = np.random.default_rng(K)
    scales = np.array([1e-4, 1e-3, 3e-3, 1.0, 50.0], np.float32)
    x = (rng.standard_normal((5, K)) * scales[:, None]).astype(np.float32)
    g = rng.uniform(0.8, 1.2, K).astype(np.float32)
    xn = orc.rmsnorm(x, g, 1e-6).astype(np.float64)
    ref = rms64(x, g, 1e-6)
    bound = ((K / 256 + 8) / 2 + 6) * U
    rel = np.abs(xn - ref) / np.abs(ref).max(axis=1, keepdims=True)
    assert rel.max() <= bound
    # eps matters for the small rows: the formula without eps is far off
    no_eps = rms64(x, g, 0.0)
    assert np.abs(no_eps[0] - ref[0]).max() > 100 * bound * np.abs(ref[0]).max()


def test_quant_amax_maps_to_127_and_symmetry(orc):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 2560)).astype(np.float32)
    g = rng.uniform(0.8, 1.2, 2560).astype(np.float32)
    q, inv, qsum = orc.act_quant(x, g, 1e-6)
    xn = orc.rmsnorm(x, g, 1e-6)
    for m in range(6):
        j = np.argmax(np.abs(xn[m]))
        assert abs(int(q[m, j])) == 127 and np.sign(q[m, j]) == np.sign(xn[m, j])
        assert inv[m] == np.float32(127.0) / np.abs(xn[m]).max()
    assert np.abs(q.astype(np.int32)).max() <= 127
    assert np.array_equal(qsum, q.astype(np.int64).sum(axis=1))
    qn, invn, qsumn = orc.act_quant(-x, g, 1e-6)
    assert np.array_equal(qn, -q) and np.array_equal(invn, inv) and np.array_equal(qsumn, -qsum)


def test_quant_zero_row(orc):
    x = np.zeros((2, 256), np.float32)
    x[1, 7] = 1.0
    q, inv, qsum = orc.act_quant(x, np.ones(256, np.float32), 1e-6)
    assert np.all(q[0] == 0) and qsum[0] == 0
    assert inv[0] == np.float32(127.0) / np.float32(1e-5)
    assert q[1, 7] == 127 and qsum[1] == 127


def tie_case():
    """A row where r = 1 exactly (x = +-1, K = 128, eps below half an ulp of
    1.0) so xn = x * gamma exactly; gamma_max = 127/64 gives inv = 64
    exactly, and the other gains are t/64, so xn * inv = t exactly."""
    K = 128
    t = np.array([2.5, 3.5, 0.5, 1.5, -2.5, -0.5, 126.5, 4.25, 4.75], np.float64)
    x = np.ones((1, K), np.float32)
    g = np.full(K, 1.0 / 64, np.float32)
    g[0] = 127.0 / 64
    g[1:1 + t.size] = (np.abs(t) / 64).astype(np.float32)
    x[0, 1:1 + t.size] = np.sign(t)
    eps = 2.0 ** -30
    expect = np.array([2, 4, 0, 2, -2, 0, 126, 4, 5], np.int8)
    return x, g, eps, expect, t.size


def test_quant_round_half_even(orc):
    x, g, eps, expect, n = tie_case()
    q, inv, qsum = orc.act_quant(x, g, eps)
    assert inv[0] == 64.0
    assert q[0, 0] == 127
    assert q[0, 1:1 + n].tolist() == expect.tolist()
    assert np.all(q[0, 1 + n:] == 1)


@pytest.mark.parametrize("K", [2560, 8192])
def test_quant_vs_fp64_pipeline(orc, K):
    """q from the fp32 pipeline equals round(xn64 * 127 / amax64) except
    where the fp64 value sits within 1e-4 of a half-integer (where the fp32
    rounding legitimately decides); such cases must be rare."""
    rng = np.random.default_rng(K + 1)
    M = 64
    x = rng.standard_normal((M, K)).astype(np.float32)
    mask = rng.random((M, K)) < 0.01
    x[mask] *= 20
    g = rng.uniform(0.8, 1.2, K).astype(np.float32)
    q, inv, qsum = orc.act_quant(x, g, 1e-6)
    xn = rms64(x, g, 1e-6)
    v = xn * (127.0 / np.abs(xn).max(axis=1, keepdims=True))
    ref = np.round(v)  # numpy rounds half to even
    near = np.abs(np.abs(v - np.floor(v)) - 0.5) < 1e-4
    diff = q.astype(np.float64) != ref
    assert np.all(~diff | near)
    assert diff.sum() <= 1e-4 * q.size + 1
    assert np.abs(q.astype(np.float64) - ref).max() <= 1


# --- the layer without RMSNorm (gamma None: use_rms_norm off) -------------

def test_quant_without_norm_hand_values(orc):
    """amax = 2 gives inv = 63.5 exactly and every product x * 63.5 below is
    exact in fp32, so the codes follow by hand: 31.75 -> 32, 15.875 -> 16,
    63.5 -> 64 (tie to even), -47.625 -> -48, 7.9375 -> 8, 95.25 -> 95."""
    x = np.array([[0.5, -2.0, 0.25, 0.0, 1.0, -0.75, 0.125, 1.5]], np.float32)
    q, inv, qsum = orc.act_quant(x, None, 1e-6)
    assert inv[0] == np.float32(63.5)
    assert q[0].tolist() == [32, -127, 16, 0, 64, -48, 8, 95]
    assert qsum[0] == 40
    # amax = 1: inv = 127 and 0.5 * 127 = 63.5 ties to 64
    x = np.array([[1.0, 0.5, -0.5, 0.25]], np.float32)
    q, inv, qsum = orc.act_quant(x, None, 1e-6)
    assert inv[0] == np.float32(127.0)
    assert q[0].tolist() == [127, 64, -64, 32] and qsum[0] == 159


def test_quant_without_norm_ignores_eps_and_is_not_normalised(orc):
    """With no RMSNorm the result depends on x alone: eps is unused, and a
    power-of-two scaling of x leaves q and qsum unchanged while inv scales
    inversely (all exact in fp32).  The normalised form differs from it on
    a row whose RMS is not 1."""
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((4, 512)) * 3).astype(np.float32)
    q, inv, qsum = orc.act_quant(x, None, 1e-6)
    q2, inv2, qsum2 = orc.act_quant(x, None, 0.5)
    assert np.array_equal(q, q2) and np.array_equal(inv, inv2)
    q4, inv4, qsum4 = orc.act_quant(x * np.float32(4.0), None, 1e-6)
    assert np.array_equal(q4, q) and np.array_equal(qsum4, qsum)
    assert np.array_equal(inv4, inv / np.float32(4.0))
    assert np.array_equal(inv, np.float32(127.0) / np.abs(x).max(axis=1))
    qn, invn, _ = orc.act_quant(x, np.ones(512, np.float32), 1e-6)
    assert not np.array_equal(invn, inv)


def test_quant_without_norm_vs_fp64(orc):
    """q = round(x * 127 / amax) from fp64 except within 1e-4 of a tie."""
    rng = np.random.default_rng(12)
    M, K = 32, 2560
    x = rng.standard_normal((M, K)).astype(np.float32)
    q, inv, qsum = orc.act_quant(x, None, 1e-6)
    v = x.astype(np.float64) * (127.0 / np.abs(x.astype(np.float64)).max(axis=1, keepdims=True))
    ref = np.round(v)
    near = np.abs(np.abs(v - np.floor(v)) - 0.5) < 1e-4
    diff = q.astype(np.float64) != ref
    assert np.all(~diff | near)
    assert np.array_equal(qsum, q.astype(np.int64).sum(axis=1))
