"""GPU parity: every stage of the HIP path against the CPU oracle.

Integer results (packed bytes, int8 q, int32 qsum/acc) and the fp32 inv are
compared bit for bit; fp32 y within 1e-5 relative of the oracle's fp64 y
(and exactly 0 where the oracle's is 0).  Shapes span several tiles and
ragged tails; the full-size workloads are checked on sampled outputs.
"""
import sys

import numpy as np
import pytest

from ternary_bit_linear_amd import workloads as wl

pytestmark = pytest.mark.gpu

RTOL = 1e-5


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


def dev(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.cpu().numpy()


def check_y(y, y64):
    y = np.asarray(y, np.float64)
    assert y.shape == y64.shape
    assert np.all(np.isfinite(y)), "unwritten or non-finite outputs"
    zero = y64 == 0
    assert np.all(y[zero] == 0)
    err = np.abs(y - y64)
    bad = err > RTOL * np.abs(y64)
    assert not bad.any(), f"{bad.sum()} outputs beyond 1e-5 rel; max rel {np.max(err[~zero] / np.abs(y64[~zero]))}"


# ---------------------------------------------------------------- packing

PACK_SHAPES = [(1, 128), (3, 256), (17, 384), (100, 1024), (640, 2560), (2560, 6912)]


@pytest.mark.parametrize("N,K", PACK_SHAPES)
def test_pack_parity(torch, bl, orc, N, K):
    announce("pack", N, K)
    w, _ = wl.ternary(100 + N, N, K, 1 / 3, 0.02)
    ref, s_ref = orc.pack_i2s(w)
    packed, s = bl.pack_i2s(dev(torch, w))
    torch.cuda.synchronize()
    assert s == s_ref
    assert np.array_equal(host(packed), ref)
    assert bl.read_scale(packed, N, K) == s_ref
    back = bl.unpack_i2s(packed, N, K)
    torch.cuda.synchronize()
    assert np.array_equal(host(back), w)


def test_pack_full_size(torch, bl, orc):
    """The packing workload: fp32 ternary x 0.02, N = 8192 x K = 28672."""
    N, K = wl.PACK_SHAPE
    announce("pack full", N, K)
    w, _ = wl.ternary(5000, N, K, 1 / 3, 0.02)
    ref, s_ref = orc.pack_i2s(w)
    packed, s = bl.pack_i2s(dev(torch, w))
    torch.cuda.synchronize()
    assert s == s_ref
    assert np.array_equal(host(packed), ref)


def test_pack_golden(torch, bl):
    from tests.test_oracle_pack import golden_weights, load_golden
    for c in load_golden():
        announce("pack golden", c["name"])
        packed, s = bl.pack_i2s(dev(torch, golden_weights(c)))
        torch.cuda.synchronize()
        nb = c["N"] * c["K"] // 4
        assert host(packed)[:nb].tolist() == c["bytes"].tolist()
        assert host(packed)[nb:].tolist() == c["trailer"].tolist()


@pytest.mark.parametrize("bad", ["two_magnitudes", "nan", "inf"])
def test_pack_not_ternary(torch, bl, bad):
    announce("pack not ternary", bad)
    w = np.zeros((4, 256), np.float32)
    w[0, 3], w[3, 255] = 0.5, -0.5
    w[2, 100] = {"two_magnitudes": 0.25, "nan": np.nan, "inf": np.inf}[bad]
    with pytest.raises(bl.BitLinearError) as e:
        bl.pack_i2s(dev(torch, w))
    assert e.value.status == bl.ERR_NOT_TERNARY


def test_pack_all_zero(torch, bl):
    announce("pack zero")
    packed, s = bl.pack_i2s(torch.zeros((5, 384), dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    p = host(packed)
    assert s == 0.0 and np.all(p[:5 * 96] == 0x55) and np.all(p[5 * 96:] == 0)


# ---------------------------------------------------------------- RMSNorm + int8

# Rows past 8192 in launches of at most one row per CU take the 1024-thread
# form (8320: a ragged last chain segment; 12288 / 16384: four float4 groups
# per thread; 28672: eight); 300 rows of 9216 keep the 256-thread form.
AQ_CASES = [(1, 128, 0.0), (1, 256, 0.0), (3, 384, 0.0), (4, 2560, 0.01), (5, 6912, 0.0),
            (16, 8192, 0.01), (64, 2560, 0.01), (7, 28672, 0.0), (33, 640, 0.0),
            (3, 8320, 0.01), (2, 12288, 0.0), (16, 16384, 0.01), (300, 9216, 0.0),
            # rows past 32768 are streamed (three passes); the longest row the
            # library takes, K = 2^22
            (3, 40960, 0.01), (2, 1 << 22, 0.0)]


@pytest.mark.parametrize("M,K,outl", AQ_CASES)
def test_act_quant_parity(torch, bl, orc, M, K, outl):
    announce("act_quant", M, K, outl)
    x = wl.activations(200 + M + K, M, K, outl)
    x[0] *= np.float32(1e-3)  # a row whose mean square is near eps
    g = wl.gamma(201, K, "u0.8-1.2")
    q_r, inv_r, qs_r = orc.act_quant(x, g, 1e-6)
    q, inv, qs = bl.act_quant(dev(torch, x), dev(torch, g), 1e-6)
    torch.cuda.synchronize()
    assert np.array_equal(host(q), q_r)
    assert np.array_equal(host(inv).view(np.uint32), inv_r.view(np.uint32))
    assert np.array_equal(host(qs), qs_r)


def test_act_quant_ties_and_zero_rows(torch, bl, orc):
    from tests.test_oracle_norm_quant import tie_case
    announce("act_quant ties")
    x, g, eps, expect, n = tie_case()
    x = np.concatenate([x, np.zeros_like(x), -x])
    q, inv, qs = bl.act_quant(dev(torch, x), dev(torch, g), eps)
    torch.cuda.synchronize()
    q = host(q)
    assert q[0, 1:1 + n].tolist() == expect.tolist()
    assert np.all(q[1] == 0) and host(qs)[1] == 0
    assert np.array_equal(q[2], -q[0])
    q_r, inv_r, qs_r = orc.act_quant(x, g, eps)
    assert np.array_equal(q, q_r) and np.array_equal(host(inv), inv_r)


# ---------------------------------------------------------------- contraction

def mm_case(M, K, N, seed):
    x = wl.activations(seed, M, K, 0.01)
    w, t = wl.ternary(seed + 1, N, K, 0.4, 0.015)
    g = wl.gamma(seed + 2, K, "u0.8-1.2")
    return x, w, t, g


MM_SHAPES = [(1, 128, 16), (1, 256, 100), (2, 384, 33), (5, 2560, 640), (16, 1024, 48),
             (17, 384, 70), (31, 256, 64), (32, 640, 129), (33, 1280, 31), (64, 2560, 256),
             (65, 384, 300), (130, 1152, 200), (16, 4096, 40), (9, 8192, 33),
             (2, 1 << 22, 16)]  # the longest row the library takes


@pytest.mark.parametrize("path", [1, 2])
@pytest.mark.parametrize("M,K,N", MM_SHAPES)
def test_matmul_parity(torch, bl, orc, path, M, K, N):
    announce("matmul", path, M, K, N)
    x, w, t, g = mm_case(M, K, N, 300 + M + N)
    packed_r, _ = orc.pack_i2s(w)
    q, inv, qs = orc.act_quant(x, g, 1e-6)
    acc_r = orc.matmul_i2s(q, qs, packed_r, N)
    assert np.array_equal(acc_r.astype(np.int64), q.astype(np.int64) @ t.astype(np.int64).T)
    P = dev(torch, packed_r)
    Q, QS = dev(torch, q), dev(torch, qs)
    for v in range(1, bl.num_variants(path) + 1):
        acc = bl.matmul_i2s(Q, QS, P, N, path=path, variant=v)
        torch.cuda.synchronize()
        assert np.array_equal(host(acc), acc_r), f"variant {v}"


FWD_SHAPES = [(1, 256, 256), (1, 2560, 640), (2, 384, 100), (3, 1024, 77), (4, 6912, 160),
              (7, 512, 513), (10, 2560, 300), (12, 1024, 129), (15, 6912, 200), (16, 2560, 256),
              (17, 256, 64), (63, 640, 333), (64, 1024, 200), (100, 384, 90),
              (1, 1 << 22, 3), (3, 65536, 40),  # rows past 32768, up to the longest
              (1, 128, 1 << 18), (20000, 256, 16),  # a wide single token, a tall batch
              # 2..4 tokens past 64 KB of q (tile route, 16x32 tiles in k groups;
              # the last with a half step of K and a step count that 4 does not divide)
              (4, 28672, 100), (2, 40960, 48), (3, 22656, 50)]


@pytest.mark.parametrize("M,K,N", FWD_SHAPES)
def test_forward_parity(torch, bl, orc, M, K, N):
    announce("forward", M, K, N)
    x, w, t, g = mm_case(M, K, N, 400 + M + K)
    packed_r, s = orc.pack_i2s(w)
    y64 = orc.forward(x, packed_r, s, g, 1e-6, N)
    X, P, G = dev(torch, x), dev(torch, packed_r), dev(torch, g)
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    ws = bl.new_workspace(M, K)
    y = bl.forward(X, P, s, G, 1e-6, N, out=out, workspace=ws)
    torch.cuda.synchronize()
    check_y(host(y), y64)
    # the workspace holds this call's q / inv / qsum
    q_r, inv_r, qs_r = orc.act_quant(x, g, 1e-6)
    q, inv, qs = bl.workspace_views(ws, M, K)
    assert np.array_equal(host(q), q_r) and np.array_equal(host(inv), inv_r)
    assert np.array_equal(host(qs), qs_r)
    # every route / fusion / launch shape gives the same bits
    ref = host(y).copy()
    opts = [(1, 0, 0), (2, 0, 0)] + [(2, 0, v) for v in range(1, bl.num_variants(2) + 1)]
    opts += [(1, 0, v) for v in range(1, bl.num_variants(1) + 1)]
    if M <= 4 and M * K <= 32768:
        opts += [(1, 1, v) for v in range(1, bl.num_variants(1) + 1)]
    for path, fuse, v in opts:
        out.fill_(float("nan"))
        y2 = bl.forward(X, P, s, G, 1e-6, N, out=out, workspace=ws, path=path, fuse=fuse, variant=v)
        torch.cuda.synchronize()
        assert np.array_equal(host(y2), ref), (path, fuse, v)


def test_forward_quant_is_applied(torch, bl, orc):
    """The output is the quantised path's, not a plain fp32 x W^T."""
    M, K, N = 2, 1024, 64
    x, w, t, g = mm_case(M, K, N, 77)
    packed_r, s = orc.pack_i2s(w)
    y = host(bl.forward(dev(torch, x), dev(torch, packed_r), s, dev(torch, g), 1e-6, N))
    xn = orc.rmsnorm(x, g, 1e-6).astype(np.float64)
    plain = xn @ w.astype(np.float64).T
    assert np.abs(y - plain).max() > 1e-4 * np.abs(plain).max()
    check_y(y, orc.forward(x, packed_r, s, g, 1e-6, N))


def test_forward_zero_weights_and_identity(torch, bl, orc):
    announce("forward special W")
    K = 256
    x = wl.activations(88, 3, K)
    g = np.ones(K, np.float32)
    P0, s0 = bl.pack_i2s(torch.zeros((16, K), dtype=torch.float32, device="cuda"))
    y0 = host(bl.forward(dev(torch, x), P0, s0, dev(torch, g), 1e-6, 16))
    assert np.all(y0 == 0)
    PI, sI = bl.pack_i2s(torch.eye(K, dtype=torch.float32, device="cuda") * 0.5)
    yI = host(bl.forward(dev(torch, x), PI, sI, dev(torch, g), 1e-6, K))
    q, inv, _ = orc.act_quant(x, g, 1e-6)
    check_y(yI, q.astype(np.float64) * (0.5 / inv.astype(np.float64))[:, None])


# ---------------------------------------------------------------- full-size workloads

def run_linear(torch, bl, orc, work, i, sample_rows=None, sample_cols=None):
    L = work.linears[i]
    announce("workload", work.name, L.name, L.M, L.K, L.N)
    x, w, t, g = work.inputs(i)
    X, G = dev(torch, x), dev(torch, g)
    P, s = bl.pack_i2s(dev(torch, w))
    ws = bl.new_workspace(L.M, L.K)
    # y starts as NaN, so an output the kernels leave unwritten cannot pass
    # as a finite leftover of the allocator.
    out = torch.full((L.M, L.N), float("nan"), dtype=torch.float32, device="cuda")
    y = host(bl.forward(X, P, s, G, work.eps, L.N, out=out, workspace=ws))
    assert np.all(np.isfinite(y)), f"{np.sum(~np.isfinite(y))} outputs unwritten or non-finite"
    q_r, inv_r, qs_r = orc.act_quant(x, g, work.eps)
    q, inv, qs = (host(a) for a in bl.workspace_views(ws, L.M, L.K))
    assert np.array_equal(q, q_r) and np.array_equal(inv, inv_r) and np.array_equal(qs, qs_r)
    # every row of the sampled columns (and the sampled rows of every
    # column when rows are sampled): |acc| < 2^24, so the fp64 products and
    # sums below are exact
    cols = np.arange(L.N) if sample_cols is None else sample_cols
    acc = q_r.astype(np.float64) @ t[cols].astype(np.float64).T
    y64 = acc * (np.float64(s) / inv_r.astype(np.float64))[:, None]
    check_y(y[:, cols], y64)
    if sample_rows is not None:
        acc = q_r[sample_rows].astype(np.float64) @ t.astype(np.float64).T
        y64 = acc * (np.float64(s) / inv_r[sample_rows].astype(np.float64))[:, None]
        check_y(y[sample_rows], y64)
    return y


@pytest.mark.parametrize("i", range(7))
def test_workload_decode_layer(torch, bl, orc, i):
    run_linear(torch, bl, orc, wl.DECODE_LAYER, i)


@pytest.mark.parametrize("i", range(7))
def test_workload_prefill_layer(torch, bl, orc, i):
    L = wl.PREFILL_LAYER.linears[i]
    rng = np.random.default_rng(i)
    rows = np.unique(np.concatenate([[0, L.M - 1], rng.integers(0, L.M, 14)]))
    cols = np.unique(np.concatenate([[0, L.N - 1], rng.integers(0, L.N, 500)]))
    run_linear(torch, bl, orc, wl.PREFILL_LAYER, i, rows, cols)


@pytest.mark.parametrize("M", [1, 16])
@pytest.mark.parametrize("i", range(3))
def test_workload_ffn70b(torch, bl, orc, M, i):
    work = wl.ffn70b(M)
    L = work.linears[i]
    rng = np.random.default_rng(i + M)
    cols = np.unique(np.concatenate([[0, L.N - 1], rng.integers(0, L.N, 3000)]))
    run_linear(torch, bl, orc, work, i, None, cols)


# M = 1024: the 128 x 256 tiles at one per CU (rows of 8192); the rest as
# the bench's sweep.
@pytest.mark.parametrize("M", list(wl.SWEEP_M) + [1024])
def test_workload_sweep(torch, bl, orc, M):
    work = wl.sweep(M)
    rng = np.random.default_rng(M)
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 12)]))
    cols = np.unique(np.concatenate([[0, 8191], rng.integers(0, 8192, 1000)]))
    run_linear(torch, bl, orc, work, 0, rows, cols)


def test_graph_replay_matches_eager(torch, bl, orc):
    """A captured HIP graph of several forwards (decode fused, decode staged,
    prefill) replayed repeatedly, with eager work in between, gives the eager
    bits every time."""
    cases = [(1, 2560, 640), (8, 1024, 96), (40, 512, 130)]
    data = []
    for i, (M, K, N) in enumerate(cases):
        x, w, t, g = mm_case(M, K, N, 900 + i)
        P, s = bl.pack_i2s(dev(torch, w))
        X, G = dev(torch, x), dev(torch, g)
        out = torch.empty((M, N), dtype=torch.float32, device="cuda")
        ws = bl.new_workspace(M, K)
        data.append((X, P, s, G, N, out, ws))
    eager = []
    for X, P, s, G, N, out, ws in data:
        eager.append(host(bl.forward(X, P, s, G, 1e-6, N, out=out, workspace=ws)).copy())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for X, P, s, G, N, out, ws in data:
            bl.forward(X, P, s, G, 1e-6, N, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for X, P, s, G, N, out, ws in data:
            bl.forward(X, P, s, G, 1e-6, N, out=out, workspace=ws)
    for rep in range(4):
        announce("graph replay", rep)
        for _, _, _, _, _, out, _ in data:
            out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for (X, P, s, G, N, out, ws), ref in zip(data, eager):
            assert np.array_equal(host(out), ref), rep
        # eager work between replays
        bl.forward(*data[0][:4], 1e-6, data[0][4], out=torch.empty_like(data[0][5]))
        torch.cuda.synchronize()


def test_act_quant_order_sensitive_rows(torch, bl, orc):
    """Rows whose fp32 sum of squares depends on the summation order (the
    hand-derived values pinned in the oracle tests), through both GPU
    quantisation paths (separate kernel and fused decode prologue)."""
    K = 2048
    rows = []
    for idx in ([0, 1], [0, 4, 12], [0, 1, 2], [0, 256, 257], [0, 1024, 1025], [0, 512, 768]):
        v = np.zeros(K, np.float32)
        v[idx[0]] = 4096 if len(idx) > 2 else 2.0 ** -12
        for i in idx[1:]:
            v[i] = 1.0 if len(idx) > 2 else 1 + 2.0 ** -12
        rows.append(v)
    x = np.stack(rows)
    g = np.ones(K, np.float32)
    q_r, inv_r, qs_r = orc.act_quant(x, g, 1e-6)
    q, inv, qs = bl.act_quant(dev(torch, x), dev(torch, g), 1e-6)
    assert np.array_equal(host(q), q_r) and np.array_equal(host(qs), qs_r)
    assert np.array_equal(host(inv).view(np.uint32), inv_r.view(np.uint32))
    P, s = bl.pack_i2s(torch.ones((16, K), dtype=torch.float32, device="cuda"))
    for m in range(len(rows)):
        ws = bl.new_workspace(1, K)
        bl.forward(dev(torch, x[m:m + 1]), P, s, dev(torch, g), 1e-6, 16, workspace=ws, path=1, fuse=1)
        torch.cuda.synchronize()
        qf, invf, qsf = bl.workspace_views(ws, 1, K)
        assert np.array_equal(host(qf)[0], q_r[m]) and host(qsf)[0] == qs_r[m]
        assert host(invf).view(np.uint32)[0] == inv_r.view(np.uint32)[m]


def test_forward_batch_matches_single_calls(torch, bl, orc):
    """A batch mixing fused decode problems (several K/N, M = 1..4), an
    unfused decode problem and a prefill problem gives, per problem, the
    bits of the single call; more than 8 fused problems span launches."""
    shapes = [(1, 2560, 640), (1, 6912, 300), (3, 1024, 77), (1, 256, 16), (8, 512, 96),
              (40, 384, 130), (1, 2560, 2560), (2, 768, 33), (1, 1024, 48), (1, 512, 1000),
              (4, 256, 17), (1, 128, 8)]
    items, singles, refs = [], [], []
    for i, (M, K, N) in enumerate(shapes):
        x, w, t, g = mm_case(M, K, N, 700 + i)
        packed_r, s = orc.pack_i2s(w)
        X, P, G = dev(torch, x), dev(torch, packed_r), dev(torch, g)
        out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        ws = bl.new_workspace(M, K)
        items.append((X, P, s, G, 1e-6, out, ws))
        singles.append(host(bl.forward(X, P, s, G, 1e-6, N)).copy())
        refs.append(orc.forward(x, packed_r, s, g, 1e-6, N))
    announce("forward_batch", len(items))
    bl.forward_batch(items)
    torch.cuda.synchronize()
    for (X, P, s, G, eps, out, ws), single, y64, (M, K, N) in zip(items, singles, refs, shapes):
        assert np.array_equal(host(out), single), (M, K, N)
        check_y(host(out), y64)
        q, inv, qs = bl.workspace_views(ws, M, K)
        q_r, inv_r, qs_r = orc.act_quant(host(X), host(G), 1e-6)
        assert np.array_equal(host(q), q_r) and np.array_equal(host(inv), inv_r)
        assert np.array_equal(host(qs), qs_r)
    # every launch shape of the fused route gives the same bits
    fused = [(it, single) for it, single, sh in zip(items, singles, shapes) if sh[0] <= 4]
    for v in range(1, bl.num_variants(1) + 1):
        for it, _ in fused:
            it[5].fill_(float("nan"))
        bl.forward_batch([it for it, _ in fused], path=1, variant=v)
        torch.cuda.synchronize()
        for it, single in fused:
            assert np.array_equal(host(it[5]), single), v


@pytest.mark.parametrize("norm", [True, False])
def test_decode_every_shape_wide_workgroups(torch, bl, orc, norm):
    """One-token decode batches whose rows take K splits of 1, 2 and 4 waves
    and ragged N, forced through every launch shape -- the 4-wave shapes and
    the 8- and 16-wave workgroups, where only the first four waves normalise
    and quantise and the others meet their barriers -- and the persistent
    form: y bit for bit the same in every shape and within 1e-5 of the
    oracle; the first workgroup's q / inv / qsum are the oracle's."""
    shapes = [(2560, 640), (6912, 2560), (8192, 1000), (1024, 200), (384, 40), (2560, 6912)]
    items, refs, xs = [], [], []
    for i, (K, N) in enumerate(shapes):
        x, w, t, g = mm_case(1, K, N, 1700 + 7 * i + (0 if norm else 3))
        gg = g if norm else None
        packed_r, s = orc.pack_i2s(w)
        refs.append(orc.forward(x, packed_r, s, gg, 1e-6, N))
        X, P = dev(torch, x), dev(torch, packed_r)
        G = dev(torch, g) if norm else None
        out = torch.full((1, N), float("nan"), dtype=torch.float32, device="cuda")
        items.append((X, P, s, G, 1e-6, out, bl.new_workspace(1, K)))
        xs.append((x, gg, K))
    announce("decode every shape", norm)
    bl.forward_batch(items)
    torch.cuda.synchronize()
    ref_bits = [host(it[5]).copy() for it in items]
    for y, y64 in zip(ref_bits, refs):
        check_y(y, y64)
    for v in range(1, bl.num_variants(1) + 1):
        for it in items:
            it[5].fill_(float("nan"))
            it[6].fill_(0)
        bl.forward_batch(items, path=1, variant=v)
        torch.cuda.synchronize()
        for it, y, (x, gg, K) in zip(items, ref_bits, xs):
            assert np.array_equal(host(it[5]), y), v
            q, inv, qs = bl.workspace_views(it[6], 1, K)
            q_r, inv_r, qs_r = orc.act_quant(x, gg, 1e-6)
            assert np.array_equal(host(q), q_r) and np.array_equal(host(inv), inv_r), v
            assert np.array_equal(host(qs), qs_r), v


# Rolling form: one token with the 1024-thread quantisation (rows up to
# 32768, K a multiple of 1024 or not), q from the workspace for up to 8
# tokens; K splits of 1..16 waves per tile group, ragged N.
ROLL_CASES = [(1, 28672, 100, True), (1, 28672, 1500, True), (1, 6912, 1000, True),
              (1, 2560, 77, False), (1, 16384, 333, True), (1, 4096, 2048, True),
              (1, 640, 9000, True), (3, 4096, 500, True), (8, 8192, 64, True),
              (2, 28672, 40, False)]


@pytest.mark.parametrize("M,K,N,norm", ROLL_CASES)
def test_roll_parity(torch, bl, orc, M, K, N, norm):
    """The rolling form, forced, fused (one token) and over q from the
    workspace: within 1e-5 of the oracle and the same bits as the automatic
    route; the fused launch's first workgroup leaves the oracle's q / inv /
    qsum in the workspace."""
    announce("roll", M, K, N, norm)
    x, w, t, g = mm_case(M, K, N, 3100 + M + K + N)
    gg = g if norm else None
    packed_r, s = orc.pack_i2s(w)
    y64 = orc.forward(x, packed_r, s, gg, 1e-6, N)
    q_r, inv_r, qs_r = orc.act_quant(x, gg, 1e-6)
    X, P = dev(torch, x), dev(torch, packed_r)
    G = dev(torch, g) if norm else None
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    ws = bl.new_workspace(M, K)
    ref = host(bl.forward(X, P, s, G, 1e-6, N, out=out, workspace=ws)).copy()
    check_y(ref, y64)
    vroll = bl.num_variants(1)
    for fuse in ((1, 0) if M == 1 else (0,)):
        out.fill_(float("nan"))
        ws.fill_(0)
        y = host(bl.forward(X, P, s, G, 1e-6, N, out=out, workspace=ws, path=1, fuse=fuse,
                            variant=vroll))
        assert np.array_equal(y, ref), fuse
        q, inv, qs = bl.workspace_views(ws, M, K)
        assert np.array_equal(host(q), q_r) and np.array_equal(host(inv), inv_r), fuse
        assert np.array_equal(host(qs), qs_r), fuse


def test_roll_batch_mixed_rows(torch, bl, orc):
    """One rolling launch over problems of different row lengths (different
    K splits and quantisation segments per problem): each output the same
    bits as its single call and within 1e-5 of the oracle."""
    shapes = [(8192, 3000), (28672, 700), (2560, 5000), (6912, 1200)]
    items, singles, refs = [], [], []
    for i, (K, N) in enumerate(shapes):
        x, w, t, g = mm_case(1, K, N, 3300 + i)
        packed_r, s = orc.pack_i2s(w)
        refs.append(orc.forward(x, packed_r, s, g, 1e-6, N))
        X, P, G = dev(torch, x), dev(torch, packed_r), dev(torch, g)
        out = torch.full((1, N), float("nan"), dtype=torch.float32, device="cuda")
        ws = bl.new_workspace(1, K)
        singles.append(host(bl.forward(X, P, s, G, 1e-6, N, out=out, workspace=ws)).copy())
        items.append((X, P, s, G, 1e-6, out, ws))
    announce("roll batch")
    for it in items:
        it[5].fill_(float("nan"))
    bl.forward_batch(items, path=1, variant=bl.num_variants(1))
    torch.cuda.synchronize()
    for it, single, y64 in zip(items, singles, refs):
        assert np.array_equal(host(it[5]), single)
        check_y(host(it[5]), y64)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_forward_io_decode_layer(torch, bl, orc, dt):
    """The decoder layer's seven BitLinears at full size, one token, x and y
    in bf16 / fp16, as one typed batch (one fused launch): y bit for bit the
    oracle's."""
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[dt]
    work = wl.DECODE_LAYER
    items, refs = [], []
    for i, L in enumerate(work.linears):
        x32, w, t, g = work.inputs(i)
        x = orc.from_f32(x32, dt)
        packed_r, s = orc.pack_i2s(w)
        refs.append(orc.forward_io(x, dt, packed_r, s, g, work.eps, L.N, dt))
        out = torch.empty((L.M, L.N), dtype=tdt, device="cuda")
        items.append((torch_io(torch, x, dt), dev(torch, packed_r), s, dev(torch, g), work.eps,
                      out, bl.io_workspace(L.M, L.K, L.N)))
    announce("forward_io decode layer", dt)
    bl.forward_io_batch(items)
    torch.cuda.synchronize()
    for it, ref, L in zip(items, refs, work.linears):
        assert np.array_equal(bits16(torch, it[5]), np.asarray(ref).view(np.uint16)), L


def test_forward_batch_grouped_prefill(torch, bl, orc):
    """Prefill-sized problems of a batch (K a whole number of 256-k steps,
    K <= 8192) go out as one batched quantisation launch and one grouped
    tile-kernel launch per 8; each gives the bits of its single call.  The
    batch spans two groups (10 such problems, ragged M and N, K from 256 to
    8192) and mixes in problems that cannot join a group (K % 256 != 0,
    K > 8192) and a fused decode problem."""
    shapes = [(64, 256, 128), (70, 2560, 200), (130, 512, 17), (257, 768, 640), (5, 6912, 96),
              (512, 2560, 130), (96, 8192, 64), (33, 1024, 1000), (300, 256, 33), (65, 2560, 640),
              (40, 384, 130), (20, 8448, 48), (1, 2560, 256)]
    items, singles, refs = [], [], []
    for i, (M, K, N) in enumerate(shapes):
        x, w, t, g = mm_case(M, K, N, 900 + i)
        packed_r, s = orc.pack_i2s(w)
        X, P, G = dev(torch, x), dev(torch, packed_r), dev(torch, g)
        out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        ws = bl.new_workspace(M, K)
        items.append((X, P, s, G, 1e-6, out, ws))
        singles.append(host(bl.forward(X, P, s, G, 1e-6, N)).copy())
        refs.append(orc.forward(x, packed_r, s, g, 1e-6, N))
    announce("forward_batch grouped prefill", len(items))
    bl.forward_batch(items)
    torch.cuda.synchronize()
    for (X, P, s, G, eps, out, ws), single, y64, (M, K, N) in zip(items, singles, refs, shapes):
        assert np.array_equal(host(out), single), (M, K, N)
        check_y(host(out), y64)
        q, inv, qs = bl.workspace_views(ws, M, K)
        q_r, inv_r, qs_r = orc.act_quant(host(X), host(G), 1e-6)
        assert np.array_equal(host(q), q_r) and np.array_equal(host(inv), inv_r)
        assert np.array_equal(host(qs), qs_r)
    # the same prefill problems forced onto the tile route one by one
    for it, single, (M, K, N) in zip(items, singles, shapes):
        if M < 5:
            continue
        it[5].fill_(float("nan"))
        bl.forward_batch([it], path=2, variant=1)
        torch.cuda.synchronize()
        assert np.array_equal(host(it[5]), single), (M, K, N)


def run_batch(torch, bl, orc, work, sample=None):
    """Every BitLinear of a workload as one forward_batch call (the launch
    configuration bench.py times); outputs checked against the oracle, on
    sampled rows and columns when `sample` (rows, cols per linear) is set."""
    items, data = [], []
    for i, L in enumerate(work.linears):
        x, w, t, g = work.inputs(i)
        X, G = dev(torch, x), dev(torch, g)
        P, s = bl.pack_i2s(dev(torch, w))
        out = torch.full((L.M, L.N), float("nan"), dtype=torch.float32, device="cuda")
        ws = bl.new_workspace(L.M, L.K)
        items.append((X, P, s, G, work.eps, out, ws))
        data.append((L, x, t, g, s))
    announce("forward_batch", work.name, len(items))
    bl.forward_batch(items)
    torch.cuda.synchronize()
    for i, ((X, P, s, G, eps, out, ws), (L, x, t, g, s_)) in enumerate(zip(items, data)):
        y = host(out)
        assert np.all(np.isfinite(y)), L.name
        q_r, inv_r, qs_r = orc.act_quant(x, g, work.eps)
        q, inv, qs = (host(a) for a in bl.workspace_views(ws, L.M, L.K))
        assert np.array_equal(q, q_r) and np.array_equal(inv, inv_r) and np.array_equal(qs, qs_r)
        rows, cols = (np.arange(L.M), np.arange(L.N)) if sample is None else sample(i, L)
        acc = q_r[rows].astype(np.int64) @ t[cols].astype(np.int64).T
        y64 = acc * (np.float64(s) / inv_r[rows].astype(np.float64))[:, None]
        check_y(y[np.ix_(rows, cols)], y64)


def test_workload_decode_layer_batched(torch, bl, orc):
    run_batch(torch, bl, orc, wl.DECODE_LAYER)


def test_workload_prefill_layer_batched(torch, bl, orc):
    def sample(i, L):
        rng = np.random.default_rng(50 + i)
        rows = np.unique(np.concatenate([[0, L.M - 1], rng.integers(0, L.M, 14)]))
        cols = np.unique(np.concatenate([[0, L.N - 1], rng.integers(0, L.N, 500)]))
        return rows, cols
    run_batch(torch, bl, orc, wl.PREFILL_LAYER, sample)


@pytest.mark.parametrize("M,K,N", [(1024, 256, 2048), (64, 4352, 16384), (2048, 256, 8192),
                                   (512, 6144, 8192),
                                   # 32x32x32 kernel below 256 tokens: 64x128 tiles,
                                   # 128x128 in two k groups, 128x256 tiles
                                   (192, 4096, 8192), (128, 4096, 24576), (192, 4096, 24576),
                                   (96, 4096, 16384)])
def test_forward_batch_group_tiles(torch, bl, orc, M, K, N):
    """The grouped tile launch with each of its larger tile shapes (by the
    group's tile counts): sampled outputs against the oracle, all outputs
    bitwise against the single call."""
    x, w, t, g = mm_case(M, K, N, 990 + M)
    packed_r, s = orc.pack_i2s(w)
    X, P, G = dev(torch, x), dev(torch, packed_r), dev(torch, g)
    single = host(bl.forward(X, P, s, G, 1e-6, N)).copy()
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    ws = bl.new_workspace(M, K)
    announce("forward_batch group tile", M, K, N)
    bl.forward_batch([(X, P, s, G, 1e-6, out, ws)])
    torch.cuda.synchronize()
    y = host(out)
    assert np.array_equal(y, single)
    rng = np.random.default_rng(M + N)
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, 30)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, 300)]))
    q_r, inv_r, qs_r = orc.act_quant(x, g, 1e-6)
    acc = q_r[rows].astype(np.int64) @ t[cols].astype(np.int64).T
    y64 = acc * (np.float64(s) / inv_r[rows].astype(np.float64))[:, None]
    check_y(y[np.ix_(rows, cols)], y64)


def test_graph_replay_forward_batch_new_inputs(torch, bl, orc):
    """forward_batch captured once in a HIP graph (one-shot decode launch plus
    a grouped prefill launch pair) and replayed with new activations copied
    into the same buffers between replays: every replay matches the eager
    batch on those inputs and the oracle, so no launch keeps state from an
    earlier one."""
    shapes = [(1, 2560, 640), (1, 6912, 256), (2, 1024, 96), (64, 2560, 200), (130, 512, 96)]
    data = []
    for i, (M, K, N) in enumerate(shapes):
        x, w, t, g = mm_case(M, K, N, 1500 + i)
        packed_r, s = orc.pack_i2s(w)
        X, P, G = dev(torch, x), dev(torch, packed_r), dev(torch, g)
        out = torch.empty((M, N), dtype=torch.float32, device="cuda")
        data.append([X, P, s, G, out, bl.new_workspace(M, K), packed_r, g])
    items = lambda: [(d[0], d[1], d[2], d[3], 1e-6, d[4], d[5]) for d in data]  # noqa: E731
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bl.forward_batch(items())
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        bl.forward_batch(items())
    for rep in range(3):
        announce("graph replay forward_batch", rep)
        xs = [wl.activations(1600 + 10 * rep + i, M, K, 0.01) for i, (M, K, N) in enumerate(shapes)]
        for d, x in zip(data, xs):
            d[0].copy_(torch.from_numpy(x))
            d[4].fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [host(d[4]).copy() for d in data]
        # eager batch on the same inputs
        outs = [torch.full_like(d[4], float("nan")) for d in data]
        bl.forward_batch([(d[0], d[1], d[2], d[3], 1e-6, o, d[5]) for d, o in zip(data, outs)])
        torch.cuda.synchronize()
        for d, x, y, o, (M, K, N) in zip(data, xs, got, outs, shapes):
            assert np.array_equal(y, host(o)), (rep, M, K, N)
            check_y(y, orc.forward(x, d[6], d[2], d[7], 1e-6, N))


# ---------------------------------------------------------------- no RMSNorm

NONORM_AQ = [(1, 128), (3, 1024), (4, 2560), (16, 8192), (2, 28672), (33, 640)]


@pytest.mark.parametrize("M,K", NONORM_AQ)
def test_act_quant_without_norm_parity(torch, bl, orc, M, K):
    """gamma None (use_rms_norm off): x is quantised as it is; the one-wave,
    block and streamed-row forms all match the oracle bit for bit."""
    announce("act_quant no-norm", M, K)
    x = wl.activations(900 + M + K, M, K, 0.01)
    x[0] *= np.float32(1e-3)
    q_r, inv_r, qs_r = orc.act_quant(x, None, 1e-6)
    q, inv, qs = bl.act_quant(dev(torch, x), None, 0.0)
    torch.cuda.synchronize()
    assert np.array_equal(host(q), q_r)
    assert np.array_equal(host(inv).view(np.uint32), inv_r.view(np.uint32))
    assert np.array_equal(host(qs), qs_r)


def test_act_quant_without_norm_hand_values(torch, bl):
    announce("act_quant no-norm hand values")
    x = np.zeros((2, 128), np.float32)
    x[0, :8] = [0.5, -2.0, 0.25, 0.0, 1.0, -0.75, 0.125, 1.5]
    x[1, :4] = [1.0, 0.5, -0.5, 0.25]
    q, inv, qs = bl.act_quant(dev(torch, x), None, 1e-6)
    torch.cuda.synchronize()
    q, inv, qs = host(q), host(inv), host(qs)
    assert inv[0] == np.float32(63.5) and inv[1] == np.float32(127.0)
    assert q[0, :8].tolist() == [32, -127, 16, 0, 64, -48, 8, 95] and qs[0] == 40
    assert q[1, :4].tolist() == [127, 64, -64, 32] and qs[1] == 159
    assert np.all(q[0, 8:] == 0) and np.all(q[1, 4:] == 0)


NONORM_FWD = [(1, 2560, 640), (1, 6912, 300), (3, 1024, 77), (4, 8192, 64), (1, 28672, 64),
              (17, 256, 64), (64, 1024, 200)]


@pytest.mark.parametrize("M,K,N", NONORM_FWD)
def test_forward_without_norm_parity(torch, bl, orc, M, K, N):
    """The layer without RMSNorm through every route, fusion and launch
    shape: the same bits each time, within 1e-5 of the oracle."""
    announce("forward no-norm", M, K, N)
    x, w, t, g = mm_case(M, K, N, 950 + M + K)
    packed_r, s = orc.pack_i2s(w)
    y64 = orc.forward(x, packed_r, s, None, 1e-6, N)
    X, P = dev(torch, x), dev(torch, packed_r)
    out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
    ws = bl.new_workspace(M, K)
    y = bl.forward(X, P, s, None, 1e-6, N, out=out, workspace=ws)
    torch.cuda.synchronize()
    check_y(host(y), y64)
    q_r, inv_r, qs_r = orc.act_quant(x, None, 1e-6)
    q, inv, qs = bl.workspace_views(ws, M, K)
    assert np.array_equal(host(q), q_r) and np.array_equal(host(inv), inv_r)
    assert np.array_equal(host(qs), qs_r)
    ref = host(y).copy()
    opts = [(1, 0, 0), (2, 0, 0)] + [(2, 0, v) for v in range(1, bl.num_variants(2) + 1)]
    opts += [(1, 0, v) for v in range(1, bl.num_variants(1) + 1)]
    if M <= 4 and M * K <= 32768:
        opts += [(1, 1, v) for v in range(1, bl.num_variants(1) + 1)]
    for path, fuse, v in opts:
        out.fill_(float("nan"))
        y2 = bl.forward(X, P, s, None, 1e-6, N, out=out, workspace=ws, path=path, fuse=fuse,
                        variant=v)
        torch.cuda.synchronize()
        assert np.array_equal(host(y2), ref), (path, fuse, v)


def test_forward_without_norm_identity_exact(torch, bl, orc):
    """Integer rows with amax 127 through W = s I: y = s x exactly, on the
    fused decode route (M = 1) and the tile route (M = 64)."""
    K = 128
    packed_r, s = orc.pack_i2s(np.eye(K, dtype=np.float32) * np.float32(0.25))
    P = dev(torch, packed_r)
    for M in (1, 64):
        announce("forward no-norm identity", M)
        x = (np.arange(M * K, dtype=np.int64).reshape(M, K) % 255 - 127).astype(np.float32)
        x[:, 0] = -127.0
        y = host(bl.forward(dev(torch, x), P, s, None, 1e-6, K))
        torch.cuda.synchronize()
        assert np.array_equal(y, x * np.float32(0.25))


def test_forward_batch_mixes_norm_and_no_norm(torch, bl, orc):
    """A batch where some problems have RMSNorm and some not, on the fused
    decode launch and the grouped prefill launches: each matches its single
    call and the oracle."""
    shapes = [(1, 2560, 640, True), (1, 2560, 640, False), (1, 6912, 256, False),
              (64, 2560, 256, False), (64, 2560, 256, True), (32, 1024, 96, False)]
    items, singles, refs = [], [], []
    for i, (M, K, N, norm) in enumerate(shapes):
        x, w, t, g = mm_case(M, K, N, 980 + i)
        packed_r, s = orc.pack_i2s(w)
        X, P = dev(torch, x), dev(torch, packed_r)
        G = dev(torch, g) if norm else None
        out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        ws = bl.new_workspace(M, K)
        items.append((X, P, s, G, 1e-6, out, ws))
        singles.append(host(bl.forward(X, P, s, G, 1e-6, N)).copy())
        refs.append(orc.forward(x, packed_r, s, g if norm else None, 1e-6, N))
    announce("forward_batch norm/no-norm", len(items))
    bl.forward_batch(items)
    torch.cuda.synchronize()
    for it, single, y64, sh in zip(items, singles, refs, shapes):
        assert np.array_equal(host(it[5]), single), sh
        check_y(host(it[5]), y64)


# ---------------------------------------------------------------- FFN block

def ffn_case(seed, M, H, F, norm=True):
    x = wl.activations(seed, M, H, 0.01)
    gi = wl.gamma(seed + 1, H, "u0.8-1.2") if norm else None
    gs = wl.gamma(seed + 2, F, "u0.8-1.2") if norm else None
    wg, _ = wl.ternary(seed + 3, F, H, 1 / 3, 0.02)
    wu, _ = wl.ternary(seed + 4, F, H, 1 / 3, 0.015)
    wd, _ = wl.ternary(seed + 5, H, F, 1 / 3, 0.025)
    return x, gi, gs, wg, wu, wd


# (M, H, F, norm): M = 1 with F <= 8192 takes the two-launch form (the down
# projection's quantisation inside the one-shot kernel); F > 8192 and M > 1
# take the separate gated quantisation; M <= 8 with M * H and M * F up to
# 64 KB the one-shot kernel for all three projections (M = 2, 3: gate and up
# with the quantisation fused in, groups of four waves per row); M = 64 the
# tile kernel.
FFN_SHAPES = [(1, 2560, 6912, True), (1, 256, 384, False), (1, 1024, 9216, True),
              (3, 512, 1280, True), (2, 2560, 6912, True), (8, 2560, 6912, True),
              (6, 1024, 2816, False),
              (17, 256, 384, True), (64, 1024, 2816, True), (64, 256, 640, False)]


@pytest.mark.parametrize("M,H,F,norm", FFN_SHAPES)
def test_ffn_parity(torch, bl, orc, M, H, F, norm):
    """Gate / up outputs and the down projection's int8 codes bit for bit,
    y within 1e-5 of the oracle's fp64 block."""
    announce("ffn", M, H, F, norm)
    x, gi, gs, wg, wu, wd = ffn_case(1000 + M + F, M, H, F, norm)
    gate, up, down = orc.pack_i2s(wg), orc.pack_i2s(wu), orc.pack_i2s(wd)
    y64, g_r, u_r, a_r = orc.ffn(x, gi, 1e-6, gate, up, down, gs)
    dv = lambda a: None if a is None else dev(torch, a)  # noqa: E731
    D = [(dev(torch, p), s) for p, s in (gate, up, down)]
    ws = torch.empty(bl.ffn_workspace_bytes(M, H, F), dtype=torch.uint8, device="cuda")
    out = torch.full((M, H), float("nan"), dtype=torch.float32, device="cuda")
    y = bl.ffn_forward(dev(torch, x), dv(gi), 1e-6, D[0], D[1], D[2], dv(gs), out=out,
                       workspace=ws)
    torch.cuda.synchronize()
    g, u = bl.ffn_workspace_views(ws, M, F)
    assert np.array_equal(host(g).view(np.uint32), g_r.view(np.uint32))
    assert np.array_equal(host(u).view(np.uint32), u_r.view(np.uint32))
    check_y(host(y), y64)
    # the same call again gives the same bits
    out2 = bl.ffn_forward(dev(torch, x), dv(gi), 1e-6, D[0], D[1], D[2], dv(gs))
    torch.cuda.synchronize()
    assert np.array_equal(host(out2), host(y))


def test_ffn_down_codes_match_oracle(torch, bl, orc):
    """The down projection's q / inv / qsum (formed from g and u inside its
    quantisation, never stored as a) equal the oracle's quantisation of
    relu2_mul(g, u), on both down routes."""
    for M, H, F in ((1, 2560, 6912), (5, 512, 1280)):
        announce("ffn down codes", M, H, F)
        x, gi, gs, wg, wu, wd = ffn_case(1100 + M, M, H, F)
        gate, up, down = orc.pack_i2s(wg), orc.pack_i2s(wu), orc.pack_i2s(wd)
        _, g_r, u_r, a_r = orc.ffn(x, gi, 1e-6, gate, up, down, gs)
        assert np.array_equal(orc.relu2_mul(g_r, u_r), a_r)
        D = [(dev(torch, p), s) for p, s in (gate, up, down)]
        ws = torch.empty(bl.ffn_workspace_bytes(M, H, F), dtype=torch.uint8, device="cuda")
        bl.ffn_forward(dev(torch, x), dev(torch, gi), 1e-6, D[0], D[1], D[2], dev(torch, gs),
                       workspace=ws)
        torch.cuda.synchronize()
        al = lambda v: (v + 255) // 256 * 256  # noqa: E731
        off = 2 * al(4 * M * F) + 2 * al(bl.workspace_bytes(M, H))
        q, inv, qs = bl.workspace_views(ws[off:], M, F)
        q_r, inv_r, qs_r = orc.act_quant(a_r, gs, 1e-6)
        assert np.array_equal(host(q), q_r)
        assert np.array_equal(host(inv).view(np.uint32), inv_r.view(np.uint32))
        assert np.array_equal(host(qs), qs_r)


def test_ffn_structured_closed_form(torch, bl, orc):
    """The selector-weight block of the oracle's pins, on the device."""
    from tests.test_oracle_ffn import structured_case
    for M, H, F, ni, ns in ((2, 128, 256, True, True), (1, 128, 384, False, True)):
        announce("ffn structured", M, H, F)
        x, gi, gs, _, (wg, wu, wd), _, _ = structured_case(40 + M + H, M, H, F, ni, ns)
        gate, up, down = orc.pack_i2s(wg), orc.pack_i2s(wu), orc.pack_i2s(wd)
        y64 = orc.ffn(x, gi, 1e-6, gate, up, down, gs)[0]
        dv = lambda a: None if a is None else dev(torch, a)  # noqa: E731
        D = [(dev(torch, p), s) for p, s in (gate, up, down)]
        y = bl.ffn_forward(dev(torch, x), dv(gi), 1e-6, D[0], D[1], D[2], dv(gs))
        torch.cuda.synchronize()
        check_y(host(y), y64)


def test_ffn_70b_shapes_sampled(torch, bl, orc):
    """The 70B FFN (H = 8192, F = 28672) at M = 1 and 16: gate / up outputs
    checked on sampled columns (the oracle over the sampled weight rows),
    the down projection's codes against the oracle's quantisation of the
    device's g and u, and y on sampled outputs."""
    H, F = 8192, 28672
    rng = np.random.default_rng(5)
    cols = np.sort(rng.choice(F, 24, replace=False))
    outs = np.sort(rng.choice(H, 24, replace=False))
    for M in (1, 16):
        announce("ffn 70b sampled", M)
        x = wl.activations(1200 + M, M, H, 0.01)
        gi = wl.gamma(1201, H, "u0.8-1.2")
        gs = wl.gamma(1202, F, "u0.8-1.2")
        gen = torch.Generator(device="cuda")
        packs = []
        for i, (n, k, sc) in enumerate(((F, H, 0.02), (F, H, 0.015), (H, F, 0.025))):
            gen.manual_seed(1203 + i)
            t = torch.randint(-1, 2, (n, k), generator=gen, device="cuda", dtype=torch.int8)
            w = t.to(torch.float32).mul_(sc)
            del t
            p, s = bl.pack_i2s(w)
            del w
            packs.append((p, s))
        torch.cuda.synchronize()
        ws = torch.empty(bl.ffn_workspace_bytes(M, H, F), dtype=torch.uint8, device="cuda")
        y = host(bl.ffn_forward(dev(torch, x), dev(torch, gi), 1e-6, packs[0], packs[1],
                                packs[2], dev(torch, gs), workspace=ws))
        torch.cuda.synchronize()
        g, u = (host(t) for t in bl.ffn_workspace_views(ws, M, F))
        # gate / up on sampled columns: fp32 outputs, bit for bit
        q, inv, qs = orc.act_quant(x, gi, 1e-6)
        for (p, s), full in ((packs[0], g), (packs[1], u)):
            sub = orc.packed_rows(host(p), H, cols)
            acc = orc.matmul_i2s(q, qs, sub, cols.size)
            assert np.array_equal(orc.rescale_f32(acc, inv, s), full[:, cols])
        # down: codes of relu2_mul(g, u) and sampled outputs
        a = orc.relu2_mul(g, u)
        qa, inva, qsa = orc.act_quant(a, gs, 1e-6)
        sub = orc.packed_rows(host(packs[2][0]), F, outs)
        y64 = orc.rescale(orc.matmul_i2s(qa, qsa, sub, outs.size), inva, packs[2][1])
        check_y(y[:, outs], y64)
        # the down projection's own q / inv / qsum in its part of the
        # workspace (at M = 1 written by the fused launch's first workgroup)
        al = lambda v: (v + 255) // 256 * 256  # noqa: E731
        off = 2 * al(4 * M * F) + 2 * al(bl.workspace_bytes(M, H))
        wq, winv, wqs = bl.workspace_views(ws[off:], M, F)
        assert np.array_equal(host(wq), qa) and np.array_equal(host(winv), inva)
        assert np.array_equal(host(wqs), qsa)
        del packs, ws
        torch.cuda.empty_cache()


def test_ffn_graph_replay(torch, bl, orc):
    """The block captured in a HIP graph and replayed with new inputs
    matches the eager call each time."""
    M, H, F = 1, 2560, 6912
    x, gi, gs, wg, wu, wd = ffn_case(1300, M, H, F)
    gate, up, down = orc.pack_i2s(wg), orc.pack_i2s(wu), orc.pack_i2s(wd)
    D = [(dev(torch, p), s) for p, s in (gate, up, down)]
    X, GI, GS = dev(torch, x), dev(torch, gi), dev(torch, gs)
    ws = torch.empty(bl.ffn_workspace_bytes(M, H, F), dtype=torch.uint8, device="cuda")
    out = torch.empty((M, H), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        bl.ffn_forward(X, GI, 1e-6, D[0], D[1], D[2], GS, out=out, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        bl.ffn_forward(X, GI, 1e-6, D[0], D[1], D[2], GS, out=out, workspace=ws)
    torch.cuda.synchronize()
    announce("ffn graph replay")
    for r in range(3):
        xr = wl.activations(1310 + r, M, H, 0.01)
        X.copy_(dev(torch, xr))
        graph.replay()
        torch.cuda.synchronize()
        got = host(out).copy()
        eager = host(bl.ffn_forward(dev(torch, xr), GI, 1e-6, D[0], D[1], D[2], GS))
        torch.cuda.synchronize()
        assert np.array_equal(got, eager), r
        check_y(got, orc.ffn(xr, gi, 1e-6, gate, up, down, gs)[0])


# ---------------------------------------------------------------- half-precision I/O

IO_SHAPES = [(1, 2560, 640), (3, 1024, 77), (17, 256, 63), (64, 1024, 200), (2, 28672, 48)]
IO_TYPES = [("bf16", "bf16"), ("f16", "f16"), ("bf16", "f32"), ("f32", "bf16"), ("f32", "f32")]


def torch_io(torch, a, dt):
    """numpy oracle-side representation -> device tensor of the I/O type."""
    if dt == "bf16":
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    if dt == "f16":
        return torch.from_numpy(np.ascontiguousarray(a, np.float16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def bits16(torch, t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("xd,yd", IO_TYPES)
@pytest.mark.parametrize("M,K,N", IO_SHAPES)
def test_forward_io_parity(torch, bl, orc, M, K, N, xd, yd):
    """x widened exactly, the int8 codes of the widened x, and y rounded
    once from the fp32 output: bit for bit against the oracle."""
    announce("forward_io", M, K, N, xd, yd)
    x32, w, t, g = mm_case(M, K, N, 1400 + M + N)
    x = orc.from_f32(x32, xd)
    packed_r, s = orc.pack_i2s(w)
    y_r = orc.forward_io(x, xd, packed_r, s, g, 1e-6, N, yd)
    X = torch_io(torch, x, xd)
    ydt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[yd]
    ws = torch.empty(bl.lib().bitlinear_io_workspace_bytes(M, K, N), dtype=torch.uint8,
                     device="cuda")
    y = bl.forward_io(X, dev(torch, packed_r), s, dev(torch, g), 1e-6, N, y_dtype=ydt, workspace=ws)
    torch.cuda.synchronize()
    if yd == "f32":
        assert np.array_equal(host(y).view(np.uint32), y_r.view(np.uint32))
    else:
        assert np.array_equal(bits16(torch, y), np.asarray(y_r).view(np.uint16))
    q_r, inv_r, qs_r = orc.act_quant(orc.to_f32(x, xd), g, 1e-6)
    q, inv, qs = bl.workspace_views(ws, M, K)
    assert np.array_equal(host(q), q_r) and np.array_equal(host(inv), inv_r)
    assert np.array_equal(host(qs), qs_r)


def test_forward_io_f32_equals_forward(torch, bl, orc):
    """With fp32 in and out the typed entry point gives forward()'s bits,
    with and without RMSNorm."""
    for M, K, N in ((1, 2560, 640), (40, 512, 130)):
        x, w, t, g = mm_case(M, K, N, 1450 + M)
        packed_r, s = orc.pack_i2s(w)
        X, P, G = dev(torch, x), dev(torch, packed_r), dev(torch, g)
        for gg in (G, None):
            announce("forward_io f32", M, K, N, gg is None)
            a = host(bl.forward(X, P, s, gg, 1e-6, N))
            b = host(bl.forward_io(X, P, s, gg, 1e-6, N))
            torch.cuda.synchronize()
            assert np.array_equal(a, b)


def test_forward_io_identity_exact(torch, bl, orc):
    """bf16 x = integers / 64 (exact), no norm, W = 0.5 I: y = x / 2 exactly
    in bf16 and fp16."""
    K = 128
    m = (np.arange(2 * K).reshape(2, K) % 255 - 127).astype(np.float32)
    m[:, 0] = -127.0
    xf = m / np.float32(64.0)
    packed_r, s = orc.pack_i2s(np.eye(K, dtype=np.float32) * np.float32(0.5))
    for dt, tdt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        announce("forward_io identity", dt)
        X = torch_io(torch, orc.from_f32(xf, dt), dt)
        y = bl.forward_io(X, dev(torch, packed_r), s, None, 1e-6, K)
        torch.cuda.synchronize()
        assert y.dtype == tdt
        assert np.array_equal(y.float().cpu().numpy(), xf / np.float32(2.0))


def test_forward_io_f16_subnormals_exact(torch, bl, orc):
    """fp16 subnormal inputs and outputs keep their exact values: x = m *
    2^-20 (subnormal below |m| = 16) widens exactly, so q = m; with
    W = s I, y = s x exactly: m * 2^-24 (all subnormal) for s = 2^-4 and
    m * 2^-10 (normal) for s = 2^10; the device's bits are checked against
    the oracle's."""
    K = 128
    m = (np.arange(2 * K).reshape(2, K) % 255 - 127).astype(np.float32)
    m[:, 0] = -127.0
    xf = m * np.float32(2.0 ** -20)
    x = orc.from_f32(xf, "f16")
    assert np.array_equal(orc.to_f32(x, "f16"), xf)  # exact in fp16, subnormals included
    for s_w in (2.0 ** -4, 2.0 ** 10):
        packed_r, s = orc.pack_i2s(np.eye(K, dtype=np.float32) * np.float32(s_w))
        y_r = orc.forward_io(x, "f16", packed_r, s, None, 1e-6, K, "f16")
        assert np.array_equal(y_r.astype(np.float32), xf * np.float32(s_w))
        sub = (y_r != 0) & (np.abs(y_r.astype(np.float32)) < 2.0 ** -14)
        assert sub.any() == (s_w < 1)
        announce("forward_io f16 subnormals", s_w)
        y = bl.forward_io(torch_io(torch, x, "f16"), dev(torch, packed_r), s, None, 1e-6, K)
        torch.cuda.synchronize()
        assert np.array_equal(bits16(torch, y), y_r.view(np.uint16))
        q, inv, qs = orc.act_quant(orc.to_f32(x, "f16"), None, 1e-6)
        assert np.array_equal(q.astype(np.float32), m)


def one_token_io(torch, bl, x, dt, packed, s, g, N):
    """forward_io of one token with x and y of type dt: the one-shot kernel
    with the quantisation inside.  -> (y bits, q, inv, qsum)."""
    K = x.shape[-1]
    ws = torch.empty(bl.lib().bitlinear_io_workspace_bytes(1, K, N), dtype=torch.uint8,
                     device="cuda")
    ydt = {"bf16": torch.bfloat16, "f16": torch.float16}[dt]
    out = torch.full((1, N), float("nan"), dtype=ydt, device="cuda")
    y = bl.forward_io(torch_io(torch, x.reshape(1, K), dt), dev(torch, packed), s,
                      None if g is None else dev(torch, g), 1e-6, N, y_dtype=ydt, out=out,
                      workspace=ws)
    torch.cuda.synchronize()
    q, inv, qs = bl.workspace_views(ws, 1, K)
    return bits16(torch, y), host(q), host(inv), host(qs)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_forward_io_one_token_fused_edges(torch, bl, orc, dt):
    """One token with the same half type in and out takes the one-shot
    kernel with the RMSNorm + quantisation inside.  Edge cases through it,
    bit for bit against the oracle: exact ties in the output rounding
    (integer accumulators rescaled by exactly 1), ties in the quantisation
    (x * inv = m + 1/2), fp16 subnormal inputs and subnormal outputs
    (including ties between subnormals), fp16 overflow to inf, with and
    without RMSNorm."""
    K = 1024
    rng = np.random.default_rng(1500)
    # x = m / 64 with m integer in [-127, 127] and amax = 127 / 64: with no
    # RMSNorm inv = 64 exactly and q = m; w_scale = 64 makes the output
    # scale w_scale / inv exactly 1, so y = acc as an fp32 integer.
    m = rng.integers(-127, 128, K).astype(np.float32)
    m[5] = -127.0
    x_int = orc.from_f32(m / np.float32(64.0), dt)
    w, t = wl.ternary(1501, 512, K, 1 / 3, 64.0)
    packed, s = orc.pack_i2s(w)
    assert s == 64.0
    acc = m.astype(np.int64) @ t.astype(np.int64).T
    half = (np.abs(acc) >= 2048) & (acc % 2 == 1) if dt == "f16" else (np.abs(acc) >= 256) & (acc % 2 == 1)
    assert half.sum() > 50, "the case must hold many exact ties of the output rounding"
    cases = [("integer acc", x_int, packed, s, None, 512)]
    cases.append(("integer acc, RMSNorm", x_int, packed, s, wl.gamma(1502, K, "u0.8-1.2"), 512))
    # quantisation ties: x = (2j + 1) / 128, so x * 64 = j + 1/2
    j = rng.integers(-64, 63, K).astype(np.float32)
    xt = (2 * j + 1) / np.float32(128.0)
    xt[0] = np.float32(-127.0 / 64.0)
    x_tie = orc.from_f32(xt, dt)
    eye, s_eye = orc.pack_i2s(np.eye(K, dtype=np.float32) * np.float32(0.5))
    cases.append(("quantisation ties", x_tie, eye, s_eye, None, K))
    if dt == "f16":
        # fp16 subnormal inputs x = m 2^-20: inv = 2^20 and q = m, so W = s I
        # gives y = m s 2^-20 exactly before rounding: subnormal (s = 2^-4),
        # ties between subnormals (s = 2^-5: odd m gives m 2^-25) and normal
        # (s = 2^10); over x = m / 64, s = 2^16 gives y = 1024 m, which
        # overflows to inf from |m| >= 64
        xs = m * np.float32(2.0 ** -20)
        x_sub = orc.from_f32(xs, "f16")
        assert np.array_equal(orc.to_f32(x_sub, "f16"), xs)
        for e in (-4, -5, 10, 16):
            pk, sk = orc.pack_i2s(np.eye(K, dtype=np.float32) * np.float32(2.0 ** e))
            cases.append((f"subnormal x, s = 2^{e}", x_sub if e < 16 else x_int, pk, sk, None, K))
    for name, x, pk, sk, g, N in cases:
        announce("forward_io one token", dt, name)
        y_r = orc.forward_io(x.reshape(1, K), dt, pk, sk, g, 1e-6, N, dt)
        yb, q, inv, qs = one_token_io(torch, bl, x, dt, pk, sk, g, N)
        assert np.array_equal(yb, np.asarray(y_r).view(np.uint16)), name
        q_r, inv_r, qs_r = orc.act_quant(orc.to_f32(x.reshape(1, K), dt), g, 1e-6)
        assert np.array_equal(q, q_r) and np.array_equal(inv, inv_r) and np.array_equal(qs, qs_r)
        if name == "quantisation ties":
            # round half to even by hand: j + 1/2 -> the even one of j, j + 1
            expect = np.where(j % 2 == 0, j, j + 1)
            assert np.array_equal(q[0, 1:].astype(np.float32), expect[1:])
        if name.endswith("2^16"):
            yh = yb.view(np.float16).astype(np.float32)
            assert np.all(np.isinf(yh[0, np.abs(m) >= 64])) and np.all(np.isfinite(yh[0, np.abs(m) < 64]))


def test_fp32_ops_correctly_rounded(torch, bl):
    """The device's fp32 square root and division, as the normalisation and
    quantisation use them, are correctly rounded: bit for bit against the
    host's IEEE arithmetic on every exponent (subnormals included) with
    65536 mantissas each, on wide random divisions, and on the RMSNorm and
    quantisation scales at every row length K % 128 == 0 up to 32768."""
    rng = np.random.default_rng(1600)
    e = np.repeat(np.arange(255, dtype=np.uint32), 65536)
    mant = (np.tile(np.arange(65536, dtype=np.uint32), 255) * 128 +
            rng.integers(0, 128, 255 * 65536, dtype=np.uint32))
    a = ((e << 23) | mant).view(np.float32)
    announce("fp32 ops sqrt", a.size)
    A = dev(torch, a)
    got = host(bl.fp32_ops(bl.FP_SQRT, A))
    torch.cuda.synchronize()
    ref = np.sqrt(a)
    bad = got.view(np.uint32) != ref.view(np.uint32)
    assert not bad.any(), f"sqrtf differs on {bad.sum()} inputs, e.g. {a[bad][:4]}"
    del A
    # division over wide random operands (normal range)
    n = 1 << 24
    num = ((rng.integers(64, 190, n, dtype=np.uint32) << 23) |
           rng.integers(0, 1 << 23, n, dtype=np.uint32)).view(np.float32)
    den = ((rng.integers(64, 190, n, dtype=np.uint32) << 23) |
           rng.integers(0, 1 << 23, n, dtype=np.uint32)).view(np.float32)
    announce("fp32 ops div", n)
    got = host(bl.fp32_ops(bl.FP_DIV, dev(torch, num), dev(torch, den)))
    torch.cuda.synchronize()
    ref = num / den
    bad = got.view(np.uint32) != ref.view(np.uint32)
    assert not bad.any(), f"division differs on {bad.sum()} pairs"
    # the RMSNorm scale 1 / sqrt(ss / K + eps) at every K, ss over the range
    # of sums of squares (and the quantisation scale 127 / max(amax, 1e-5))
    Ks = np.arange(128, 32768 + 1, 128, dtype=np.float32)
    per = 1 << 16
    ss = np.exp(rng.uniform(np.log(1e-12), np.log(1e9), Ks.size * per)).astype(np.float32)
    kk = np.repeat(Ks, per)
    for eps in (1e-6, 1e-5):
        announce("fp32 ops rms scale", eps)
        got = host(bl.fp32_ops(bl.FP_RMS_SCALE, dev(torch, ss), dev(torch, kk), eps))
        torch.cuda.synchronize()
        ref = np.float32(1.0) / np.sqrt(ss / kk + np.float32(eps))
        bad = got.view(np.uint32) != ref.view(np.uint32)
        assert not bad.any(), f"rms scale differs on {bad.sum()} rows"
    amax = np.exp(rng.uniform(np.log(1e-7), np.log(1e6), 1 << 22)).astype(np.float32)
    amax[:3] = (0.0, 1e-5, np.float32(127.0 / 64.0))
    announce("fp32 ops quant scale")
    got = host(bl.fp32_ops(bl.FP_QUANT_SCALE, dev(torch, amax)))
    torch.cuda.synchronize()
    ref = np.float32(127.0) / np.maximum(amax, np.float32(1e-5))
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert got[2] == np.float32(64.0)


def test_forward_io_batch_mixed(torch, bl, orc):
    """A typed batch mixing bf16, fp16 and fp32 decode problems (fused per
    type), prefill problems (grouped per type pair) and staged ones (mixed
    types, M = 2..4, K > 8192): each equals its single forward_io call and
    the oracle, bit for bit."""
    cases = [(1, 2560, 640, "bf16", "bf16"), (1, 6912, 256, "bf16", "bf16"),
             (1, 2560, 96, "f16", "f16"), (1, 1024, 48, "f32", "f32"),
             (1, 2560, 64, "bf16", "f32"), (5, 512, 33, "bf16", "bf16"),
             (1, 9216, 40, "f16", "f16"), (1, 256, 16, "bf16", "bf16"),
             (64, 2560, 256, "bf16", "bf16"), (40, 512, 130, "f16", "bf16"),
             (96, 1024, 64, "bf16", "f32"), (33, 768, 50, "bf16", "bf16"),
             (70, 256, 40, "f32", "f16")]
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
    items, refs, singles = [], [], []
    for i, (M, K, N, xd, yd) in enumerate(cases):
        x32, w, t, g = mm_case(M, K, N, 1500 + i)
        x = orc.from_f32(x32, xd)
        packed_r, s = orc.pack_i2s(w)
        refs.append(orc.forward_io(x, xd, packed_r, s, g, 1e-6, N, yd))
        X, P, G = torch_io(torch, x, xd), dev(torch, packed_r), dev(torch, g)
        out = torch.empty((M, N), dtype=tdt[yd], device="cuda")
        ws = bl.io_workspace(M, K, N)
        items.append((X, P, s, G, 1e-6, out, ws))
        singles.append(bl.forward_io(X, P, s, G, 1e-6, N, y_dtype=tdt[yd]).clone())
    announce("forward_io_batch", len(items))
    bl.forward_io_batch(items)
    torch.cuda.synchronize()
    for it, single, ref, c in zip(items, singles, refs, cases):
        out = it[5]
        if c[4] == "f32":
            assert np.array_equal(host(out).view(np.uint32), ref.view(np.uint32)), c
            assert torch.equal(out, single), c
        else:
            assert np.array_equal(bits16(torch, out), np.asarray(ref).view(np.uint16)), c
            assert np.array_equal(bits16(torch, out), bits16(torch, single)), c


@pytest.mark.parametrize("M", [2, 3, 4, 5, 8])
def test_few_token_batches(torch, bl, orc, M):
    """The decoder layer's seven BitLinears at M = 2..8 tokens: fp32 through
    forward_batch (one batched quantisation and one one-shot contraction
    launch), bf16 and fp16 through forward_io_batch, with a problem whose
    x and y types differ: every output the oracle's (fp32 within 1e-5,
    half types bit for bit) and each fp32 one equal to its single call."""
    work = wl.DECODE_LAYER
    items, refs, singles = [], [], []
    for i, L in enumerate(work.linears):
        x, w, t, g = mm_case(M, L.K, L.N, 1800 + 10 * M + i)
        packed_r, s = orc.pack_i2s(w)
        X, P, G = dev(torch, x), dev(torch, packed_r), dev(torch, g)
        out = torch.full((M, L.N), float("nan"), dtype=torch.float32, device="cuda")
        items.append((X, P, s, G, 1e-6, out, bl.new_workspace(M, L.K)))
        refs.append(orc.forward(x, packed_r, s, g, 1e-6, L.N))
        singles.append(host(bl.forward(X, P, s, G, 1e-6, L.N)).copy())
    announce("few-token batch", M)
    bl.forward_batch(items)
    torch.cuda.synchronize()
    for it, ref, single in zip(items, refs, singles):
        check_y(host(it[5]), ref)
        assert np.array_equal(host(it[5]), single)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
    types = [("bf16", "bf16"), ("f16", "f16"), ("bf16", "f32"), ("f16", "bf16")]
    titems, trefs = [], []
    for i, L in enumerate(work.linears):
        xd, yd = types[i % len(types)]
        x32, w, t, g = mm_case(M, L.K, L.N, 1900 + 10 * M + i)
        x = orc.from_f32(x32, xd)
        packed_r, s = orc.pack_i2s(w)
        trefs.append((orc.forward_io(x, xd, packed_r, s, g, 1e-6, L.N, yd), yd))
        out = torch.empty((M, L.N), dtype=tdt[yd], device="cuda")
        titems.append((torch_io(torch, x, xd), dev(torch, packed_r), s, dev(torch, g), 1e-6, out,
                       bl.io_workspace(M, L.K, L.N)))
    announce("few-token typed batch", M)
    bl.forward_io_batch(titems)
    torch.cuda.synchronize()
    for it, (ref, yd) in zip(titems, trefs):
        if yd == "f32":
            assert np.array_equal(host(it[5]).view(np.uint32), ref.view(np.uint32))
        else:
            assert np.array_equal(bits16(torch, it[5]), np.asarray(ref).view(np.uint16))


# Few-token sets with the quantisation fused in: (M, K, N) per problem.  The
# first set fits the 16-wave one-shot shape in one round (groups of four
# waves quantise the rows of 2- and 3-token problems side by side, beside a
# one-token problem); the second needs two rounds, so its one-token problem
# goes out fused alone and the others as the batched quantisation +
# contraction pair.
FEW_FUSED_SETS = [
    [(1, 2560, 2560), (2, 2560, 640), (3, 6912, 2560), (2, 1024, 1000)],
    [(1, 2560, 2560), (2, 2560, 20480), (2, 4096, 16384), (3, 512, 72)],
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(len(FEW_FUSED_SETS)))
def test_few_token_fused_sets(torch, bl, orc, case):
    """Automatic forward_batch over a few-token set: every y the oracle's
    (fp32 within 1e-5, NaN-prefilled so an unwritten output fails), each
    workspace holding the oracle's q / inv / qsum, and each output equal to
    its single forward."""
    items, refs, aqs, singles = [], [], [], []
    for i, (M, K, N) in enumerate(FEW_FUSED_SETS[case]):
        x, w, t, g = mm_case(M, K, N, 2100 + 10 * case + i)
        packed_r, s = orc.pack_i2s(w)
        X, P, G = dev(torch, x), dev(torch, packed_r), dev(torch, g)
        out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        items.append((X, P, s, G, 1e-6, out, bl.new_workspace(M, K)))
        refs.append(orc.forward(x, packed_r, s, g, 1e-6, N))
        aqs.append(orc.act_quant(x, g, 1e-6))
        singles.append(host(bl.forward(X, P, s, G, 1e-6, N)).copy())
    announce("few-token fused set", case)
    bl.forward_batch(items)
    torch.cuda.synchronize()
    for it, ref, (q_r, inv_r, qs_r), single, (M, K, N) in zip(items, refs, aqs, singles,
                                                               FEW_FUSED_SETS[case]):
        check_y(host(it[5]), ref)
        assert np.array_equal(host(it[5]), single)
        q, inv, qs = bl.workspace_views(it[6], M, K)
        assert np.array_equal(host(q), q_r) and np.array_equal(host(inv), inv_r)
        assert np.array_equal(host(qs), qs_r)


# ---------------------------------------------------------------- dequantisation

@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("N,K", [(1, 128), (17, 384), (640, 2560), (2560, 6912)])
def test_dequant_parity(torch, bl, orc, N, K, dt):
    """Dense W in each type, bit for bit against the oracle's unpack
    rounded once."""
    announce("dequant", N, K, dt)
    w, _ = wl.ternary(1600 + N, N, K, 1 / 3, 0.0137)
    packed_r, s = orc.pack_i2s(w)
    ref = orc.dequant_i2s(packed_r, N, K, dt)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dt]
    got = bl.dequant_i2s(dev(torch, packed_r), N, K, tdt)
    torch.cuda.synchronize()
    if dt == "f32":
        assert np.array_equal(host(got).view(np.uint32), ref.view(np.uint32))
    else:
        assert np.array_equal(bits16(torch, got), np.asarray(ref).view(np.uint16))


def test_forward_batch_few_token_tiles(torch, bl, orc):
    """Prefill-route problems of 5..32 tokens take 16-row tiles (grouped and
    single, each width): the oracle's outputs within 1e-5, the single calls'
    bits."""
    shapes = [(5, 1024, 96), (16, 2560, 6912), (17, 512, 300), (32, 2048, 8192), (9, 9216, 64),
              (16, 768, 4000)]
    items, singles, refs = [], [], []
    for i, (M, K, N) in enumerate(shapes):
        x, w, t, g = mm_case(M, K, N, 1700 + i)
        packed_r, s = orc.pack_i2s(w)
        X, P, G = dev(torch, x), dev(torch, packed_r), dev(torch, g)
        out = torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")
        ws = bl.new_workspace(M, K)
        items.append((X, P, s, G, 1e-6, out, ws))
        singles.append(host(bl.forward(X, P, s, G, 1e-6, N)).copy())
        rows = np.arange(0, N, max(1, N // 97))
        refs.append((rows, orc.forward(x, orc.packed_rows(packed_r, K, rows), s, g, 1e-6,
                                       rows.size)))
    announce("forward_batch few-token tiles", len(items))
    bl.forward_batch(items)
    torch.cuda.synchronize()
    for it, single, (rows, y64), sh in zip(items, singles, refs, shapes):
        got = host(it[5])
        assert np.array_equal(got, single), sh
        check_y(got[:, rows], y64)


# ---------------------------------------------------------------- calibration probes

def test_probe_read_reads_every_byte(torch, bl):
    """The read-ceiling probe reads every byte once: each workgroup's sink
    word is the XOR of the 32-bit words of its 32 KB share (a ragged last
    share included)."""
    announce("probe read")
    nb = 3 * 32768 + 48
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    buf = torch.randint(0, 256, (nb,), generator=g, dtype=torch.uint8, device="cuda")
    sink = bl.probe_read(buf)
    torch.cuda.synchronize()
    h = buf.cpu().numpy()
    expect = [np.bitwise_xor.reduce(h[i:i + 32768].view(np.uint32)) for i in range(0, nb, 32768)]
    assert host(sink).view(np.uint32).tolist() == [int(e) for e in expect]


def test_probe_mfma_deterministic(torch, bl):
    announce("probe mfma")
    a = host(bl.probe_mfma(64, 8)).copy()
    b = host(bl.probe_mfma(64, 8))
    torch.cuda.synchronize()
    assert np.array_equal(a, b) and np.any(a != 0)
