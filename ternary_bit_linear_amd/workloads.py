"""Seeded synthetic inputs for the BitLinear forward path.

This module only draws random numbers: activations, ternary weight patterns
times a scale, and RMSNorm gains.  It holds none of the method's arithmetic
(no packing, normalisation, quantisation or contraction) and imports neither
the HIP binding nor the oracle, so both sides can take their inputs from it.

Every draw uses numpy's PCG64 with an explicit seed, ``seed = 1000 * workload
id + tensor index``, so a tensor is reproducible on any host.

Workload shapes (a decoder layer of a ~2.5B-parameter BitNet, a 70B-shaped
FFN, and a square 8192 sweep) follow the tensor sizes discussed on the
llama.cpp discussion #8722 page "More BitNet-like IQ1_S quantizations"
(per-tensor sizes of a 3B BitNet b1.58; FFN weights dominate) -- the pages
measure on real checkpoints, which these synthetic tensors stand in for.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def ternary(seed: int, N: int, K: int, p0: float, scale: float):
    """Ternary pattern t in {-1, 0, +1} (int8 [N][K]) with P(0) = p0 and
    P(+1) = P(-1) = (1 - p0) / 2, and W = t * scale as fp32."""
    u = rng(seed).random((N, K), dtype=np.float64)
    t = np.ones((N, K), dtype=np.int8)
    t[u >= p0 + (1.0 - p0) / 2.0] = -1
    t[u < p0] = 0
    w = t.astype(np.float32) * np.float32(scale)
    return w, t


def activations(seed: int, M: int, K: int, outlier_frac: float = 0.0,
                outlier_mult: float = 20.0) -> np.ndarray:
    """x ~ N(0, 1) as fp32 [M][K]; with outlier_frac > 0 each entry is, with
    that probability, multiplied by outlier_mult after the normal draw."""
    g = rng(seed)
    x = g.standard_normal((M, K), dtype=np.float64).astype(np.float32)
    if outlier_frac > 0.0:
        mask = g.random((M, K)) < outlier_frac
        x[mask] *= np.float32(outlier_mult)
    return x


def gamma(seed: int, K: int, kind: str) -> np.ndarray:
    """RMSNorm gain: 'ones' or 'u0.8-1.2' (uniform on [0.8, 1.2))."""
    if kind == "ones":
        return np.ones(K, dtype=np.float32)
    if kind == "u0.8-1.2":
        return rng(seed).uniform(0.8, 1.2, K).astype(np.float32)
    raise ValueError(kind)


@dataclass(frozen=True)
class Linear:
    """One BitLinear of a workload: K inputs -> N outputs at M tokens."""
    name: str
    M: int
    K: int
    N: int
    p0: float
    scale: float
    gamma: str
    outlier_frac: float = 0.0


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    linears: tuple = field(default_factory=tuple)
    eps: float = 1e-6

    def seeds(self, i: int):
        """(x seed, W seed, gamma seed) of linear i."""
        base = 1000 * self.wid + 3 * i
        return base, base + 1, base + 2

    def inputs(self, i: int):
        """(x fp32 [M][K], W fp32 [N][K], t int8 [N][K], gamma fp32 [K])."""
        L = self.linears[i]
        sx, sw, sg = self.seeds(i)
        x = activations(sx, L.M, L.K, L.outlier_frac)
        w, t = ternary(sw, L.N, L.K, L.p0, L.scale)
        g = gamma(sg, L.K, L.gamma)
        return x, w, t, g

    def algorithmic_bytes(self) -> int:
        """Bytes a forward must move at least once: packed W (N*K/4), x
        (4*M*K), gamma (4*K) and y (4*M*N), summed over the linears."""
        return sum(L.N * L.K // 4 + 4 * L.M * L.K + 4 * L.K + 4 * L.M * L.N
                   for L in self.linears)

    def int_ops(self) -> int:
        """2*M*N*K multiply-adds of the int8 contraction, summed."""
        return sum(2 * L.M * L.N * L.K for L in self.linears)


def _layer(M, p0, scale, gamma_kind, outlier=0.0):
    shapes = [("q", 2560, 2560), ("k", 2560, 640), ("v", 2560, 640),
              ("o", 2560, 2560), ("gate", 2560, 6912), ("up", 2560, 6912),
              ("down", 6912, 2560)]
    return tuple(Linear(n, M, K, N, p0, scale, gamma_kind, outlier) for n, K, N in shapes)


# The five workloads: a tiny single BitLinear; one decoder layer at decode
# (M = 1) and at prefill (M = 512); a 70B-shaped FFN; a square sweep.
TINY = Workload(1, "single BitLinear M=1 K=256 N=256",
                (Linear("tiny", 1, 256, 256, 1.0 / 3.0, 0.02, "ones"),))
DECODE_LAYER = Workload(2, "decoder-layer BitLinears, decode M=1 (2560/640/6912)",
                        _layer(1, 0.4, 0.015, "u0.8-1.2"))
PREFILL_LAYER = Workload(3, "decoder-layer BitLinears, prefill M=512 (2560/640/6912)",
                         _layer(512, 0.4, 0.015, "u0.8-1.2", outlier=0.01))


def decode_layer(M: int) -> Workload:
    """The decoder layer's seven BitLinears at M tokens (few-token decode:
    batched serving or draft tokens), with the decode layer's weights and
    activations recipe."""
    return Workload(6, f"decoder-layer BitLinears, decode M={M} (2560/640/6912)",
                    _layer(M, 0.4, 0.015, "u0.8-1.2"))


def ffn70b(M: int) -> Workload:
    return Workload(4, f"70B-shaped FFN BitLinears M={M}",
                    (Linear("gate", M, 8192, 28672, 0.35, 0.01, "ones"),
                     Linear("up", M, 8192, 28672, 0.35, 0.01, "ones"),
                     Linear("down", M, 28672, 8192, 0.35, 0.01, "ones")))


def sweep(M: int) -> Workload:
    return Workload(5, f"square BitLinear K=N=8192 M={M}",
                    (Linear(f"sq{M}", M, 8192, 8192, 1.0 / 3.0, 0.02, "ones"),))


PACK_SHAPE = (8192, 28672)  # N x K of the packing workload (p0 = 1/3, s = 0.02)
SWEEP_M = (1, 4, 16, 64, 256, 512, 2048)
