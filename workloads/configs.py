"""Shapes, seeds and value distributions of the synthetic workloads.

Weights W are bf16 [N][K] (output features x input features); activations x
are bf16 [M][K]. Each tensor is a slice of a seeded counter-based stream
(``gen.bf16_tensor``), so the same bits are reproducible anywhere.

Workloads (sizes follow the decode and prefill shapes of a Qwen3-0.6B-like
model, a 27B-class dense layer, and a 151936-entry vocabulary head):

* ``gemv_1024``        single 1024x1024 projection, M=1, W ~ N(0, 0.02) seed 0,
                        x ~ N(0,1) seed 1000.
* ``qwen3_0p6b_decode`` 28 layers; layer l (1..28) draws q 2048x1024, k 1024x1024,
                        v 1024x1024, o 1024x2048, gate 3072x1024, up 3072x1024,
                        down 1024x3072 in that order from stream l (N(0,0.02));
                        x rows of width 1024, 2048, 3072 in that order from
                        stream 10000+l. M=1.
* ``dense27b_layer``   gate 17408x5120 (seed 100), up 17408x5120 (seed 101),
                        down 5120x17408 (seed 102), N(0, 0.015) with each entry
                        independently scaled x20 with probability 0.001; x of
                        width 5120 from seed 200 and of width 17408 from seed 201.
* ``dense27b_smallm``  the same weights, M in {2,4,8,16}; x row m (0-based) is
                        drawn from seed 300+m (width 5120, then width 17408).
* ``lm_head``          151936x1024, N(0, 0.02) seed 400; x row m from seed 410+m,
                        M in {1, 8}.
* ``prefill``          the gate/up weights of ``dense27b_layer`` with
                        x 2048x5120 ~ N(0,1) from seed 500.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .gen import bf16_tensor


@dataclass(frozen=True)
class Tensor:
    name: str
    N: int
    K: int
    seed: int
    start: int = 0
    sigma: float = 0.02
    outlier_p: float = 0.0
    outlier_scale: float = 1.0

    @property
    def numel(self) -> int:
        return self.N * self.K


@dataclass(frozen=True)
class XRows:
    """M activation rows of width K; row m comes from stream seeds[m] at offset start
    (or, with a single seed, the whole [M][K] matrix is one row-major stream)."""
    name: str
    M: int
    K: int
    seeds: tuple
    start: int = 0
    sigma: float = 1.0


@dataclass(frozen=True)
class Workload:
    name: str
    tensors: tuple
    xs: tuple = field(default_factory=tuple)

    def tensor(self, name: str) -> Tensor:
        for t in self.tensors:
            if t.name == name:
                return t
        raise KeyError(name)

    def x(self, name: str) -> XRows:
        for t in self.xs:
            if t.name == name:
                return t
        raise KeyError(name)


def tensor_bits(t: Tensor) -> np.ndarray:
    """uint16 bf16 bits of shape [N][K]."""
    return bf16_tensor((t.N, t.K), t.seed, t.sigma, t.start, t.outlier_p, t.outlier_scale)


def x_bits(x: XRows) -> np.ndarray:
    """uint16 bf16 bits of shape [M][K]."""
    if len(x.seeds) == 1:
        return bf16_tensor((x.M, x.K), x.seeds[0], x.sigma, x.start)
    assert len(x.seeds) == x.M
    return np.stack([bf16_tensor((x.K,), s, x.sigma, x.start) for s in x.seeds])


def _qwen_layer(l: int):
    shapes = [("q", 2048, 1024), ("k", 1024, 1024), ("v", 1024, 1024), ("o", 1024, 2048),
              ("gate", 3072, 1024), ("up", 3072, 1024), ("down", 1024, 3072)]
    ts, off = [], 0
    for name, n, k in shapes:
        ts.append(Tensor(f"L{l}.{name}", n, k, seed=l, start=off, sigma=0.02))
        off += n * k
    xs = [XRows(f"L{l}.x1024", 1, 1024, (10000 + l,), 0),
          XRows(f"L{l}.x2048", 1, 2048, (10000 + l,), 1024),
          XRows(f"L{l}.x3072", 1, 3072, (10000 + l,), 3072)]
    return ts, xs


def _build():
    w = {}
    w["gemv_1024"] = Workload("gemv_1024", (Tensor("w", 1024, 1024, seed=0, sigma=0.02),),
                              (XRows("x", 1, 1024, (1000,)),))
    ts, xs = [], []
    for l in range(1, 29):
        a, b = _qwen_layer(l)
        ts += a
        xs += b
    w["qwen3_0p6b_decode"] = Workload("qwen3_0p6b_decode", tuple(ts), tuple(xs))
    big = dict(sigma=0.015, outlier_p=0.001, outlier_scale=20.0)
    dense = (Tensor("gate", 17408, 5120, seed=100, **big),
             Tensor("up", 17408, 5120, seed=101, **big),
             Tensor("down", 5120, 17408, seed=102, **big))
    w["dense27b_layer"] = Workload("dense27b_layer", dense,
                                   (XRows("x_in", 1, 5120, (200,)), XRows("x_mid", 1, 17408, (201,))))
    sm = []
    for M in (2, 4, 8, 16):
        seeds = tuple(300 + m for m in range(M))
        sm += [XRows(f"x_in_m{M}", M, 5120, seeds, 0), XRows(f"x_mid_m{M}", M, 17408, seeds, 5120)]
    w["dense27b_smallm"] = Workload("dense27b_smallm", dense, tuple(sm))
    w["lm_head"] = Workload("lm_head", (Tensor("w", 151936, 1024, seed=400, sigma=0.02),),
                            (XRows("x_m1", 1, 1024, (410,)),
                             XRows("x_m8", 8, 1024, tuple(410 + m for m in range(8)))))
    w["prefill"] = Workload("prefill", dense[:2], (XRows("x", 2048, 5120, (500,)),))
    return w


WORKLOADS = _build()


def workload(name: str) -> Workload:
    return WORKLOADS[name]
