"""Seeded synthetic inputs for the Muon update step.

This module holds the five workload descriptions (matrix shapes, dtypes,
value distributions, hyperparameters) and the seeded generators that draw
their weights and gradients.  It contains none of the optimizer's
arithmetic: both the fp64 oracle side and the HIP side receive the arrays
it produces, and neither side imports the other.

Every matrix of every step is drawn from its own numpy PCG64 stream, seeded
with ``SeedSequence([0, cfg, mat_idx, step, kind])`` (``kind`` 0 = weights,
1 = gradient), so any single matrix can be regenerated on its own.  Values
are drawn in fp64 and stored in the parameter dtype: fp64 -> fp32 by numpy's
round-to-nearest-even, then fp32 -> bf16 by round-to-nearest-even on the
bit pattern.  The stored value *is* the input; consumers read it exactly.

Shapes come from the published workload descriptions of the Muon / DMuon
pages (transformer blocks, an embodied VLA backbone with an action expert,
a Llama-style 7B matrix set and an MoE expert stack); the pages give no
values, so weights are N(0, 0.02^2) everywhere and gradients follow each
workload's stated law.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Sequence, Tuple

import numpy as np

F32 = "f32"
BF16 = "bf16"

KIND_W = 0
KIND_G = 1


@dataclass(frozen=True)
class Hyper:
    lr: float = 0.02
    beta: float = 0.95
    wd: float = 0.01
    ns_steps: int = 5
    coeffs: Tuple[float, float, float] = (3.4445, -4.7750, 2.0315)
    eps: float = 1e-7
    rms_scale: float = 0.2


@dataclass(frozen=True)
class Workload:
    cfg: int                      # 1-based workload number (part of every seed)
    name: str
    shapes: Tuple[Tuple[int, int], ...]   # (rows, cols) per matrix, in plan order
    dtype: str                    # parameter / gradient dtype: "f32" or "bf16"
    grad_law: str                 # "normal" or "student_t"
    grad_scale: float
    w_scale: float = 0.02
    steps: int = 1
    hyper: Hyper = field(default_factory=Hyper)

    @property
    def n_matrices(self) -> int:
        return len(self.shapes)

    @property
    def n_elements(self) -> int:
        return int(sum(r * c for r, c in self.shapes))


def _transformer(layers: int, shapes_per_layer: Sequence[Tuple[int, int]]):
    out: List[Tuple[int, int]] = []
    for _ in range(layers):
        out.extend(shapes_per_layer)
    return tuple(out)


def _c5_shapes():
    out: List[Tuple[int, int]] = []
    for _layer in range(8):
        for _expert in range(64):
            out.append((1408, 2048))   # gate
            out.append((1408, 2048))   # up
            out.append((2048, 1408))   # down
    out.extend([(512, 16384)] * 8)     # tall-skinny Gram-space cases
    return tuple(out)


WORKLOADS = {
    1: Workload(1, "single fp32 256x512", ((256, 512),), F32, "normal", 0.02),
    2: Workload(2, "4-layer transformer d=1024 ffn=4096",
                _transformer(4, [(3072, 1024), (1024, 1024), (4096, 1024), (1024, 4096)]),
                BF16, "normal", 0.02, steps=3),
    3: Workload(3, "VLA mixed shapes: 24-layer d=2048 backbone + 12-layer d=512 action expert",
                _transformer(24, [(6144, 2048), (2048, 2048), (8192, 2048), (2048, 8192)])
                + _transformer(12, [(1536, 512), (512, 512), (2048, 512), (512, 2048)]),
                BF16, "student_t", 0.01),
    4: Workload(4, "Llama-style 7B matrix set (32 layers, d=4096, ffn=11008)",
                _transformer(32, [(12288, 4096), (4096, 4096), (11008, 4096), (11008, 4096),
                                  (4096, 11008)]),
                BF16, "normal", 0.01),
    5: Workload(5, "MoE stack: 8 layers x 64 experts (1408x2048, 2048x1408) + 8 x 512x16384",
                _c5_shapes(), BF16, "normal", 0.02),
}


def workload(cfg: int) -> Workload:
    return WORKLOADS[cfg]


def rng_for(cfg: int, mat_idx: int, step: int, kind: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([0, cfg, mat_idx, step, kind])))


def f64_to_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bit patterns.

    Finite inputs only (the generated values are far from overflow)."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return u.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def f32_to_bf16_values(x32: np.ndarray) -> np.ndarray:
    """The fp64 value of each stored bf16 element (exact)."""
    return bf16_bits_to_f64(f32_to_bf16_bits(x32))


@dataclass
class Stored:
    """One stored matrix: its exact value in fp64 plus the raw storage array.

    ``raw`` is float32 for f32 workloads and uint16 bf16 bit patterns for bf16."""
    value: np.ndarray
    raw: np.ndarray
    dtype: str


def _store(x64: np.ndarray, dtype: str) -> Stored:
    x32 = f64_to_f32(x64)
    if dtype == F32:
        return Stored(x32.astype(np.float64), x32, F32)
    bits = f32_to_bf16_bits(x32)
    return Stored(bf16_bits_to_f64(bits), bits, BF16)


def draw(wl: Workload, mat_idx: int, step: int, kind: int,
         shape: Tuple[int, int] | None = None) -> Stored:
    """Draw weights (kind 0, step ignored -> 0) or the gradient of ``step`` (kind 1)."""
    rows, cols = shape if shape is not None else wl.shapes[mat_idx]
    if kind == KIND_W:
        rng = rng_for(wl.cfg, mat_idx, 0, KIND_W)
        x = rng.standard_normal((rows, cols)) * wl.w_scale
    else:
        rng = rng_for(wl.cfg, mat_idx, step, KIND_G)
        if wl.grad_law == "normal":
            x = rng.standard_normal((rows, cols)) * wl.grad_scale
        elif wl.grad_law == "student_t":
            x = rng.standard_t(3.0, (rows, cols)) * wl.grad_scale
        else:
            raise ValueError(wl.grad_law)
    return _store(x, wl.dtype)


def draw_custom(seed: Sequence[int], shape: Tuple[int, int], dtype: str,
                law: str = "normal", scale: float = 0.02) -> Stored:
    """A seeded matrix outside the five workloads (tests: ragged shapes, edge cases)."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(seed))))
    if law == "normal":
        x = rng.standard_normal(shape) * scale
    elif law == "student_t":
        x = rng.standard_t(3.0, shape) * scale
    elif law == "zeros":
        x = np.zeros(shape)
    else:
        raise ValueError(law)
    return _store(x, dtype)
