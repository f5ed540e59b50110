"""Seeded synthetic inputs for the FP8 block-scaled decode GEMM.

This module is shared by the tests, the bench and the smoke check. It holds
no arithmetic of the method itself (no FP8 encoding, no scaling, no GEMM):
only random draws, the fp32 -> bf16 rounding that turns a draw into a bf16
tensor, and the table of workload shapes.

Workload shapes follow the pages: decode batches of about eight rows
("A 23% faster GPU kernel, and a model that did not move", section "Why this
shape is hard") and the 248,320 x 5,120 vocabulary output layer ("The
profiler said the kernel ran zero times", section "The output layer, which
did run"). The square, MLP and step-mix shapes are the synthetic stand-ins
used for the pages' unnamed Qwen layers; the weights are random because the
pages' checkpoint is not available.

Every array is produced on the host with numpy; callers move it to the GPU.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "bf16_from_f32",
    "f32_from_bf16",
    "weight_bf16",
    "act_bf16",
    "Workload",
    "WORKLOADS",
    "STEP_SHAPES",
    "step_order",
]


def bf16_from_f32(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round to nearest, ties to even); returns uint16 bit patterns.

    Inputs are finite by construction (normal draws times small factors).
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def f32_from_bf16(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 (exact)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def weight_bf16(seed: int, n: int, k: int, sigma: float = 0.02,
                row_chunk: int | None = None) -> np.ndarray:
    """W[n][k] as bf16 bits: sigma * N(0,1) drawn in fp32, then rounded once.

    With ``row_chunk`` set, each chunk of ``row_chunk`` rows is drawn from its
    own stream ``default_rng([seed, chunk_index])`` so that any block row of a
    very large weight can be regenerated alone (used for sampled checks of the
    vocabulary layer).
    """
    if row_chunk is None:
        rng = np.random.default_rng(seed)
        w = rng.standard_normal((n, k), dtype=np.float32)
        w *= np.float32(sigma)
        return bf16_from_f32(w)
    assert n % row_chunk == 0
    out = np.empty((n, k), dtype=np.uint16)
    for c in range(n // row_chunk):
        out[c * row_chunk:(c + 1) * row_chunk] = weight_rows_bf16(seed, c, row_chunk, k, sigma)
    return out


def weight_rows_bf16(seed: int, chunk: int, row_chunk: int, k: int,
                     sigma: float = 0.02) -> np.ndarray:
    """One independently seeded row chunk of a chunked weight (see weight_bf16)."""
    rng = np.random.default_rng([seed, chunk])
    w = rng.standard_normal((row_chunk, k), dtype=np.float32)
    w *= np.float32(sigma)
    return bf16_from_f32(w)


def act_bf16(seed: int, col_seed: int, m: int, k: int, n_outlier: int,
             factor: float) -> np.ndarray:
    """X[m][k] as bf16 bits: N(0,1) in fp32, ``n_outlier`` distinct columns times
    ``factor``, then rounded to bf16 once."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((m, k), dtype=np.float32)
    if n_outlier > 0:
        cols = np.random.default_rng(col_seed).choice(k, size=n_outlier, replace=False)
        x[:, cols] *= np.float32(factor)
    return bf16_from_f32(x)


@dataclass(frozen=True)
class Workload:
    """One GEMM workload: Y[m][n] = X[m][k] . W[n][k]^T."""
    name: str
    m_values: tuple
    n: int
    k: int
    w_seed: int
    x_seed: int
    col_seed: int
    n_outlier: int
    outlier_factor: float
    row_chunk: int | None = None
    note: str = field(default="", compare=False)

    def weight(self) -> np.ndarray:
        return weight_bf16(self.w_seed, self.n, self.k, row_chunk=self.row_chunk)

    def act(self, m: int | None = None) -> np.ndarray:
        """Activations for ``m`` rows: the leading rows of the largest draw."""
        mmax = max(self.m_values)
        x = act_bf16(self.x_seed, self.col_seed, mmax, self.k, self.n_outlier,
                     self.outlier_factor)
        return x if m is None else x[:m].copy()

    def algorithmic_bytes(self, m: int) -> int:
        """Bytes one GEMM must move at minimum: e4m3 weight codes, fp32 block
        scales, bf16 activations in, bf16 output."""
        return (self.n * self.k + 4 * (self.n // 128) * (self.k // 128)
                + 2 * m * self.k + 2 * m * self.n)


def _pct_cols(k: int) -> int:
    return int(round(0.01 * k))


WORKLOADS = {
    "tiny": Workload("tiny", (8,), 512, 1024, 100, 101, 102, 4, 20.0,
                     note="M=8, K=1024, N=512; 4 outlier columns x20"),
    "square": Workload("square", (1, 8), 5120, 5120, 110, 111, 112, 4, 20.0,
                       note="M in {1,8}, K=N=5120"),
    "mlp_up": Workload("mlp_up", (8,), 34816, 5120, 120, 122, 124, _pct_cols(5120), 10.0,
                       note="up/gate, M=8, K=5120, N=34816; 1% of columns x10"),
    "mlp_down": Workload("mlp_down", (8,), 5120, 17408, 121, 123, 125, _pct_cols(17408), 10.0,
                         note="down, M=8, K=17408, N=5120; 1% of columns x10"),
    "vocab": Workload("vocab", (1, 8, 16), 248320, 5120, 130, 131, 132, 4, 20.0,
                      row_chunk=128,
                      note="vocabulary output layer, M in {1,8,16}, K=5120, N=248320"),
}

# Decode-step mix: the four GEMM shapes, drawn uniformly in a seeded order.
STEP_SHAPES = ("square", "mlp_up", "mlp_down", "vocab")
STEP_M_VALUES = (1, 2, 4, 8, 16, 32)


def step_order(n_gemms: int = 256, seed: int = 0) -> list:
    """Seeded order of the step mix: a list of workload names."""
    idx = np.random.default_rng(seed).integers(0, len(STEP_SHAPES), size=n_gemms)
    return [STEP_SHAPES[i] for i in idx]
