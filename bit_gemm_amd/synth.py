"""Seeded synthetic inputs: weight matrices with planted outliers and activations.

This module only draws random numbers; it holds none of the quantiser's
arithmetic. Tests, the benchmark and the smoke check take their inputs from
here, so the HIP path and the CPU oracle always see identical bytes.

Recipe (numpy ``default_rng``):
  W = fp16_RNE(0.02 * N(0, 1)) drawn in float32; the outlier entries are
      multiplied by 20 in float32 before the fp16 rounding.
  outlier placement
      uniform  : round(0.005 N K) positions drawn without replacement;
      columns  : c columns drawn without replacement, then
                 min(round(0.005 N K), c N) positions among those columns;
      rows     : the same with r rows.
  X = fp16_RNE(N(0, 1)) drawn in float32; optionally h activation channels
      (drawn without replacement) multiplied by 50 before the rounding.
  seed of a tensor = 1000 * workload + 10 * matrix + role, role 0 = W,
  1 = X, 2 = outlier positions, 3 = hot activation channels, 4 = calibration
  activations, 5 = held-out evaluation activations (both with the layer's
  hot channels, role 3, so they share one activation profile).

The shapes are Llama-family linear layers; they stand in for the real models'
weights, which are not available (no trained checkpoints are used).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

W_STD = 0.02
OUTLIER_MULT = 20.0
OUTLIER_FRAC = 0.005
HOT_MULT = 50.0


def seed_of(workload: int, matrix: int, role: int) -> int:
    return 1000 * workload + 10 * matrix + role


def _positions(rng, N, K, mode, count_lines, frac):
    total = int(round(frac * N * K))
    if mode == "none":
        return np.zeros(0, dtype=np.int64)
    if mode == "uniform":
        return rng.choice(N * K, size=min(total, N * K), replace=False).astype(np.int64)
    if mode == "columns":
        cols = np.sort(rng.choice(K, size=count_lines, replace=False)).astype(np.int64)
        cand = (np.arange(N, dtype=np.int64)[:, None] * K + cols[None, :]).ravel()
    elif mode == "rows":
        rows = np.sort(rng.choice(N, size=count_lines, replace=False)).astype(np.int64)
        cand = (rows[:, None] * K + np.arange(K, dtype=np.int64)[None, :]).ravel()
    else:
        raise ValueError(f"unknown outlier mode {mode!r}")
    if total >= cand.size:
        return cand
    return cand[rng.choice(cand.size, size=total, replace=False)]


def weight(N: int, K: int, seed_w: int, seed_pos: int, mode: str = "columns",
           count_lines: int = 8, frac: float = OUTLIER_FRAC) -> np.ndarray:
    """fp16 [N, K] weight with planted outliers (see the module recipe)."""
    w = np.random.default_rng(seed_w).standard_normal((N, K), dtype=np.float32)
    w *= np.float32(W_STD)
    pos = _positions(np.random.default_rng(seed_pos), N, K, mode, count_lines, frac)
    flat = w.reshape(-1)
    flat[pos] *= np.float32(OUTLIER_MULT)
    return w.astype(np.float16)


def activations(M: int, K: int, seed_x: int, seed_ch: int | None = None,
                hot_channels: int = 0) -> np.ndarray:
    """fp16 [M, K] activations, N(0,1), optionally with hot channels x50."""
    x = np.random.default_rng(seed_x).standard_normal((M, K), dtype=np.float32)
    if hot_channels:
        ch = np.random.default_rng(seed_ch).choice(K, size=hot_channels, replace=False)
        x[:, ch] *= np.float32(HOT_MULT)
    return x.astype(np.float16)


@dataclass(frozen=True)
class Layer:
    """One linear layer of a workload: shape, outlier recipe and packing knobs."""
    name: str
    N: int
    K: int
    mode: str
    count_lines: int
    group: int
    rho: float
    workload: int
    matrix: int
    hot_channels: int = 0

    def W(self) -> np.ndarray:
        return weight(self.N, self.K, seed_of(self.workload, self.matrix, 0),
                      seed_of(self.workload, self.matrix, 2), self.mode, self.count_lines)

    def X(self, M: int) -> np.ndarray:
        return activations(M, self.K, seed_of(self.workload, self.matrix, 1),
                           seed_of(self.workload, self.matrix, 3), self.hot_channels)

    def calibration(self, M: int, hot_channels: int, held_out: bool = False) -> np.ndarray:
        """Calibration (or held-out evaluation) activations with hot channels."""
        return activations(M, self.K, seed_of(self.workload, self.matrix, 5 if held_out else 4),
                           seed_of(self.workload, self.matrix, 3), hot_channels)


@dataclass(frozen=True)
class Workload:
    name: str
    layers: tuple
    batch: tuple = field(default=(1,))


def _cols(K: int) -> int:
    # "outliers in 0.2 % of the input columns"
    return int(round(0.002 * K))


WORKLOADS = {
    # 1024x1024, 8 outlier columns, 0.5 % of entries x20, rho 1 %, one token
    "tiny-1024x1024": Workload("tiny-1024x1024", (
        Layer("w", 1024, 1024, "columns", 8, 128, 0.01, 1, 0),), (1,)),
    # Llama-7B-shaped MLP up-projection, decode batches 1 / 4 / 16
    "decode-11008x4096": Workload("decode-11008x4096", (
        Layer("up", 11008, 4096, "columns", _cols(4096), 128, 0.005, 2, 0),), (1, 4, 16)),
    # the seven linears of one 4096-hidden transformer block at M = 16
    "block-4096h": Workload("block-4096h", tuple(
        Layer(n, N, K, "columns", _cols(K), 128, 0.005, 3, m)
        for m, (n, N, K) in enumerate([
            ("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
            ("gate", 11008, 4096), ("up", 11008, 4096), ("down", 4096, 11008)])), (16,)),
    # 70B-shaped MLP prefill, column-clustered outliers, 4 hot activation channels
    "prefill-28672x8192": Workload("prefill-28672x8192", (
        Layer("up", 28672, 8192, "columns", _cols(8192), 128, 0.01, 4, 0, hot_channels=4),),
        (512, 2048)),
}

# residual sweep at 14336x4096: outlier placement x density x batch
SWEEP_MODES = (("uniform", 0), ("columns", _cols(4096)), ("rows", int(round(0.002 * 14336))))
SWEEP_RHOS = (0.001, 0.005, 0.02, 0.05)
SWEEP_BATCH = (1, 64, 512)


def sweep_layer(mode: str, rho: float) -> Layer:
    m = [x for x, _ in SWEEP_MODES].index(mode)
    lines = dict(SWEEP_MODES)[mode]
    return Layer(f"sweep-{mode}", 14336, 4096, mode, lines, 128, rho, 5, m)
