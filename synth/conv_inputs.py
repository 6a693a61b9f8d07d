"""Seeded inputs for the short causal conv over the [q|k|v] channels.

The pages give no distributions for this step; the recipe below is the plain
reading (a unit-variance activation stream and the default initialisation of
a depthwise conv layer, whose fan-in is the kernel width W):

  stream  tensor   distribution
  21      x        N(0, 1)                              [T, dim]
  22      weight   U(-1/sqrt(W), 1/sqrt(W))             [dim, W]   fp32
  23      bias     U(-1/sqrt(W), 1/sqrt(W))             [dim]      fp32
  24      state    N(0, 1) where a carried state is used [N, W - 1, dim]
  25      lengths  integers in [lo, hi] (see seeded_conv_lengths)

x and the state are rounded once (RNE) to the storage dtype, as the KDA
inputs are; weight and bias stay fp32.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

from .kda_inputs import _store, _widen

STREAM = {"x": 21, "weight": 22, "bias": 23, "state": 24, "lengths": 25}


def _rng(seed: int, stream: str) -> np.random.Generator:
    return np.random.default_rng([int(seed), STREAM[stream]])


@dataclass
class ConvInputs:
    dtype: str
    x: np.ndarray                 # [T, dim] storage dtype (bf16 as uint16 bits)
    weight: np.ndarray            # [dim, W] fp32
    bias: np.ndarray              # [dim] fp32
    state: Optional[np.ndarray]   # [N, W - 1, dim] storage dtype, or None
    cu_seqlens: np.ndarray        # [N + 1] int32

    @property
    def T(self) -> int:
        return int(self.x.shape[0])

    @property
    def dim(self) -> int:
        return int(self.x.shape[1])

    @property
    def W(self) -> int:
        return int(self.weight.shape[1])

    @property
    def N(self) -> int:
        return len(self.cu_seqlens) - 1

    def f64(self) -> dict:
        return dict(x=_widen(self.x, self.dtype), weight=self.weight.astype(np.float64),
                    bias=self.bias.astype(np.float64),
                    state=None if self.state is None else _widen(self.state, self.dtype),
                    cu_seqlens=self.cu_seqlens.astype(np.int64))


def make_conv_inputs(seed: int, lengths: Sequence[int], dim: int, W: int = 4,
                     dtype: str = "bf16", with_state: bool = True) -> ConvInputs:
    lengths = [int(n) for n in lengths]
    T = sum(lengths)
    bound = 1.0 / np.sqrt(W)
    x = _rng(seed, "x").standard_normal((T, dim))
    w = _rng(seed, "weight").uniform(-bound, bound, (dim, W))
    b = _rng(seed, "bias").uniform(-bound, bound, dim)
    st = _rng(seed, "state").standard_normal((len(lengths), W - 1, dim)) if with_state else None
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return ConvInputs(dtype=dtype, x=_store(x, dtype), weight=w.astype(np.float32),
                      bias=b.astype(np.float32), state=None if st is None else _store(st, dtype),
                      cu_seqlens=cu)


def seeded_conv_lengths(seed: int, n: int, lo: int, hi: int) -> list:
    return [int(v) for v in _rng(seed, "lengths").integers(lo, hi + 1, n)]
