"""Seeded input generator for the KDA workloads.

Recipe (one numpy PCG64 stream per tensor, keyed by [seed, stream id], so
adding a tensor never shifts the others):

  stream  tensor   distribution
  1       q        N(0, 1), then L2-normalised over dk per (token, head)
                   (left raw when the kernels are to normalise it)
  2       k        N(0, 1), likewise; q and k have n_k_heads heads (= H by
                   default), v, g, beta and the state H
  3       v        N(0, 1)
  4       beta     sigmoid(N(0, 1))                                [T, H]
  5       gate x   N(0, 1)                                         [T, H, dk]
  6       a        U(-3, 0)                                        [H]
  7       b        N(0, 0.5) (standard deviation 0.5)              [H, dk]
  8       h0       N(0, std) (std 0.02 where an initial state is used)
  9       lengths  integers in [lo, hi], both ends inclusive

Gates.  "softplus": g = -softplus(x).  "kimi": g = -exp(a_h) * softplus(x + b),
the Kimi-Linear gate with a per-head a and a per-(head, channel) bias b.

Values are drawn in fp64 and rounded once, round-to-nearest-even, to the
storage dtype: fp32, or bf16 (kept as uint16 bit patterns).  The log-decay g
and the states are always fp32.  The oracle consumes the rounded values
widened to fp64, so any measured difference is the GPU path's own.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Tuple, Optional, Sequence

import numpy as np

STREAM = {"q": 1, "k": 2, "v": 3, "beta": 4, "x": 5, "a": 6, "b": 7, "h0": 8, "lengths": 9}


def _rng(seed: int, stream: str) -> np.random.Generator:
    return np.random.default_rng([int(seed), STREAM[stream]])


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 (8 significant bits, ties to even) and return
    the bit patterns as uint16.  Values must lie in the normal bf16 range or be
    zero (true for every distribution above).

    The rounding works on the fp64 bit pattern: the 45 low mantissa bits are
    dropped with round-to-nearest-even (add 2^44 - 1 plus the lowest kept bit,
    then clear them); the result is exact in fp32, whose top 16 bits are the
    bf16."""
    b = np.ascontiguousarray(np.asarray(x, dtype=np.float64)).view(np.uint64)
    keep = (b >> np.uint64(45)) & np.uint64(1)
    r = (b + (np.uint64((1 << 44) - 1) + keep)) & ~np.uint64((1 << 45) - 1)
    f = r.view(np.float64).astype(np.float32)  # exact: at most 8 significant bits
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x64.astype(np.float32))
    if dtype == "bf16":
        return np.ascontiguousarray(f64_to_bf16_bits(x64))
    raise ValueError(f"unknown dtype {dtype!r}")


def _widen(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16" and x.dtype == np.uint16:
        return bf16_bits_to_f64(x)
    return np.asarray(x, dtype=np.float64)


def _l2norm(x: np.ndarray, eps: float = 1e-12) -> np.ndarray:
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, eps)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


@dataclass
class KdaInputs:
    """One packed batch.  Storage arrays are what the GPU path receives."""

    q: np.ndarray  # [T, Hg, dk]  f32 or bf16 bits (Hg = H unless key heads are grouped)
    k: np.ndarray  # [T, Hg, dk]
    v: np.ndarray  # [T, H, dv]
    g: np.ndarray  # [T, H, dk]   fp32 natural-log decay, <= 0
    beta: np.ndarray  # [T, H]
    h0: Optional[np.ndarray]  # [N, H, dk, dv] fp32 or None (zero state)
    cu_seqlens: np.ndarray  # [N + 1] int32
    dtype: str  # "f32" or "bf16": dtype of q, k, v, beta and o
    chunk: int = 64
    scale: float = 0.0
    meta: dict = field(default_factory=dict)
    # The raw gate behind g, for the fused-gate path: x [T, H, dk] rounded to
    # the storage dtype, a_log [H] and dt_bias [H, dk] rounded to fp32 ("softplus"
    # gates have a_log = 0 and dt_bias = 0).  g above was made from the
    # unrounded values; a fused-gate reference recomputes it from these.
    gate_x: Optional[np.ndarray] = None
    gate_a_log: Optional[np.ndarray] = None
    gate_dt_bias: Optional[np.ndarray] = None

    @property
    def T(self) -> int:
        return int(self.q.shape[0])

    @property
    def H(self) -> int:
        return int(self.v.shape[1])

    @property
    def Hg(self) -> int:
        return int(self.q.shape[1])

    @property
    def dk(self) -> int:
        return int(self.q.shape[2])

    @property
    def dv(self) -> int:
        return int(self.v.shape[2])

    @property
    def N(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)

    def gate_f64(self) -> tuple:
        """(x, a_log, dt_bias) of the raw gate as stored, widened to fp64."""
        return (_widen(self.gate_x, self.dtype), np.asarray(self.gate_a_log, dtype=np.float64),
                np.asarray(self.gate_dt_bias, dtype=np.float64))

    def f64(self) -> dict:
        """The same values widened to fp64, as the oracle consumes them."""
        d = self.dtype
        return {
            "q": _widen(self.q, d),
            "k": _widen(self.k, d),
            "v": _widen(self.v, d),
            "g": np.asarray(self.g, dtype=np.float64),
            "beta": _widen(self.beta, d),
            "h0": None if self.h0 is None else np.asarray(self.h0, dtype=np.float64),
            "cu_seqlens": self.cu_seqlens.astype(np.int64),
            "scale": self.scale,
        }


def make_inputs(
    seed: int,
    lengths: Sequence[int],
    H: int,
    dk: int,
    dv: Optional[int] = None,
    dtype: str = "bf16",
    gate: str = "kimi",
    h0_std: float = 0.0,
    chunk: int = 64,
    scale: Optional[float] = None,
    n_k_heads: Optional[int] = None,
    qk_prenorm: bool = True,
    a_range: Tuple[float, float] = (-3.0, 0.0),
) -> KdaInputs:
    """Packed varlen batch with the recipe in the module docstring.
    n_k_heads: q/k heads (a divisor of H; default H).  qk_prenorm = False
    leaves q and k unnormalised (for kernels that normalise them).
    a_range: the interval a_h is drawn from for the Kimi gate (the workloads'
    U(-3, 0); U(1, 3) gives per-token log-decays of about -2 to -40, the strong
    per-channel decay that takes the chunked path's exact diagonal tiles)."""
    dv = dk if dv is None else dv
    Hg = H if n_k_heads is None else int(n_k_heads)
    if Hg < 1 or H % Hg:
        raise ValueError(f"n_k_heads {Hg} must divide H = {H}")
    qk = _l2norm if qk_prenorm else (lambda a: a)
    lengths = [int(x) for x in lengths]
    if any(x < 0 for x in lengths):
        raise ValueError("negative sequence length")
    T = int(sum(lengths))
    N = len(lengths)
    cu = np.zeros(N + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)

    # The independent streams are drawn on worker threads (numpy's generators
    # release the GIL); each stream's values do not depend on the threading.
    def draw_q():
        return _store(qk(_rng(seed, "q").standard_normal((T, Hg, dk))), dtype)

    def draw_k():
        return _store(qk(_rng(seed, "k").standard_normal((T, Hg, dk))), dtype)

    def draw_v():
        return _store(_rng(seed, "v").standard_normal((T, H, dv)), dtype)

    def draw_g():
        x = _rng(seed, "x").standard_normal((T, H, dk))
        if gate == "softplus":
            a = np.zeros(H)
            b = np.zeros((H, dk))
            g = -_softplus(x)
        elif gate == "kimi":
            a = _rng(seed, "a").uniform(a_range[0], a_range[1], size=(H,))
            b = _rng(seed, "b").normal(0.0, 0.5, size=(H, dk))
            g = -np.exp(a)[None, :, None] * _softplus(x + b[None, :, :])
        else:
            raise ValueError(f"unknown gate {gate!r}")
        return (np.ascontiguousarray(g.astype(np.float32)), _store(x, dtype),
                a.astype(np.float32), np.ascontiguousarray(b.astype(np.float32)))

    if gate not in ("softplus", "kimi"):
        raise ValueError(f"unknown gate {gate!r}")
    with ThreadPoolExecutor(max_workers=4) as pool:
        futs = [pool.submit(f) for f in (draw_q, draw_k, draw_v, draw_g)]
        q_s, k_s, v_s, (g_s, x_s, a_s, b_s) = (f.result() for f in futs)
    beta = 1.0 / (1.0 + np.exp(-_rng(seed, "beta").standard_normal((T, H))))
    h0 = None
    if h0_std > 0.0:
        h0 = _rng(seed, "h0").normal(0.0, h0_std, size=(N, H, dk, dv)).astype(np.float32)
    return KdaInputs(
        q=q_s,
        k=k_s,
        v=v_s,
        g=g_s,
        beta=_store(beta, dtype),
        h0=h0,
        cu_seqlens=cu,
        dtype=dtype,
        chunk=chunk,
        scale=float(dk ** -0.5) if scale is None else float(scale),
        meta={"seed": seed, "lengths": lengths, "gate": gate, "h0_std": h0_std,
              "qk_prenorm": qk_prenorm},
        gate_x=x_s,
        gate_a_log=a_s,
        gate_dt_bias=b_s,
    )


def seeded_lengths(seed: int, n: int, lo: int, hi: int) -> list:
    return [int(x) for x in _rng(seed, "lengths").integers(lo, hi + 1, n)]


# The five workloads.  decode-64x256 is generated as 64 sequences of 1280 tokens;
# the prefill uses tokens [0, 1024) of each and decode step s uses token
# 1024 + s of every sequence.
CONFIGS = {
    0: dict(name="tiny-f32", H=2, d=32, chunk=16, dtype="f32", gate="softplus",
            lengths=[128], h0_std=0.0),
    1: dict(name="prefill-4k", H=32, d=128, chunk=64, dtype="bf16", gate="kimi",
            lengths=[4096], h0_std=0.0),
    2: dict(name="prefill-32k", H=32, d=128, chunk=64, dtype="bf16", gate="kimi",
            lengths=[32768], h0_std=0.02),
    3: dict(name="varlen-8", H=32, d=128, chunk=64, dtype="bf16", gate="kimi",
            lengths=None, n_seqs=8, len_lo=300, len_hi=8192, h0_std=0.02),
    4: dict(name="decode-64x256", H=32, d=128, chunk=64, dtype="bf16", gate="kimi",
            lengths=[1280] * 64, h0_std=0.0, prefill_len=1024, decode_steps=256),
}


def config_lengths(cfg_id: int) -> list:
    c = CONFIGS[cfg_id]
    if c["lengths"] is not None:
        return list(c["lengths"])
    return seeded_lengths(cfg_id, c["n_seqs"], c["len_lo"], c["len_hi"])


def make_config(cfg_id: int, heads: Optional[Sequence[int]] = None) -> KdaInputs:
    """Inputs of workload cfg_id (seed = cfg_id).  `heads` keeps only the listed
    heads (after generation, so the kept values are identical)."""
    c = CONFIGS[cfg_id]
    inp = make_inputs(cfg_id, config_lengths(cfg_id), c["H"], c["d"], c["d"], c["dtype"],
                      c["gate"], c["h0_std"], c["chunk"])
    inp.meta["config"] = cfg_id
    inp.meta["name"] = c["name"]
    if heads is not None:
        inp = slice_heads(inp, heads)
    return inp


def slice_heads(inp: KdaInputs, heads: Sequence[int]) -> KdaInputs:
    if inp.Hg != inp.H:
        raise ValueError("slice_heads needs one key head per head")
    hs = np.asarray(list(heads), dtype=np.int64)
    return KdaInputs(
        q=np.ascontiguousarray(inp.q[:, hs]),
        k=np.ascontiguousarray(inp.k[:, hs]),
        v=np.ascontiguousarray(inp.v[:, hs]),
        g=np.ascontiguousarray(inp.g[:, hs]),
        beta=np.ascontiguousarray(inp.beta[:, hs]),
        h0=None if inp.h0 is None else np.ascontiguousarray(inp.h0[:, hs]),
        cu_seqlens=inp.cu_seqlens.copy(),
        dtype=inp.dtype,
        chunk=inp.chunk,
        scale=inp.scale,
        meta=dict(inp.meta, heads=[int(h) for h in hs]),
        gate_x=None if inp.gate_x is None else np.ascontiguousarray(inp.gate_x[:, hs]),
        gate_a_log=None if inp.gate_a_log is None else inp.gate_a_log[hs].copy(),
        gate_dt_bias=None if inp.gate_dt_bias is None else np.ascontiguousarray(inp.gate_dt_bias[hs]),
    )
