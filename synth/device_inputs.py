"""Seeded synthetic KDA inputs drawn on the device, for shapes too large to
draw on the host (billions of values per tensor).

Same distributions as the host recipe in kda_inputs.py, drawn with torch's
device generator (one generator per tensor, seeded with 16 * seed + stream
id, the stream ids of the host recipe) and computed in fp32 before the one
rounding to the storage dtype:
  q, k    N(0, 1), L2-normalised over dk per (token, head), stored bf16
  v       N(0, 1), bf16
  beta    sigmoid(N(0, 1)), bf16                                   [T, H]
  g       -exp(a_h) * softplus(x + b_h), x ~ N(0, 1), a ~ U(-3, 0) [H],
          b ~ N(0, 0.5) [H, dk]; fp32
  h0      N(0, h0_std), fp32                                       [N, H, dk, dv]
The values differ from the host recipe's (another generator); the oracle is
given the same device values, copied to the host and widened to fp64
(`host_f64`).  Only random numbers and roundings happen here.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from .kda_inputs import STREAM


def _gen(torch, device, seed: int, stream: str):
    g = torch.Generator(device=device)
    g.manual_seed(16 * int(seed) + STREAM[stream])
    return g


def make_device_inputs(seed: int, lengths: Sequence[int], H: int, D: int, h0_std: float = 0.0,
                       device: str = "cuda") -> dict:
    """Packed bf16 batch on `device`: q, k, v, beta (bf16), g (fp32), h0
    (fp32 or None), cu_seqlens (int32), scale; T tokens in len(lengths)
    sequences.  Peak extra memory is two fp32 copies of one [T, H, D] tensor."""
    import torch

    lengths = [int(x) for x in lengths]
    if any(x < 0 for x in lengths):
        raise ValueError("negative sequence length")
    T, N = int(sum(lengths)), len(lengths)
    cu = torch.zeros(N + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    f32, b16 = torch.float32, torch.bfloat16

    def unit_rows(stream):
        x = torch.randn((T, H, D), generator=_gen(torch, device, seed, stream), dtype=f32,
                        device=device)
        x.div_(x.norm(dim=-1, keepdim=True).clamp_min_(1e-12))
        return x.to(b16)

    q = unit_rows("q")
    k = unit_rows("k")
    v = torch.randn((T, H, D), generator=_gen(torch, device, seed, "v"), dtype=f32,
                    device=device).to(b16)
    beta = torch.sigmoid(torch.randn((T, H), generator=_gen(torch, device, seed, "beta"),
                                     dtype=f32, device=device)).to(b16)
    a = torch.rand((H,), generator=_gen(torch, device, seed, "a"), dtype=f32, device=device) * -3.0
    b = 0.5 * torch.randn((H, D), generator=_gen(torch, device, seed, "b"), dtype=f32,
                          device=device)
    g = torch.randn((T, H, D), generator=_gen(torch, device, seed, "x"), dtype=f32, device=device)
    g.add_(b)
    g = torch.nn.functional.softplus(g)
    g.mul_(-torch.exp(a)[None, :, None])
    h0 = None
    if h0_std > 0.0:
        h0 = h0_std * torch.randn((N, H, D, D), generator=_gen(torch, device, seed, "h0"),
                                  dtype=f32, device=device)
    return {"q": q, "k": k, "v": v, "g": g, "beta": beta, "h0": h0,
            "cu_seqlens": cu.to(device), "cu_host": cu.numpy().astype(np.int64),
            "scale": float(D ** -0.5)}


def host_f64(d: dict, n: int, heads: Sequence[int], t_end: Optional[int] = None) -> dict:
    """Sequence n of a device batch, heads `heads`, tokens [start, t_end) of it
    (default: all), copied to the host as fp64 arrays in the oracle's layout,
    with h0 of that sequence and those heads."""
    cu = d["cu_host"]
    s, e = int(cu[n]), int(cu[n + 1])
    e = e if t_end is None else min(e, s + int(t_end))
    hs = list(heads)

    def take(x):
        return x[s:e][:, hs].double().cpu().numpy()

    h0 = None if d["h0"] is None else d["h0"][n:n + 1][:, hs].double().cpu().numpy()
    return {"q": take(d["q"]), "k": take(d["k"]), "v": take(d["v"]), "g": take(d["g"]),
            "beta": take(d["beta"]), "h0": h0,
            "cu_seqlens": np.array([0, e - s], dtype=np.int64), "scale": d["scale"],
            "range": (s, e)}


def make_device_conv_inputs(seed: int, lengths: Sequence[int], dim: int, W: int,
                            device: str = "cuda") -> dict:
    """The short conv's recipe (conv_inputs.py) drawn on `device`: x [T, dim]
    and carried taps [N, W - 1, dim] N(0, 1) stored bf16; weight [dim, W] and
    bias [dim] U(-1/sqrt(W), 1/sqrt(W)) fp32; cu_seqlens int32.  Generators
    seeded with 16 * seed + the conv stream ids."""
    import torch

    from .conv_inputs import STREAM as CSTREAM

    def gen(stream):
        g = torch.Generator(device=device)
        g.manual_seed(16 * int(seed) + CSTREAM[stream])
        return g

    lengths = [int(x) for x in lengths]
    T, N = int(sum(lengths)), len(lengths)
    cu = torch.zeros(N + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    lim = float(W) ** -0.5
    f32 = torch.float32
    x = torch.randn((T, dim), generator=gen("x"), dtype=f32, device=device).to(torch.bfloat16)
    weight = (torch.rand((dim, W), generator=gen("weight"), dtype=f32, device=device) * 2 - 1) * lim
    bias = (torch.rand((dim,), generator=gen("bias"), dtype=f32, device=device) * 2 - 1) * lim
    state = torch.randn((N, W - 1, dim), generator=gen("state"), dtype=f32,
                        device=device).to(torch.bfloat16)
    return {"x": x, "weight": weight, "bias": bias, "state": state, "cu_seqlens": cu.to(device),
            "cu_host": cu.numpy().astype(np.int64)}
