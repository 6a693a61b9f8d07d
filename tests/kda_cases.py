"""Helpers shared by the GPU tests: move seeded inputs to the device, run the
oracle on the same (rounded) values, and compare."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth

TOL = {"f32": 1e-4, "bf16": 1e-2}  # relative L2 bars for o and the final state


def rel_l2(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (n if n > 0 else 1.0))


def to_dev(arr: np.ndarray, dtype: str, dev="cuda") -> torch.Tensor:
    if arr.dtype == np.uint16:
        t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr))
    return t.to(dev)


def to_host64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def dev_inputs(inp: synth.KdaInputs, dev="cuda") -> dict:
    d = inp.dtype
    return {
        "q": to_dev(inp.q, d, dev), "k": to_dev(inp.k, d, dev), "v": to_dev(inp.v, d, dev),
        "g": to_dev(inp.g, "f32", dev), "beta": to_dev(inp.beta, d, dev),
        "h0": None if inp.h0 is None else to_dev(inp.h0, "f32", dev),
        "cu_seqlens": torch.from_numpy(inp.cu_seqlens).to(dev),
    }


def dev_gate(inp: synth.KdaInputs, dev="cuda") -> tuple:
    """The raw gate (x, a_log, dt_bias) on the device, as the fused-gate path takes it."""
    return (to_dev(inp.gate_x, inp.dtype, dev), to_dev(inp.gate_a_log, "f32", dev),
            to_dev(inp.gate_dt_bias, "f32", dev))


def oracle_qk(inp: synth.KdaInputs, f: dict, qk_l2norm: bool = False):
    """q and k as the oracle consumes them: normalised when the kernels are
    asked to normalise, and expanded from Hg key heads to the H heads."""
    q, k = f["q"], f["k"]
    if qk_l2norm:
        q, k = oracle.l2norm(q), oracle.l2norm(k)
    return oracle.expand_key_heads(q, inp.H), oracle.expand_key_heads(k, inp.H)


def oracle_prefill(inp: synth.KdaInputs, fused_gate: bool = False, qk_l2norm: bool = False):
    """fp64 oracle on the rounded inputs; with fused_gate, g is recomputed by
    the oracle from the stored raw gate (what the fused-gate path receives);
    with qk_l2norm, q and k are normalised by the oracle first."""
    f = inp.f64()
    g = oracle.kimi_gate(*inp.gate_f64()) if fused_gate else f["g"]
    q, k = oracle_qk(inp, f, qk_l2norm)
    return oracle.prefill(q, k, f["v"], g, f["beta"], f["h0"], f["cu_seqlens"], f["scale"])


# Per-token bound on o: each (token, head) row's error against
#   TOK_FACTOR x the whole-tensor bar x (|ref row| + 0.1 x rms of the ref rows),
# so a single wrong token fails even when the whole-tensor rel-L2 of a long
# sequence would hide it; the 0.1 rms floor keeps rows whose reference is
# near zero from turning rounding noise into a large relative error.
TOK_FACTOR = 10.0


def token_errors(o, ref) -> np.ndarray:
    """Per-row error ratio err / (|ref| + 0.1 rms) over the last axis."""
    o = np.asarray(o, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.linalg.norm(o - ref, axis=-1)
    rn = np.linalg.norm(ref, axis=-1)
    rms = float(np.sqrt(np.mean(rn ** 2))) if rn.size else 0.0
    return err / (rn + 0.1 * rms + 1e-300)


def check_tokens(o, ref, tol: float) -> float:
    """Assert the per-token bound; returns the worst row's ratio."""
    if np.asarray(ref).size == 0:
        return 0.0
    worst = float(token_errors(o, ref).max())
    assert worst <= TOK_FACTOR * tol, f"worst token row {worst:.3e} > {TOK_FACTOR * tol:.1e}"
    return worst


def worst_head(o, ref) -> float:
    """Largest rel-L2 over the head axis (axis 1 of [T, H, d] or [N, H, d, d])."""
    o = np.asarray(o, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return max(rel_l2(o[:, i], ref[:, i]) for i in range(ref.shape[1]))


def say(msg: str):
    print(msg, flush=True)
