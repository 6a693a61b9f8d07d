"""PyTorch-facing entry points of libkda: argument marshalling only.

Every step of the KDA forward runs in the HIP kernels behind the C ABI
(include/kda.h); torch supplies device memory and the current stream.
"""
from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _abi

_DTYPES = {torch.float32: _abi.KDA_DTYPE_F32, torch.bfloat16: _abi.KDA_DTYPE_BF16}


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _check(t: torch.Tensor, name: str, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


_PLANS = {"auto": _abi.KDA_PLAN_AUTO, "fused": _abi.KDA_PLAN_FUSED,
          "two_pass": _abi.KDA_PLAN_TWO_PASS}


def _gate_tuple(gate):
    if gate is None:
        return (_abi.KDA_GATE_GIVEN, None, None, None)
    x, a_log, dt_bias = gate
    return (_abi.KDA_GATE_KIMI, _ptr(x), _ptr(a_log), _ptr(dt_bias))


def _check_gate(gate, g, lead, H, dk, dtype, dev):
    """g [*lead, H, dk] fp32, or gate = (x [*lead, H, dk] in dtype, a_log [H]
    fp32, dt_bias [H, dk] fp32)."""
    if gate is None:
        if g is None:
            raise ValueError("g is required unless gate = (x, a_log, dt_bias) is given")
        _check(g, "g", (*lead, H, dk), torch.float32, dev)
        return
    if len(gate) != 3:
        raise ValueError("gate must be (x, a_log, dt_bias)")
    x, a_log, dt_bias = gate
    _check(x, "gate x", (*lead, H, dk), dtype, dev)
    _check(a_log, "gate a_log", (H,), torch.float32, dev)
    _check(dt_bias, "gate dt_bias", (H, dk), torch.float32, dev)


def prefill_desc(q, k, v, g, beta, h0=None, cu_seqlens=None, scale=None, chunk=64, o=None,
                 ht=None, plan="auto", gate=None, state_indices=None,
                 n_slots=0, qk_l2norm=False) -> _abi.PrefillDesc:
    st = h0 if h0 is not None else ht
    T, Hg, dk = q.shape
    H, dv = v.shape[1], v.shape[-1]
    N = 1 if cu_seqlens is None else int(cu_seqlens.shape[0]) - 1
    return _abi.prefill_desc(
        dtype=_DTYPES[q.dtype], n_seqs=N, n_heads=H, dk=dk, dv=dv, chunk=int(chunk),
        plan=_PLANS[plan], t_total=T, scale=0.0 if scale is None else float(scale), q=_ptr(q), k=_ptr(k),
        v=_ptr(v), g=_ptr(g), beta=_ptr(beta), h0=_ptr(h0), cu_seqlens=_ptr(cu_seqlens),
        o=_ptr(o), ht=_ptr(ht), gate=_gate_tuple(gate), state_indices=_ptr(state_indices),
        n_slots=int(n_slots), n_k_heads=Hg, qk_l2norm=int(bool(qk_l2norm)),
        state_dtype=_DTYPES[st.dtype] if st is not None else _abi.KDA_DTYPE_F32)


def _state_dtype(h0, ht, state_dtype):
    """dtype of the states of one call: that of h0 or ht when given (they must
    agree), else `state_dtype` (fp32 by default) for a newly allocated ht."""
    given = [t.dtype for t in (h0, ht) if t is not None]
    sd = given[0] if given else (state_dtype or torch.float32)
    if sd not in _DTYPES or any(x != sd for x in given):
        raise TypeError(f"states must share one dtype of fp32/bf16, got {given or [sd]}")
    if state_dtype is not None and state_dtype != sd:
        raise TypeError(f"state_dtype {state_dtype} but the states are {sd}")
    return sd


def _prefill_args(q, k, v, g, beta, h0, cu_seqlens, out, ht, output_final_state, gate,
                  state_indices, state_dtype):
    """Shared checks of the prefill entry points; returns (N, n_slots, out, ht)."""
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("the KDA prefill runs on the GPU only")
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    T, Hg, dk = q.shape
    if v.dim() != 3:
        raise ValueError(f"v must be [T, H, dv], got {tuple(v.shape)}")
    H, dv = int(v.shape[1]), int(v.shape[2])
    if H % Hg:
        raise ValueError(f"q/k heads {Hg} must divide the value heads {H}")
    N = 1 if cu_seqlens is None else int(cu_seqlens.shape[0]) - 1
    _check(q, "q", (T, Hg, dk), q.dtype, dev)
    _check(k, "k", (T, Hg, dk), q.dtype, dev)
    _check(v, "v", (T, H, dv), q.dtype, dev)
    _check_gate(gate, g, (T,), H, dk, q.dtype, dev)
    _check(beta, "beta", (T, H), q.dtype, dev)
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, dev)
    S = N
    if state_indices is not None:
        _check(state_indices, "state_indices", (N,), torch.int32, dev)
        pool = h0 if h0 is not None else ht
        if pool is None:
            raise ValueError("state_indices needs a state pool (h0 and/or ht)")
        S = int(pool.shape[0])
    sd = _state_dtype(h0, ht, state_dtype)
    if h0 is not None:
        _check(h0, "h0", (S, H, dk, dv), sd, dev)
    if out is None:
        out = torch.empty((T, H, dv), dtype=q.dtype, device=dev)
    else:
        _check(out, "out", (T, H, dv), q.dtype, dev)
    if ht is None and output_final_state:
        ht = h0 if state_indices is not None else torch.empty((N, H, dk, dv), dtype=sd,
                                                                device=dev)
    if ht is not None:
        _check(ht, "ht", (S, H, dk, dv), sd, dev)
    return N, (S if state_indices is not None else 0), out, ht


def prefill_workspace_bytes(T: int, H: int, d: int, n_seqs: int = 1, chunk: int = 64,
                            dtype: torch.dtype = torch.bfloat16) -> int:
    desc = _abi.prefill_desc(dtype=_DTYPES[dtype], n_seqs=n_seqs, n_heads=H, dk=d, dv=d,
                             chunk=chunk, t_total=T)
    return _abi.workspace_bytes(desc)


def chunk_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: Optional[torch.Tensor],
                  beta: torch.Tensor, h0: Optional[torch.Tensor] = None,
                  cu_seqlens: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                  chunk: int = 64, out: Optional[torch.Tensor] = None,
                  ht: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  output_final_state: bool = True, stream=None, events=None,
                  plan: str = "auto", gate=None,
                  state_indices: Optional[torch.Tensor] = None, qk_l2norm: bool = False,
                  state_dtype: Optional[torch.dtype] = None, noalloc: bool = False,
                  check: bool = False) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked KDA prefill.  q, k: [T, Hg, dk] (Hg key heads, each shared by
    H / Hg consecutive value heads; Hg = H by default); g: [T, H, dk]; v: [T, H, dv]; beta: [T, H];
    h0: [N, H, dk, dv] fp32 or None; cu_seqlens: int32 [N + 1] on the device or
    None (one sequence).  Returns (o [T, H, dv], ht [N, H, dk, dv] or None).
    `ht` may be h0 itself (in-place carry).  `events`: four torch.cuda.Event
    objects recorded before the first launch and after each of the three
    launches (chunk map, chunk-local stage, state scan), for stage timing.
    `plan`: "auto" or "two_pass" (the same plan; "fused" is a reserved value
    the library refuses).  `gate`: None
    (g given), or (x [T, H, dk] in q's dtype, a_log [H] fp32, dt_bias [H, dk]
    fp32) to compute g = -exp(a_log) softplus(x + dt_bias) in the kernels
    (g may then be None).  `state_indices` (int32 [N] on the device): h0 and
    ht are then state pools [S, H, dk, dv] (ht defaults to h0: in place) and
    sequence n uses slot state_indices[n]; a negative slot skips it.
    `qk_l2norm`: L2-normalise every q and k row in the kernels (eps 1e-6).
    States (h0, ht) are fp32, or bf16 with bf16 inputs: their dtype is that of
    h0 / ht when given, else `state_dtype` (fp32 by default) for a new ht.  The
    arithmetic is fp32 either way; a bf16 ht is rounded once when written.
    `noalloc`: call kda_chunk_prefill_noalloc, whose workspace is the library's
    static per-device buffer (KDA_NOALLOC_WORKSPACE_BYTES) -- nothing is
    allocated for it; `workspace` and `events` must then be None, and `out`
    (and `ht`) should be passed by callers that allocate nothing at all.
    `cu_seqlens` is read on the device: when it is invalid (not starting at 0,
    decreasing, or ending elsewhere than T) the kernels write neither o nor ht
    and set the workspace's status word instead.  `check=True` reads that word
    after the launches (this synchronises the stream) and raises KdaError if it
    is set; without it, and with a workspace this function allocated, the
    failure is not visible to the caller (pass `workspace` and call
    workspace_status to read it later).  `check` needs a workspace, so it
    cannot be combined with `noalloc`."""
    dev = q.device
    N, n_slots, out, ht = _prefill_args(q, k, v, g, beta, h0, cu_seqlens, out, ht,
                                        output_final_state, gate, state_indices, state_dtype)
    desc = prefill_desc(q, k, v, g, beta, h0, cu_seqlens, scale, chunk, out, ht, plan, gate,
                        state_indices, n_slots, qk_l2norm)
    if noalloc:
        if workspace is not None or events is not None or check:
            raise ValueError("noalloc takes no workspace, no events and no check")
        st = _abi.chunk_prefill_noalloc_raw(desc, _stream(stream))
        if st != _abi.KDA_OK:
            raise _abi.KdaError(st, "kda_chunk_prefill_noalloc")
        return out, ht
    need = _abi.workspace_bytes(desc)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    handles = None
    if events is not None:
        if len(events) != 4:
            raise ValueError("events must be four torch.cuda.Event objects")
        for e in events:  # torch creates the HIP event on its first record
            if e.cuda_event == 0:
                e.record(torch.cuda.current_stream() if stream is None else stream)
        handles = [e.cuda_event for e in events]
    st = _abi.chunk_prefill_timed_raw(desc, workspace.data_ptr(),
                                      workspace.numel() * workspace.element_size(),
                                      _stream(stream), handles)
    if st != _abi.KDA_OK:
        raise _abi.KdaError(st, "kda_chunk_prefill")
    if check:
        st = _abi.workspace_status(workspace.data_ptr(), _stream(stream))
        if st != _abi.KDA_OK:
            raise _abi.KdaError(st, "kda_chunk_prefill (device status)")
    return out, ht


def recurrent_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                      g: Optional[torch.Tensor], beta: torch.Tensor,
                      h0: Optional[torch.Tensor] = None,
                      cu_seqlens: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                      out: Optional[torch.Tensor] = None, ht: Optional[torch.Tensor] = None,
                      output_final_state: bool = True, stream=None, gate=None,
                      state_indices: Optional[torch.Tensor] = None, qk_l2norm: bool = False,
                      state_dtype: Optional[torch.dtype] = None
                      ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """The prefill of chunk_prefill computed token by token with the state held
    on chip (for continuing prefills of a few tokens on a carried state).  Same
    arguments and results; no chunk, plan or workspace."""
    N, n_slots, out, ht = _prefill_args(q, k, v, g, beta, h0, cu_seqlens, out, ht,
                                        output_final_state, gate, state_indices, state_dtype)
    desc = prefill_desc(q, k, v, g, beta, h0, cu_seqlens, scale, 64, out, ht, "auto", gate,
                        state_indices, n_slots, qk_l2norm)
    st = _abi.recurrent_prefill_raw(desc, _stream(stream))
    if st != _abi.KDA_OK:
        raise _abi.KdaError(st, "kda_recurrent_prefill")
    return out, ht


def recurrent_decode(state: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                     g: Optional[torch.Tensor], beta: torch.Tensor, scale: Optional[float] = None,
                     out: Optional[torch.Tensor] = None, stream=None, gate=None,
                     state_indices: Optional[torch.Tensor] = None,
                     qk_l2norm: bool = False) -> torch.Tensor:
    """One recurrent decode step; `state` [N, H, dk, dv] is updated in place.
    The state is fp32, or bf16 with bf16 inputs (fp32 arithmetic, rounded once
    when written back).
    q, k: [N, Hg, dk] (Hg divides H); g: [N, H, dk]; v: [N, H, dv]; beta: [N, H].
    Returns o [N, H, dv].  `qk_l2norm` as in chunk_prefill.
    `gate` as in chunk_prefill (x is [N, H, dk]).  `state_indices` (int32 [N]
    on the device): `state` is then a pool [S, H, dk, dv] and sequence n
    updates slot state_indices[n]; a negative slot skips it (its o is left as
    it was)."""
    dev = state.device
    if dev.type != "cuda":
        raise ValueError("recurrent_decode runs on the GPU only")
    if q.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {q.dtype}")
    S, H, dk, dv = state.shape
    N = S if state_indices is None else int(q.shape[0])
    if state.dtype not in _DTYPES:
        raise TypeError(f"state must be fp32 or bf16, got {state.dtype}")
    _check(state, "state", (S, H, dk, dv), state.dtype, dev)
    if state_indices is not None:
        _check(state_indices, "state_indices", (N,), torch.int32, dev)
    Hg = int(q.shape[1]) if q.dim() == 3 else H
    if Hg < 1 or H % Hg:
        raise ValueError(f"q/k heads {Hg} must divide the value heads {H}")
    _check(q, "q", (N, Hg, dk), q.dtype, dev)
    _check(k, "k", (N, Hg, dk), q.dtype, dev)
    _check(v, "v", (N, H, dv), q.dtype, dev)
    _check_gate(gate, g, (N,), H, dk, q.dtype, dev)
    _check(beta, "beta", (N, H), q.dtype, dev)
    if out is None:
        out = torch.empty((N, H, dv), dtype=q.dtype, device=dev)
    else:
        _check(out, "out", (N, H, dv), q.dtype, dev)
    desc = _abi.decode_desc(dtype=_DTYPES[q.dtype], n_seqs=N, n_heads=H, dk=dk, dv=dv,
                            scale=0.0 if scale is None else float(scale), state=state.data_ptr(),
                            q=q.data_ptr(), k=k.data_ptr(), v=v.data_ptr(), g=_ptr(g),
                            beta=beta.data_ptr(), o=out.data_ptr(), gate=_gate_tuple(gate),
                            state_indices=_ptr(state_indices),
                            n_slots=S if state_indices is not None else 0, n_k_heads=Hg,
                            qk_l2norm=int(bool(qk_l2norm)), state_dtype=_DTYPES[state.dtype])
    st = _abi.recurrent_decode_raw(desc, _stream(stream))
    if st != _abi.KDA_OK:
        raise _abi.KdaError(st, "kda_recurrent_decode")
    return out


def workspace_status(workspace: torch.Tensor, stream=None) -> int:
    """Device status word of the last prefill that used `workspace`."""
    return _abi.workspace_status(workspace.data_ptr(), _stream(stream))


_ACTS = {None: _abi.KDA_CONV_ACT_NONE, "none": _abi.KDA_CONV_ACT_NONE,
         "silu": _abi.KDA_CONV_ACT_SILU}


def _conv_args(x, weight, bias, state_in, state_out, state_indices, n_seqs, split, out,
               activation):
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("the causal conv runs on the GPU only")
    if x.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {x.dtype}")
    if activation not in _ACTS:
        raise ValueError(f"activation must be one of {list(_ACTS)}")
    rows, dim = x.shape
    _check(x, "x", (rows, dim), x.dtype, dev)
    if weight.dim() != 2 or weight.shape[0] != dim:
        raise ValueError(f"weight must be [dim={dim}, W], got {tuple(weight.shape)}")
    W = int(weight.shape[1])
    _check(weight, "weight", (dim, W), torch.float32, dev)
    if bias is not None:
        _check(bias, "bias", (dim,), torch.float32, dev)
    S = n_seqs if state_indices is None else None
    for name, st in (("state_in", state_in), ("state_out", state_out)):
        if st is not None:
            if S is None:
                S = int(st.shape[0])
            _check(st, name, (S, W - 1, dim), x.dtype, dev)
    if state_indices is not None:
        if state_in is None and state_out is None:
            raise ValueError("state_indices needs a tap pool (state_in and/or state_out)")
        _check(state_indices, "state_indices", (n_seqs,), torch.int32, dev)
    widths = (dim,) if split is None else tuple(int(w) for w in split)
    if sum(widths) != dim or not 1 <= len(widths) <= 3:
        raise ValueError(f"split {widths} must be 1..3 widths summing to dim={dim}")
    if out is None:
        ys = tuple(torch.empty((rows, w), dtype=x.dtype, device=dev) for w in widths)
    else:
        ys = (out,) if isinstance(out, torch.Tensor) else tuple(out)
        if len(ys) != len(widths):
            raise ValueError("out must match split")
        for i, (y, w) in enumerate(zip(ys, widths)):
            _check(y, f"out[{i}]", (rows, w), x.dtype, dev)
    desc = _abi.conv_desc(dtype=_DTYPES[x.dtype], n_seqs=n_seqs, dim=dim, width=W,
                          activation=_ACTS[activation], x=x.data_ptr(),
                          weight=weight.data_ptr(), bias=_ptr(bias), state_in=_ptr(state_in),
                          state_out=_ptr(state_out), state_indices=_ptr(state_indices),
                          n_slots=S if state_indices is not None else 0, n_out=len(widths),
                          y=[y.data_ptr() for y in ys] + [None] * (3 - len(ys)),
                          y_width=list(widths) + [0] * (3 - len(widths)))
    return desc, (ys[0] if split is None else ys)


def causal_conv1d_fwd(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor] = None,
                      cu_seqlens: Optional[torch.Tensor] = None,
                      state_in: Optional[torch.Tensor] = None,
                      state_out: Optional[torch.Tensor] = None,
                      state_indices: Optional[torch.Tensor] = None, activation="silu",
                      split=None, out=None, stream=None):
    """Short causal depthwise conv over a packed batch with carried taps.

    x [T, dim] (fp32 or bf16); weight [dim, W] fp32, W in 2..4; bias [dim]
    fp32; cu_seqlens int32 [N + 1] (None for one sequence); state_in /
    state_out [S, W - 1, dim] in x.dtype (None: zero taps in / none out; may be
    the same tensor), S = N or the pool size with state_indices (int32 [N],
    negative = skip the sequence).  split: None returns y [T, dim]; a tuple of
    1..3 widths returns that many dense [T, w] tensors (e.g. q, k, v)."""
    N = 1 if cu_seqlens is None else int(cu_seqlens.shape[0]) - 1
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", (N + 1,), torch.int32, x.device)
    desc, y = _conv_args(x, weight, bias, state_in, state_out, state_indices, N, split, out,
                         activation)
    desc.t_total = int(x.shape[0])
    desc.cu_seqlens = _ptr(cu_seqlens)
    st = _abi.conv_fwd_raw(desc, _stream(stream))
    if st != _abi.KDA_OK:
        raise _abi.KdaError(st, "kda_causal_conv1d_fwd")
    return y


def causal_conv1d_update(x: torch.Tensor, weight: torch.Tensor,
                         bias: Optional[torch.Tensor] = None,
                         state: Optional[torch.Tensor] = None,
                         state_indices: Optional[torch.Tensor] = None, activation="silu",
                         split=None, out=None, stream=None):
    """One token per sequence: x [N, dim]; `state` [S, W - 1, dim] is read and
    shifted in place (S = N, or the pool size with state_indices).  Returns y
    as causal_conv1d_fwd does."""
    desc, y = _conv_args(x, weight, bias, state, state, state_indices, int(x.shape[0]), split,
                         out, activation)
    st = _abi.conv_update_raw(desc, _stream(stream))
    if st != _abi.KDA_OK:
        raise _abi.KdaError(st, "kda_causal_conv1d_update")
    return y
