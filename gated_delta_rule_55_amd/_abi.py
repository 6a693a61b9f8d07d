"""ctypes mirror of include/kda.h and include/kda_conv.h.  Loads the in-tree libkda.so; there is no
other implementation to fall back to, so a missing library is an error."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkda.so")

KDA_ABI_VERSION = 5
KDA_OK = 0
KDA_ERR_NULL = -1
KDA_ERR_SHAPE = -2
KDA_ERR_DTYPE = -3
KDA_ERR_UNSUPPORTED = -4
KDA_ERR_ALIGN = -5
KDA_ERR_WORKSPACE = -6
KDA_ERR_HIP = -7
KDA_ERR_VERSION = -8
KDA_ERR_ALIAS = -9
KDA_ERR_SEQLENS = -10
KDA_ERR_SYNC = -11

KDA_PLAN_AUTO = 0
KDA_PLAN_FUSED = 1
KDA_PLAN_TWO_PASS = 2

KDA_DTYPE_F32 = 1
KDA_DTYPE_BF16 = 2

KDA_GATE_GIVEN = 0
KDA_GATE_KIMI = 1

KDA_CONV_ACT_NONE = 0
KDA_CONV_ACT_SILU = 1


class GateDesc(ctypes.Structure):
    _fields_ = [
        ("mode", ctypes.c_int32),
        ("x", ctypes.c_void_p),
        ("a_log", ctypes.c_void_p),
        ("dt_bias", ctypes.c_void_p),
    ]


class PrefillDesc(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
        ("n_seqs", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("dk", ctypes.c_int32),
        ("dv", ctypes.c_int32),
        ("chunk", ctypes.c_int32),
        ("plan", ctypes.c_int32),
        ("t_total", ctypes.c_int64),
        ("scale", ctypes.c_float),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p),
        ("beta", ctypes.c_void_p),
        ("h0", ctypes.c_void_p),
        ("cu_seqlens", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("ht", ctypes.c_void_p),
        ("gate", GateDesc),
        ("state_indices", ctypes.c_void_p),
        ("n_slots", ctypes.c_int32),
        ("n_k_heads", ctypes.c_int32),
        ("qk_l2norm", ctypes.c_int32),
        ("state_dtype", ctypes.c_int32),
    ]


class DecodeDesc(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
        ("n_seqs", ctypes.c_int32),
        ("n_heads", ctypes.c_int32),
        ("dk", ctypes.c_int32),
        ("dv", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("state", ctypes.c_void_p),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("g", ctypes.c_void_p),
        ("beta", ctypes.c_void_p),
        ("o", ctypes.c_void_p),
        ("gate", GateDesc),
        ("state_indices", ctypes.c_void_p),
        ("n_slots", ctypes.c_int32),
        ("n_k_heads", ctypes.c_int32),
        ("qk_l2norm", ctypes.c_int32),
        ("state_dtype", ctypes.c_int32),
    ]


class ConvDesc(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int32),
        ("n_seqs", ctypes.c_int32),
        ("dim", ctypes.c_int32),
        ("width", ctypes.c_int32),
        ("activation", ctypes.c_int32),
        ("t_total", ctypes.c_int64),
        ("x", ctypes.c_void_p),
        ("weight", ctypes.c_void_p),
        ("bias", ctypes.c_void_p),
        ("cu_seqlens", ctypes.c_void_p),
        ("state_in", ctypes.c_void_p),
        ("state_out", ctypes.c_void_p),
        ("state_indices", ctypes.c_void_p),
        ("n_slots", ctypes.c_int32),
        ("n_out", ctypes.c_int32),
        ("y", ctypes.c_void_p * 3),
        ("y_width", ctypes.c_int32 * 3),
    ]


class KdaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status}"
                         + (f", hipError {lib().kda_last_hip_error()})" if status == KDA_ERR_HIP
                            else ")"))


_LIB = None


def lib():
    """The loaded libkda.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -m gated_delta_rule_55_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        L.kda_abi_version.argtypes = []
        L.kda_abi_version.restype = ctypes.c_int
        L.kda_status_string.argtypes = [ctypes.c_int]
        L.kda_status_string.restype = ctypes.c_char_p
        L.kda_last_hip_error.argtypes = []
        L.kda_last_hip_error.restype = ctypes.c_int
        L.kda_chunk_prefill_workspace_bytes.argtypes = [ctypes.POINTER(PrefillDesc),
                                                        ctypes.POINTER(ctypes.c_int)]
        L.kda_chunk_prefill_workspace_bytes.restype = ctypes.c_size_t
        L.kda_chunk_prefill.argtypes = [ctypes.POINTER(PrefillDesc), ctypes.c_void_p,
                                        ctypes.c_size_t, ctypes.c_void_p]
        L.kda_chunk_prefill.restype = ctypes.c_int
        L.kda_chunk_prefill_timed.argtypes = [ctypes.POINTER(PrefillDesc), ctypes.c_void_p,
                                              ctypes.c_size_t, ctypes.c_void_p,
                                              ctypes.POINTER(ctypes.c_void_p)]
        L.kda_chunk_prefill_timed.restype = ctypes.c_int
        L.kda_chunk_prefill_noalloc.argtypes = [ctypes.POINTER(PrefillDesc), ctypes.c_void_p]
        L.kda_chunk_prefill_noalloc.restype = ctypes.c_int
        L.kda_workspace_status.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        L.kda_workspace_status.restype = ctypes.c_int
        L.kda_recurrent_decode.argtypes = [ctypes.POINTER(DecodeDesc), ctypes.c_void_p]
        L.kda_recurrent_decode.restype = ctypes.c_int
        L.kda_recurrent_prefill.argtypes = [ctypes.POINTER(PrefillDesc), ctypes.c_void_p]
        L.kda_recurrent_prefill.restype = ctypes.c_int
        for name in ("kda_causal_conv1d_fwd", "kda_causal_conv1d_update"):
            fn = getattr(L, name)
            fn.argtypes = [ctypes.POINTER(ConvDesc), ctypes.c_void_p]
            fn.restype = ctypes.c_int
        if L.kda_abi_version() != KDA_ABI_VERSION:
            raise RuntimeError(f"libkda ABI {L.kda_abi_version()} != {KDA_ABI_VERSION}")
        _LIB = L
    return _LIB


def status_string(status: int) -> str:
    return lib().kda_status_string(int(status)).decode()


def _fill(d, kw):
    for key, val in kw.items():
        if key == "gate":  # (mode, x, a_log, dt_bias)
            mode, x, a_log, dt_bias = val
            d.gate = GateDesc(mode, x, a_log, dt_bias)
        else:
            setattr(d, key, val)
    return d


def prefill_desc(**kw) -> PrefillDesc:
    d = PrefillDesc()
    d.struct_size = ctypes.sizeof(PrefillDesc)
    return _fill(d, kw)


def decode_desc(**kw) -> DecodeDesc:
    d = DecodeDesc()
    d.struct_size = ctypes.sizeof(DecodeDesc)
    return _fill(d, kw)


def conv_desc(**kw) -> ConvDesc:
    d = ConvDesc()
    d.struct_size = ctypes.sizeof(ConvDesc)
    for key, val in kw.items():
        if key in ("y", "y_width"):
            for i, v in enumerate(val):
                getattr(d, key)[i] = v
        else:
            setattr(d, key, val)
    return d


def workspace_bytes(desc: PrefillDesc) -> int:
    st = ctypes.c_int(0)
    n = lib().kda_chunk_prefill_workspace_bytes(ctypes.byref(desc), ctypes.byref(st))
    if st.value != KDA_OK:
        raise KdaError(st.value, "kda_chunk_prefill_workspace_bytes")
    return int(n)


def chunk_prefill_raw(desc: PrefillDesc, workspace: int, workspace_bytes: int, stream: int) -> int:
    return int(lib().kda_chunk_prefill(ctypes.byref(desc), workspace, workspace_bytes, stream))


def chunk_prefill_timed_raw(desc: PrefillDesc, workspace: int, workspace_bytes: int,
                            stream: int, events) -> int:
    """events: four raw hipEvent_t handles (ints) or None."""
    arr = None
    if events is not None:
        arr = (ctypes.c_void_p * 4)(*[int(e) for e in events])
    return int(lib().kda_chunk_prefill_timed(ctypes.byref(desc), workspace, workspace_bytes,
                                             stream, arr))


# Bytes of the static workspace kda_chunk_prefill_noalloc uses (one per device).
KDA_NOALLOC_WORKSPACE_BYTES = 64 << 20


def chunk_prefill_noalloc_raw(desc: PrefillDesc, stream: int) -> int:
    return int(lib().kda_chunk_prefill_noalloc(ctypes.byref(desc), stream))


def recurrent_decode_raw(desc: DecodeDesc, stream: int) -> int:
    return int(lib().kda_recurrent_decode(ctypes.byref(desc), stream))


def recurrent_prefill_raw(desc: PrefillDesc, stream: int) -> int:
    return int(lib().kda_recurrent_prefill(ctypes.byref(desc), stream))


def workspace_status(workspace: int, stream: int) -> int:
    return int(lib().kda_workspace_status(workspace, stream))


def conv_fwd_raw(desc: ConvDesc, stream: int) -> int:
    return int(lib().kda_causal_conv1d_fwd(ctypes.byref(desc), stream))


def conv_update_raw(desc: ConvDesc, stream: int) -> int:
    return int(lib().kda_causal_conv1d_update(ctypes.byref(desc), stream))
