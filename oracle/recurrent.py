"""ctypes binding to the fp64 token-by-token oracle in kda_oracle.c.

Test infrastructure only.  Arrays are widened to contiguous fp64 here; the C
side does all of the arithmetic.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.path.join(HERE, "liboracle.so")


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


class OracleLib:
    """One loaded copy of the C oracle (the test suite also loads deliberately
    broken builds of the same source through this class)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        i64, dp = ctypes.c_int64, ctypes.POINTER(ctypes.c_double)
        lib.kda_oracle_prefill_f64.argtypes = [i64, i64, i64, i64, ctypes.POINTER(i64), dp, dp,
                                               dp, dp, dp, dp, ctypes.c_double, dp, dp]
        lib.kda_oracle_prefill_f64.restype = ctypes.c_int
        lib.kda_oracle_decode_f64.argtypes = [i64, i64, i64, i64, dp, dp, dp, dp, dp, dp,
                                              ctypes.c_double, dp]
        lib.kda_oracle_decode_f64.restype = ctypes.c_int
        lib.kda_oracle_num_threads.argtypes = []
        lib.kda_oracle_num_threads.restype = ctypes.c_int
        # the fp32 twin (absent from the single-source builds the tests plant
        # mistakes in)
        self.has_f32 = hasattr(lib, "kda_oracle_prefill_f32")
        if self.has_f32:
            i64, fp = ctypes.c_int64, ctypes.POINTER(ctypes.c_float)
            lib.kda_oracle_prefill_f32.argtypes = [i64, i64, i64, i64, ctypes.POINTER(i64), fp,
                                                   fp, fp, fp, fp, fp, ctypes.c_float, fp, fp]
            lib.kda_oracle_prefill_f32.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def num_threads(self) -> int:
        return int(self.lib.kda_oracle_num_threads())

    def set_num_threads(self, n: int) -> None:
        """Threads of later calls (OpenMP over the independent chains)."""
        if hasattr(self.lib, "kda_oracle_set_num_threads"):
            self.lib.kda_oracle_set_num_threads(ctypes.c_int(int(n)))

    def prefill(self, q, k, v, g, beta, h0=None, cu_seqlens=None, scale=None):
        """Token-by-token KDA prefill in fp64.

        q, k, g: [T, H, dk]; v: [T, H, dv]; beta: [T, H]; h0: [N, H, dk, dv] or None;
        cu_seqlens: [N + 1] token offsets (default: one sequence of T tokens).
        Returns (o [T, H, dv], hT [N, H, dk, dv]), both fp64."""
        q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
        T, H, dk = q.shape
        dv = v.shape[2]
        if k.shape != (T, H, dk) or g.shape != (T, H, dk) or v.shape[:2] != (T, H) \
                or beta.shape != (T, H):
            raise ValueError("inconsistent shapes")
        cu = np.array([0, T], dtype=np.int64) if cu_seqlens is None else \
            np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        N = cu.shape[0] - 1
        if cu[-1] != T:
            raise ValueError("cu_seqlens[-1] must equal T")
        h0a = None if h0 is None else _f64(h0)
        if h0a is not None and h0a.shape != (N, H, dk, dv):
            raise ValueError("h0 shape")
        sc = float(dk ** -0.5) if scale is None else float(scale)
        o = np.zeros((T, H, dv), dtype=np.float64)
        ht = np.zeros((N, H, dk, dv), dtype=np.float64)
        rc = self.lib.kda_oracle_prefill_f64(
            N, H, dk, dv, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _ptr(q), _ptr(k),
            _ptr(v), _ptr(g), _ptr(beta), _ptr(h0a), sc, _ptr(o), _ptr(ht))
        if rc != 0:
            raise RuntimeError(f"oracle prefill failed ({rc})")
        return o, ht

    def prefill_f32(self, q, k, v, g, beta, h0=None, cu_seqlens=None, scale=None):
        """The fp32 twin of prefill(): the same token loop with every value and
        every accumulation in fp32 (inputs rounded to fp32 first).  A
        diagnostic of the fp32 floor; returns fp64 copies of the fp32 results."""
        f32 = lambda x: np.ascontiguousarray(np.asarray(x, dtype=np.float32))  # noqa: E731
        q, k, v, g, beta = f32(q), f32(k), f32(v), f32(g), f32(beta)
        T, H, dk = q.shape
        dv = v.shape[2]
        cu = np.array([0, T], dtype=np.int64) if cu_seqlens is None else \
            np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        N = cu.shape[0] - 1
        h0a = None if h0 is None else f32(h0)
        sc = float(dk ** -0.5) if scale is None else float(scale)
        o = np.zeros((T, H, dv), dtype=np.float32)
        ht = np.zeros((N, H, dk, dv), dtype=np.float32)
        fp = lambda a: None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))  # noqa: E731
        rc = self.lib.kda_oracle_prefill_f32(
            N, H, dk, dv, cu.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), fp(q), fp(k), fp(v),
            fp(g), fp(beta), fp(h0a), sc, fp(o), fp(ht))
        if rc != 0:
            raise RuntimeError(f"oracle fp32 prefill failed ({rc})")
        return o.astype(np.float64), ht.astype(np.float64)

    def decode(self, state, q, k, v, g, beta, scale=None):
        """One decode step.  state: [N, H, dk, dv]; q, k, g: [N, H, dk]; v: [N, H, dv];
        beta: [N, H].  Returns (o [N, H, dv], new_state) in fp64; `state` is untouched."""
        st = _f64(state).copy()
        q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
        N, H, dk, dv = st.shape
        if q.shape != (N, H, dk) or k.shape != (N, H, dk) or g.shape != (N, H, dk) \
                or v.shape != (N, H, dv) or beta.shape != (N, H):
            raise ValueError("inconsistent shapes")
        sc = float(dk ** -0.5) if scale is None else float(scale)
        o = np.zeros((N, H, dv), dtype=np.float64)
        rc = self.lib.kda_oracle_decode_f64(N, H, dk, dv, _ptr(st), _ptr(q), _ptr(k), _ptr(v),
                                            _ptr(g), _ptr(beta), sc, _ptr(o))
        if rc != 0:
            raise RuntimeError(f"oracle decode failed ({rc})")
        return o, st


_DEFAULT: Optional[OracleLib] = None


def default() -> OracleLib:
    global _DEFAULT
    if _DEFAULT is None:
        if not os.path.exists(lib_path()):
            from .build import build

            build()
        _DEFAULT = OracleLib(lib_path())
    return _DEFAULT


def prefill(*args, **kwargs):
    return default().prefill(*args, **kwargs)


def decode(*args, **kwargs):
    return default().decode(*args, **kwargs)


def prefill_f32(*args, **kwargs):
    return default().prefill_f32(*args, **kwargs)


def num_threads() -> int:
    return default().num_threads()


def set_num_threads(n: int) -> None:
    default().set_num_threads(n)
