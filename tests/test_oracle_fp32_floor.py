"""The oracle's fp32 twin: the same token recurrence (the same C source
instantiated with float) run in plain fp32, against the fp64 oracle.

First pinned as a twin: on the hand-worked goldens and on random cases it
agrees with the fp64 oracle to fp32 rounding, and a mistake planted in the
shared source shows up in both.  Then it documents the floor under the
acceptance bars: what plain fp32 arithmetic of the definition itself reaches
at each workload (sampled heads of the bf16 workloads, every head of the tiny
fp32 one) -- far inside 1e-4 (fp32 inputs) and 1e-2 (bf16 inputs), so the
bars leave room for the chunked GPU path's own rounding (bf16 matrix-core
operands)."""
import json
import os
import tempfile

import numpy as np
import pytest

import oracle
import synth
from oracle.build import SRC, compile_oracle
from oracle.recurrent import OracleLib
from pins import GOLDEN, _rand_case


def rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


class _F32:
    """prefill() of the fp32 twin, for the golden checks below."""

    def __init__(self, lib):
        self.lib = lib

    def prefill(self, *a, **kw):
        return self.lib.prefill_f32(*a, **kw)


def test_twin_on_goldens():
    """Hand-worked examples (exact binary fractions) hold in fp32 to fp32
    rounding."""
    lib = oracle.recurrent.default()
    assert lib.has_f32
    for name, shape in (("scalar_kda.json", None), ("two_channel_kda.json", None)):
        fx = json.load(open(os.path.join(GOLDEN, name)))
        if name.startswith("scalar"):
            sh = lambda x: np.asarray(x, dtype=np.float64).reshape(-1, 1, 1)  # noqa: E731
            args = (sh(fx["q"]), sh(fx["k"]), sh(fx["v"]), np.log(sh(fx["decay"])),
                    np.asarray(fx["beta"]).reshape(-1, 1), np.full((1, 1, 1, 1), fx["h0"]))
        else:
            args = (np.asarray(fx["q"])[:, None, :], np.asarray(fx["k"])[:, None, :],
                    np.asarray(fx["v"])[:, None, :], np.log(np.asarray(fx["decay"]))[:, None, :],
                    np.asarray(fx["beta"])[:, None], np.asarray(fx["h0"])[None, None])
        o, ht = lib.prefill_f32(*args, None, fx["scale"])
        ref_o = np.asarray(fx["o"]).reshape(o.shape)
        assert np.allclose(o, ref_o, rtol=1e-6, atol=1e-6), (name, o.ravel(), ref_o.ravel())
        assert np.allclose(ht.ravel(), np.ravel(fx["hT"]), rtol=1e-6, atol=1e-6), name


@pytest.mark.parametrize("T,dk,strong", [(50, 8, 1.0), (120, 16, 4.0)])
def test_twin_tracks_fp64(T, dk, strong):
    """Random varlen cases: the twin's error against fp64 stays at fp32
    rounding (a few ulp per token accumulated over the sequence)."""
    rng = np.random.default_rng([7, T, dk])
    q, k, v, g, beta, s0 = _rand_case(rng, T, 3, dk, dk, strong=strong)
    h0 = np.repeat(s0, 2, axis=0)
    cu = np.array([0, T // 3, T])
    o, ht = oracle.prefill(q, k, v, g, beta, h0, cu, 0.3)
    o32, ht32 = oracle.prefill_f32(q, k, v, g, beta, h0, cu, 0.3)
    assert rel(o32, o) < 2e-6 and rel(ht32, ht) < 2e-6
    assert rel(o32, o) > 0  # it really is the fp32 arithmetic


def test_twin_shares_the_source():
    """A mistake planted in the shared source shows in the twin as well (here:
    the erase sign), so the twin cannot drift from the definition."""
    src = open(SRC).read()
    old = "u[j] = beta * (v[j] - u[j]);"
    assert old in src
    with tempfile.TemporaryDirectory() as td:
        path = os.path.join(td, "mut.c")
        open(path, "w").write(src.replace(old, "u[j] = beta * (v[j] + u[j]);"))
        lib = OracleLib(compile_oracle(path, os.path.join(td, "libmut.so"), werror=False, twin=True))
        rng = np.random.default_rng(3)
        q, k, v, g, beta, s0 = _rand_case(rng, 20, 1, 4, 4)
        o_good, _ = oracle.prefill(q, k, v, g, beta, s0, None, 0.5)
        o_bad32, _ = lib.prefill_f32(q, k, v, g, beta, s0, None, 0.5)
        assert rel(o_bad32, o_good) > 1e-2


# (config, sampled heads, bound the floor must stay under)
FLOOR_CASES = [(0, [0, 1], 1e-6), (1, [9], 1e-5), (2, [17], 1e-5), (3, [22], 1e-5), (4, [27], 1e-5)]


@pytest.mark.parametrize("cfg,heads,bound", FLOOR_CASES)
def test_fp32_floor_per_config(cfg, heads, bound):
    inp = synth.slice_heads(synth.make_config(cfg), heads)
    f = inp.f64()
    o, ht = oracle.prefill(f["q"], f["k"], f["v"], f["g"], f["beta"], f["h0"], f["cu_seqlens"],
                           f["scale"])
    o32, ht32 = oracle.prefill_f32(f["q"], f["k"], f["v"], f["g"], f["beta"], f["h0"],
                                   f["cu_seqlens"], f["scale"])
    eo, es = rel(o32, o), rel(ht32, ht)
    print(f"fp32 floor {synth.CONFIGS[cfg]['name']} (heads {heads}): "
          f"rel-L2 o={eo:.3e} state={es:.3e}", flush=True)
    assert eo < bound and es < bound
