"""GPU parity of the fused gate activation: the kernels compute
g = -exp(a_log) softplus(x + dt_bias) from the raw gate; the reference is the
fp64 oracle run on g recomputed (oracle/gate.py) from the same stored x, a_log
and dt_bias.  Bars as elsewhere: relative L2 <= 1e-4 (fp32) and <= 1e-2 (bf16)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from kda_cases import TOL, dev_gate, dev_inputs, oracle_prefill, rel_l2, say, to_host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_55_amd as m

    return m


def gated_prefill(kda, inp):
    d = dev_inputs(inp)
    o, ht = kda.chunk_prefill(d["q"], d["k"], d["v"], None, d["beta"], d["h0"], d["cu_seqlens"],
                              scale=inp.scale, chunk=inp.chunk, gate=dev_gate(inp))
    torch.cuda.synchronize()
    return to_host64(o), to_host64(ht)


@pytest.mark.parametrize("dtype,d,chunk,lengths,h0,gate", [
    ("f32", 32, 16, [128], False, "softplus"),
    ("f32", 64, 32, [77, 0, 130], True, "kimi"),
    ("bf16", 128, 64, [300], True, "kimi"),
    ("bf16", 128, 64, [64, 1, 129, 0, 200], True, "kimi"),
    ("bf16", 32, 16, [70], True, "kimi"),
])
def test_gated_prefill_small(kda, dtype, d, chunk, lengths, h0, gate):
    say(f"gated prefill dtype={dtype} d={d} C={chunk} lengths={lengths} gate={gate}")
    inp = synth.make_inputs(51, lengths, 3, d, dtype=dtype, gate=gate,
                            h0_std=0.05 if h0 else 0.0, chunk=chunk)
    o, hT = gated_prefill(kda, inp)
    o_ref, hT_ref = oracle_prefill(inp, fused_gate=True)
    eo, es = rel_l2(o, o_ref), rel_l2(hT, hT_ref)
    say(f"  rel-L2 o={eo:.3e} state={es:.3e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_gated_prefill_4k_sampled_heads(kda):
    """The 4k single-sequence workload with the fused gate, on sampled heads."""
    inp = synth.make_config(1)
    o, hT = gated_prefill(kda, inp)
    heads = [0, 9, 31]
    sub = synth.slice_heads(inp, heads)
    o_ref, hT_ref = oracle_prefill(sub, fused_gate=True)
    eo, es = rel_l2(o[:, heads], o_ref), rel_l2(hT[:, heads], hT_ref)
    say(f"prefill-4k gated, heads {heads}: rel-L2 o={eo:.3e} state={es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


@pytest.mark.parametrize("dtype,d", [("f32", 32), ("bf16", 128)])
def test_gated_decode(kda, dtype, d):
    say(f"gated decode dtype={dtype} d={d}")
    inp = synth.make_inputs(52, [1] * 6, 4, d, dtype=dtype, h0_std=0.5, gate="kimi")
    dev = dev_inputs(inp)
    state = dev["h0"].clone()
    o = kda.recurrent_decode(state, dev["q"], dev["k"], dev["v"], None, dev["beta"],
                             scale=inp.scale, gate=dev_gate(inp))
    torch.cuda.synchronize()
    f = inp.f64()
    g_ref = oracle.kimi_gate(*inp.gate_f64())
    o_ref, st_ref = oracle.decode(f["h0"], f["q"], f["k"], f["v"], g_ref, f["beta"], f["scale"])
    eo, es = rel_l2(to_host64(o), o_ref), rel_l2(to_host64(state), st_ref)
    say(f"  rel-L2 o={eo:.3e} state={es:.3e}")
    # the state of one step is exact up to fp32 rounding; the in-kernel gate
    # adds the rounding of its exp2 / log2 (about 1e-7 relative per factor)
    assert eo <= TOL[dtype] and es <= 1e-5
