"""The no-allocation entry point, kda_chunk_prefill_noalloc, on the GPU: two
calls in a row (the second with fewer tokens and sequences, so it runs over
the contents the first left in the shared static workspace) against the
workspace entry point kda_chunk_prefill on the same inputs -- the same
kernels, so the results must agree bit for bit, and both must meet the oracle
bar -- and an oversize request refused before anything is launched."""
import numpy as np
import pytest
import torch

import synth
from kda_cases import TOL, dev_inputs, oracle_prefill, rel_l2, say, to_host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_55_amd as m

    return m


def _run(kda, inp, noalloc):
    d = dev_inputs(inp)
    N = len(inp.cu_seqlens) - 1
    o = torch.full((inp.T, inp.H, inp.dk), 3.0, dtype=d["v"].dtype, device="cuda")
    ht = torch.full((N, inp.H, inp.dk, inp.dk), 3.0, dtype=torch.float32, device="cuda")
    kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"],
                      scale=inp.scale, chunk=inp.chunk, out=o, ht=ht, noalloc=noalloc)
    torch.cuda.synchronize()
    return to_host64(o), to_host64(ht)


@pytest.mark.parametrize("dtype,d,chunk,H", [("bf16", 128, 64, 32), ("f32", 32, 16, 2)])
def test_noalloc_matches_workspace_entry_point(kda, dtype, d, chunk, H):
    for seed, lengths in ((71, [1000, 300, 0, 77]), (72, [200, 57])):
        say(f"noalloc {dtype} d={d} C={chunk} H={H} lengths={lengths}")
        inp = synth.make_inputs(seed, lengths, H, d, dtype=dtype, h0_std=0.02, chunk=chunk,
                                gate="softplus" if dtype == "f32" else "kimi")
        o1, s1 = _run(kda, inp, noalloc=False)
        o2, s2 = _run(kda, inp, noalloc=True)
        assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
        o_ref, s_ref = oracle_prefill(inp)
        eo, es = rel_l2(o2, o_ref), rel_l2(s2, s_ref)
        say(f"  bitwise equal to kda_chunk_prefill; vs oracle rel-L2 o={eo:.3e} state={es:.3e}")
        assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_noalloc_refuses_oversize(kda):
    inp = synth.make_inputs(73, [1600], 32, 128, dtype="bf16", chunk=64)
    with pytest.raises(kda.KdaError) as e:
        _run(kda, inp, noalloc=True)
    assert e.value.status == -6  # KDA_ERR_WORKSPACE
