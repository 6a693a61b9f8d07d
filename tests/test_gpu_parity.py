"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the
same seeded inputs.  Bars: relative L2 <= 1e-4 (fp32 inputs) and <= 1e-2 (bf16
inputs, fp32 accumulation) for o and for the final state."""
import numpy as np
import pytest
import torch

import synth
from kda_cases import (TOL, check_tokens, dev_inputs, oracle_prefill, rel_l2, say, to_host64,
                       worst_head)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_55_amd as m

    return m


def run_prefill(kda, inp, chunk=None, ht_inplace=False):
    d = dev_inputs(inp)
    ht = None
    if ht_inplace and d["h0"] is not None:
        ht = d["h0"]
    o, hT = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"],
                              d["cu_seqlens"], scale=inp.scale, chunk=chunk or inp.chunk, ht=ht)
    torch.cuda.synchronize()
    return to_host64(o), to_host64(hT)


@pytest.mark.parametrize("dtype,d,chunk,lengths,h0", [
    ("f32", 32, 16, [128], False),        # the tiny fp32 workload
    ("f32", 64, 32, [77, 0, 130], True),
    ("f32", 128, 16, [45], True),
    ("bf16", 128, 64, [300], True),
    ("bf16", 128, 64, [64, 1, 129, 0, 200], True),
    ("bf16", 64, 32, [100, 33], False),
    ("bf16", 32, 16, [70], True),
    ("bf16", 128, 16, [90, 17], True),
    ("bf16", 128, 32, [150], False),
])
def test_prefill_small(kda, dtype, d, chunk, lengths, h0):
    say(f"prefill dtype={dtype} d={d} C={chunk} lengths={lengths} h0={h0}")
    inp = synth.make_inputs(11, lengths, 3, d, dtype=dtype,
                            gate="softplus" if dtype == "f32" else "kimi",
                            h0_std=0.05 if h0 else 0.0, chunk=chunk)
    o, hT = run_prefill(kda, inp)
    o_ref, hT_ref = oracle_prefill(inp)
    eo, es = rel_l2(o, o_ref), rel_l2(hT, hT_ref)
    who, whs = worst_head(o, o_ref), worst_head(hT, hT_ref)
    tok = check_tokens(o, o_ref, TOL[dtype])
    say(f"  rel-L2 o={eo:.3e} state={es:.3e} worst head o={who:.3e} state={whs:.3e} "
        f"worst token {tok:.3e}")
    assert max(eo, es, who, whs) <= TOL[dtype]


@pytest.mark.parametrize("dtype,d", [("f32", 32), ("f32", 128), ("bf16", 64), ("bf16", 128)])
def test_decode_matches_oracle(kda, dtype, d):
    say(f"decode dtype={dtype} d={d}")
    import oracle

    inp = synth.make_inputs(21, [1] * 5, 4, d, dtype=dtype, h0_std=0.5)
    dev = dev_inputs(inp)
    state = dev["h0"].clone()
    o = kda.recurrent_decode(state, dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"],
                             scale=inp.scale)
    torch.cuda.synchronize()
    f = inp.f64()
    o_ref, st_ref = oracle.decode(f["h0"], f["q"], f["k"], f["v"], f["g"], f["beta"], f["scale"])
    eo, es = rel_l2(to_host64(o), o_ref), rel_l2(to_host64(state), st_ref)
    say(f"  rel-L2 o={eo:.3e} state={es:.3e}")
    assert eo <= TOL[dtype] and es <= 1e-6


def test_tiny_config_prefill_vs_decode_by_decode(kda):
    """The tiny fp32 workload: chunked prefill = token-by-token decode on the GPU."""
    say("tiny-f32 chunked vs decode-by-decode")
    inp = synth.make_config(0)
    o_c, s_c = run_prefill(kda, inp)
    dev = dev_inputs(inp)
    T, H, D = inp.T, inp.H, inp.dk
    state = torch.zeros((1, H, D, D), dtype=torch.float32, device="cuda")
    outs = []
    for t in range(T):
        outs.append(kda.recurrent_decode(state, dev["q"][t:t + 1], dev["k"][t:t + 1],
                                         dev["v"][t:t + 1], dev["g"][t:t + 1],
                                         dev["beta"][t:t + 1], scale=inp.scale))
    o_d = to_host64(torch.cat(outs, 0))
    s_d = to_host64(state)
    o_ref, s_ref = oracle_prefill(inp)
    say(f"  chunk vs oracle {rel_l2(o_c, o_ref):.3e}/{rel_l2(s_c, s_ref):.3e}; "
        f"decode vs oracle {rel_l2(o_d, o_ref):.3e}/{rel_l2(s_d, s_ref):.3e}; "
        f"chunk vs decode {rel_l2(o_c, o_d):.3e}/{rel_l2(s_c, s_d):.3e}")
    for e in [rel_l2(o_c, o_ref), rel_l2(s_c, s_ref), rel_l2(o_d, o_ref), rel_l2(s_d, s_ref),
              rel_l2(o_c, o_d), rel_l2(s_c, s_d)]:
        assert e <= 1e-4


def test_inplace_carry_and_determinism(kda):
    say("in-place ht = h0 and bitwise determinism")
    inp = synth.make_inputs(31, [200, 90], 2, 128, dtype="bf16", h0_std=0.02)
    o1, s1 = run_prefill(kda, inp)
    o2, s2 = run_prefill(kda, inp)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
    o3, s3 = run_prefill(kda, inp, ht_inplace=True)
    assert np.array_equal(o1, o3) and np.array_equal(s1, s3)


def test_bad_cu_seqlens_reported(kda):
    say("invalid cu_seqlens -> device status")
    inp = synth.make_inputs(41, [10, 20], 2, 64, dtype="bf16")
    d = dev_inputs(inp)
    bad = torch.tensor([0, 25, 20], dtype=torch.int32, device="cuda")  # decreasing
    o = torch.full((30, 2, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(kda.prefill_workspace_bytes(30, 2, 64, n_seqs=2), dtype=torch.uint8,
                     device="cuda")
    kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], None, bad, out=o, workspace=ws)
    assert kda.workspace_status(ws) == -10
    assert torch.all(o == 7.0)
    good = d["cu_seqlens"]
    kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], None, good, out=o, workspace=ws)
    assert kda.workspace_status(ws) == 0
    # a workspace the binding allocates itself: the status is read with check=True
    with pytest.raises(kda.KdaError):
        kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], None, bad, check=True)
    kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], None, good, check=True)


@pytest.mark.parametrize("dtype,d,chunk,n,hi", [
    ("f32", 32, 16, 600, 40),     # more than 256 sequences: several passes of the offset scan
    ("bf16", 128, 64, 300, 150),  # the workload head shape, many partial chunks
])
def test_many_short_sequences(kda, dtype, d, chunk, n, hi):
    """Hundreds of packed sequences, about a tenth of them empty: every chunk's
    table entry (its sequence found by search over the chunk offsets) must
    send it to the right sequence, so o and every final state match the
    oracle run sequence by sequence."""
    lengths = synth.seeded_lengths(17 + n, n, 0, hi)
    lengths = [0 if i % 10 == 3 else L for i, L in enumerate(lengths)]
    say(f"prefill {n} sequences dtype={dtype} d={d} C={chunk} tokens={sum(lengths)}")
    inp = synth.make_inputs(19, lengths, 2, d, dtype=dtype,
                            gate="softplus" if dtype == "f32" else "kimi", h0_std=0.05,
                            chunk=chunk)
    o, hT = run_prefill(kda, inp)
    o_ref, hT_ref = oracle_prefill(inp)
    eo, es = rel_l2(o, o_ref), rel_l2(hT, hT_ref)
    say(f"  rel-L2 o={eo:.3e} state={es:.3e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]
    # empty sequences carry h0 through unchanged
    empty = [i for i, L in enumerate(lengths) if L == 0]
    assert np.array_equal(hT[empty], inp.h0[empty].astype(np.float64))
