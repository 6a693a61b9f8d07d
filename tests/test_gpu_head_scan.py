"""The per-head scan: the two-pass plan's scan for batches with more
(sequence, head) pairs than half the device's CUs (bf16, d = 128, chunk 64).
One workgroup per (sequence, head) reads each chunk-local block once; the
chunk-local stage writes U and Ol for it in the per-head layout (Ol as the
transposed product).

Each case asserts on the host that the batch reaches that scan (2 x pairs > CUs)
and compares sampled heads with the fp64 oracle (whole-tensor, worst-head and
per-token bounds).  The same sequences run one call each take the
column-block scan: the sums run in the same order and the transposed Ol
product rounds like the other, so the two agree bit for bit."""
import numpy as np
import pytest
import torch

import synth
from kda_cases import (TOL, check_tokens, dev_gate, dev_inputs, oracle_prefill, rel_l2, say,
                       to_host64, worst_head)

pytestmark = pytest.mark.gpu

HEADS = [0, 13, 31]


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_55_amd as m

    return m


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _slice(inp, heads):
    """Value heads `heads` with their key heads as one key head each."""
    if inp.Hg == inp.H:
        return synth.slice_heads(inp, heads)
    hs = np.asarray(heads)
    kh = hs // (inp.H // inp.Hg)
    return synth.KdaInputs(
        q=np.ascontiguousarray(inp.q[:, kh]), k=np.ascontiguousarray(inp.k[:, kh]),
        v=np.ascontiguousarray(inp.v[:, hs]), g=np.ascontiguousarray(inp.g[:, hs]),
        beta=np.ascontiguousarray(inp.beta[:, hs]),
        h0=None if inp.h0 is None else np.ascontiguousarray(inp.h0[:, hs]),
        cu_seqlens=inp.cu_seqlens.copy(), dtype=inp.dtype, chunk=inp.chunk, scale=inp.scale)


def _check(o, s, inp, tag, fused_gate=False, qk_l2norm=False, heads=HEADS):
    sub = _slice(inp, heads)
    o_ref, s_ref = oracle_prefill(sub, fused_gate=fused_gate, qk_l2norm=qk_l2norm)
    o, s = o[:, heads], s[:, heads]
    eo, es = rel_l2(o, o_ref), rel_l2(s, s_ref)
    who, whs = worst_head(o, o_ref), worst_head(s, s_ref)
    tok = check_tokens(o, o_ref, TOL["bf16"])
    say(f"  {tag}: rel-L2 o={eo:.3e} state={es:.3e} worst head o={who:.3e} state={whs:.3e} "
        f"worst token {tok:.3e}")
    assert max(eo, es, who, whs) <= TOL["bf16"]


@pytest.mark.parametrize("lengths,h0", [
    ([70, 1, 64, 0, 130, 5, 33, 900], True),       # empty, one-token, ragged, one long
    ([300, 200, 64, 65, 128, 129, 10, 400], False),
    ([400, 0, 64, 130, 77], True),                 # 160 pairs: between half and all CUs
])
def test_head_scan_matches_oracle_and_column_scan(kda, lengths, h0):
    H = 32
    assert 2 * len(lengths) * H > _cus(), "the batch must reach the per-head scan"
    say(f"per-head scan: lengths={lengths} H={H} h0={h0}")
    inp = synth.make_inputs(101, lengths, H, 128, dtype="bf16", gate="kimi",
                            h0_std=0.05 if h0 else 0.0, chunk=64)
    d = dev_inputs(inp)
    o, ht = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"],
                              d["cu_seqlens"], scale=inp.scale)
    torch.cuda.synchronize()
    _check(to_host64(o), to_host64(ht), inp, "vs oracle")
    # the same sequences one call each (32 pairs: the column-block scan)
    cu = inp.cu_seqlens
    for n in range(len(lengths)):
        s, e = int(cu[n]), int(cu[n + 1])
        h0n = None if d["h0"] is None else d["h0"][n:n + 1]
        o1, h1 = kda.chunk_prefill(d["q"][s:e], d["k"][s:e], d["v"][s:e], d["g"][s:e],
                                   d["beta"][s:e], h0n, None, scale=inp.scale)
        torch.cuda.synchronize()
        assert torch.equal(o1, o[s:e]) and torch.equal(h1, ht[n:n + 1]), n
    say("  batch (per-head scan) = one call per sequence (column-block scan), bit for bit")


def test_head_scan_state_forms(kda):
    """Pool slots with a skipped sequence, in place; bf16 states; no final
    state."""
    H = 32
    lengths = [260, 0, 190, 64, 1, 333, 70, 128]
    assert 2 * len(lengths) * H > _cus()
    say("per-head scan: pool slots, bf16 states, no ht")
    inp = synth.make_inputs(102, lengths, H, 128, dtype="bf16", h0_std=0.05)
    d = dev_inputs(inp)
    o1, ht1 = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"],
                                d["cu_seqlens"], scale=inp.scale)
    o2, ht2 = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"],
                                d["cu_seqlens"], scale=inp.scale, output_final_state=False)
    torch.cuda.synchronize()
    assert ht2 is None and torch.equal(o1, o2)
    _check(to_host64(o1), to_host64(ht1), inp, "fp32 states")
    # pool of 10 slots: sequence n in slot 9 - n, sequence 3 skipped
    N = len(lengths)
    pool = torch.zeros((10, H, 128, 128), dtype=torch.float32, device="cuda")
    for n in range(N):
        pool[9 - n] = d["h0"][n]
    idx = torch.tensor([9 - n if n != 3 else -1 for n in range(N)], dtype=torch.int32,
                       device="cuda")
    o3 = torch.full_like(o1, 5.0)
    kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], pool, d["cu_seqlens"],
                      scale=inp.scale, out=o3, state_indices=idx)
    torch.cuda.synchronize()
    cu = inp.cu_seqlens
    for n in range(N):
        s, e = int(cu[n]), int(cu[n + 1])
        if n == 3:
            assert torch.equal(pool[9 - n], d["h0"][n]), "skipped slot changed"
            assert bool((o3[s:e] == 5.0).all()), "skipped sequence wrote o"
        else:
            assert torch.equal(pool[9 - n], ht1[n]) and torch.equal(o3[s:e], o1[s:e]), n
    # bf16 states: read widened, written rounded once
    h0b = d["h0"].to(torch.bfloat16)
    o4, ht4 = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], h0b,
                                d["cu_seqlens"], scale=inp.scale)
    torch.cuda.synchronize()
    assert ht4.dtype == torch.bfloat16
    inp_b = synth.make_inputs(102, lengths, H, 128, dtype="bf16", h0_std=0.05)
    inp_b.h0 = to_host64(h0b).astype(np.float32)  # the oracle starts from the rounded h0
    _check(to_host64(o4), to_host64(ht4), inp_b, "bf16 states")


def test_head_scan_gate_and_heads(kda):
    """The fused Kimi gate; two key heads shared by 32 value heads with
    in-kernel q/k normalisation."""
    H = 32
    lengths = [333, 190, 64, 250, 5, 129, 80, 200]
    assert 2 * len(lengths) * H > _cus()
    say("per-head scan: fused gate; grouped heads with qk_l2norm")
    inp = synth.make_inputs(103, lengths, H, 128, dtype="bf16", h0_std=0.02)
    d = dev_inputs(inp)
    o, ht = kda.chunk_prefill(d["q"], d["k"], d["v"], None, d["beta"], d["h0"], d["cu_seqlens"],
                              scale=inp.scale, gate=dev_gate(inp))
    torch.cuda.synchronize()
    _check(to_host64(o), to_host64(ht), inp, "fused gate", fused_gate=True)
    inp = synth.make_inputs(104, lengths, H, 128, dtype="bf16", h0_std=0.02, n_k_heads=2,
                            qk_prenorm=False)
    d = dev_inputs(inp)
    o, ht = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"],
                              d["cu_seqlens"], scale=inp.scale, qk_l2norm=True)
    torch.cuda.synchronize()
    _check(to_host64(o), to_host64(ht), inp, "Hg = 2, H = 32, qk_l2norm", qk_l2norm=True,
           heads=[0, 15, 16, 31])
