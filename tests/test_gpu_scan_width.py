"""The state scan's column-block width (16, 32 or 64 value columns per
workgroup) is chosen from the batch: the widest that still leaves every CU a
workgroup.  The width changes which workgroup computes a column, not the
arithmetic, so a batch must equal the same sequences run one call each (one
sequence at H = 32 always takes the narrowest width) bit for bit, and match
the oracle.  Batches here reach each width on a 256-CU part: 3 x 32 heads at
d = 128 take 32 columns; at d = 64, 8 x 32 heads take 64.  At d = 128 a batch
of more (sequence, head) pairs than half the CUs (8 x 32 here) takes the
per-head scan instead (tests/test_gpu_head_scan.py covers it in full): its sums
run in the same order and its transposed Ol product rounds like the other, so
that batch too equals the one-call runs bit for bit."""
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


@pytest.mark.parametrize("d,lengths", [
    (128, [100, 37, 64]),                          # 96 heads
    (128, [70, 1, 64, 0, 130, 5, 33, 90]),         # 256 heads
    (64, [40, 64, 65, 3, 17, 100, 2, 50]),         # 256 heads
])
def test_batch_equals_one_call_per_sequence(kda, d, lengths):
    say(f"scan width: d={d} lengths={lengths}")
    inp = synth.make_inputs(61, lengths, 32, d, dtype="bf16", gate="kimi", h0_std=0.05, chunk=64)
    dv = dev_inputs(inp)
    o, ht = kda.chunk_prefill(dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"], dv["h0"],
                              dv["cu_seqlens"], scale=inp.scale)
    cu = inp.cu_seqlens
    for n in range(len(lengths)):
        s, e = int(cu[n]), int(cu[n + 1])
        o1, h1 = kda.chunk_prefill(dv["q"][s:e], dv["k"][s:e], dv["v"][s:e], dv["g"][s:e],
                                   dv["beta"][s:e], dv["h0"][n:n + 1], None, scale=inp.scale)
        torch.cuda.synchronize()
        assert torch.equal(o1, o[s:e]) and torch.equal(h1, ht[n:n + 1]), n
    sub = synth.slice_heads(inp, [0, 13, 31])
    o_ref, ht_ref = oracle_prefill(sub)
    eo = rel_l2(to_host64(o)[:, [0, 13, 31]], o_ref)
    es = rel_l2(to_host64(ht)[:, [0, 13, 31]], ht_ref)
    say(f"  rel-L2 o={eo:.3e} state={es:.3e} (heads 0, 13, 31)")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
