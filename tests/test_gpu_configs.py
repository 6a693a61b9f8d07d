"""The five workloads at full size on the GPU against the fp64 oracle.

The oracle runs on a sample of heads (heads are independent chains, so the
sampled heads' results are exact references for those heads); the GPU always
runs every head, in the same launch configuration the benchmark times."""
import numpy as np
import pytest
import torch

import oracle
import synth
from kda_cases import TOL, check_tokens, dev_inputs, rel_l2, say, to_host64, worst_head

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_55_amd as m

    return m


def gpu_prefill(kda, inp, d=None):
    d = d or dev_inputs(inp)
    o, ht = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], d["cu_seqlens"],
                              scale=inp.scale, chunk=inp.chunk)
    torch.cuda.synchronize()
    return o, ht


def check_sampled(inp, o, ht, heads, tol):
    """o and the final state of the sampled heads against the oracle: the
    whole-tensor rel-L2, the worst head's, and a bound on every token row
    (so one wrong token cannot hide in a long sequence's norm)."""
    sub = synth.slice_heads(inp, heads)
    f = sub.f64()
    o_ref, ht_ref = oracle.prefill(f["q"], f["k"], f["v"], f["g"], f["beta"], f["h0"],
                                   f["cu_seqlens"], f["scale"])
    o_g = to_host64(o[:, heads])
    ht_g = to_host64(ht[:, heads])
    eo, es = rel_l2(o_g, o_ref), rel_l2(ht_g, ht_ref)
    who, whs = worst_head(o_g, o_ref), worst_head(ht_g, ht_ref)
    tok = check_tokens(o_g, o_ref, tol)
    say(f"  heads {list(heads)}: rel-L2 o={eo:.3e} state={es:.3e} worst head o={who:.3e} "
        f"state={whs:.3e} worst token {tok:.3e} max|o|={np.abs(o_ref).max():.3f}")
    assert max(eo, es, who, whs) <= tol
    return eo, es


@pytest.mark.parametrize("cfg,heads", [(0, [0, 1]), (1, [0, 9, 31]), (2, [3, 17, 30]),
                                       (3, [5, 22])])
def test_config_prefill(kda, cfg, heads):
    say(f"workload {synth.CONFIGS[cfg]['name']}")
    inp = synth.make_config(cfg)
    say(f"  T={inp.T} N={inp.N} H={inp.H} d={inp.dk} C={inp.chunk} dtype={inp.dtype}")
    o, ht = gpu_prefill(kda, inp)
    check_sampled(inp, o, ht, heads, TOL[inp.dtype])


@pytest.fixture(scope="module")
def decode_inputs():
    say("decode-64x256: generating 64 x 1280 tokens")
    return synth.make_config(4)


def test_decode_workload_prefill_then_decode(kda, decode_inputs):
    """Chunked prefill of tokens [0, 1024) of 64 sequences, then 256 recurrent
    decode steps on the carried state; checked against the oracle (sampled
    heads) and against a 1280-token chunked prefill on the GPU (all heads)."""
    inp = decode_inputs
    N, L, P, S = 64, 1280, 1024, 256
    H, D = inp.H, inp.dk
    d = dev_inputs(inp)
    view = lambda t: t.view(N, L, *t.shape[1:])  # noqa: E731
    pre = {k: view(d[k])[:, :P].reshape(N * P, *d[k].shape[1:]).contiguous()
           for k in ["q", "k", "v", "g", "beta"]}
    dec = {k: view(d[k])[:, P:].transpose(0, 1).contiguous() for k in ["q", "k", "v", "g", "beta"]}
    cu = torch.arange(0, N * P + 1, P, dtype=torch.int32, device="cuda")
    say("  prefill 64 x 1024")
    o_pre, state = kda.chunk_prefill(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], None, cu,
                                     scale=inp.scale, chunk=64)
    say("  256 decode steps")
    o_dec = torch.empty((S, N, H, D), dtype=torch.bfloat16, device="cuda")
    for s in range(S):
        kda.recurrent_decode(state, dec["q"][s], dec["k"][s], dec["v"][s], dec["g"][s],
                             dec["beta"][s], scale=inp.scale, out=o_dec[s])
    torch.cuda.synchronize()
    say("  1280-token chunked prefill (all heads)")
    o_full, ht_full = gpu_prefill(kda, inp, d)
    o_full_dec = view(o_full)[:, P:].transpose(0, 1)
    e_o = rel_l2(to_host64(o_dec), to_host64(o_full_dec))
    e_s = rel_l2(to_host64(state), to_host64(ht_full))
    say(f"  decode vs 1280-prefill: rel-L2 o={e_o:.3e} state={e_s:.3e}")
    assert e_o <= TOL["bf16"] and e_s <= TOL["bf16"]
    heads = [4, 27]
    sub = synth.slice_heads(inp, heads)
    f = sub.f64()
    o_ref, ht_ref = oracle.prefill(f["q"], f["k"], f["v"], f["g"], f["beta"], None,
                                   f["cu_seqlens"], f["scale"])
    o_ref_dec = o_ref.reshape(N, L, len(heads), D)[:, P:].transpose(1, 0, 2, 3)
    e_o2 = rel_l2(to_host64(o_dec[:, :, heads]), o_ref_dec)
    e_s2 = rel_l2(to_host64(state[:, heads]), ht_ref)
    o_ref_pre = o_ref.reshape(N, L, len(heads), D)[:, :P].reshape(N * P, len(heads), D)
    e_p = rel_l2(to_host64(o_pre[:, heads]), o_ref_pre)
    who = worst_head(to_host64(o_dec[:, :, heads]).transpose(1, 0, 2, 3).reshape(N * S, len(heads), D),
                     o_ref_dec.transpose(1, 0, 2, 3).reshape(N * S, len(heads), D))
    tok = check_tokens(to_host64(o_dec[:, :, heads]), o_ref_dec, TOL["bf16"])
    tokp = check_tokens(to_host64(o_pre[:, heads]), o_ref_pre, TOL["bf16"])
    say(f"  vs oracle heads {heads}: prefill o={e_p:.3e}; decode o={e_o2:.3e} state={e_s2:.3e} "
        f"worst head decode o={who:.3e}; worst token prefill {tokp:.3e} decode {tok:.3e}")
    assert max(e_o2, e_s2, e_p, who) <= TOL["bf16"]
