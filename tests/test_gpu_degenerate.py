"""The method's degenerate cases on the GPU, against the oracle.

  beta = 0     no write: the state only decays (and the GPU state, whose
               update is then exactly a per-channel scaling in fp32, is held
               to 1e-5 in bf16 runs too)
  g = 0        no decay: the plain delta rule
  g = -1000    a decay that underflows to zero at every token: each state
               is the last token's write alone, beta k v^T
  no tokens    every sequence empty: ht = h0 bit for bit, in both scans

through the chunked prefill (fp32 d = 32 C = 16 and bf16 d = 128 C = 64) and
a few decode steps."""
import numpy as np
import pytest
import torch

import oracle
import synth
from kda_cases import TOL, check_tokens, dev_inputs, oracle_prefill, rel_l2, say, to_host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_55_amd as m

    return m


def _store(x64, dtype):
    if dtype == "bf16":
        return synth.f64_to_bf16_bits(x64)
    return np.ascontiguousarray(x64.astype(np.float32))


def _inputs(case, dtype, d, chunk, lengths, seed=61):
    inp = synth.make_inputs(seed, lengths, 3, d, dtype=dtype, gate="kimi", h0_std=0.1,
                            chunk=chunk)
    if case == "beta0":
        inp.beta = _store(np.zeros(inp.beta.shape), dtype)
    elif case == "g0":
        inp.g = np.zeros(inp.g.shape, dtype=np.float32)
    elif case == "g_underflow":
        inp.g = np.full(inp.g.shape, -1000.0, dtype=np.float32)
    return inp


@pytest.mark.parametrize("dtype,d,chunk", [("f32", 32, 16), ("bf16", 128, 64)])
@pytest.mark.parametrize("case", ["beta0", "g0", "g_underflow"])
def test_degenerate_prefill(kda, case, dtype, d, chunk):
    lengths = [150, 0, 77]
    say(f"degenerate prefill {case}: dtype={dtype} d={d} C={chunk} lengths={lengths}")
    inp = _inputs(case, dtype, d, chunk, lengths)
    dv = dev_inputs(inp)
    o, ht = kda.chunk_prefill(dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"], dv["h0"],
                              dv["cu_seqlens"], scale=inp.scale, chunk=chunk)
    torch.cuda.synchronize()
    o, ht = to_host64(o), to_host64(ht)
    o_ref, s_ref = oracle_prefill(inp)
    eo, es = rel_l2(o, o_ref), rel_l2(ht, s_ref)
    tok = check_tokens(o, o_ref, TOL[dtype])
    say(f"  rel-L2 o={eo:.3e} state={es:.3e} worst token {tok:.3e}")
    assert np.isfinite(o).all() and np.isfinite(ht).all()
    assert eo <= TOL[dtype] and es <= TOL[dtype]
    if case == "beta0":
        assert es <= 1e-5, "with beta = 0 the state is only scaled, in fp32"
    if case == "g_underflow":
        # the last token's write alone: beta k v^T (the empty sequence keeps h0)
        f = inp.f64()
        for n, (s, e) in enumerate(zip(inp.cu_seqlens[:-1], inp.cu_seqlens[1:])):
            if e > s:
                t = e - 1
                w = f["beta"][t][:, None, None] * f["k"][t][:, :, None] * f["v"][t][:, None, :]
                assert rel_l2(s_ref[n], w) <= 1e-12  # the oracle itself
                assert rel_l2(ht[n], w) <= TOL[dtype]
            else:
                assert np.array_equal(ht[n], f["h0"][n])


@pytest.mark.parametrize("case", ["beta0", "g0", "g_underflow"])
def test_degenerate_decode(kda, case):
    say(f"degenerate decode {case}: bf16 d=128, 4 steps on 5 sequences")
    inp = _inputs(case, "bf16", 128, 64, [4] * 5, seed=62)
    d = dev_inputs(inp)
    N, H, D = 5, inp.H, inp.dk
    view = lambda t: t.view(N, 4, *t.shape[1:])  # noqa: E731
    state = d["h0"].clone()
    f = inp.f64()
    st_ref = f["h0"].copy()
    fv = {k2: f[k2].reshape(N, 4, *f[k2].shape[1:]) for k2 in ("q", "k", "v", "g", "beta")}
    for s in range(4):
        o = kda.recurrent_decode(state, *(view(d[x])[:, s].contiguous()
                                          for x in ("q", "k", "v", "g", "beta")),
                                 scale=inp.scale)
        o_ref, st_ref = oracle.decode(st_ref, *(fv[x][:, s] for x in ("q", "k", "v", "g", "beta")),
                                      inp.scale)
        torch.cuda.synchronize()
        eo, es = rel_l2(to_host64(o), o_ref), rel_l2(to_host64(state), st_ref)
        say(f"  step {s}: rel-L2 o={eo:.3e} state={es:.3e}")
        assert eo <= TOL["bf16"] and es <= 1e-6


@pytest.mark.parametrize("n_seqs,H,scan", [(3, 3, "column-block"), (8, 32, "per-head")])
def test_no_tokens_keeps_h0(kda, n_seqs, H, scan):
    """Every sequence empty (T = 0): o has no rows and ht = h0 bit for bit."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert (2 * n_seqs * H > cus) == (scan == "per-head")
    say(f"no tokens: {n_seqs} empty sequences, H={H} ({scan} scan)")
    D = 128
    z = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device="cuda")  # noqa: E731
    h0 = 0.1 * torch.randn((n_seqs, H, D, D), generator=torch.Generator().manual_seed(63)).cuda()
    cu = torch.zeros(n_seqs + 1, dtype=torch.int32, device="cuda")
    g = torch.zeros((0, H, D), dtype=torch.float32, device="cuda")
    o, ht = kda.chunk_prefill(z(0, H, D), z(0, H, D), z(0, H, D), g, z(0, H), h0, cu,
                              scale=D ** -0.5, chunk=64)
    torch.cuda.synchronize()
    assert o.shape == (0, H, D)
    assert torch.equal(ht, h0)
