"""Every descriptor option at once, through each path.

The options are tested one or two at a time elsewhere; here they are all on
together, so that no path depends on an option being off: the fused Kimi gate
(raw x, a_log, dt_bias), 8 key heads shared by 32 value heads with in-kernel
q/k normalisation (raw q, k), and a bf16 state pool read and written in place
through a slot table that skips one sequence.  Paths: the chunked prefill
through the column-block scan (3 sequences) and through the per-head scan
(8 sequences), the recurrent prefill, and decode.  Expected values: the fp64
oracle on the gate the oracle computes from the stored raw gate, q and k
normalised and expanded by the oracle, and the pool slots widened; skipped
sequences must leave their o rows and their slot untouched, unused slots
keep their bits."""
import numpy as np
import pytest
import torch

import oracle
import synth
from kda_cases import (TOL, check_tokens, dev_gate, dev_inputs, oracle_qk, rel_l2, say, to_dev,
                       to_host64)

pytestmark = pytest.mark.gpu

H, HG, D = 32, 8, 128


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_55_amd as m

    return m


def _pool(S, std, seed):
    bits = synth.f64_to_bf16_bits(np.random.default_rng(seed).normal(0.0, std, (S, H, D, D)))
    return bits, to_dev(bits, "bf16")


def _expected(inp, pool_bits, slots, decode=False):
    """Oracle results per sequence; a skipped sequence runs from slot 0 (its
    results are not compared)."""
    f = inp.f64()
    g = oracle.kimi_gate(*inp.gate_f64())
    q, k = oracle_qk(inp, f, True)
    h0 = synth.bf16_bits_to_f64(pool_bits)[[s if s >= 0 else 0 for s in slots]]
    if decode:
        return oracle.decode(h0, q, k, f["v"], g, f["beta"], f["scale"])
    return oracle.prefill(q, k, f["v"], g, f["beta"], h0, f["cu_seqlens"], f["scale"])


def _check_pool(pool, before, slots, ht_ref, tol):
    used = set(s for s in slots if s >= 0)
    for n, s in enumerate(slots):
        if s >= 0:
            es = rel_l2(to_host64(pool[s]), ht_ref[n])
            say(f"  seq {n} slot {s}: rel-L2 state={es:.3e}")
            assert es <= tol
    for s in range(pool.shape[0]):
        if s not in used:
            assert torch.equal(pool[s].view(torch.int16), before[s].view(torch.int16)), s


@pytest.mark.parametrize("lengths,slots,scan", [
    ([300, 70, 129], [4, -1, 1], "column-block"),
    ([100, 64, 0, 90, 1, 120, 77, 65], [9, 2, 7, -1, 0, 5, 3, 10], "per-head"),
])
@pytest.mark.parametrize("path", ["chunk", "recurrent"])
def test_all_options_prefill(kda, lengths, slots, scan, path):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if path == "chunk":
        assert (2 * len(lengths) * H > cus) == (scan == "per-head"), "the batch reaches the scan"
    say(f"all options, {path} prefill ({scan} batch): lengths={lengths} slots={slots}")
    inp = synth.make_inputs(71 + len(lengths), lengths, H, D, dtype="bf16", gate="kimi",
                            h0_std=0.0, chunk=64, n_k_heads=HG, qk_prenorm=False)
    dv = dev_inputs(inp)
    S = max(slots) + 3
    pool_bits, pool = _pool(S, 0.05, 81)
    before = pool.clone()
    idx = torch.tensor(slots, dtype=torch.int32, device="cuda")
    o = torch.full((inp.T, H, D), 3.0, dtype=torch.bfloat16, device="cuda")
    run = kda.chunk_prefill if path == "chunk" else kda.recurrent_prefill
    kw = {"chunk": 64} if path == "chunk" else {}
    _, ht = run(dv["q"], dv["k"], dv["v"], None, dv["beta"], pool, dv["cu_seqlens"],
                scale=inp.scale, out=o, gate=dev_gate(inp), state_indices=idx, qk_l2norm=True,
                **kw)
    torch.cuda.synchronize()
    assert ht.data_ptr() == pool.data_ptr()
    o_ref, ht_ref = _expected(inp, pool_bits, slots)
    cu = inp.cu_seqlens
    for n, s in enumerate(slots):
        rows = slice(int(cu[n]), int(cu[n + 1]))
        og = to_host64(o[rows])
        if s < 0:
            assert bool((o[rows] == 3.0).all()), "a skipped sequence wrote o"
            continue
        if og.size:
            eo = rel_l2(og, o_ref[rows])
            tok = check_tokens(og, o_ref[rows], TOL["bf16"])
            say(f"  seq {n}: rel-L2 o={eo:.3e} worst token {tok:.3e}")
            assert eo <= TOL["bf16"]
    _check_pool(pool, before, slots, ht_ref, TOL["bf16"])


def test_all_options_decode(kda):
    slots = [3, -1, 0, 6, 2]
    N = len(slots)
    say(f"all options, decode: {N} sequences, slots={slots}")
    inp = synth.make_inputs(79, [1] * N, H, D, dtype="bf16", gate="kimi", h0_std=0.0,
                            n_k_heads=HG, qk_prenorm=False)
    dv = dev_inputs(inp)
    pool_bits, pool = _pool(8, 0.5, 82)
    before = pool.clone()
    idx = torch.tensor(slots, dtype=torch.int32, device="cuda")
    o = torch.full((N, H, D), 3.0, dtype=torch.bfloat16, device="cuda")
    kda.recurrent_decode(pool, dv["q"], dv["k"], dv["v"], None, dv["beta"], scale=inp.scale,
                         out=o, gate=dev_gate(inp), state_indices=idx, qk_l2norm=True)
    torch.cuda.synchronize()
    o_ref, st_ref = _expected(inp, pool_bits, slots, decode=True)
    for n, s in enumerate(slots):
        if s < 0:
            assert bool((o[n] == 3.0).all()), "a skipped sequence wrote o"
            continue
        eo = rel_l2(to_host64(o[n]), o_ref[n])
        say(f"  seq {n}: rel-L2 o={eo:.3e}")
        assert eo <= TOL["bf16"]
    _check_pool(pool, before, slots, st_ref, TOL["bf16"])
