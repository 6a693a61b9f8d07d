"""GPU parity of bf16 KDA states (the state pool's dtype follows the cache
dtype setting on the pages; the arithmetic stays fp32).

The initial states are drawn in fp32 and rounded to bf16 on the host; the
fp64 oracle runs from those rounded values, so the only differences left are
the kernels' fp32 arithmetic and the one rounding of the state written back.
Bars: relative L2 <= 1e-2 (the bf16 bar) for o and the final state.  Decode
with a bf16 state runs the same fp32 step as with an fp32 state holding the
same values: its o and its state rounded to bf16 must agree with that run's
to fp32 rounding."""
import numpy as np
import pytest
import torch

import oracle
import synth
from kda_cases import TOL, dev_inputs, oracle_qk, rel_l2, say, to_dev, to_host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_55_amd as m

    return m


def bf16_state(inp):
    """(device bf16 h0, its fp64 values) from the fp32 draw, or (None, None)."""
    if inp.h0 is None:
        return None, None
    bits = synth.f64_to_bf16_bits(inp.h0.astype(np.float64))
    return to_dev(bits, "bf16"), synth.bf16_bits_to_f64(bits)


def oracle_run(inp, h0_64, norm):
    f = inp.f64()
    q, k = oracle_qk(inp, f, norm)
    return oracle.prefill(q, k, f["v"], f["g"], f["beta"], h0_64, f["cu_seqlens"], f["scale"])


CASES = [
    # d, chunk, lengths, H, h0_std, norm
    (128, 64, [300, 0, 77], 4, 0.05, False),
    (64, 32, [129, 5], 4, 0.05, True),
    (32, 16, [90], 6, 0.05, False),
    (128, 64, [200], 2, 0.0, False),          # no h0: ht allocated as bf16
]


@pytest.mark.parametrize("d,chunk,lengths,H,h0_std,norm", CASES)
@pytest.mark.parametrize("path", ["chunked", "recurrent"])
def test_prefill_bf16_state(kda, path, d, chunk, lengths, H, h0_std, norm):
    say(f"{path} prefill, bf16 state: d={d} C={chunk} lengths={lengths} H={H} h0={h0_std > 0}")
    inp = synth.make_inputs(61, lengths, H, d, dtype="bf16", gate="kimi", h0_std=h0_std,
                            chunk=chunk, qk_prenorm=not norm)
    dev = dev_inputs(inp)
    h0, h0_64 = bf16_state(inp)
    args = (dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], h0, dev["cu_seqlens"])
    kw = dict(scale=inp.scale, qk_l2norm=norm, state_dtype=torch.bfloat16)
    if path == "chunked":
        o, ht = kda.chunk_prefill(*args, chunk=chunk, **kw)
    else:
        o, ht = kda.recurrent_prefill(*args, **kw)
    torch.cuda.synchronize()
    assert ht.dtype == torch.bfloat16
    o_ref, ht_ref = oracle_run(inp, h0_64, norm)
    eo, es = rel_l2(to_host64(o), o_ref), rel_l2(to_host64(ht), ht_ref)
    say(f"  rel-L2 o={eo:.3e} state={es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_prefill_bf16_state_pool_in_place(kda):
    """A bf16 pool carried in place through a slot table: untouched slots keep
    their bits, used slots hold the final states."""
    say("chunked prefill, bf16 pool in place with a slot table")
    lengths, H, d, S = [150, 40, 90], 4, 128, 6
    inp = synth.make_inputs(62, lengths, H, d, dtype="bf16", gate="kimi", h0_std=0.0, chunk=64)
    dev = dev_inputs(inp)
    pool_bits = synth.f64_to_bf16_bits(
        np.random.default_rng(5).normal(0.0, 0.05, (S, H, d, d)))
    pool = to_dev(pool_bits, "bf16")
    before = pool.clone()
    slots = [4, -1, 1]
    idx = torch.tensor(slots, dtype=torch.int32, device="cuda")
    o, ht = kda.chunk_prefill(dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"], pool,
                              dev["cu_seqlens"], scale=inp.scale, state_indices=idx)
    torch.cuda.synchronize()
    assert ht.data_ptr() == pool.data_ptr()
    h0_64 = synth.bf16_bits_to_f64(pool_bits)[[4, 0, 1]]   # slot 0 stands in for the skip
    o_ref, ht_ref = oracle_run(inp, h0_64, False)
    cu = inp.cu_seqlens
    for n, s in enumerate(slots):
        if s < 0:
            continue
        rows = slice(cu[n], cu[n + 1])
        eo = rel_l2(to_host64(o[rows]), o_ref[rows])
        es = rel_l2(to_host64(pool[s]), ht_ref[n])
        say(f"  seq {n} slot {s}: rel-L2 o={eo:.3e} state={es:.3e}")
        assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    for s in (0, 2, 3, 5):
        assert torch.equal(pool[s].view(torch.int16), before[s].view(torch.int16))


@pytest.mark.parametrize("d,H,Hg,norm", [(128, 8, 2, True), (64, 4, 4, False), (32, 4, 1, True)])
def test_decode_bf16_state(kda, d, H, Hg, norm):
    say(f"decode, bf16 state: d={d} H={H} Hg={Hg} norm={norm}")
    N = 5
    inp = synth.make_inputs(63, [1] * N, H, d, dtype="bf16", h0_std=0.5, n_k_heads=Hg,
                            qk_prenorm=not norm)
    dev = dev_inputs(inp)
    st16, h0_64 = bf16_state(inp)
    st32 = st16.float()                      # the same values held in fp32
    step = (dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"])
    o16 = kda.recurrent_decode(st16, *step, scale=inp.scale, qk_l2norm=norm)
    o32 = kda.recurrent_decode(st32, *step, scale=inp.scale, qk_l2norm=norm)
    torch.cuda.synchronize()
    f = inp.f64()
    q, k = oracle_qk(inp, f, norm)
    o_ref, st_ref = oracle.decode(h0_64, q, k, f["v"], f["g"], f["beta"], f["scale"])
    eo, es = rel_l2(to_host64(o16), o_ref), rel_l2(to_host64(st16), st_ref)
    say(f"  rel-L2 o={eo:.3e} state={es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    # against the fp32-state step on the same values
    e_o = rel_l2(to_host64(o16), to_host64(o32))
    e_s = rel_l2(to_host64(st16), to_host64(st32.to(torch.bfloat16)))
    say(f"  vs fp32 state: rel-L2 o={e_o:.3e} state (rounded)={e_s:.3e}")
    assert e_o <= 1e-6 and e_s <= 1e-6


def test_decode_bf16_state_pool(kda):
    """Decode on a bf16 pool through a slot table: skipped and unused slots
    keep their bits."""
    say("decode, bf16 pool with a slot table")
    N, H, d, S = 4, 4, 128, 7
    inp = synth.make_inputs(64, [1] * N, H, d, dtype="bf16", h0_std=0.5)
    dev = dev_inputs(inp)
    bits = synth.f64_to_bf16_bits(np.random.default_rng(6).normal(0.0, 0.5, (S, H, d, d)))
    pool = to_dev(bits, "bf16")
    before = pool.clone()
    slots = [6, 2, -1, 0]
    idx = torch.tensor(slots, dtype=torch.int32, device="cuda")
    o = kda.recurrent_decode(pool, dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"],
                             scale=inp.scale, state_indices=idx)
    torch.cuda.synchronize()
    f = inp.f64()
    st0 = synth.bf16_bits_to_f64(bits)[[6, 2, 0, 0]]
    o_ref, st_ref = oracle.decode(st0, f["q"], f["k"], f["v"], f["g"], f["beta"], f["scale"])
    for n, s in enumerate(slots):
        if s < 0:
            continue
        eo = rel_l2(to_host64(o[n]), o_ref[n])
        es = rel_l2(to_host64(pool[s]), st_ref[n])
        say(f"  seq {n} slot {s}: rel-L2 o={eo:.3e} state={es:.3e}")
        assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    for s in (1, 3, 4, 5):
        assert torch.equal(pool[s].view(torch.int16), before[s].view(torch.int16))
