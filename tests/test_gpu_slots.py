"""GPU parity of the state pool (slot-indexed states) and of the recurrent
prefill (token-by-token over a carried state), against the fp64 oracle and
against the chunked path.  Bars: relative L2 <= 1e-4 (fp32), <= 1e-2 (bf16)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from kda_cases import TOL, dev_inputs, oracle_prefill, rel_l2, say, to_dev, to_host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_55_amd as m

    return m


def test_decode_state_pool(kda):
    say("decode over a state pool: slots [5, 0, -1, 3] of 7")
    H, D, S = 4, 64, 7
    inp = synth.make_inputs(61, [1] * 4, H, D, dtype="bf16", h0_std=0.5)
    pool = np.random.default_rng(7).normal(0.0, 0.5, (S, H, D, D)).astype(np.float32)
    slots = np.array([5, 0, -1, 3], dtype=np.int32)
    dev = dev_inputs(inp)
    state = torch.from_numpy(pool.copy()).cuda()
    out = torch.full((4, H, D), 3.0, dtype=torch.bfloat16, device="cuda")
    kda.recurrent_decode(state, dev["q"], dev["k"], dev["v"], dev["g"], dev["beta"],
                         scale=inp.scale, out=out, state_indices=torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    f = inp.f64()
    live = [0, 1, 3]
    o_ref, st_ref = oracle.decode(pool[slots[live]].astype(np.float64), f["q"][live], f["k"][live],
                                  f["v"][live], f["g"][live], f["beta"][live], f["scale"])
    o_g, st_g = to_host64(out), to_host64(state)
    eo, es = rel_l2(o_g[live], o_ref), rel_l2(st_g[slots[live]], st_ref)
    say(f"  rel-L2 o={eo:.3e} state={es:.3e}")
    assert eo <= TOL["bf16"] and es <= 1e-6
    assert np.all(o_g[2] == 3.0)                                   # skipped: o untouched
    for s in (1, 2, 4, 6):                                         # unused slots untouched
        assert np.array_equal(st_g[s], pool[s].astype(np.float64))


def test_chunk_prefill_state_pool_in_place(kda):
    say("chunked prefill, h0 = ht = pool, slots [4, 1, -1]")
    H, D, S = 3, 128, 5
    inp = synth.make_inputs(62, [90, 33, 20], H, D, dtype="bf16", chunk=64)
    pool = np.random.default_rng(8).normal(0.0, 0.05, (S, H, D, D)).astype(np.float32)
    slots = np.array([4, 1, -1], dtype=np.int32)
    d = dev_inputs(inp)
    pool_d = torch.from_numpy(pool.copy()).cuda()
    out = torch.full((inp.T, H, D), 5.0, dtype=torch.bfloat16, device="cuda")
    kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], pool_d, d["cu_seqlens"],
                      scale=inp.scale, chunk=64, out=out, ht=pool_d,
                      state_indices=torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    # reference: the first two sequences alone, h0 gathered from the pool
    sub = synth.make_inputs(62, [90, 33, 20], H, D, dtype="bf16", chunk=64)
    f = sub.f64()
    T2 = 123
    cu2 = np.array([0, 90, 123], dtype=np.int64)
    o_ref, st_ref = oracle.prefill(f["q"][:T2], f["k"][:T2], f["v"][:T2], f["g"][:T2],
                                   f["beta"][:T2], pool[slots[:2]].astype(np.float64), cu2,
                                   f["scale"])
    o_g, st_g = to_host64(out), to_host64(pool_d)
    eo, es = rel_l2(o_g[:T2], o_ref), rel_l2(st_g[slots[:2]], st_ref)
    say(f"  rel-L2 o={eo:.3e} state={es:.3e}")
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
    assert np.all(o_g[T2:] == 5.0)
    for s in (0, 2, 3):
        assert np.array_equal(st_g[s], pool[s].astype(np.float64))


@pytest.mark.parametrize("dtype,d,lengths,h0", [
    ("f32", 32, [5, 12, 0, 1], True),
    ("bf16", 128, [17, 0, 40], True),
    ("bf16", 64, [64], False),
])
def test_recurrent_prefill_matches_oracle(kda, dtype, d, lengths, h0):
    say(f"recurrent prefill dtype={dtype} d={d} lengths={lengths}")
    inp = synth.make_inputs(63, lengths, 3, d, dtype=dtype, h0_std=0.05 if h0 else 0.0,
                            gate="softplus" if dtype == "f32" else "kimi")
    dv = dev_inputs(inp)
    o, ht = kda.recurrent_prefill(dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"], dv["h0"],
                                  dv["cu_seqlens"], scale=inp.scale)
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle_prefill(inp)
    eo, es = rel_l2(to_host64(o), o_ref), rel_l2(to_host64(ht), ht_ref)
    say(f"  rel-L2 o={eo:.3e} state={es:.3e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_recurrent_prefill_one_token_equals_decode(kda):
    """One token per sequence: the recurrent prefill computes the decode step.
    The two kernels are compiled separately (the compiler may fuse multiply-adds
    differently), so they agree to fp32 rounding: the state to 1e-6, o to a
    bf16 rounding flip in a few elements."""
    inp = synth.make_inputs(64, [1] * 5, 4, 128, dtype="bf16", h0_std=0.3)
    dv = dev_inputs(inp)
    o1, s1 = kda.recurrent_prefill(dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"], dv["h0"],
                                   dv["cu_seqlens"], scale=inp.scale)
    state = dv["h0"].clone()
    o2 = kda.recurrent_decode(state, dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"],
                              scale=inp.scale)
    torch.cuda.synchronize()
    eo = rel_l2(to_host64(o1), to_host64(o2))
    es = rel_l2(to_host64(s1), to_host64(state))
    say(f"recurrent(1 token) vs decode: rel-L2 o={eo:.3e} state={es:.3e}")
    assert eo <= 1e-3 and es <= 1e-6


def test_continuing_prefill_through_the_pool(kda):
    """Chunked prefill of 200 tokens into slot 2, then a 24-token recurrent
    continuation from that slot (the serving pattern), equals one prefill of
    all 224 tokens (oracle) and the chunked path."""
    H, D = 4, 128
    full = synth.make_inputs(65, [224], H, D, dtype="bf16", chunk=64)
    dv = dev_inputs(full)
    pool = torch.zeros((3, H, D, D), dtype=torch.float32, device="cuda")
    slot = torch.tensor([2], dtype=torch.int32, device="cuda")
    cut = lambda t, a, b: t[a:b].contiguous()  # noqa: E731
    o_a, _ = kda.chunk_prefill(*(cut(dv[n], 0, 200) for n in ("q", "k", "v", "g", "beta")),
                               pool, None, scale=full.scale, chunk=64, ht=pool,
                               state_indices=slot)
    o_b, _ = kda.recurrent_prefill(*(cut(dv[n], 200, 224) for n in ("q", "k", "v", "g", "beta")),
                                   pool, None, scale=full.scale, ht=pool, state_indices=slot)
    o_c, s_c = kda.chunk_prefill(dv["q"], dv["k"], dv["v"], dv["g"], dv["beta"], None, None,
                                 scale=full.scale, chunk=64)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_prefill(full)
    o_ab = np.concatenate([to_host64(o_a), to_host64(o_b)], 0)
    s_ab = to_host64(pool)[2:3]
    e1, e2 = rel_l2(o_ab, o_ref), rel_l2(s_ab, s_ref)
    e3 = rel_l2(o_ab, to_host64(o_c))
    say(f"continuing prefill: vs oracle o={e1:.3e} state={e2:.3e}; vs one chunked pass o={e3:.3e}")
    assert e1 <= TOL["bf16"] and e2 <= TOL["bf16"] and e3 <= TOL["bf16"]
    assert np.all(to_host64(pool)[:2] == 0.0)
