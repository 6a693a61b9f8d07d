"""GPU parity of the short causal conv (kda_causal_conv1d_fwd / _update)
against the fp64 oracle (oracle/conv.py) on the same seeded, rounded inputs.

Bars.  y: relative L2 <= 1e-4 (fp32) / 1e-2 (bf16), and per element
|y - ref| <= 2^-8 |ref| + 1e-4 in bf16 (one rounding of the fp32 result) or
1e-5 |ref| + 1e-5 in fp32.  The new taps are copies of inputs, so they must
equal the oracle's exactly.  Properties that hold bit for bit: the split
output equals the single one, in-place and separate state agree, the update
equals the forward with every length 1, and prefill + updates equal one
forward over the whole sequence."""
import numpy as np
import pytest
import torch

import oracle
import synth
from kda_cases import TOL, rel_l2, say, to_dev, to_host64

pytestmark = pytest.mark.gpu

DTY = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_55_amd as m

    return m


def dev_conv(inp):
    return dict(x=to_dev(inp.x, inp.dtype), weight=to_dev(inp.weight, "f32"),
                bias=to_dev(inp.bias, "f32"),
                state=None if inp.state is None else to_dev(inp.state, inp.dtype),
                cu=torch.from_numpy(inp.cu_seqlens).cuda())


def check_y(y, ref, dtype, rows=None):
    y = np.asarray(y, dtype=np.float64)
    if rows is not None:
        y, ref = y[rows], ref[rows]
    e = rel_l2(y, ref)
    if dtype == "bf16":
        bound = 2.0 ** -8 * np.abs(ref) + 1e-4
    else:
        bound = 1e-5 * np.abs(ref) + 1e-5
    worst = float(np.max(np.abs(y - ref) - bound)) if y.size else -1.0
    say(f"  rel-L2 y={e:.3e}, worst excess over element bound {worst:.2e}")
    assert e <= TOL[dtype] and worst <= 0.0


ACT = ["none", "silu"]


@pytest.mark.parametrize("dtype,dim,W,lengths,state,act", [
    ("f32", 8, 4, [37], True, "silu"),
    ("f32", 24, 2, [1, 0, 40, 2], True, "none"),
    ("f32", 264, 3, [17, 16, 15, 33], False, "silu"),
    ("bf16", 8, 4, [5], True, "silu"),
    ("bf16", 64, 4, [64, 1, 129, 0, 200], True, "silu"),
    ("bf16", 2056, 4, [31, 2, 70], True, "none"),     # a partial channel block
    ("bf16", 4096, 3, [16, 17, 1, 1, 3], True, "silu"),
    ("bf16", 384, 2, [0, 0, 9], False, "silu"),
])
def test_fwd_matches_oracle(kda, dtype, dim, W, lengths, state, act):
    say(f"conv fwd dtype={dtype} dim={dim} W={W} lengths={lengths} state={state} act={act}")
    inp = synth.make_conv_inputs(3, lengths, dim, W, dtype, with_state=state)
    d = dev_conv(inp)
    st_out = torch.full((inp.N, W - 1, dim), 9.0, dtype=DTY[dtype], device="cuda")
    y = kda.causal_conv1d_fwd(d["x"], d["weight"], d["bias"], d["cu"], state_in=d["state"],
                              state_out=st_out, activation=act)
    torch.cuda.synchronize()
    f = inp.f64()
    y_ref, st_ref = oracle.causal_conv1d(f["x"], f["weight"], f["bias"], f["cu_seqlens"],
                                         f["state"], act)
    check_y(to_host64(y), y_ref, dtype)
    assert np.array_equal(to_host64(st_out), st_ref)


def test_split_inplace_and_no_bias(kda):
    say("conv fwd: [q|k|v] split = single output; in-place state = separate; bias None")
    dim = 3 * 4 * 64
    inp = synth.make_conv_inputs(4, [50, 3, 77], dim, 4, "bf16")
    d = dev_conv(inp)
    st_sep = torch.empty_like(d["state"])
    y = kda.causal_conv1d_fwd(d["x"], d["weight"], d["bias"], d["cu"], d["state"], st_sep)
    q, k, v = kda.causal_conv1d_fwd(d["x"], d["weight"], d["bias"], d["cu"], d["state"], None,
                                    split=(256, 256, 256))
    st_in = d["state"].clone()
    y2 = kda.causal_conv1d_fwd(d["x"], d["weight"], d["bias"], d["cu"], st_in, st_in)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([q, k, v], 1), y) and torch.equal(y2, y)
    assert torch.equal(st_in, st_sep)
    assert q.is_contiguous() and q.shape == (130, 256)
    yb = kda.causal_conv1d_fwd(d["x"], d["weight"], None, d["cu"], d["state"], None)
    torch.cuda.synchronize()
    f = inp.f64()
    ref, _ = oracle.causal_conv1d(f["x"], f["weight"], None, f["cu_seqlens"], f["state"], "silu")
    check_y(to_host64(yb), ref, "bf16")


def test_state_pool_and_skips(kda):
    say("conv fwd with a state pool: slots, negative slot skips")
    dim, W = 128, 4
    inp = synth.make_conv_inputs(5, [20, 7, 33], dim, W, "bf16")
    d = dev_conv(inp)
    pool = torch.randn((6, W - 1, dim), device="cuda").to(torch.bfloat16)
    pool[4] = d["state"][0]
    pool[1] = d["state"][2]
    before = pool.clone()
    slots = torch.tensor([4, -1, 1], dtype=torch.int32, device="cuda")
    y = torch.full((60, dim), 5.0, dtype=torch.bfloat16, device="cuda")
    kda.causal_conv1d_fwd(d["x"], d["weight"], d["bias"], d["cu"], pool, pool,
                          state_indices=slots, out=y)
    torch.cuda.synchronize()
    f = inp.f64()
    ref, st_ref = oracle.causal_conv1d(f["x"], f["weight"], f["bias"], f["cu_seqlens"],
                                       f["state"], "silu")
    rows = np.r_[0:20, 27:60]
    check_y(to_host64(y), ref, "bf16", rows)
    assert torch.all(y[20:27] == 5.0)                      # the skipped sequence
    assert np.array_equal(to_host64(pool[4]), st_ref[0])
    assert np.array_equal(to_host64(pool[1]), st_ref[2])
    for s in (0, 2, 3, 5):
        assert torch.equal(pool[s], before[s])


@pytest.mark.parametrize("dtype,W,act", [("f32", 4, "silu"), ("bf16", 4, "silu"),
                                         ("bf16", 2, "none"), ("bf16", 3, "silu")])
def test_update_matches_oracle_and_fwd(kda, dtype, W, act):
    say(f"conv update dtype={dtype} W={W} act={act}")
    dim, N = 768, 9
    inp = synth.make_conv_inputs(6, [1] * N, dim, W, dtype)
    d = dev_conv(inp)
    st = d["state"].clone()
    y = kda.causal_conv1d_update(d["x"], d["weight"], d["bias"], st, activation=act)
    st_f = torch.empty_like(st)
    y_f = kda.causal_conv1d_fwd(d["x"], d["weight"], d["bias"], d["cu"], d["state"], st_f,
                                activation=act)
    torch.cuda.synchronize()
    f = inp.f64()
    ref, st_ref = oracle.causal_conv1d(f["x"], f["weight"], f["bias"], f["cu_seqlens"],
                                       f["state"], act)
    check_y(to_host64(y), ref, dtype)
    assert np.array_equal(to_host64(st), st_ref)
    assert torch.equal(y, y_f) and torch.equal(st, st_f)


def test_prefill_then_updates_equal_one_pass(kda):
    say("conv: prefill 100 tokens + 12 updates = one forward over 112 (bitwise)")
    dim, W, N = 1536, 4, 3
    L0, steps = 100, 12
    inp = synth.make_conv_inputs(7, [L0 + steps] * N, dim, W, "bf16")
    d = dev_conv(inp)
    x = d["x"].view(N, L0 + steps, dim)
    st_all = torch.empty_like(d["state"])
    y_all = kda.causal_conv1d_fwd(d["x"], d["weight"], d["bias"], d["cu"], d["state"], st_all)
    pre = x[:, :L0].reshape(N * L0, dim).contiguous()
    cu = torch.arange(0, N * L0 + 1, L0, dtype=torch.int32, device="cuda")
    pool = torch.zeros((5, W - 1, dim), dtype=torch.bfloat16, device="cuda")
    slots = torch.tensor([3, 0, 4], dtype=torch.int32, device="cuda")
    pool[slots.long()] = d["state"]
    y_pre = kda.causal_conv1d_fwd(pre, d["weight"], d["bias"], cu, pool, pool,
                                  state_indices=slots)
    ys = [kda.causal_conv1d_update(x[:, L0 + s].contiguous(), d["weight"], d["bias"], pool,
                                   state_indices=slots) for s in range(steps)]
    torch.cuda.synchronize()
    y_all = y_all.view(N, L0 + steps, dim)
    assert torch.equal(y_pre.view(N, L0, dim), y_all[:, :L0])
    for s in range(steps):
        assert torch.equal(ys[s], y_all[:, L0 + s])
    assert torch.equal(pool[slots.long()], st_all)


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_full_size_sampled(kda, cfg):
    """The [q|k|v] conv at the workload shapes (H = 32, d = 128: dim 12288,
    W = 4, SiLU, bf16), in the launch bench.py times; sampled rows against
    the oracle run on the rows each needs."""
    lengths = synth.kda_inputs.config_lengths(cfg)
    if cfg == 4:
        lengths = [1024] * 64
    dim, W = 3 * 32 * 128, 4
    say(f"conv full size cfg={cfg} T={sum(lengths)} dim={dim}")
    inp = synth.make_conv_inputs(8 + cfg, lengths, dim, W, "bf16")
    d = dev_conv(inp)
    st = d["state"].clone()
    q, k, v = kda.causal_conv1d_fwd(d["x"], d["weight"], d["bias"], d["cu"], st, st,
                                    split=(4096, 4096, 4096))
    torch.cuda.synchronize()
    y = torch.cat([q, k, v], 1)
    f = inp.f64()
    cu = inp.cu_seqlens
    rng = np.random.default_rng(cfg)
    for n in sorted(set([0, inp.N - 1] + list(rng.integers(0, inp.N, 3)))):
        s, e = int(cu[n]), int(cu[n + 1])
        # first rows (carried taps), a random window, the last rows (new taps)
        a = int(rng.integers(s + 3, max(s + 4, e - 40)))
        for lo, hi in [(s, min(e, s + 40)), (a, min(e, a + 40)), (max(s, e - 40), e)]:
            if lo == s:
                stn = f["state"][n:n + 1]
            else:  # the W - 1 inputs before lo stand in for the carried taps
                stn = f["x"][lo - (W - 1):lo][None]
            ref, _ = oracle.causal_conv1d(f["x"][lo:hi], f["weight"], f["bias"], [0, hi - lo],
                                          stn, "silu")
            check_y(to_host64(y[lo:hi]), ref, "bf16")
        _, st_ref = oracle.causal_conv1d(f["x"][max(s, e - 8):e], f["weight"], f["bias"],
                                         [0, e - max(s, e - 8)],
                                         f["state"][n:n + 1] if e - s < 8 else
                                         f["x"][e - 8 - (W - 1):e - 8][None], "silu")
        assert np.array_equal(to_host64(st[n]), st_ref[0])


def test_update_full_decode_shape(kda):
    """The one-token update at the decode workload's shape: 64 sequences, dim
    12288, W = 4, SiLU, bf16, taps in a 64-slot pool in shuffled order; three
    steps against the oracle."""
    N, dim, W = 64, 3 * 32 * 128, 4
    say(f"conv update full decode shape N={N} dim={dim}")
    inp = synth.make_conv_inputs(12, [3] * N, dim, W, "bf16")
    d = dev_conv(inp)
    x = d["x"].view(N, 3, dim)
    slots = torch.from_numpy(np.random.default_rng(1).permutation(N).astype(np.int32)).cuda()
    pool = torch.empty_like(d["state"])
    pool[slots.long()] = d["state"]
    ys = [kda.causal_conv1d_update(x[:, s].contiguous(), d["weight"], d["bias"], pool,
                                   state_indices=slots, split=(4096, 4096, 4096))
          for s in range(3)]
    torch.cuda.synchronize()
    f = inp.f64()
    ref, st_ref = oracle.causal_conv1d(f["x"], f["weight"], f["bias"], f["cu_seqlens"],
                                       f["state"], "silu")
    ref = ref.reshape(N, 3, dim)
    for s in range(3):
        check_y(to_host64(torch.cat(ys[s], 1)), ref[:, s], "bf16")
    assert np.array_equal(to_host64(pool[slots.long()]), st_ref)
