"""Shapes whose element offsets pass 2^31.

The chunked prefill with a batch whose last sequence starts beyond element
2^31 of q, k, v and o (and beyond byte 2^33 of g, with a workspace of ~22 GB),
through each scan the launch can pick: the 16-column and the 32-column
column-block scans and the per-head scan; the token-by-token prefill on such a
batch; one decode step on a state of more than 2^31 fp32 values; the short
conv with x and y past element 2^31.  Inputs are drawn on the device
(synth.device_inputs: the workload recipe's distributions, for tensors too
large to draw on the host); the oracle checks the sequences past the boundary
on sampled heads, from the same values copied back to the host.  Each case
holds ~60 GB of device memory and frees it before the next."""
import gc

import numpy as np
import pytest
import torch

import oracle
from kda_cases import TOL, check_tokens, rel_l2, say, to_host64, worst_head
from synth.device_inputs import host_f64, make_device_inputs

pytestmark = pytest.mark.gpu

ELEM_LIMIT = 1 << 31


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_55_amd as m

    return m


def _cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def _release():
    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _scan_of(N, H, D=128):
    """The scan the launch picks for N sequences of H heads: the per-head scan
    for more (sequence, head) pairs than half the CUs, else the widest
    column block (64, 32, 16 columns) that leaves every CU a workgroup."""
    cus = _cus()
    if 2 * N * H > cus:
        return "per-head scan"
    for nj in (4, 2):
        if N * H * (D // 16 // nj) >= cus:
            return f"{16 * nj}-column blocks"
    return "16-column blocks"


def _past(H, D=128):
    """First token whose row starts at element 2^31 or later."""
    return -(-ELEM_LIMIT // (H * D))


@pytest.mark.parametrize("H,lengths,which", [
    (16, [_past(16) + 1000, 3000], "16-column blocks"),
    (32, [_past(32) + 1000, 3000], "32-column blocks"),
    (32, [75000] * 7 + [3000], "per-head scan"),
])
def test_prefill_past_2e31_elements(kda, H, lengths, which):
    D = 128
    N = len(lengths)
    start_last = sum(lengths[:-1])
    assert start_last * H * D >= ELEM_LIMIT, "the last sequence must start past element 2^31"
    assert _scan_of(N, H, D) == which, "the batch reaches the named scan"
    say(f"large prefill ({which}): H={H} lengths={lengths} T={sum(lengths)}, last sequence "
        f"from element {start_last * H * D} (2^31 = {ELEM_LIMIT})")
    d = make_device_inputs(301 + H + N, lengths, H, D, h0_std=0.02)
    o, ht = kda.chunk_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"],
                              d["cu_seqlens"], scale=d["scale"], chunk=64)
    torch.cuda.synchronize()
    heads = [0, H - 1]
    f = host_f64(d, N - 1, heads)
    s, e = f["range"]
    o_ref, s_ref = oracle.prefill(f["q"], f["k"], f["v"], f["g"], f["beta"], f["h0"],
                                  f["cu_seqlens"], f["scale"])
    o_g = to_host64(o[s:e][:, heads])
    s_g = to_host64(ht[N - 1:N][:, heads])
    del o, ht, d
    _release()
    eo, es = rel_l2(o_g, o_ref), rel_l2(s_g, s_ref)
    who, whs = worst_head(o_g, o_ref), worst_head(s_g, s_ref)
    tok = check_tokens(o_g, o_ref, TOL["bf16"])
    say(f"  last sequence, heads {heads}: rel-L2 o={eo:.3e} state={es:.3e} worst head "
        f"o={who:.3e} state={whs:.3e} worst token {tok:.3e}")
    assert max(eo, es, who, whs) <= TOL["bf16"]


def test_decode_state_past_2e31_elements(kda):
    H, D = 32, 128
    N = -(-ELEM_LIMIT // (H * D * D)) + 64  # the last sequences' states start past 2^31
    assert (N - 1) * H * D * D >= ELEM_LIMIT
    say(f"large decode: N={N} H={H}: state of {N * H * D * D} fp32 values")
    d = make_device_inputs(401, [1] * N, H, D, h0_std=0.5)
    ns, hs = [0, N - 1], [0, H - 1]
    pick = lambda x: x[ns][:, hs].double().cpu().numpy()  # noqa: E731
    st0 = pick(d["h0"])
    q, k, v, g, beta = (pick(d[x]) for x in ("q", "k", "v", "g", "beta"))
    state = d["h0"]  # updated in place
    o = kda.recurrent_decode(state, d["q"], d["k"], d["v"], d["g"], d["beta"], scale=d["scale"])
    torch.cuda.synchronize()
    o_g, st_g = to_host64(o[ns][:, hs]), to_host64(state[ns][:, hs])
    del o, state, d
    _release()
    o_ref, st_ref = oracle.decode(st0, q, k, v, g, beta, float(D ** -0.5))
    eo, es = rel_l2(o_g, o_ref), rel_l2(st_g, st_ref)
    say(f"  sequences {ns}, heads {hs}: rel-L2 o={eo:.3e} state={es:.3e}")
    assert eo <= TOL["bf16"] and es <= 1e-6
    assert np.isfinite(o_g).all()


def test_recurrent_prefill_past_2e31_elements(kda):
    """The token-by-token prefill over a batch whose last sequence starts past
    element 2^31 (H = 32: 528 K tokens)."""
    H, D = 32, 128
    lengths = [_past(H) + 1000, 3000]
    N = len(lengths)
    assert lengths[0] * H * D >= ELEM_LIMIT
    say(f"large recurrent prefill: H={H} lengths={lengths}")
    d = make_device_inputs(311, lengths, H, D, h0_std=0.02)
    o, ht = kda.recurrent_prefill(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"],
                                  d["cu_seqlens"], scale=d["scale"])
    torch.cuda.synchronize()
    heads = [0, H - 1]
    f = host_f64(d, N - 1, heads)
    s, e = f["range"]
    o_ref, s_ref = oracle.prefill(f["q"], f["k"], f["v"], f["g"], f["beta"], f["h0"],
                                  f["cu_seqlens"], f["scale"])
    o_g = to_host64(o[s:e][:, heads])
    s_g = to_host64(ht[N - 1:N][:, heads])
    del o, ht, d
    _release()
    eo, es = rel_l2(o_g, o_ref), rel_l2(s_g, s_ref)
    tok = check_tokens(o_g, o_ref, TOL["bf16"])
    say(f"  last sequence, heads {heads}: rel-L2 o={eo:.3e} state={es:.3e} worst token {tok:.3e}")
    assert eo <= TOL["bf16"] and es <= 1e-5


def test_conv_past_2e31_elements(kda):
    """The short conv over [q|k|v] channels (dim = 12,288, W = 4, bf16) with
    the last sequence starting past element 2^31 of x and y; sampled channels
    against the oracle (per-element bound), new taps bit for bit."""
    from synth.device_inputs import make_device_conv_inputs

    dim, W = 12288, 4
    lengths = [-(-ELEM_LIMIT // dim) + 100, 500]
    assert lengths[0] * dim >= ELEM_LIMIT
    say(f"large conv: dim={dim} W={W} lengths={lengths}")
    c = make_device_conv_inputs(321, lengths, dim, W)
    new = torch.empty_like(c["state"])
    y = kda.causal_conv1d_fwd(c["x"], c["weight"], c["bias"], cu_seqlens=c["cu_seqlens"],
                              state_in=c["state"], state_out=new, activation="silu")
    torch.cuda.synchronize()
    s, e = int(c["cu_host"][1]), int(c["cu_host"][2])
    ch = [0, 1, dim // 2, dim - 2, dim - 1]
    host = lambda t: t.double().cpu().numpy()  # noqa: E731
    x_s = host(c["x"][s:e][:, ch])
    y_ref, st_ref = oracle.causal_conv1d(x_s, host(c["weight"][ch]), host(c["bias"][ch]),
                                         np.array([0, e - s]), host(c["state"][1:2][:, :, ch]),
                                         activation="silu")
    y_g = host(y[s:e][:, ch])
    st_g = host(new[1:2][:, :, ch])
    del y, new, c
    _release()
    err = rel_l2(y_g, y_ref)
    excess = float(np.max(np.abs(y_g - y_ref) - (2.0 ** -8 * np.abs(y_ref) + 1e-4)))
    say(f"  last sequence, channels {ch}: rel-L2 y={err:.3e}, worst excess over element bound "
        f"{excess:.2e}")
    assert err <= TOL["bf16"] and excess <= 0.0
    assert np.array_equal(st_g, st_ref)
