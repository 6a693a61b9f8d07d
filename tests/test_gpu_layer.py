"""The short conv feeding the KDA step, as the pages run them in a layer: the
conv over the [q|k|v] channels writes q, k and v as separate tensors, the
chunked prefill reads them with the gate activation fused and q, k
normalised in the kernels, and decode continues with the conv update and a
recurrent step on the carried taps and state.  The oracle composes its own
fp64 conv, normalisation, gate and recurrence from the same stored inputs
(no value it uses comes from the GPU); the bar is the bf16 one, 1e-2."""
import numpy as np
import pytest
import torch

import oracle
import synth
from kda_cases import TOL, rel_l2, say, to_dev, to_host64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_55_amd as m

    return m


@pytest.mark.parametrize("H,d,lengths", [(4, 64, [150, 37]), (2, 128, [200])])
def test_conv_then_prefill_then_decode(kda, H, d, lengths):
    say(f"layer: conv -> prefill (fused gate, in-kernel norm) -> decode; H={H} d={d} {lengths}")
    dim, W, N = 3 * H * d, 4, len(lengths)
    T = sum(lengths)
    cin = synth.make_conv_inputs(71, [n + 1 for n in lengths], dim, W, "bf16")
    kin = synth.make_inputs(72, [n + 1 for n in lengths], H, d, dtype="bf16", gate="kimi",
                            h0_std=0.02, qk_prenorm=False)
    cu_all = cin.cu_seqlens  # each sequence: its prefill tokens, then one decode token
    pre_rows = np.concatenate([np.arange(cu_all[n], cu_all[n + 1] - 1) for n in range(N)])
    dec_rows = np.array([cu_all[n + 1] - 1 for n in range(N)])
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)

    # GPU: conv forward on the prefill rows (taps carried into a pool), prefill
    x = to_dev(cin.x, "bf16")
    w, b = to_dev(cin.weight, "f32"), to_dev(cin.bias, "f32")
    taps = to_dev(cin.state, "bf16")
    cu_d = torch.from_numpy(cu).cuda()
    pre_idx = torch.from_numpy(pre_rows).cuda()
    q, k, v = kda.causal_conv1d_fwd(x[pre_idx].contiguous(), w, b, cu_d, taps, taps,
                                    split=(H * d,) * 3)
    gx = to_dev(kin.gate_x, "bf16")
    gate = (gx[pre_idx].contiguous(), to_dev(kin.gate_a_log, "f32"),
            to_dev(kin.gate_dt_bias, "f32"))
    beta = to_dev(kin.beta, "bf16")
    h0 = to_dev(kin.h0, "f32")
    o, ht = kda.chunk_prefill(q.view(T, H, d), k.view(T, H, d), v.view(T, H, d), None,
                              beta[pre_idx].contiguous(), h0, cu_d, gate=gate, qk_l2norm=True)
    # decode: conv update on the carried taps, then one recurrent step
    dec_idx = torch.from_numpy(dec_rows).cuda()
    qd, kd, vd = kda.causal_conv1d_update(x[dec_idx].contiguous(), w, b, taps,
                                          split=(H * d,) * 3)
    gd = (gx[dec_idx].contiguous(), gate[1], gate[2])
    od = kda.recurrent_decode(ht, qd.view(N, H, d), kd.view(N, H, d), vd.view(N, H, d), None,
                              beta[dec_idx].contiguous(), gate=gd, qk_l2norm=True)
    torch.cuda.synchronize()

    # oracle: the same composition in fp64 from the stored inputs
    fc, fk = cin.f64(), kin.f64()
    y, _ = oracle.causal_conv1d(fc["x"], fc["weight"], fc["bias"], cu_all, fc["state"], "silu")
    y = y.reshape(-1, 3, H, d)
    qo, ko, vo = oracle.l2norm(y[:, 0]), oracle.l2norm(y[:, 1]), y[:, 2]
    g = oracle.kimi_gate(*kin.gate_f64())
    o_ref, ht_ref = oracle.prefill(qo[pre_rows], ko[pre_rows], vo[pre_rows], g[pre_rows],
                                   fk["beta"][pre_rows], fk["h0"], cu, fk["scale"])
    od_ref, st_ref = oracle.decode(ht_ref, qo[dec_rows], ko[dec_rows], vo[dec_rows],
                                   g[dec_rows], fk["beta"][dec_rows], fk["scale"])
    e = [rel_l2(to_host64(o), o_ref), rel_l2(to_host64(od), od_ref),
         rel_l2(to_host64(ht), st_ref)]
    say(f"  rel-L2 prefill o={e[0]:.3e} decode o={e[1]:.3e} state={e[2]:.3e}")
    assert max(e) <= TOL["bf16"]
