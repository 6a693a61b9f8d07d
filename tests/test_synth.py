"""The seeded input generator: determinism, stream independence and the
rounding to bf16.  No GPU."""
import numpy as np
import torch

import synth


def test_deterministic_and_stream_keyed():
    a = synth.make_inputs(7, [10, 5], 2, 8, dtype="bf16")
    b = synth.make_inputs(7, [10, 5], 2, 8, dtype="bf16")
    for name in ["q", "k", "v", "g", "beta"]:
        assert np.array_equal(getattr(a, name), getattr(b, name))
    c = synth.make_inputs(7, [10, 5], 2, 8, dtype="bf16", h0_std=0.02)
    assert np.array_equal(a.q, c.q) and c.h0 is not None and a.h0 is None


def test_bf16_rounding_is_rne():
    """fp64 -> bf16 rounding agrees with torch's fp32 -> bf16 (round to nearest
    even) on values that are exact in fp32, including exact ties."""
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000).astype(np.float32)
    ties = (np.arange(1, 200, dtype=np.float32) * 2.0 ** -7 + 2.0 ** -9).astype(np.float32)
    x = np.concatenate([x, ties, -ties])
    mine = synth.f64_to_bf16_bits(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    back = synth.bf16_bits_to_f64(mine)
    assert np.all(np.abs(back - x) <= np.abs(x) * 2.0 ** -8)


def test_config_shapes_and_ranges():
    inp = synth.make_config(0)
    assert inp.q.shape == (128, 2, 32) and inp.q.dtype == np.float32 and inp.chunk == 16
    assert np.all(inp.g <= 0)
    n = np.linalg.norm(inp.q.astype(np.float64), axis=-1)
    assert np.allclose(n, 1.0, atol=1e-6)
    lens = synth.kda_inputs.config_lengths(3)
    assert len(lens) == 8 and all(300 <= x <= 8192 for x in lens)
    assert lens == synth.kda_inputs.config_lengths(3)


def test_kimi_gate_is_negative():
    inp = synth.make_inputs(3, [100], 4, 16, dtype="bf16", gate="kimi")
    assert np.all(inp.g <= 0) and np.all(np.isfinite(inp.g))
    b = synth.bf16_bits_to_f64(inp.beta)
    assert np.all((b > 0) & (b < 1))


def test_device_inputs_recipe_and_slices():
    """The device-side generator (run here on the CPU device): shapes, dtypes,
    unit q/k rows, g <= 0, beta in (0, 1), the same values for the same seed,
    and host_f64 returning one sequence's rows of the sampled heads."""
    from synth.device_inputs import host_f64, make_device_inputs

    a = make_device_inputs(5, [70, 0, 33], 4, 16, h0_std=0.02, device="cpu")
    b = make_device_inputs(5, [70, 0, 33], 4, 16, h0_std=0.02, device="cpu")
    assert a["q"].shape == (103, 4, 16) and a["q"].dtype == torch.bfloat16
    assert a["g"].dtype == torch.float32 and a["h0"].shape == (3, 4, 16, 16)
    assert a["cu_seqlens"].tolist() == [0, 70, 70, 103]
    for x in ("q", "k", "v", "g", "beta", "h0"):
        assert torch.equal(a[x], b[x]), x
    n = a["q"].double().norm(dim=-1)
    assert torch.allclose(n, torch.ones_like(n), atol=1e-2)
    assert bool((a["g"] <= 0).all()) and bool(torch.isfinite(a["g"]).all())
    assert bool(((a["beta"] > 0) & (a["beta"] < 1)).all())
    f = host_f64(a, 2, [1, 3])
    assert f["range"] == (70, 103) and f["q"].shape == (33, 2, 16)
    assert np.array_equal(f["v"], a["v"][70:103][:, [1, 3]].double().numpy())
    assert f["h0"].shape == (1, 2, 16, 16) and list(f["cu_seqlens"]) == [0, 33]


def test_device_conv_inputs_recipe():
    from synth.device_inputs import make_device_conv_inputs

    a = make_device_conv_inputs(7, [20, 0, 9], 24, 4, device="cpu")
    b = make_device_conv_inputs(7, [20, 0, 9], 24, 4, device="cpu")
    assert a["x"].shape == (29, 24) and a["x"].dtype == torch.bfloat16
    assert a["weight"].shape == (24, 4) and a["state"].shape == (3, 3, 24)
    for x in ("x", "weight", "bias", "state"):
        assert torch.equal(a[x], b[x]), x
    lim = 4 ** -0.5
    assert float(a["weight"].abs().max()) <= lim and float(a["bias"].abs().max()) <= lim
    assert a["cu_seqlens"].tolist() == [0, 20, 20, 29]
