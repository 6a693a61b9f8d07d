"""Pins of the fp64 Kimi gate activation (oracle/gate.py) against facts that
do not come from the oracle itself: closed forms of softplus, an independent
scalar evaluation with Python's math module, and the orientation of a_log and
dt_bias fixed by special inputs."""
import math

import numpy as np

import oracle


def test_softplus_closed_forms():
    # softplus(0) = ln 2; softplus(z) - softplus(-z) = z; asymptotes
    assert oracle.softplus(np.array([0.0]))[0] == math.log(2.0)
    z = np.linspace(-40.0, 40.0, 801)
    assert np.max(np.abs(oracle.softplus(z) - oracle.softplus(-z) - z)) < 1e-13
    big = np.array([50.0, 200.0, 700.0])
    assert np.allclose(oracle.softplus(big), big + np.exp(-big), rtol=0, atol=1e-15)
    small = np.array([-50.0, -200.0, -700.0])
    assert np.allclose(oracle.softplus(small), np.exp(small), rtol=1e-12, atol=0)


def test_softplus_matches_scalar_math():
    # an independent evaluation: log1p(exp(z)) one scalar at a time, where it
    # cannot overflow
    for z in np.linspace(-30.0, 30.0, 241):
        ref = math.log1p(math.exp(float(z)))
        assert abs(oracle.softplus(np.array([z]))[0] - ref) <= 1e-15 * max(1.0, ref)


def test_gate_orientation_and_scaling():
    rng = np.random.default_rng(5)
    H, D = 3, 8
    a = rng.uniform(-3.0, 0.0, H)
    b = rng.normal(0.0, 0.5, (H, D))
    # x = -dt_bias puts every softplus at 0: g = -exp(a_log[h]) ln 2, per head
    g = oracle.kimi_gate(-np.broadcast_to(b, (4, H, D)), a, b)
    assert np.allclose(g, -np.exp(a)[None, :, None] * math.log(2.0) * np.ones((4, H, D)),
                       rtol=1e-15, atol=0)
    # a_log enters as exp(a_log): shifting it by log 2 doubles g
    x = rng.normal(size=(5, H, D))
    assert np.allclose(oracle.kimi_gate(x, a + math.log(2.0), b), 2.0 * oracle.kimi_gate(x, a, b),
                       rtol=1e-14, atol=0)
    # a decay: g < 0, decreasing in x
    g1, g2 = oracle.kimi_gate(x, a, b), oracle.kimi_gate(x + 0.1, a, b)
    assert np.all(g1 < 0) and np.all(g2 < g1)


def test_gate_matches_the_workload_recipe():
    """The synthetic workloads build g from the same formula in their own code
    (from the unrounded x); with fp32 inputs the oracle's gate reproduces that g
    up to the fp32 rounding of x, a_log and dt_bias."""
    import synth

    inp = synth.make_inputs(9, [40], 4, 32, dtype="f32", gate="kimi")
    x, a, b = inp.gate_f64()
    g = oracle.kimi_gate(x, a, b)
    assert np.max(np.abs(g - inp.g)) < 1e-5 * max(1.0, float(np.max(np.abs(g))))
