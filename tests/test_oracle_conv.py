"""Pins of the fp64 causal conv (oracle/conv.py): numpy's own convolution on a
single zero-started sequence, the identity kernel, the carried-state invariant
(one pass = two passes with the taps carried), varlen = separate runs, and the
SiLU closed form."""
import math

import numpy as np

import oracle


def _case(seed, T, dim, W):
    rng = np.random.default_rng(seed)
    return (rng.normal(size=(T, dim)), rng.normal(size=(dim, W)), rng.normal(size=dim))


def test_matches_numpy_convolve():
    x, w, b = _case(1, 37, 5, 4)
    y, st = oracle.causal_conv1d(x, w, b, [0, 37], None)
    for c in range(5):
        # causal: y[t] = sum_j w[j] x[t - 3 + j]  ==  full convolution with the
        # reversed kernel, first 37 outputs
        ref = np.convolve(x[:, c], w[c, ::-1])[:37] + b[c]
        assert np.max(np.abs(y[:, c] - ref)) < 1e-12
    assert np.array_equal(st[0], x[-3:])


def test_identity_kernel_and_silu():
    x, _, b = _case(2, 20, 6, 3)
    w = np.zeros((6, 3))
    w[:, -1] = 1.0
    y, _ = oracle.causal_conv1d(x, w, b, [0, 20], None, activation="silu")
    z = x + b
    assert np.max(np.abs(y - z / (1.0 + np.exp(-z)))) < 1e-15
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    assert abs(oracle.silu(np.array([1.0]))[0] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16


def test_carried_state_equals_one_pass():
    for W in (2, 3, 4):
        x, w, b = _case(3 + W, 41, 4, W)
        rng = np.random.default_rng(W)
        st0 = rng.normal(size=(1, W - 1, 4))
        y_all, st_all = oracle.causal_conv1d(x, w, b, [0, 41], st0)
        for cut in (0, 1, 2, 17, 40, 41):
            y1, st1 = oracle.causal_conv1d(x[:cut], w, b, [0, cut], st0)
            y2, st2 = oracle.causal_conv1d(x[cut:], w, b, [0, 41 - cut], st1)
            assert np.max(np.abs(np.concatenate([y1, y2]) - y_all)) < 1e-13
            assert np.max(np.abs(st2 - st_all)) == 0.0


def test_varlen_equals_separate_runs_and_short_sequences_keep_taps():
    x, w, b = _case(7, 30, 5, 4)
    rng = np.random.default_rng(9)
    st0 = rng.normal(size=(4, 3, 5))  # [N, W - 1, dim]
    cu = [0, 12, 12, 13, 30]  # an empty and a one-token sequence
    y, st = oracle.causal_conv1d(x, w, b, cu, st0)
    for n in range(4):
        s, e = cu[n], cu[n + 1]
        yn, sn = oracle.causal_conv1d(x[s:e], w, b, [0, e - s], st0[n:n + 1])
        assert np.array_equal(y[s:e], yn)
        assert np.array_equal(st[n], sn[0])
    assert np.array_equal(st[1], st0[1])                       # empty: unchanged
    assert np.array_equal(st[2][:2], st0[2][1:])              # one token: taps shift
    assert np.array_equal(st[2][2], x[12])
