"""Short causal depthwise convolution with carried taps, fp64 -- TEST
INFRASTRUCTURE ONLY (see the package docstring).

The pages run a short causal conv over the [q|k|v] channels before the KDA
step, as a varlen forward over a prefill and a one-token update in decode,
both carrying the last taps in a conv state (page "model(kimi_linear):
ONE-SURFACE ROW 7 -- fold Kimi-Linear onto the shared paged runner", B2:
CausalConv1dFwd (varlen) / CausalConv1dUpdate (decode) in the [q|k|v]
conv-state layout).  Reading taken here (the pages give names, not the
formula): for channel c, kernel width W, weight w[c, 0..W-1]:

    y[t, c] = act(bias[c] + sum_j w[c, j] * x[t - (W - 1) + j, c])

where a position before its sequence's start reads the carried state
state[n, i, c] = the input at position start - (W - 1) + i (oldest first, a
row of taps per position over all channels);
after the sequence the state holds its last W - 1 inputs (carried values
still among them when the sequence is shorter than W - 1).  act is the
identity or SiLU (z * sigmoid(z)).
"""
import numpy as np


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def causal_conv1d(x, weight, bias, cu_seqlens, state, activation="none"):
    """x [T, dim]; weight [dim, W]; bias [dim] or None; cu_seqlens [N + 1];
    state [N, W - 1, dim] or None (zeros).  Returns (y [T, dim], new state
    [N, W - 1, dim])."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    dim, W = w.shape
    N = len(cu_seqlens) - 1
    st = np.zeros((N, W - 1, dim)) if state is None else np.array(state, dtype=np.float64)
    b = np.zeros(dim) if bias is None else np.asarray(bias, dtype=np.float64)
    y = np.zeros_like(x)
    new = st.copy()
    for n in range(N):
        s, e = int(cu_seqlens[n]), int(cu_seqlens[n + 1])
        # the sequence's inputs preceded by its carried taps: row i of `ext` is
        # position s - (W - 1) + i
        ext = np.concatenate([st[n], x[s:e]], axis=0)
        for t in range(s, e):
            i = t - s + (W - 1)  # row of position t in ext
            acc = b.copy()
            for j in range(W):
                acc = acc + w[:, j] * ext[i - (W - 1) + j]
            y[t] = acc
        new[n] = ext[len(ext) - (W - 1):]
    if activation == "silu":
        y = silu(y)
    elif activation != "none":
        raise ValueError(activation)
    return y, new
