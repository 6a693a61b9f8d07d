"""The Kimi gate activation in fp64 -- TEST INFRASTRUCTURE ONLY (see the
package docstring).

The pages run the gate activation fused into the chunked forward (page
"spike(kimi-linear): chunk_kda prefill AOT port -- kernel set + pinned-config
recipe (S17)", commit message: the gate/cumsum kernel of
chunk_kda_with_fused_gate); the formula itself is the workload's Kimi-Linear
gate:

    g[t, h, c] = -exp(a_log[h]) * softplus(x[t, h, c] + dt_bias[h, c]),
    softplus(z) = log(1 + e^z).

softplus is evaluated as log(1 + e^z) = max(z, 0) + log1p(e^-|z|), which is
exact to rounding for every z (no overflow for large z, no cancellation for
very negative z).
"""
import numpy as np


def softplus(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def kimi_gate(x: np.ndarray, a_log: np.ndarray, dt_bias: np.ndarray) -> np.ndarray:
    """x [..., H, dk], a_log [H], dt_bias [H, dk] -> g [..., H, dk] (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    a_log = np.asarray(a_log, dtype=np.float64)
    dt_bias = np.asarray(dt_bias, dtype=np.float64)
    return -np.exp(a_log)[:, None] * softplus(x + dt_bias)
