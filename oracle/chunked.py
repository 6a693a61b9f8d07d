"""fp64 chunked re-derivation of the KDA forward pass -- TEST INFRASTRUCTURE.

The pages name the chunked prefill as a pipeline of stages: a chunk-local
cumulative sum of the per-channel log-decay, a beta-scaled decayed K K^T
inside the chunk, a unit-lower-triangular solve, a recompute of W and U with
the per-key-channel decay, the inter-chunk state recurrence (delta_h), and a
GLA-style output (page "spike(kimi-linear): chunk_kda prefill AOT port",
commit message and section Delivered).  This module takes those stages in that
order for each chunk of at most C tokens, with start state S0:

  1. G = cumulative sum of g over the chunk's tokens (per key channel; restarts
     at every chunk and every sequence start).
  2. A[r, i] = beta_r * sum_c k[r,c] k[i,c] exp(G[r,c] - G[i,c])   for i < r.
  3. T = (I + A)^-1  (unit lower triangular; forward substitution).
  4. W = T diag(beta) (K * exp(G));   U = T diag(beta) V.
  5. V_new = U - W S0.
  6. P[r, i] = sum_c q[r,c] k[i,c] exp(G[r,c] - G[i,c])   for i <= r.
  7. O = scale * ((Q * exp(G)) S0 + P V_new).
  8. S_end = diag(exp(G_last)) S0 + (K * exp(G_last - G))^T V_new.

In exact arithmetic this equals the token recurrence for any C (the step
S_r = D_r S_{r-1} + k_r u_r^T unrolled over the chunk and solved for all u_r
at once), so it is checked against the recurrence, not trusted on its own.
The exponent differences in steps 2 and 6 are formed before exp, so nothing
overflows.
"""
from __future__ import annotations

import numpy as np


def unit_lower_inverse(A: np.ndarray) -> np.ndarray:
    """(I + A)^-1 for strictly lower-triangular A, by forward substitution:
    row r of the inverse is e_r - A[r, :r] @ (rows 0..r-1 of the inverse)."""
    L = A.shape[0]
    T = np.zeros((L, L), dtype=np.float64)
    for r in range(L):
        T[r, r] = 1.0
        if r:
            T[r, :r] -= A[r, :r] @ T[:r, :r]
    return T


def _chunk(q, k, v, g, beta, S0, scale):
    """One chunk of one head.  q, k, g: [L, dk]; v: [L, dv]; beta: [L]."""
    L = q.shape[0]
    G = np.cumsum(g, axis=0)
    diff = G[:, None, :] - G[None, :, :]  # [r, i, c] = G[r,c] - G[i,c]
    strict = np.tril(np.ones((L, L), dtype=bool), -1)
    incl = np.tril(np.ones((L, L), dtype=bool), 0)
    decay_strict = np.exp(np.where(strict[:, :, None], diff, -np.inf))
    decay_incl = np.exp(np.where(incl[:, :, None], diff, -np.inf))
    A = beta[:, None] * np.einsum("rc,ic,ric->ri", k, k, decay_strict)
    T = unit_lower_inverse(A)
    W = T @ (beta[:, None] * k * np.exp(G))
    U = T @ (beta[:, None] * v)
    V_new = U - W @ S0
    P = np.einsum("rc,ic,ric->ri", q, k, decay_incl)
    O = scale * ((q * np.exp(G)) @ S0 + P @ V_new)
    G_last = G[-1]
    S_end = np.exp(G_last)[:, None] * S0 + (k * np.exp(G_last[None, :] - G)).T @ V_new
    return O, S_end


def chunked_prefill(q, k, v, g, beta, h0=None, cu_seqlens=None, scale=None, chunk=64):
    """Same signature and result as recurrent.prefill, computed chunk by chunk."""
    q, k, v, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, v, g, beta))
    T, H, dk = q.shape
    dv = v.shape[2]
    cu = np.array([0, T]) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    sc = float(dk ** -0.5) if scale is None else float(scale)
    o = np.zeros((T, H, dv))
    ht = np.zeros((N, H, dk, dv))
    for n in range(N):
        for h in range(H):
            S = np.zeros((dk, dv)) if h0 is None else np.array(h0[n, h], dtype=np.float64)
            for s in range(int(cu[n]), int(cu[n + 1]), chunk):
                e = min(s + chunk, int(cu[n + 1]))
                O, S = _chunk(q[s:e, h], k[s:e, h], v[s:e, h], g[s:e, h], beta[s:e, h], S, sc)
                o[s:e, h] = O
            ht[n, h] = S
    return o, ht
