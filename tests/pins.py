"""Pins of the CPU oracle: results fixed by the mathematics of the recurrence,
not by the oracle itself.  Each check takes an object with `prefill` and
`decode` (the oracle, or a deliberately broken build of it) and raises
AssertionError when the object disagrees with the pinned value.

The recurrence (per-channel-decay KDA, page "spike(kimi-linear): chunk_kda
prefill AOT port", section Delivered): S_t = (I - b_t k_t k_t^T) Diag(exp g_t)
S_{t-1} + b_t k_t v_t^T and o_t = scale S_t^T q_t.
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rel(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (nb if nb > 0 else 1.0)


def _rand_case(rng, T, H, dk, dv, h0=True, strong=1.0):
    q = rng.standard_normal((T, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    g = -strong * np.logaddexp(0.0, rng.standard_normal((T, H, dk)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    s0 = rng.standard_normal((1, H, dk, dv)) * 0.5 if h0 else None
    return q, k, v, g, beta, s0


def golden_scalar(orc):
    """Hand-worked dk = dv = 1 example (tests/golden/scalar_kda.json)."""
    fx = json.load(open(os.path.join(GOLDEN, "scalar_kda.json")))
    sh = lambda x: np.asarray(x, dtype=np.float64).reshape(-1, 1, 1)  # noqa: E731
    o, ht = orc.prefill(sh(fx["q"]), sh(fx["k"]), sh(fx["v"]), np.log(sh(fx["decay"])),
                        np.asarray(fx["beta"]).reshape(-1, 1),
                        np.full((1, 1, 1, 1), fx["h0"]), None, fx["scale"])
    assert np.allclose(o.ravel(), fx["o"], rtol=1e-14, atol=0), (o.ravel(), fx["o"])
    assert abs(ht.ravel()[0] - fx["hT"]) <= 1e-14 * abs(fx["hT"]), (ht.ravel(), fx["hT"])


def golden_two_channel(orc):
    """Hand-worked dk = 2, dv = 1 example with per-channel decay
    (tests/golden/two_channel_kda.json)."""
    fx = json.load(open(os.path.join(GOLDEN, "two_channel_kda.json")))
    q = np.asarray(fx["q"])[:, None, :]
    k = np.asarray(fx["k"])[:, None, :]
    v = np.asarray(fx["v"])[:, None, :]
    g = np.log(np.asarray(fx["decay"]))[:, None, :]
    beta = np.asarray(fx["beta"])[:, None]
    h0 = np.asarray(fx["h0"])[None, None]
    o, ht = orc.prefill(q, k, v, g, beta, h0, None, fx["scale"])
    assert np.allclose(o[:, 0, :], fx["o"], rtol=1e-14, atol=1e-15), o
    assert np.allclose(ht[0, 0], fx["hT"], rtol=1e-14, atol=1e-15), ht


def p1_beta_zero(orc):
    """beta = 0: no writes, so the state is the decayed initial state:
    S_t = diag(exp(G_t)) h0 with G_t the running sum of g; o_t = scale (exp(G_t) * q_t)^T h0."""
    rng = np.random.default_rng(101)
    T, H, dk, dv = 37, 3, 6, 5
    q, k, v, g, _, h0 = _rand_case(rng, T, H, dk, dv)
    beta = np.zeros((T, H))
    scale = 0.7
    o, ht = orc.prefill(q, k, v, g, beta, h0, None, scale)
    G = np.cumsum(g, axis=0)  # [T, H, dk]
    o_ref = scale * np.einsum("thc,hcj->thj", np.exp(G) * q, h0[0])
    ht_ref = np.exp(G[-1])[:, :, None] * h0[0]
    assert _rel(o, o_ref) < 1e-13, _rel(o, o_ref)
    assert _rel(ht[0], ht_ref) < 1e-13, _rel(ht[0], ht_ref)


def p2_basis_keys(orc):
    """Keys are distinct standard basis vectors and h0 = 0: the erase term is
    always zero and the result is per-channel gated linear attention,
    o_t = scale sum_{s<=t} beta_s q_t[c_s] exp(G_t[c_s] - G_s[c_s]) v_s."""
    rng = np.random.default_rng(202)
    H, dk, dv = 2, 9, 4
    T = 7
    q, _, v, g, beta, _ = _rand_case(rng, T, H, dk, dv, h0=False)
    chans = np.stack([rng.permutation(dk)[:T] for _ in range(H)], axis=1)  # [T, H]
    k = np.zeros((T, H, dk))
    for t in range(T):
        for h in range(H):
            k[t, h, chans[t, h]] = 1.0
    scale = 1.3
    o, ht = orc.prefill(q, k, v, g, beta, None, None, scale)
    G = np.cumsum(g, axis=0)
    o_ref = np.zeros((T, H, dv))
    for t in range(T):
        for h in range(H):
            for s in range(t + 1):
                c = chans[s, h]
                o_ref[t, h] += beta[s, h] * q[t, h, c] * np.exp(G[t, h, c] - G[s, h, c]) * v[s, h]
    o_ref *= scale
    assert _rel(o, o_ref) < 1e-13, _rel(o, o_ref)
    ht_ref = np.zeros((H, dk, dv))
    for h in range(H):
        for s in range(T):
            c = chans[s, h]
            ht_ref[h, c] = beta[s, h] * np.exp(G[-1, h, c] - G[s, h, c]) * v[s, h]
    assert _rel(ht[0], ht_ref) < 1e-13, _rel(ht[0], ht_ref)


def p3_exact_overwrite(orc):
    """g = 0, beta = 1 and keys from an orthonormal basis {e_j}: a write at key
    e_j replaces what is stored there, so S_t^T e_j is the last value written at
    e_j (h0^T e_j if none) and o_t = scale sum_j (q_t . e_j) value_j(t)."""
    rng = np.random.default_rng(303)
    H, dk, dv, T = 2, 6, 3, 25
    basis = [np.linalg.qr(rng.standard_normal((dk, dk)))[0] for _ in range(H)]  # columns
    idx = rng.integers(0, dk, size=(T, H))
    k = np.zeros((T, H, dk))
    for t in range(T):
        for h in range(H):
            k[t, h] = basis[h][:, idx[t, h]]
    q = rng.standard_normal((T, H, dk))
    v = rng.standard_normal((T, H, dv))
    g = np.zeros((T, H, dk))
    beta = np.ones((T, H))
    h0 = rng.standard_normal((1, H, dk, dv))
    scale = 0.9
    o, ht = orc.prefill(q, k, v, g, beta, h0, None, scale)
    for h in range(H):
        B = basis[h]
        val = B.T @ h0[0, h]  # [dk, dv]: value stored at each basis key
        for t in range(T):
            val[idx[t, h]] = v[t, h]
            o_ref = scale * (B.T @ q[t, h]) @ val
            assert _rel(o[t, h], o_ref) < 1e-12, (t, h, _rel(o[t, h], o_ref))
        S_ref = B @ val
        assert _rel(ht[0, h], S_ref) < 1e-12, (h, _rel(ht[0, h], S_ref))


def p5_prefill_then_decode(orc):
    """Prefill of T1 tokens, then T2 single-token decode steps from the carried
    state, equals one prefill of T1 + T2 tokens (bitwise: same operation order)."""
    rng = np.random.default_rng(505)
    T1, T2, H, dk, dv = 11, 6, 3, 5, 4
    q, k, v, g, beta, h0 = _rand_case(rng, T1 + T2, H, dk, dv)
    o_full, ht_full = orc.prefill(q, k, v, g, beta, h0, None, 0.8)
    o1, st = orc.prefill(q[:T1], k[:T1], v[:T1], g[:T1], beta[:T1], h0, None, 0.8)
    outs = [o1]
    for t in range(T1, T1 + T2):
        o_t, st = orc.decode(st, q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1],
                             beta[t:t + 1], 0.8)
        outs.append(o_t)
    assert np.array_equal(np.concatenate(outs, axis=0), o_full)
    assert np.array_equal(st, ht_full)


def p6_varlen_is_separate(orc):
    """A packed batch of sequences equals running each sequence alone from its
    own initial state (bitwise), including an empty sequence (hT = h0)."""
    rng = np.random.default_rng(606)
    lens = [5, 0, 9, 1]
    H, dk, dv = 2, 4, 3
    T = sum(lens)
    q, k, v, g, beta, _ = _rand_case(rng, T, H, dk, dv, h0=False)
    h0 = rng.standard_normal((len(lens), H, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, ht = orc.prefill(q, k, v, g, beta, h0, cu, 0.6)
    for n in range(len(lens)):
        s, e = cu[n], cu[n + 1]
        o_n, ht_n = orc.prefill(q[s:e], k[s:e], v[s:e], g[s:e], beta[s:e], h0[n:n + 1], None,
                                0.6)
        assert np.array_equal(o[s:e], o_n)
        assert np.array_equal(ht[n], ht_n[0])
    assert np.array_equal(ht[1], h0[1])


def p7_brute_force(orc):
    """Explicit matrix products on tiny sizes: with A_s = (I - b_s k_s k_s^T)
    diag(exp(g_s)), S_t = A_t...A_1 h0 + sum_{s<=t} A_t...A_{s+1} b_s k_s v_s^T,
    built as dense matrices; o_t = scale S_t^T q_t."""
    rng = np.random.default_rng(707)
    for (T, dk, dv) in [(12, 4, 3), (9, 3, 4), (1, 2, 2)]:
        H = 2
        q, k, v, g, beta, h0 = _rand_case(rng, T, H, dk, dv)
        scale = 1.1
        o, ht = orc.prefill(q, k, v, g, beta, h0, None, scale)
        for h in range(H):
            A = [(np.eye(dk) - beta[s, h] * np.outer(k[s, h], k[s, h])) @ np.diag(np.exp(g[s, h]))
                 for s in range(T)]
            for t in range(T):
                prod_all = np.eye(dk)
                for s in range(t + 1):
                    prod_all = A[s] @ prod_all
                S = prod_all @ h0[0, h]
                for s in range(t + 1):
                    M = np.eye(dk)
                    for r in range(s + 1, t + 1):
                        M = A[r] @ M
                    S = S + M @ (beta[s, h] * np.outer(k[s, h], v[s, h]))
                o_ref = scale * S.T @ q[t, h]
                assert _rel(o[t, h], o_ref) < 1e-13, (T, t, h, _rel(o[t, h], o_ref))
            assert _rel(ht[0, h], S) < 1e-13


def p8_scalar_closed_form_decode(orc):
    """The decode entry point on the scalar golden example reproduces the
    hand-worked outputs step by step."""
    fx = json.load(open(os.path.join(GOLDEN, "scalar_kda.json")))
    st = np.full((1, 1, 1, 1), fx["h0"])
    for t in range(3):
        one = lambda x: np.full((1, 1, 1), x[t])  # noqa: E731
        o, st = orc.decode(st, one(fx["q"]), one(fx["k"]), one(fx["v"]),
                           np.log(one(fx["decay"])), np.full((1, 1), fx["beta"][t]),
                           fx["scale"])
        assert abs(o.ravel()[0] - fx["o"][t]) <= 1e-14 * abs(fx["o"][t]), (t, o)
    assert abs(st.ravel()[0] - fx["hT"]) <= 1e-14 * abs(fx["hT"])


def p10_linearity(orc):
    """For fixed q, k, g, beta the map (v, h0) -> (o, hT) is linear."""
    rng = np.random.default_rng(1010)
    T, H, dk, dv = 20, 2, 5, 3
    q, k, v1, g, beta, h01 = _rand_case(rng, T, H, dk, dv)
    v2 = rng.standard_normal(v1.shape)
    h02 = rng.standard_normal(h01.shape)
    a, b = 0.75, -1.5
    o1, s1 = orc.prefill(q, k, v1, g, beta, h01, None, 0.5)
    o2, s2 = orc.prefill(q, k, v2, g, beta, h02, None, 0.5)
    o3, s3 = orc.prefill(q, k, a * v1 + b * v2, g, beta, a * h01 + b * h02, None, 0.5)
    assert _rel(o3, a * o1 + b * o2) < 1e-12
    assert _rel(s3, a * s1 + b * s2) < 1e-12


def p11_head_permutation(orc):
    """Heads are independent: permuting the heads of every input permutes the
    outputs (bitwise)."""
    rng = np.random.default_rng(1111)
    T, H, dk, dv = 15, 5, 4, 4
    q, k, v, g, beta, h0 = _rand_case(rng, T, H, dk, dv)
    perm = rng.permutation(H)
    o, ht = orc.prefill(q, k, v, g, beta, h0, None, 0.5)
    op, htp = orc.prefill(q[:, perm], k[:, perm], v[:, perm], g[:, perm], beta[:, perm],
                          h0[:, perm], None, 0.5)
    assert np.array_equal(op, o[:, perm])
    assert np.array_equal(htp, ht[:, perm])


def p12_contraction_bound(orc):
    """With |k| = 1, beta in [0, 1] and g <= 0 one step satisfies
    |S_t|_F <= |S_{t-1}|_F + beta_t |v_t|: (I - b k k^T) and Diag(exp g) are
    contractions.  Checked step by step through the decode entry point."""
    rng = np.random.default_rng(1212)
    T, H, dk, dv = 40, 3, 6, 5
    q, k, v, g, beta, h0 = _rand_case(rng, T, H, dk, dv)
    st = h0 * 4.0
    for t in range(T):
        prev = np.linalg.norm(st[0], axis=(1, 2))
        _, st = orc.decode(st, q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], beta[t:t + 1],
                           0.5)
        now = np.linalg.norm(st[0], axis=(1, 2))
        bound = prev + beta[t] * np.linalg.norm(v[t], axis=-1)
        assert np.all(now <= bound * (1 + 1e-12)), (t, now, bound)


def p12b_erase_shrinks(orc):
    """A write with beta = 1 and v equal to what is stored at k leaves the state
    unchanged (g = 0): the erase removes exactly the stored value."""
    rng = np.random.default_rng(1213)
    H, dk, dv = 2, 5, 3
    st = rng.standard_normal((1, H, dk, dv))
    k = rng.standard_normal((1, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = np.einsum("hij,hi->hj", st[0], k[0])[None]
    q = rng.standard_normal((1, H, dk))
    o, st2 = orc.decode(st, q, k, v, np.zeros((1, H, dk)), np.ones((1, H)), 1.0)
    assert _rel(st2, st) < 1e-14
    assert _rel(o[0], np.einsum("hij,hi->hj", st[0], q[0])) < 1e-14


ALL_PINS = [golden_scalar, golden_two_channel, p1_beta_zero, p2_basis_keys, p3_exact_overwrite,
            p5_prefill_then_decode, p6_varlen_is_separate, p7_brute_force,
            p8_scalar_closed_form_decode, p10_linearity, p11_head_permutation,
            p12_contraction_bound, p12b_erase_shrinks]
