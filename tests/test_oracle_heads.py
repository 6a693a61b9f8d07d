"""Pins of oracle/heads.py: the L2 normalisation on worked values (3-4-5 rows,
a zero row, row independence, scale invariance) and the key-head mapping on
an array that carries its own head index; then the grouped prefill against a
head-by-head run of the single-head oracle."""
import numpy as np

import oracle


def test_l2norm_worked_values():
    x = np.array([[3.0, 4.0], [0.0, 5.0], [0.0, 0.0]])
    y = oracle.l2norm(x, eps=0.0 + 1e-300)
    assert np.allclose(y[0], [0.6, 0.8], rtol=0, atol=1e-15)
    assert np.allclose(y[1], [0.0, 1.0], rtol=0, atol=1e-15)
    assert np.array_equal(oracle.l2norm(x)[2], [0.0, 0.0])          # zero row stays zero
    e = oracle.L2NORM_EPS
    assert abs(oracle.l2norm(x)[0, 0] - 3.0 / np.sqrt(25.0 + e)) < 1e-16
    assert e == 1e-6


def test_l2norm_rows_and_scale():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 3, 64)) * rng.uniform(0.5, 20.0, (5, 3, 1))
    y = oracle.l2norm(x)
    n2 = np.sum(x * x, axis=-1)
    # |y|^2 = s / (s + eps) per row
    assert np.max(np.abs(np.sum(y * y, -1) - n2 / (n2 + oracle.L2NORM_EPS))) < 1e-14
    assert np.max(np.abs(oracle.l2norm(7.0 * x) - y)) < 1e-8          # scale only through eps
    assert np.max(np.abs(y[:, :, :5] * np.sqrt(n2 + 1e-6)[..., None] - x[:, :, :5])) < 1e-12


def test_key_head_mapping():
    T, Hg, H, d = 3, 2, 6, 4
    x = np.broadcast_to(np.arange(Hg, dtype=np.float64)[None, :, None], (T, Hg, d))
    y = oracle.expand_key_heads(x, H)
    assert y.shape == (T, H, d)
    assert list(y[0, :, 0]) == [0, 0, 0, 1, 1, 1]                      # h -> h // (H / Hg)
    assert np.array_equal(oracle.expand_key_heads(x, Hg), x)


def test_grouped_prefill_equals_headwise_single_head():
    rng = np.random.default_rng(3)
    T, Hg, H, d = 37, 2, 4, 16
    q = oracle.l2norm(rng.standard_normal((T, Hg, d)))
    k = oracle.l2norm(rng.standard_normal((T, Hg, d)))
    v = rng.standard_normal((T, H, d))
    g = -np.log1p(np.exp(rng.standard_normal((T, H, d))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    h0 = 0.1 * rng.standard_normal((1, H, d, d))
    o, ht = oracle.prefill(oracle.expand_key_heads(q, H), oracle.expand_key_heads(k, H), v, g,
                           beta, h0, None, d ** -0.5)
    for h in range(H):
        kh = h // (H // Hg)
        o1, h1 = oracle.prefill(q[:, kh:kh + 1], k[:, kh:kh + 1], v[:, h:h + 1], g[:, h:h + 1],
                                beta[:, h:h + 1], h0[:, h:h + 1], None, d ** -0.5)
        assert np.max(np.abs(o1[:, 0] - o[:, h])) < 1e-12
        assert np.max(np.abs(h1[:, 0] - ht[:, h])) < 1e-12
