"""The fp64 chunked re-derivation (oracle/chunked.py) against the token
recurrence, and its triangular solve against a library routine.  No GPU."""
import numpy as np
import pytest
import scipy.linalg

import pins
from oracle import chunked_prefill, unit_lower_inverse


@pytest.mark.parametrize("C", [1, 2, 3, 5, 16, 64, 200])
def test_chunked_equals_recurrent_any_chunk(orc, C):
    """Chunked form = recurrence for any chunk size, including chunk sizes that
    do not divide T (a partial last chunk) and strong decays."""
    rng = np.random.default_rng(44)
    T, H, dk, dv = 200, 2, 8, 6
    q, k, v, g, beta, h0 = pins._rand_case(rng, T, H, dk, dv, strong=3.0)
    o_r, s_r = orc.prefill(q, k, v, g, beta, h0, None, 0.4)
    o_c, s_c = chunked_prefill(q, k, v, g, beta, h0, None, 0.4, chunk=C)
    assert pins._rel(o_c, o_r) < 1e-11
    assert pins._rel(s_c, s_r) < 1e-11


def test_chunked_varlen(orc):
    rng = np.random.default_rng(45)
    lens = [70, 0, 64, 1, 129]
    T, H, dk, dv = sum(lens), 2, 8, 8
    q, k, v, g, beta, _ = pins._rand_case(rng, T, H, dk, dv)
    h0 = rng.standard_normal((len(lens), H, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o_r, s_r = orc.prefill(q, k, v, g, beta, h0, cu, 0.4)
    o_c, s_c = chunked_prefill(q, k, v, g, beta, h0, cu, 0.4, chunk=64)
    assert pins._rel(o_c, o_r) < 1e-11
    assert pins._rel(s_c, s_r) < 1e-11


def test_unit_lower_inverse_matches_library():
    """(I + A)^-1 by forward substitution = scipy's triangular solve."""
    rng = np.random.default_rng(46)
    for L in [1, 2, 16, 64]:
        A = np.tril(rng.standard_normal((L, L)) * 0.3, -1)
        T = unit_lower_inverse(A)
        ref = scipy.linalg.solve_triangular(np.eye(L) + A, np.eye(L), lower=True,
                                            unit_diagonal=True)
        assert np.max(np.abs(T - ref)) < 1e-13 * max(1.0, np.max(np.abs(ref)))
