"""The CPU oracle against results the mathematics fixes (closed forms,
hand-worked examples, invariants, brute force).  No GPU."""
import numpy as np
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_decode_matches_prefill_on_batch(orc):
    """Decode over a batch of N sequences equals N one-token prefills."""
    rng = np.random.default_rng(9)
    N, H, dk, dv = 3, 2, 4, 5
    st = rng.standard_normal((N, H, dk, dv))
    q, k, v, g, beta, _ = pins._rand_case(rng, N, H, dk, dv, h0=False)
    o, st2 = orc.decode(st, q, k, v, g, beta, 0.3)
    o_p, st_p = orc.prefill(q, k, v, g, beta, st, np.arange(N + 1), 0.3)
    assert np.array_equal(o, o_p)
    assert np.array_equal(st2, st_p)


def test_oracle_rejects_bad_offsets(orc):
    q = np.zeros((4, 1, 2))
    with pytest.raises((RuntimeError, ValueError)):
        orc.prefill(q, q, q, q, np.zeros((4, 1)), None, np.array([0, 3, 2, 4]))
