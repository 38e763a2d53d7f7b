"""CPU tests of the GPTQ code checker (tests/_gptq_check.py): it accepts a
channel that parts at an exact rounding boundary and follows the other side
faithfully, and it rejects a wrong code anywhere after such a parting."""
import numpy as np
import pytest

import oracle
from _gptq_check import check_gptq_codes


def _tie_case():
    """Row 0 is rounded before any update reaches it.  Every channel's largest
    value is 127/128 (in the last row), so the step is 2^-7 exactly, and
    W[0, n] = (m + 1/2)/128 puts row 0's quotient exactly on a half-integer."""
    rng = np.random.default_rng(3)
    T, K, N = 160, 48, 6
    x = rng.standard_normal((T, K)).astype(np.float32)
    x[:, 1:] += 0.6 * x[:, :-1]                        # correlated inputs
    w = rng.uniform(-0.9, 0.9, (K, N)).astype(np.float32)
    w[K - 1] = 127.0 / 128.0
    w[0] = ((rng.integers(-100, 100, N) + np.float32(0.5)) / np.float32(128)).astype(np.float32)
    U, dead = oracle.gptq_factor(oracle.smoothed_act(x))
    q, ws, quot = oracle.gptq_round(w, U, dead, return_quotients=True)
    assert (ws == np.float32(2.0 ** -7)).all()
    assert (np.abs(quot[0] - np.floor(quot[0])) == 0.5).all()
    return w, U, dead, q


def _other_side(w, U, dead, q, c):
    """The codes an evaluation that rounded channel c's row-0 tie the other
    way would produce: that code forced, everything after it recomputed."""
    alt = q.copy()
    alt[c, 0] = q[c, 0] + (1 if q[c, 0] % 2 == 0 and w[0, c] > 0 else -1)
    r, _ = oracle.gptq_round(w[:, [c]], U, dead, force_codes=alt[[c]], force_rows=np.array([1]))
    alt[c] = r[0]
    return alt


def test_checker_accepts_identical_codes():
    w, U, dead, q = _tie_case()
    assert check_gptq_codes(q, w, U, dead) == 0


def test_checker_accepts_a_parting_at_a_tie_and_checks_what_follows():
    w, U, dead, q = _tie_case()
    alt = _other_side(w, U, dead, q, 2)
    assert (alt[2, 1:] != q[2, 1:]).any()       # the trajectory really moved
    assert check_gptq_codes(alt, w, U, dead) == 1


@pytest.mark.parametrize("row", [1, 5, 47])
def test_checker_rejects_a_wrong_code_after_a_tie(row):
    # the earlier check compared only each column's first difference: a
    # wrong code later in a column that had parted at a tie went unseen
    w, U, dead, q = _tie_case()
    alt = _other_side(w, U, dead, q, 2)
    alt[2, row] = alt[2, row] + (1 if alt[2, row] < 127 else -1)
    with pytest.raises(AssertionError):
        check_gptq_codes(alt, w, U, dead)


def test_checker_rejects_a_parting_away_from_a_tie():
    w, U, dead, q = _tie_case()
    bad = q.copy()
    bad[4, 3] += 1 if bad[4, 3] < 127 else -1
    with pytest.raises(AssertionError):
        check_gptq_codes(bad, w, U, dead)
