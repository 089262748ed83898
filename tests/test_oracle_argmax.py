"""Pins of the oracle's greedy arg-max rule (CPU only).

Greedy decoding takes the arg-max of the step's logits ("Model-agnostic LLM inference",
section "Notes": greedy by default).  The pages do not say which index wins a tie; the
reading taken here is the lowest index, with -0.0 equal to +0.0, and a NaN logit is an
error.  The cases are worked by hand, so a rule that returns the last tied index, compares
signed zeros by their bits, or lets a NaN through fails one of them.
"""
import numpy as np
import pytest

from oracle import greedy_argmax


@pytest.mark.parametrize("logits,want", [
    ([1.0, 3.0, 3.0, 2.0], 1),                  # a tie at the top: the lower index
    ([5.0, 4.0, 5.0, 5.0], 0),
    ([-1.0, -0.0, 0.0, -2.0], 1),               # -0.0 and +0.0 tie: the lower index
    ([-1.0, 0.0, -0.0, -2.0], 1),
    ([-3.0, -0.0, -1.0], 1),                    # -0.0 is the maximum here
    ([np.inf, 1.0, np.inf], 0),                 # infinities tie too
    ([-np.inf, -np.inf, -7.5], 2),
    ([2.0], 0),
])
def test_lowest_index_among_equal_maxima(logits, want):
    assert greedy_argmax(np.asarray(logits, dtype=np.float32)) == want
    assert greedy_argmax(np.asarray(logits, dtype=np.float64)) == want


def test_planted_ties_in_a_full_vocabulary_row():
    """151,936 logits with the maximum planted at three indices: the first one wins, and
    one fp32 ulp below the maximum does not count as a tie."""
    rng = np.random.default_rng(11)
    v = rng.standard_normal(151936).astype(np.float32)
    top = np.float32(9.0)
    for i in (151935, 77777, 4242):
        v[i] = top
    v[10] = np.nextafter(top, np.float32(0))      # just below: not a tie
    assert greedy_argmax(v) == 4242
    v[4242] = np.nextafter(top, np.float32(0))
    assert greedy_argmax(v) == 77777


def test_nan_is_an_error():
    with pytest.raises(FloatingPointError):
        greedy_argmax(np.array([1.0, np.nan, 0.5], dtype=np.float32))
    with pytest.raises(FloatingPointError):
        greedy_argmax(np.array([np.nan], dtype=np.float32))
