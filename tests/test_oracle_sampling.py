"""Pins of the sampling oracle ("Model-agnostic LLM inference", section "Sampling")
against things other than itself: numpy's Philox4x64-10 (run as a library), closed
forms of the softmax CDF, hand-worked filter and penalty cases, and the pages' stated
properties (same seed, same tokens; top-k = 1 is greedy at any temperature)."""
import numpy as np
import pytest

from oracle.sampling import SamplingParams, draw_uniform, penalize, philox4x64, sample_token


@pytest.mark.parametrize("key,ctr", [((5, 7), 0), ((0, 0), 0), ((2 ** 64 - 1, 3), 41),
                                     ((123456789, 2 ** 63), 2 ** 40)])
def test_philox_matches_numpy(key, ctr):
    # numpy advances the counter before each block of four words
    bg = np.random.Philox(key=np.array(key, dtype=np.uint64),
                          counter=np.array([ctr, 0, 0, 0], dtype=np.uint64))
    got = [int(v) for v in bg.random_raw(8)]
    assert got[:4] == list(philox4x64((ctr + 1, 0, 0, 0), key))
    assert got[4:] == list(philox4x64((ctr + 2, 0, 0, 0), key))


def test_uniform_draws_are_24_bit_and_uniform():
    us = np.array([draw_uniform(99, n) for n in range(20000)])
    assert np.all((us >= 0) & (us < 1))
    assert np.all(us * 2 ** 24 == np.floor(us * 2 ** 24))
    hist = np.histogram(us, bins=20, range=(0, 1))[0]
    chi2 = np.sum((hist - 1000.0) ** 2 / 1000.0)
    assert chi2 < 45  # 19 degrees of freedom, p ~ 1e-3
    assert draw_uniform(99, 5) == draw_uniform(99, 5) != draw_uniform(100, 5)


def _softmax(x):
    e = np.exp(np.asarray(x, np.float64) - np.max(x))
    return e / e.sum()


def test_full_vocabulary_draw_inverts_the_softmax_cdf():
    rng = np.random.default_rng(0)
    logits = rng.normal(size=6)
    p = SamplingParams(temperature=1.0, top_k=6)
    probs = _softmax(logits)
    order = np.argsort(-logits, kind="stable")
    edges = np.cumsum(probs[order])
    for k in range(4096):
        u = (k + 0.5) / 4096
        if np.min(np.abs(edges - u)) < 1e-9:
            continue
        want = order[int(np.searchsorted(edges, u, side="right"))]
        assert sample_token(logits, np.zeros(6), p, u) == want


def test_seeded_draws_follow_the_tempered_distribution():
    logits = np.array([0.3, -1.0, 1.2, 0.0])
    p = SamplingParams(temperature=0.7, top_k=4)
    n = 20000
    toks = [sample_token(logits, np.zeros(4), p, draw_uniform(7, i)) for i in range(n)]
    freq = np.bincount(toks, minlength=4) / n
    want = _softmax(logits / 0.7)
    assert np.all(np.abs(freq - want) < 4 * np.sqrt(want * (1 - want) / n) + 1e-3)


@pytest.mark.parametrize("T", [0.1, 0.8, 5.0])
def test_top_k_one_is_greedy_at_any_temperature(T):
    rng = np.random.default_rng(1)
    for _ in range(20):
        logits = rng.normal(size=50)
        counts = rng.integers(0, 3, size=50)
        p = SamplingParams(temperature=T, top_k=1, repeat_penalty=1.3, presence_penalty=0.2,
                           frequency_penalty=0.1)
        want = int(np.argmax(penalize(logits, counts, p)))
        for u in (0.0, 0.5, 1 - 2 ** -24):
            assert sample_token(logits, counts, p, u) == want


def test_top_k_ties_go_to_the_lower_id():
    p = SamplingParams(top_k=1)
    assert sample_token([1.0, 3.0, 3.0, 2.0], np.zeros(4), p, 0.9) == 1
    p = SamplingParams(top_k=2)
    toks = {sample_token([1.0, 3.0, 3.0, 3.0], np.zeros(4), p, u) for u in np.linspace(0, 0.999, 50)}
    assert toks == {1, 2}


def test_min_p_drops_the_unlikely_tail():
    probs = np.array([0.4, 0.25, 0.2, 0.1, 0.05])
    logits = np.log(probs)
    p = SamplingParams(top_k=5, min_p=0.5)     # keeps p >= 0.2: tokens 0, 1, 2
    toks = {sample_token(logits, np.zeros(5), p, u) for u in np.linspace(0, 0.9999, 400)}
    assert toks == {0, 1, 2}
    # the kept mass is renormalized: token 0 wins below 0.4 / 0.85 of the unit interval
    assert sample_token(logits, np.zeros(5), p, 0.4 / 0.85 - 1e-6) == 0
    assert sample_token(logits, np.zeros(5), p, 0.4 / 0.85 + 1e-6) == 1


def test_top_p_keeps_the_shortest_prefix_reaching_the_mass():
    logits = np.log([0.5, 0.3, 0.15, 0.05])
    p = SamplingParams(top_k=4, top_p=0.79)     # 0.5 + 0.3 reaches 0.79; 0.5 alone does not
    assert {sample_token(logits, np.zeros(4), p, u) for u in np.linspace(0, 0.9999, 400)} == {0, 1}
    assert sample_token(logits, np.zeros(4), p, 0.62) == 0   # 0.62 * 0.8 = 0.496 < 0.5
    assert sample_token(logits, np.zeros(4), p, 0.63) == 1   # 0.504 > 0.5
    p = SamplingParams(top_k=4, top_p=0.81)
    assert {sample_token(logits, np.zeros(4), p, u) for u in np.linspace(0, 0.9999, 400)} == {0, 1, 2}
    p = SamplingParams(top_k=4, top_p=0.01)     # at least one token
    assert {sample_token(logits, np.zeros(4), p, u) for u in (0.0, 0.99)} == {0}


def test_penalties_hand_worked():
    p = SamplingParams(repeat_penalty=2.0, presence_penalty=0.5, frequency_penalty=0.1)
    z = penalize([2.0, -2.0, 1.0, 0.5], [1, 2, 0, 3], p)
    np.testing.assert_allclose(z, [2 / 2 - 0.5 - 0.1, -2 * 2 - 0.5 - 0.2, 1.0, 0.5 / 2 - 0.5 - 0.3])
