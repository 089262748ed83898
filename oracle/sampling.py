"""CPU oracle for the sampled decode path.

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never calls it.

"Model-agnostic LLM inference", section "Sampling": with a temperature above zero
every token, the first one included, is drawn from the model's own distribution
through the chain repetition / presence / frequency penalties -> temperature ->
top-k -> min-p -> top-p -> seeded weighted draw; the same prompt, parameters and seed
reproduce the same tokens, and top-k = 1 reproduces the greedy sequence at any
temperature.  The pages name the steps but not their formulas; the readings taken
(each also listed in the design notes):

* counts c_t: occurrences of token t in the sequence so far (prompt and generated);
  for every t with c_t > 0 the repetition penalty r divides a positive logit and
  multiplies a non-positive one, then presence + frequency * c_t is subtracted;
* temperature T divides the penalized logits;
* top-k keeps the k largest (equal values: the lower token id first);
* min-p keeps the candidates whose probability is at least min_p times the largest;
* top-p keeps the shortest prefix, in that order, whose probability mass reaches
  top_p of what min-p left (at least one token);
* the draw: u in [0, 1) from Philox4x64-10 (Salmon et al., "Parallel random numbers:
  as easy as 1, 2, 3", SC 2011) with key (seed, 0) and counter (n, 0, 0, 0), where n
  counts the tokens already drawn for the sequence; u is the top 24 bits of the first
  output word times 2^-24.  The drawn token is the first candidate, in the order above,
  whose cumulative weight exceeds u times the kept weight.

Arithmetic is float64; the Philox words are exact integers.
"""
from __future__ import annotations

import numpy as np

__all__ = ["philox4x64", "draw_uniform", "penalize", "sample_token", "SamplingParams"]

_M0, _M1 = 0xD2E7470EE14C6C93, 0xCA5A826395121157      # Philox4x64 round multipliers
_W0, _W1 = 0x9E3779B97F4A7C15, 0xBB67AE8584CAA73B      # Weyl key increments
_MASK = (1 << 64) - 1


def philox4x64(counter, key, rounds: int = 10):
    """Philox4x64-R: four 64-bit counter words and two key words in, four words out.
    Each round multiplies words 0 and 2 by the two constants, crosses the high halves
    with words 1 and 3 and the key, and the key advances by the Weyl constants."""
    x0, x1, x2, x3 = (int(v) & _MASK for v in counter)
    k0, k1 = (int(v) & _MASK for v in key)
    for _ in range(rounds):
        p0, p1 = _M0 * x0, _M1 * x2
        x0, x1, x2, x3 = ((p1 >> 64) ^ x1 ^ k0) & _MASK, p1 & _MASK, ((p0 >> 64) ^ x3 ^ k1) & _MASK, p0 & _MASK
        k0, k1 = (k0 + _W0) & _MASK, (k1 + _W1) & _MASK
    return x0, x1, x2, x3


def draw_uniform(seed: int, n: int) -> float:
    """u in [0, 1) for the n-th draw of a sequence seeded ``seed`` (a multiple of 2^-24)."""
    w = philox4x64((n, 0, 0, 0), (seed, 0))[0]
    return (w >> 40) * 2.0 ** -24


class SamplingParams:
    def __init__(self, temperature=1.0, top_k=40, min_p=0.0, top_p=1.0, repeat_penalty=1.0,
                 presence_penalty=0.0, frequency_penalty=0.0):
        self.temperature, self.top_k, self.min_p, self.top_p = temperature, top_k, min_p, top_p
        self.repeat_penalty = repeat_penalty
        self.presence_penalty, self.frequency_penalty = presence_penalty, frequency_penalty


def penalize(logits, counts, p: SamplingParams) -> np.ndarray:
    z = np.asarray(logits, dtype=np.float64).copy()
    c = np.asarray(counts)
    seen = c > 0
    z[seen] = np.where(z[seen] > 0, z[seen] / p.repeat_penalty, z[seen] * p.repeat_penalty)
    z[seen] -= p.presence_penalty + p.frequency_penalty * c[seen]
    return z


def sample_token(logits, counts, p: SamplingParams, u: float, detail: bool = False):
    """The token drawn from one logits row with uniform u (and, with ``detail``, the
    candidate order, their weights and how many each filter kept)."""
    z = penalize(logits, counts, p) / p.temperature
    order = np.argsort(-z, kind="stable")[: p.top_k]          # top-k, lower id first on ties
    zs = z[order]
    w = np.exp(zs - zs[0])                                      # probabilities times a constant
    n_minp = int(np.count_nonzero(w >= p.min_p))                # non-increasing: a prefix
    cum = np.cumsum(w[:n_minp])
    n_topp = int(np.searchsorted(cum, p.top_p * cum[-1], side="left")) + 1
    n_topp = min(n_topp, n_minp)
    t = u * cum[n_topp - 1]
    i = int(np.searchsorted(cum[:n_topp], t, side="right"))    # first cumulative weight > t
    tok = int(order[min(i, n_topp - 1)])
    if not detail:
        return tok
    return tok, {"order": order, "z": zs, "w": w, "n_minp": n_minp, "n_topp": n_topp,
                 "cum": cum, "t": t, "pick": i}
