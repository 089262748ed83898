"""Pins for the oracle's quantizer and rounding helpers (CPU only).

Per-row int8 weights with row scales: "Model-agnostic LLM inference", section
"The quantized load cache".  The cache sizes printed in that section's table
(0.598 GB for Qwen3-0.6B-Base, 1.724 GB for Qwen3-1.7B) pin the byte layout.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import quantize_rows, bf16, packed_weight_bytes
from workloads import SHAPES

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _parse_cases():
    cases = []
    for line in open(os.path.join(GOLDEN, "quant_hand_cases.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        w, s, q = (part.split(":", 1)[1].split() for part in line.split("|"))
        cases.append((np.array([float(v) for v in w], dtype=np.float32),
                      np.float32(float(s[0])), np.array([int(v) for v in q])))
    return cases


@pytest.mark.parametrize("case", range(len(_parse_cases())))
def test_hand_worked_rows(case):
    w, s, q = _parse_cases()[case]
    qq, ss = quantize_rows(w[None, :])
    assert ss[0] == s
    np.testing.assert_array_equal(qq[0].astype(int), q)


# ---- exact rational brute force of the same rule ---------------------------------------

def _round_half_even(fr: Fraction) -> int:
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl


def _to_fp32(fr: Fraction) -> Fraction:
    """Round a rational to the nearest fp32 (ties to even); normal range only."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    assert -126 <= e <= 127
    ulp = Fraction(2) ** (e - 23)
    m = _round_half_even(a / ulp)
    return sign * m * ulp


def _quant_rational(row):
    absmax = max(abs(Fraction(float(v))) for v in row)
    s = _to_fp32(absmax / 127)
    if s == 0:
        return [0] * len(row), 0.0
    q = [max(-127, min(127, _round_half_even(_to_fp32(Fraction(float(v)) / s)))) for v in row]
    return q, float(s)


def test_matches_exact_rational_rounding():
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((24, 96)) * 0.02).astype(np.float32)
    # plant exact ties w / s = k + 1/2 in a few rows
    planted = 0
    for r in range(0, 24, 4):
        s = np.float32(np.max(np.abs(w[r])) / np.float32(127))
        for j, k in enumerate((3, -7, 12, 100)):
            cand = np.float32((k + 0.5) * np.float64(s))
            if np.float32(cand / s) == np.float32(k + 0.5) and abs(cand) < np.max(np.abs(w[r])):
                w[r, j + 1] = cand
                planted += 1
    assert planted >= 10
    q, s = quantize_rows(w)
    for r in range(w.shape[0]):
        qr, sr = _quant_rational(w[r])
        assert float(s[r]) == sr
        np.testing.assert_array_equal(q[r].astype(int), qr)


def test_ties_round_to_even_not_away():
    w = np.array([[127.0, 0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5]], dtype=np.float32)
    q, s = quantize_rows(w)
    assert s[0] == 1.0
    np.testing.assert_array_equal(q[0], [127, 0, 2, 2, 4, 0, -2, -2])


def test_invariants_and_requantization_is_exact():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((64, 256)) * 0.02).astype(np.float32)
    w[5] = 0.0
    q, s = quantize_rows(w)
    assert q.dtype == np.int8 and s.dtype == np.float32
    assert np.all(np.abs(q.astype(int)) <= 127)
    nz = s != 0
    assert np.all(np.max(np.abs(q[nz].astype(int)), axis=1) == 127)
    assert s[5] == 0 and np.all(q[5] == 0)
    deq = (q.astype(np.float32) * s[:, None]).astype(np.float32)
    q2, s2 = quantize_rows(deq)
    np.testing.assert_array_equal(s2, s)
    np.testing.assert_array_equal(q2, q)


def test_cache_footprint_matches_pages():
    # Table in "The quantized load cache": cache 0.598 GB (0.6B), 1.724 GB (1.7B)
    b06 = packed_weight_bytes(SHAPES["qwen3-0.6b"])
    b17 = packed_weight_bytes(SHAPES["qwen3-1.7b"])
    assert round(b06 / 1e9, 3) == 0.598
    assert round(b17 / 1e9, 3) == 1.724
    assert b06 == 598_230_528 and b17 == 1_723_848_192


# ---- bf16 rounding vs the library conversion ---------------------------------------------

def test_bf16_matches_torch_conversion():
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-6, 6, 20000),
        # exact ties between two bf16 neighbours
        (1.0 + np.arange(1, 256) * 2.0 ** -8).astype(np.float32),
        -(1.0 + np.arange(1, 256) * 2.0 ** -8).astype(np.float32),
        np.array([0.0, -0.0, 3.4e38, -3.4e38, 1e-40], dtype=np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(bf16(x), ref)


def test_bf16_hand_cases():
    assert bf16(np.float32(1 + 2 ** -8)) == 1.0                 # tie -> even mantissa
    assert bf16(np.float32(1 + 3 * 2 ** -8)) == 1 + 2 ** -6     # tie -> even mantissa
    assert bf16(np.float32(1 + 2 ** -8 + 2 ** -20)) == 1 + 2 ** -7
