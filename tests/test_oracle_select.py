"""Pins for the oracle's token and key selection (CPU only).

Page "FlashLoop: Fast and Memory-Efficient Looped Transformers via Lazy
Updates", section "FlashLoop combines three kinds of savings", paragraphs 1-2
(rank tokens by hidden-state change; choose keys from previous-loop
statistics).
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import token_scores, topk_ascending, select_keys


def brute_topk(scores, k):
    order = sorted(range(len(scores)), key=lambda i: (-float(scores[i]), i))
    return sorted(order[:k])


@pytest.mark.parametrize("seed", range(8))
def test_topk_matches_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 300))
    scores = rng.integers(0, 6, n).astype(np.float64)          # many exact ties
    for k in {0, 1, n // 3, n // 2, n}:
        assert topk_ascending(scores, k).tolist() == brute_topk(scores, k)


def test_topk_special_cases():
    s = np.full(50, 3.25)
    assert topk_ascending(s, 7).tolist() == list(range(7))
    assert topk_ascending(s, 0).tolist() == []
    assert topk_ascending(s, 50).tolist() == list(range(50))
    # -0.0 and +0.0 are the same score: the lower index wins
    z = np.array([0.0, -0.0, 0.0, 1.0])
    z[0] = -0.0
    assert topk_ascending(z, 2).tolist() == [0, 3]
    f32 = np.array([1e-45, 0.0, 5e-45], np.float32)           # float32 subnormals order
    assert topk_ascending(f32, 1).tolist() == [2]
    with pytest.raises(ValueError):
        topk_ascending(np.array([1.0, np.nan]), 1)


def test_select_keys_per_head():
    rng = np.random.default_rng(3)
    c = rng.random((4, 64))
    keys = select_keys(c, 7)
    assert keys.shape == (4, 7)
    for h in range(4):
        assert keys[h].tolist() == brute_topk(c[h], 7)


def test_token_scores_closed_form_and_carry():
    rng = np.random.default_rng(0)
    n, d = 40, 96
    prev = rng.standard_normal((n, d)).astype(np.float32)
    cur = prev.copy()
    cval = np.float32(0.375)                                   # exact binary fraction
    cur[5] = prev[5] + cval                                     # every element moved by c
    u = token_scores(cur, prev)
    # exact: each difference is c up to float32 rounding of prev+c; recompute exactly
    diff5 = [Fraction(float(a)) - Fraction(float(b)) for a, b in zip(cur[5], prev[5])]
    exact = sum(x * x for x in diff5)
    assert abs(u[5] - float(exact)) <= 1e-15 * float(exact)
    assert abs(u[5] - d * 0.375 ** 2) < 1e-5 * d * 0.375 ** 2
    # carried rows (unchanged) score exactly zero
    others = np.delete(np.arange(n), 5)
    assert np.all(u[others] == 0.0)


def test_token_scores_match_exact_sum():
    rng = np.random.default_rng(1)
    a = rng.standard_normal((16, 512)).astype(np.float32)
    b = rng.standard_normal((16, 512)).astype(np.float32)
    u = token_scores(a, b)
    for i in range(16):
        exact = math.fsum((float(x) - float(y)) ** 2 for x, y in zip(a[i], b[i]))
        assert abs(u[i] - exact) <= 4e-15 * exact


def test_nesting_after_lazy_loop():
    """Rows not recomputed score 0, so a non-increasing schedule nests (I9, I10)."""
    rng = np.random.default_rng(2)
    n, d = 100, 32
    h0 = rng.standard_normal((n, d)).astype(np.float32)
    h1 = h0 + rng.standard_normal((n, d)).astype(np.float32)
    a2 = topk_ascending(token_scores(h1, h0), 30)
    h2 = h1.copy()
    h2[a2] = h1[a2] + 0.1 * rng.standard_normal((30, d)).astype(np.float32)
    u3 = token_scores(h2, h1)
    assert np.all(u3[np.setdiff1d(np.arange(n), a2)] == 0.0)
    a3 = topk_ascending(u3, 20)
    assert set(a3.tolist()) <= set(a2.tolist())
