"""Pins of the sampling oracle: the draw follows softmax(z / T) over the top-k
candidates (the Gumbel-max identity, checked by frequency), candidate sets of
hand-made rows, greedy and k = 1 limits."""
import math

import numpy as np
import pytest

from oracle import sampling as S
from workload.sample import gumbel_noise


def test_hand_computed_distribution():
    # z = [2, 1, 0, -1], top 2, T = 1: p = (e^2, e^1) / (e^2 + e^1)
    p = S.distribution(np.array([2.0, 1.0, 0.0, -1.0], np.float32), 2, 1.0)
    e2, e1 = math.exp(2.0), math.exp(1.0)
    assert np.allclose(p, [e2 / (e1 + e2), e1 / (e1 + e2), 0.0, 0.0], atol=1e-15)
    # T = 2 halves the logits first
    p = S.distribution(np.array([2.0, 1.0, 0.0, -1.0], np.float32), 0, 2.0)
    w = np.exp(np.array([1.0, 0.5, 0.0, -0.5]))
    assert np.allclose(p, w / w.sum(), atol=1e-15)


@pytest.mark.parametrize("k,t", [(4, 0.7), (0, 1.0), (2, 2.5), (6, 0.3)])
def test_draws_follow_softmax_over_candidates(k, t):
    z = np.array([1.2, -0.4, 2.0, 0.3, 2.0, -3.0], np.float32)
    n = 200_000
    g = gumbel_noise(np.random.Generator(np.random.PCG64(1)), (n, z.size))
    tok = S.topk_sample(np.broadcast_to(z, (n, z.size)), g, k, t)
    freq = np.bincount(tok, minlength=z.size) / n
    p = S.distribution(z, k, t)
    assert np.all(freq[p == 0] == 0)
    assert np.all(np.abs(freq - p) <= 5 * np.sqrt(p * (1 - p) / n) + 1e-12)


def test_candidates_keep_ties_and_order_signed_zeros():
    z = np.array([1.0, 3.0, 3.0, 2.0, 3.0], np.float32)
    assert S.candidates(z, 2).tolist() == [False, True, True, False, True]
    assert S.candidates(z, 4).tolist() == [False, True, True, True, True]
    assert S.candidates(z, 0).all() and S.candidates(z, 5).all() and S.candidates(z, 9).all()
    assert S.candidates(np.array([0.0, -0.0, -1.0], np.float32), 1).tolist() == [True, False, False]
    assert S.candidates(np.array([-np.inf, 0.5, -np.inf], np.float32), 2).tolist() == [True, True, True]


def test_candidates_match_brute_force():
    rng = np.random.Generator(np.random.PCG64(2))
    for _ in range(200):
        v = int(rng.integers(1, 12))
        z = rng.integers(-3, 3, size=v).astype(np.float32)  # many ties
        k = int(rng.integers(0, v + 2))
        order = sorted(range(v), key=lambda i: -float(z[i]))
        if 0 < k < v:
            kth = float(z[order[k - 1]])
            want = [float(x) >= kth for x in z]
        else:
            want = [True] * v
        assert S.candidates(z, k).tolist() == want


def test_greedy_and_single_candidate():
    z = np.array([0.5, 4.0, 4.0, -1.0], np.float32)
    g = np.array([9.0, -5.0, 0.0, 30.0], np.float32)
    assert S.sample_row(z, g, 0, 0.0) == 1          # T <= 0: first maximum, noise ignored
    assert S.sample_row(z, g, 1, 0.9) == 2          # k = 1 keeps both tied 4.0 entries; noise decides
    z2 = np.array([0.5, 4.0, 3.0, -1.0], np.float32)
    for seed in range(20):
        g2 = gumbel_noise(np.random.Generator(np.random.PCG64(seed)), (4,))
        assert S.sample_row(z2, g2, 1, 1.3) == 1    # a single candidate is always taken
