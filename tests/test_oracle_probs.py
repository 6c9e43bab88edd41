"""Pins for the oracle's attention distribution (orc_probs).

The attention distribution pi_j = exp(s_j) / sum_k exp(s_k), s_j = scale * q.k_j,
is what the precision ablation compares between formats (a stand-in for the
shared-prefix conditional KL of the news summary "Async RL squeezes context
into fewer decode steps; ...", Interpretation paragraph 2).  Pins: a closed
form worked by hand, brute force with math.fsum and no max shift, torch's
float64 softmax at scores where an unshifted exponential overflows, and the
invariants (sum 1, shift invariance, ordering).
"""
import math

import numpy as np
import pytest


def test_hand_worked_closed_form(orc):
    """D = 1, q = 1, keys ln 1 .. ln 4: weights 1, 2, 3, 4 -> 0.1, 0.2, 0.3, 0.4."""
    K = np.log(np.array([[1.0], [2.0], [3.0], [4.0]]))
    p = orc.probs(np.array([1.0]), K)
    np.testing.assert_allclose(p, [0.1, 0.2, 0.3, 0.4], rtol=1e-14, atol=0)
    # the softmax scale multiplies the score: scale 2 squares the weights (1, 4, 9, 16)
    p2 = orc.probs(np.array([1.0]), K, sm_scale=2.0)
    np.testing.assert_allclose(p2, np.array([1.0, 4.0, 9.0, 16.0]) / 30.0, rtol=1e-14, atol=0)
    # two channels: s = q0*k0 + q1*k1 with q = (1, -1), keys (ln 6, ln 2), (ln 3, 0): weights 3, 3
    p3 = orc.probs(np.array([1.0, -1.0]), np.log(np.array([[6.0, 2.0], [3.0, 1.0]])))
    np.testing.assert_allclose(p3, [0.5, 0.5], rtol=1e-14, atol=0)


@pytest.mark.parametrize("seed", range(10))
def test_brute_force_fsum_no_shift(orc, seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 60))
    D = int(rng.choice([1, 3, 8, 16]))
    q = rng.standard_normal(D)
    K = rng.standard_normal((n, D)) * 2.0
    sm = float(rng.choice([1.0, 0.125, 0.7]))
    s = [sm * math.fsum(float(q[c]) * float(K[j, c]) for c in range(D)) for j in range(n)]
    e = [math.exp(x) for x in s]
    tot = math.fsum(e)
    want = np.array([x / tot for x in e])
    got = orc.probs(q, K, sm_scale=sm)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-300)
    assert abs(math.fsum(got) - 1.0) <= 1e-14


def test_large_scores_against_torch_softmax(orc):
    """Scores near 700-1000 overflow exp() without the shift by the maximum
    (exp(710) is inf in float64); torch's float64 softmax is the reference."""
    import torch

    rng = np.random.default_rng(5)
    n, D = 50, 4
    q = np.array([10.0, -3.0, 2.0, 0.5])
    K = rng.standard_normal((n, D)) * 3.0
    K[:, 0] += 90.0                      # scores around 900
    s = K @ q
    assert s.max() > 750
    got = orc.probs(q, K)
    want = torch.softmax(torch.tensor(s, dtype=torch.float64), dim=0).numpy()
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-300)
    # very negative scores underflow exp() without the shift (exp(-800) is 0)
    got_neg = orc.probs(-q, K)
    want_neg = torch.softmax(torch.tensor(-s, dtype=torch.float64), dim=0).numpy()
    assert np.all(np.isfinite(got_neg)) and abs(got_neg.sum() - 1.0) < 1e-14
    np.testing.assert_allclose(got_neg, want_neg, rtol=1e-11, atol=1e-300)


def test_invariants(orc):
    rng = np.random.default_rng(11)
    n, D = 33, 8
    q = rng.standard_normal(D)
    K = rng.standard_normal((n, D))
    p = orc.probs(q, K)
    assert abs(p.sum() - 1.0) < 1e-14
    s = K @ q
    # order of the weights follows the order of the scores
    assert np.array_equal(np.argsort(p, kind="stable"), np.argsort(s, kind="stable"))
    # adding a constant to every score leaves the distribution unchanged:
    # an extra channel with q = 1 and the same key value c in every row
    q2 = np.concatenate([q, [1.0]])
    K2 = np.concatenate([K, np.full((n, 1), 37.0)], axis=1)
    np.testing.assert_allclose(orc.probs(q2, K2), p, rtol=1e-12)
    # one position: probability 1; equal scores: uniform
    assert orc.probs(q, K[:1]).tolist() == [1.0]
    np.testing.assert_allclose(orc.probs(np.zeros(D), K), np.full(n, 1.0 / n), rtol=1e-15)
