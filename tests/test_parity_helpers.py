"""The decision-margin helper the GPU parity tests use to accept a differing
sampled id (CPU only)."""
import numpy as np

from oracle.dualar_oracle import Sampling, sample_token
from tests.parity import decision_margin


def _flips(z, s, u, dz, trials=400, seed=0):
    """Does any perturbation of z within +-dz change the sampled id?"""
    rng = np.random.default_rng(seed)
    base = sample_token(z, s, u)
    for _ in range(trials):
        zp = z + rng.choice([-dz, dz], size=z.shape)
        if sample_token(zp, s, u) != base:
            return True
    return False


def test_topp_margin_covers_neighbour_swap():
    # tokens 3 and 5 nearly tied; u falls in the middle of token 3's interval,
    # far from every cumulative boundary
    z = np.array([0.0, -3.0, -3.0, 2.0, -4.0, 2.0 - 1e-4, -5.0, -6.0])
    s = Sampling(greedy=False, temperature=1.0, top_p=0.99)
    p = np.exp(z - z.max()); p /= p.sum()
    u = 0.5 * p[3] / p.sum()
    assert sample_token(z, s, u) == 3
    mg = decision_margin(z, False, 1.0, 0.99, u)
    assert mg <= 1.1e-4
    assert _flips(z, s, u, 1e-4)


def test_topp_margin_large_when_decision_is_stable():
    z = np.array([3.0, 0.0, -1.0, -2.0, -4.0])
    s = Sampling(greedy=False, temperature=0.8, top_p=0.9)
    u = 0.4
    mg = decision_margin(z, False, 0.8, 0.9, u)
    assert mg > 0.05
    assert not _flips(z, s, u, 0.4 * mg * 0.8)


def test_greedy_margin_is_top1_gap():
    z = np.array([1.0, 3.0, -np.inf, 2.5])
    assert abs(decision_margin(z, True) - 0.5) < 1e-6
