"""Pins for oracle.sampler.

* the pages' worked example: the V=5 toy of [P3], replayed from its seed,
  must print the page's frequencies and acceptance rate;
* brute force on V <= 4, gamma <= 3: the oracle's exact outcome law (extracted
  by bisection, tests/_law.py) must equal the target distribution at every
  position (Chen et al. Theorem 1, [P1] / [P2] distribution-preservation
  argument), and P(n_accepted >= k) must equal the product of sum_x min(p, q);
* special cases that reduce to a library routine: q = p (bonus = numpy's
  inverse-CDF ``Generator.choice``), disjoint supports, one-hot drafts;
* edge conventions: strict <, zero-mass tokens never drawn, q(x) = 0, p = q = 0,
  the zero-residual fallback, temperature and shift invariance.
"""

import json
import os

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

from oracle import formulas as F
from oracle import sampler as S
from tests import _law, _replay

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _log(p):
    with np.errstate(divide="ignore"):
        return np.log(np.asarray(p, np.float64))


# ----------------------------------------------------------------------------
# the pages' worked example
# ----------------------------------------------------------------------------


def test_page_toy_replay_prints_page_values():
    with open(os.path.join(GOLDEN, "p3_toy_v5.json")) as f:
        g = json.load(f)
    r = _replay.build(g["p"], g["q"], g["N"], seed=g["seed"])
    freq = np.bincount(r["first_token"], minlength=g["V"]) / g["N"]
    assert list(np.round(freq, 3)) == g["printed_observed_freq_round3"]
    assert round(r["accepted"].mean(), 3) == g["printed_accept_rate_round3"]
    # alpha = sum min(p, q) = 0.78 is also the acceptance probability; the
    # observed rate sits within 4 sigma of it.
    a = F.acceptance_alpha(g["p"], g["q"])
    sigma = np.sqrt(a * (1 - a) / g["N"])
    assert abs(r["accepted"].mean() - a) < 4 * sigma


# ----------------------------------------------------------------------------
# brute force: the oracle's exact law
# ----------------------------------------------------------------------------


def _dirichlet_rows(rng, n, V, zero_frac=0.0):
    rows = rng.dirichlet(np.ones(V), size=n)
    if zero_frac:
        mask = rng.random((n, V)) < zero_frac
        mask[np.arange(n), rng.integers(0, V, n)] = False  # keep one entry alive
        rows = np.where(mask, 0.0, rows)
        rows /= rows.sum(axis=1, keepdims=True)
    return rows


CASES = [
    # (V, gamma, seed, zero fraction)
    (2, 1, 0, 0.0),
    (3, 2, 1, 0.0),
    (4, 2, 2, 0.3),
    (3, 3, 3, 0.2),
    (4, 3, 4, 0.0),
]


@pytest.mark.parametrize("V,gamma,seed,zf", CASES)
def test_bruteforce_law_preserves_target_distribution(V, gamma, seed, zf):
    rng = np.random.default_rng(seed)
    P = _dirichlet_rows(rng, gamma + 1, V, zf)
    Q = _dirichlet_rows(rng, gamma, V, zf)
    T = [1.0, 0.7, 1.3][seed % 3]
    # logits T * log(prob) + an arbitrary per-row shift give softmax(z/T) = prob
    zt = T * _log(P) + rng.normal(size=(gamma + 1, 1))
    zd = T * _log(Q) + rng.normal(size=(gamma, 1))
    law = _law.full_law(zt, zd, Q, T)
    alpha = [F.acceptance_alpha(P[i], Q[i]) for i in range(gamma)]
    reach = np.cumprod([1.0] + alpha)
    assert np.allclose(law["n_law"].sum(), 1.0, atol=1e-12)
    assert np.allclose(law["reach"], reach, atol=1e-12, rtol=0)
    for k in range(gamma + 1):
        # position k is emitted iff n >= k; given that, it is distributed as p_k
        assert np.allclose(law["pos"][k], reach[k] * P[k], atol=1e-12, rtol=0), k


def test_bruteforce_n_accepted_law_is_truncated_geometric():
    # Every position has the toy's (p, q) restricted to 4 tokens.
    rng = np.random.default_rng(7)
    p = rng.dirichlet(np.ones(4))
    q = rng.dirichlet(np.ones(4))
    gamma = 3
    zt = np.stack([_log(p)] * (gamma + 1))
    zd = np.stack([_log(q)] * gamma)
    law = _law.full_law(zt, zd, [q] * gamma, 1.0)
    a = F.acceptance_alpha(p, q)
    assert np.allclose(law["n_law"], F.n_accepted_law(a, gamma), atol=1e-12, rtol=0)
    e = np.dot(np.arange(gamma + 1) + 1, law["n_law"])
    assert abs(e - F.expected_committed(a, gamma)) < 1e-12


# ----------------------------------------------------------------------------
# special cases reducing to a library routine
# ----------------------------------------------------------------------------


def test_q_equal_p_accepts_all_and_bonus_is_numpy_choice():
    rng = np.random.default_rng(11)
    V, gamma = 37, 4
    for s in range(300):
        z = rng.normal(scale=2.0, size=(gamma + 1, V))
        x = rng.integers(0, V, gamma)
        u_acc = list(rng.random(gamma))
        u_fin = np.random.default_rng(s).random()
        r = S.verify_sequence(z, z[:gamma], x, u_acc + [u_fin], 1.0)
        assert r["n_accepted"] == gamma
        assert r["tokens"][:gamma] == list(x)
        want = np.random.default_rng(s).choice(V, p=sp_softmax(z[gamma]))
        assert r["tokens"][-1] == want


def test_disjoint_supports_reject_first_and_draw_from_p():
    V = 8
    p = np.array([0.5, 0.3, 0.2, 0, 0, 0, 0, 0])
    q = np.array([0, 0, 0, 0.1, 0.2, 0.3, 0.25, 0.15])
    for s in range(200):
        x = 3 + s % 5
        u_fin = np.random.default_rng(s).random()
        r = S.verify_sequence(_log([p, p]), _log([q]), [x], [0.0, u_fin], 1.0)
        assert r["n_accepted"] == 0
        assert r["tokens"] == [np.random.default_rng(s).choice(V, p=p)]


def test_one_hot_draft_accepts_with_p_and_resamples_p_without_x():
    V = 6
    rng = np.random.default_rng(5)
    p = rng.dirichlet(np.ones(V))
    for s in range(300):
        x = s % V
        q = np.zeros(V)
        q[x] = 1.0
        u_acc = np.random.default_rng(1000 + s).random()
        u_fin = np.random.default_rng(s).random()
        r = S.verify_sequence(_log([p, p]), _log([q]), [x], [u_acc, u_fin], 1.0)
        assert r["n_accepted"] == int(u_acc < p[x])
        if r["n_accepted"] == 0:
            rest = p.copy()
            rest[x] = 0.0
            assert r["tokens"] == [np.random.default_rng(s).choice(V, p=rest / rest.sum())]


# ----------------------------------------------------------------------------
# edge conventions
# ----------------------------------------------------------------------------


def test_accept_test_is_strict():
    # p(x) = 1/4 and q(x) = 1/2 exactly: the threshold is exactly 0.5.
    zt = np.zeros((2, 4))
    zd = np.array([[0.0, 0.0, -np.inf, -np.inf]])
    assert S.verify_sequence(zt, zd, [0], [0.5, 0.1], 1.0)["n_accepted"] == 0
    assert S.verify_sequence(zt, zd, [0], [np.nextafter(0.5, 0), 0.1], 1.0)["n_accepted"] == 1


def test_zero_mass_tokens_never_drawn():
    # Residual puts zero mass on tokens 0 and 1; u = 0 must not pick token 0.
    p = np.array([0.0, 0.0, 0.5, 0.5])
    zt = _log([p, p])
    zd = _log([[0.0, 0.0, 0.0, 1.0]])
    r = S.verify_sequence(zt, zd, [3], [0.9, 0.0], 1.0)
    assert r["n_accepted"] == 0 and r["tokens"] == [2]
    # bonus with zero mass at the front
    r = S.verify_sequence(zt, _log([p]), [2], [0.1, 0.0], 1.0)
    assert r["n_accepted"] == 1 and r["tokens"] == [2, 2]


def test_q_zero_accepts_and_p_q_zero_rejects():
    zt = _log([[0.5, 0.5, 0.0], [1 / 3, 1 / 3, 1 / 3]])
    # draft probability of token 0 is zero while p(0) > 0: p/q = inf -> accept
    r = S.verify_sequence(zt, _log([[0.0, 0.0, 1.0]]), [0], [0.999, 0.2], 1.0)
    assert r["n_accepted"] == 1
    # token 2 has p = q = 0: 0/0 -> reject for every u
    zt2 = _log([[0.5, 0.5, 0.0], [1 / 3, 1 / 3, 1 / 3]])
    r = S.verify_sequence(zt2, _log([[0.5, 0.5, 0.0]]), [2], [0.0, 0.2], 1.0)
    assert r["n_accepted"] == 0


def test_zero_residual_falls_back_to_p():
    # q = p, and the draft is a token with p = q = 0: the test rejects (0/0),
    # the residual max(0, p - q) is identically zero, and the draw uses p.
    p = np.array([0.2, 0.8, 0.0])
    for s in range(50):
        u_fin = np.random.default_rng(s).random()
        r = S.verify_sequence(_log([p, p]), _log([p]), [2], [0.3, u_fin], 1.0)
        assert r["n_accepted"] == 0 and r["fallback"]
        assert r["tokens"] == [np.random.default_rng(s).choice(3, p=p)]


def test_temperature_and_shift_invariance():
    rng = np.random.default_rng(3)
    V, gamma = 50, 3
    for _ in range(50):
        zt = rng.normal(size=(gamma + 1, V))
        zd = zt[:gamma] + rng.normal(size=(gamma, V))
        x = rng.integers(0, V, gamma)
        u = rng.random(gamma + 1)
        T = rng.uniform(0.3, 2.0)
        a = S.verify_sequence(zt, zd, x, u, T)
        b = S.verify_sequence(zt / T, zd / T, x, u, 1.0)
        c = S.verify_sequence(zt + 7.0, zd - 3.0, x, u, T)
        for o in (b, c):
            if min(a["accept_margins"] + [a["draw_margin"]]) > 1e-9:
                assert o["tokens"] == a["tokens"] and o["n_accepted"] == a["n_accepted"]
            assert np.allclose(o["p_x"], a["p_x"], rtol=1e-12)
