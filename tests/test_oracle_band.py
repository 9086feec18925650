"""Pins for the 1e-6 band of the GPU comparison (oracle.sampler margins).

The parity rule compares the GPU's tokens with the oracle's except for
sequences with a decision whose uniform lies within 1e-6 of its threshold
(the accept test's min(1, p/q), or a CDF boundary of the drawn token); [P3]
section 受理・棄却の規則と出力分布が変わらない理由 notes that floating-point
differences can change such outputs.  The helpers that measure those margins
decide which sequences are compared at all, so they are pinned here against
what the margins mean, not against their own formulas:

* a margin below eps is exactly a decision that a shift of the uniform by
  eps would change (the accept test flips, the drawn token changes, or the
  uniform leaves [0, 1)), checked with the pinned ``inverse_cdf`` and
  ``accepts`` on random weights;
* constructed cases: u exactly on a boundary and 1e-7 to either side, an
  accept threshold of exactly 0.5, a NaN threshold;
* the band probability: the closed form 2 * eps * V for uniform weights, the
  one-hot case, and a Monte Carlo count of uniforms whose margin is below eps;
* a mutated margin (always 0, or read one CDF index too far) fails these pins,
  and with a zero margin the GPU comparison's bound on the excluded count
  rejects a comparison that would otherwise pass without comparing anything.
"""

import numpy as np
import pytest

from oracle import sampler as S


def _flips_draw(w, u, eps):
    t = S.inverse_cdf(w, u)
    if u - eps < 0.0 or u + eps >= 1.0:
        return True
    return S.inverse_cdf(w, u - eps) != t or S.inverse_cdf(w, u + eps) != t


def _flips_accept(u, thr, eps):
    return S.accepts(u - eps, thr) != S.accepts(u + eps, thr)


# ----------------------------------------------------------------------------
# constructed cases
# ----------------------------------------------------------------------------


def test_cdf_margin_on_and_beside_boundaries():
    w = np.array([1.0, 1.0, 2.0])  # C / C_last = 0.25, 0.5, 1
    assert S.inverse_cdf(w, 0.25) == 1 and S.cdf_margin(w, 1, 0.25) == 0.0
    assert S.inverse_cdf(w, 0.5) == 2 and S.cdf_margin(w, 2, 0.5) == 0.0
    assert S.inverse_cdf(w, 0.0) == 0 and S.cdf_margin(w, 0, 0.0) == 0.0
    for u, t in ((0.25 + 1e-7, 1), (0.25 - 1e-7, 0), (0.5 - 1e-7, 1), (0.5 + 1e-7, 2), (1 - 1e-7, 2), (1e-7, 0)):
        assert S.inverse_cdf(w, u) == t
        assert S.cdf_margin(w, t, u) == pytest.approx(1e-7, abs=1e-15)
    # the middle of a token's interval: the distance to its nearer end
    assert S.cdf_margin(w, 2, 0.8) == pytest.approx(0.2, abs=1e-15)
    assert S.cdf_margin(w, 0, 0.1) == pytest.approx(0.1, abs=1e-15)


def test_accept_margin_cases():
    assert S.accept_margin(0.5 + 1e-7, 0.5) == pytest.approx(1e-7, abs=1e-15)
    assert S.accept_margin(0.5 - 1e-7, 0.5) == pytest.approx(1e-7, abs=1e-15)
    assert S.accept_margin(0.3, np.float64(np.nan)) == float("inf")
    assert S.accept_margin(0.9, 1.0) == pytest.approx(0.1, abs=1e-15)


def _threshold_half_case(u_accept):
    """V = 2: p = [1/2, 1/2] and q = [1, 0] at the drafted token 0, so the
    threshold is exactly 0.5; the bonus/residual draw sits far from its
    boundaries (u = 0.25 on p or on the residual [0, 1])."""
    zt = np.array([[0.0, 0.0], [0.0, 0.0]])
    zd = np.array([[0.0, -np.inf]])
    return S.verify_sequence(zt, zd, [0], [u_accept, 0.25], 1.0)


def test_threshold_of_one_half_within_and_outside_the_band():
    r = _threshold_half_case(0.5 + 1e-7)  # rejects, 1e-7 from the threshold
    assert r["n_accepted"] == 0 and r["accept_margins"][0] == pytest.approx(1e-7, abs=1e-15)
    assert min(r["accept_margins"] + [r["draw_margin"]]) < S.BAND
    r = _threshold_half_case(0.5 - 1e-7)  # accepts
    assert r["n_accepted"] == 1 and min(r["accept_margins"] + [r["draw_margin"]]) < S.BAND
    r = _threshold_half_case(0.5 + 1e-5)  # rejects, outside the band
    assert r["n_accepted"] == 0 and min(r["accept_margins"] + [r["draw_margin"]]) > S.BAND
    assert r["draw_margin"] == pytest.approx(0.25, abs=1e-15)  # residual [0, 1]: boundaries 0, 0, 1


def test_nan_threshold_has_no_band():
    # p = q = 0 at the drafted token: 0/0 rejects for every u, so the accept
    # margin is infinite and only the draw's margin counts.
    zt = np.array([[0.0, -np.inf], [0.0, 0.0]])
    zd = np.array([[0.0, -np.inf]])
    r = S.verify_sequence(zt, zd, [1], [0.3, 0.5], 1.0)
    assert r["n_accepted"] == 0 and r["accept_margins"] == [float("inf")]


# ----------------------------------------------------------------------------
# the margins mean "a shift of eps changes the decision"
# ----------------------------------------------------------------------------


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_cdf_margin_below_eps_iff_a_shift_changes_the_draw(seed):
    rng = np.random.default_rng([41, seed])
    for _ in range(400):
        V = int(rng.integers(1, 9))
        w = rng.dirichlet(np.ones(V))
        w[rng.random(V) < 0.25] = 0.0
        if w.sum() == 0.0:
            w[int(rng.integers(V))] = 1.0
        eps = float(rng.choice([1e-3, 1e-2, 5e-2]))
        u = float(rng.random())
        t = S.inverse_cdf(w, u)
        assert (S.cdf_margin(w, t, u) < eps) == _flips_draw(w, u, eps), (w, u, eps)


@pytest.mark.parametrize("seed", [0, 1])
def test_accept_margin_below_eps_iff_a_shift_changes_the_test(seed):
    rng = np.random.default_rng([42, seed])
    for _ in range(400):
        p, q = rng.random(2) * (rng.random(2) < 0.9)
        thr = S.accept_threshold(p, q)
        eps = float(rng.choice([1e-3, 1e-2, 5e-2]))
        u = float(rng.random())
        assert (S.accept_margin(u, thr) < eps) == _flips_accept(u, thr, eps), (p, q, u, eps)


def test_sequence_margins_are_those_of_its_decisions():
    """verify_sequence's margins are the margins of the tests it evaluated and
    of its final draw, at the same uniforms (the shift criterion above)."""
    rng = np.random.default_rng(43)
    for _ in range(200):
        V, gamma = 5, 3
        zt, zd = rng.normal(size=(gamma + 1, V)), rng.normal(size=(gamma, V))
        x = rng.integers(0, V, size=gamma)
        u = rng.random(gamma + 1)
        r = S.verify_sequence(zt, zd, x, u, 1.0)
        n = r["n_accepted"]
        assert len(r["accept_margins"]) == min(n + 1, gamma)
        for i, m in enumerate(r["accept_margins"]):
            thr = S.accept_threshold(r["p_x"][i], r["q_x"][i])
            assert (m < 1e-2) == _flips_accept(u[i], thr, 1e-2)
        p = S.softmax_t(zt[n], 1.0)
        w = S.residual(p, S.softmax_t(zd[n], 1.0)) if n < gamma else p
        assert (r["draw_margin"] < 1e-2) == _flips_draw(w, u[gamma], 1e-2)


# ----------------------------------------------------------------------------
# band probability
# ----------------------------------------------------------------------------


@pytest.mark.parametrize("V", [1, 2, 5, 96])
def test_band_probability_closed_form_uniform_weights(V):
    # boundaries at k/V: eps at 0, eps below 1, 2 eps around each inner one
    eps = 1e-6
    assert S.band_probability(np.ones(V), eps) == pytest.approx(2 * eps * V, rel=1e-9)


def test_band_probability_limits():
    assert S.band_probability([0.0, 3.0, 0.0], 0.01) == pytest.approx(0.02, rel=1e-12)  # boundaries 0, 0, 1, 1
    assert S.band_probability([1.0, 1.0, 2.0], 0.3) == pytest.approx(1.0)  # the intervals cover [0, 1)
    assert S.accept_band_probability(0.5, 1e-6) == pytest.approx(2e-6, rel=1e-9)
    assert S.accept_band_probability(1.0, 1e-6) == pytest.approx(1e-6, rel=1e-9)
    assert S.accept_band_probability(np.nan, 1e-6) == 0.0


@pytest.mark.parametrize("seed", [0, 1])
def test_band_probability_matches_monte_carlo(seed):
    rng = np.random.default_rng([44, seed])
    V, eps, N = 7, 0.01, 200_000
    w = rng.dirichlet(np.ones(V) * 0.5)
    u = rng.random(N)
    c = np.cumsum(w) / np.sum(w)
    t = np.searchsorted(c, u, side="right")
    lo = np.where(t > 0, c[np.maximum(t - 1, 0)], 0.0)
    inside = np.minimum(np.abs(u - lo), np.abs(u - c[np.minimum(t, V - 1)])) < eps
    # the same count through the oracle's own margin on a subsample
    for k in range(0, N, 20_000):
        assert (S.cdf_margin(w, int(t[k]), float(u[k])) < eps) == bool(inside[k])
    prob = S.band_probability(w, eps)
    sigma = np.sqrt(prob * (1 - prob) / N)
    assert abs(inside.mean() - prob) < 5 * sigma, (inside.mean(), prob)


# ----------------------------------------------------------------------------
# mutations of the margins are caught
# ----------------------------------------------------------------------------


def _zero_margin(w, t, u):
    return 0.0


def _shifted_margin(w, t, u):  # C_t and C_{t+1}: one index too far
    c = np.cumsum(w)
    c = c / c[-1]
    return float(min(abs(u - c[t]), abs(u - c[min(t + 1, len(c) - 1)])))


@pytest.mark.parametrize("mutant", [_zero_margin, _shifted_margin])
def test_mutated_cdf_margin_is_caught(monkeypatch, mutant):
    monkeypatch.setattr(S, "cdf_margin", mutant)
    with pytest.raises(AssertionError):
        test_cdf_margin_below_eps_iff_a_shift_changes_the_draw(0)


def test_mutated_accept_margin_is_caught(monkeypatch):
    monkeypatch.setattr(S, "accept_margin", lambda u, thr: 0.0)
    with pytest.raises(AssertionError):
        test_threshold_of_one_half_within_and_outside_the_band()


def test_band_probability_missing_the_zero_boundary_is_caught(monkeypatch):
    orig = S.band_probability

    def no_zero(w, eps):
        return orig(w, eps) - eps

    monkeypatch.setattr(S, "band_probability", no_zero)
    with pytest.raises(AssertionError):
        test_band_probability_closed_form_uniform_weights(5)


def _small_batch():
    rng = np.random.default_rng(45)
    B, gamma, V = 64, 4, 96
    zt = rng.normal(0, 2, size=(B, gamma + 1, V))
    zd = zt[:, :gamma] + rng.normal(size=(B, gamma, V))
    x = rng.integers(0, V, size=(B, gamma))
    u = rng.random((B, gamma + 1))
    return zt, zd, x, u


def test_zero_margin_cannot_empty_the_gpu_comparison(monkeypatch):
    """With every margin 0 the band would take every sequence out of the
    comparison; the bound on the excluded count must refuse that."""
    from tests import _gpu

    zt, zd, x, u = _small_batch()
    orc = S.verify_batch(zt, zd, x, u, 1.0)
    wrong = orc["out_tokens"].copy()
    wrong[:, 0] = (wrong[:, 0] + 1) % 96  # every sequence disagrees
    with pytest.raises(AssertionError):
        _gpu.compare_sampler(orc, orc["n_accepted"], wrong)
    monkeypatch.setattr(S, "cdf_margin", _zero_margin)
    orc0 = S.verify_batch(zt, zd, x, u, 1.0)
    assert (orc0["min_margin"] == 0).all()
    with pytest.raises(AssertionError, match="band"):
        _gpu.compare_sampler(orc0, orc0["n_accepted"], wrong)
    # the unmutated oracle with the right tokens passes, and reports its counts
    st = _gpu.compare_sampler(orc, orc["n_accepted"], orc["out_tokens"])
    assert st["in_band"] <= st["band_bound"]
