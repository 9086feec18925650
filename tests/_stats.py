"""Goodness-of-fit helpers for the statistical checks of the sampler."""

import numpy as np
from scipy import stats

P_MIN = 1e-4  # smallest chi-square p-value accepted (inputs are seeded: a fixed draw)


def chi2_pvalue(counts, probs):
    """Pearson goodness of fit of token counts to probs; cells expecting < 5 are pooled."""
    counts = np.asarray(counts, np.float64)
    exp = np.asarray(probs, np.float64) / np.sum(probs) * counts.sum()
    big = exp >= 5
    obs = counts[big]
    ex = exp[big]
    if (~big).any() and exp[~big].sum() > 0:
        obs = np.append(obs, counts[~big].sum())
        ex = np.append(ex, exp[~big].sum())
    return float(stats.chisquare(obs, ex).pvalue)


def tvd_noise(p, n):
    """Expected TVD of an n-draw empirical distribution from p (normal approximation
    of each count: E|N(0, s^2)| = s sqrt(2/pi))."""
    p = np.asarray(p, np.float64)
    return float(0.5 * np.sum(np.sqrt(2.0 * p * (1.0 - p) / (np.pi * n))))
