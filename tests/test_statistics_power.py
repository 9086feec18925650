"""The statistical checks of the sampler can tell a wrong rule from a right one.

The GPU statistics tests judge 200,000 draws by a chi-square fit of the
emitted tokens to p and of the accepted length to its geometric law.  Here the
same checks run on the oracle's draws of the same seeded inputs (10,000 of
them, to stay quick): the oracle passes, and the oracle with a plausible
mistake planted in it fails.  [P2] section 20万回の標本で確かめる (the check),
[P1] section 高速化はどこから来るか：受理長と期待値 (the length law).
"""

import numpy as np
import pytest
from scipy import stats

import workloads as W
from oracle import formulas as F
from oracle import sampler as S
from tests._stats import P_MIN, chi2_pvalue, tvd_noise

N = 10_000
V = 65


def _rows(inp):
    T = inp["temperature"]
    return (S.softmax_t(inp["target_row"].astype(np.float64), T),
            S.softmax_t(inp["draft_row"].astype(np.float64), T))


def _draws(inp):
    r = S.verify_batch(inp["target_logits"], inp["draft_logits"], inp["draft_tokens"], inp["uniforms"],
                       inp["temperature"])
    return r["n_accepted"], r["out_tokens"]


def _first_token_fit(inp):
    _, tok = _draws(inp)
    p, _ = _rows(inp)
    c = np.bincount(tok[:, 0], minlength=V)
    return chi2_pvalue(c, p), F.tvd(c / c.sum(), p), tvd_noise(p, N)


def _length_fit(inp, gamma):
    n, _ = _draws(inp)
    p, q = _rows(inp)
    law = F.n_accepted_law(F.acceptance_alpha(p, q), gamma)
    return float(stats.chisquare(np.bincount(n, minlength=gamma + 1).astype(np.float64), law * N).pvalue)


@pytest.fixture(scope="module")
def tvd_inputs():
    return W.repeated_row_inputs(1, V, 1, N, 1.0)


@pytest.fixture(scope="module")
def law_inputs():
    return W.repeated_row_inputs(14, V, 4, N, 1.0)


def test_the_oracle_passes_both_checks(tvd_inputs, law_inputs):
    pv, tvd, noise = _first_token_fit(tvd_inputs)
    assert pv > P_MIN and tvd < 2.0 * noise
    assert _length_fit(law_inputs, 4) > P_MIN


@pytest.mark.parametrize("mistake", ["residual_is_p", "residual_is_q"])
def test_wrong_correction_distribution_fails_the_token_check(tvd_inputs, monkeypatch, mistake):
    # After a rejection the token must come from normalize(max(0, p - q)).
    if mistake == "residual_is_p":
        monkeypatch.setattr(S, "residual", lambda p, q: p)
    else:
        monkeypatch.setattr(S, "residual", lambda p, q: q)
    pv, tvd, noise = _first_token_fit(tvd_inputs)
    assert pv < P_MIN and tvd > 2.0 * noise


def test_transposed_accept_ratio_fails_the_length_check(law_inputs, monkeypatch):
    # min(1, q/p) in place of min(1, p/q): another acceptance rate per position.
    real = S.accept_threshold
    monkeypatch.setattr(S, "accept_threshold", lambda p_x, q_x: real(q_x, p_x))
    assert _length_fit(law_inputs, 4) < P_MIN
