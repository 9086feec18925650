"""Statistical checks of the GPU sampler on many draws of one verification.

[P2] section 20万回の標本で確かめる checks the accept/reject rule by running
it 200,000 times on one (p, q) pair and measuring the total-variation distance
of the results from p, next to the distance that drawing from p directly
gives (the sampling noise) and the distance of the draft alone.  The first
test does that through the GPU path, on synthetic rows over a 65-token
vocabulary (no trained character model exists here).  The second checks the
law of the accepted length for gamma > 1 on repeated rows, against the
geometric law behind [P1] section 高速化はどこから来るか：受理長と期待値, and
that the token emitted at every position is distributed as p.  Both also
compare a sample of the sequences one by one with the oracle.
"""

import numpy as np
import pytest
import torch
from scipy import stats

import speculative_decoding_verification_spec_amd as sv
import workloads as W
from oracle import formulas as F
from oracle import sampler as S
from tests import _gpu
from tests._stats import P_MIN, chi2_pvalue, tvd_noise

pytestmark = pytest.mark.gpu
N = 200_000
V = 65


def _case(name, **kw):
    print(f"\n[case] {name} {kw}", flush=True)


def _run(inp):
    dev = {k: _gpu.to_dev(inp[k]) for k in ("target_logits", "draft_logits", "draft_tokens", "uniforms")}
    n, tok, p, q = sv.spec_reject_sample(**dev, temperature=inp["temperature"], want_probs=True)
    torch.cuda.synchronize()
    return _gpu.to_host(n), _gpu.to_host(tok), _gpu.to_host(p), _gpu.to_host(q)


def _rows(inp):
    T = inp["temperature"]
    p = S.softmax_t(inp["target_row"].astype(np.float64), T)
    q = S.softmax_t(inp["draft_row"].astype(np.float64), T)
    return p, q


def _parity_sample(inp, n, tok, p_x, q_x, count=4000):
    seqs = np.linspace(0, len(n) - 1, count).astype(np.int64)
    orc = S.verify_batch(inp["target_logits"], inp["draft_logits"], inp["draft_tokens"], inp["uniforms"],
                         inp["temperature"], seqs)
    return _gpu.compare_sampler(orc, n, tok, p_x, q_x, seqs=seqs)


@pytest.mark.parametrize("seed,T", [(1, 1.0), (2, 1.0), (3, 1.0), (1, 0.7)])
def test_two_hundred_thousand_draws_follow_the_target(seed, T):
    _case("tvd", seed=seed, T=T, N=N, V=V)
    inp = W.repeated_row_inputs(seed, V, 1, N, T)
    n, tok, p_x, q_x = _run(inp)
    p, q = _rows(inp)
    alpha = F.acceptance_alpha(p, q)
    rate = float(np.mean(n == 1))
    spec = np.bincount(tok[:, 0], minlength=V) / N
    direct = np.bincount(np.random.default_rng([seed, 3]).choice(V, N, p=p), minlength=V) / N
    draft = np.bincount(inp["draft_tokens"][:, 0], minlength=V) / N
    noise = tvd_noise(p, N)
    pv = chi2_pvalue(np.bincount(tok[:, 0], minlength=V), p)
    print(f"accept={rate:.4f} theory_sum_min(p,q)={alpha:.4f} TVD(spec,p)={F.tvd(spec, p):.4f} "
          f"TVD(direct,p)={F.tvd(direct, p):.4f} TVD(draft_only,p)={F.tvd(draft, p):.4f} "
          f"expected_noise={noise:.4f} chi2_p={pv:.3g}", flush=True)
    assert abs(rate - alpha) < 4.0 * np.sqrt(alpha * (1.0 - alpha) / N)
    assert pv > P_MIN
    assert F.tvd(spec, p) < 2.0 * noise
    assert F.tvd(draft, p) > 10.0 * noise  # the draft alone is far from p
    assert np.all(tok[:, 1][n == 0] == -1) and np.all(tok[:, 1][n == 1] >= 0)
    _parity_sample(inp, n, tok, p_x, q_x)


@pytest.mark.parametrize("gamma,T", [(4, 1.0), (8, 0.7)])
def test_accepted_length_law_on_repeated_rows(gamma, T):
    _case("length-law", gamma=gamma, T=T, N=N, V=V)
    inp = W.repeated_row_inputs(10 + gamma, V, gamma, N, T)
    n, tok, p_x, q_x = _run(inp)
    p, q = _rows(inp)
    alpha = F.acceptance_alpha(p, q)
    law = F.n_accepted_law(alpha, gamma)
    counts = np.bincount(n, minlength=gamma + 1)
    assert counts.size == gamma + 1 and n.min() >= 0
    pv = float(stats.chisquare(counts.astype(np.float64), law * N).pvalue)
    committed = n.astype(np.float64) + 1.0
    k = np.arange(gamma + 1) + 1.0
    var = float(np.sum(law * k * k) - np.sum(law * k) ** 2)
    want = F.expected_committed(alpha, gamma)
    print(f"alpha={alpha:.4f} counts={counts.tolist()} law*N={np.round(law * N).astype(int).tolist()} "
          f"chi2_p={pv:.3g} E[n+1]={committed.mean():.4f} closed_form={want:.4f}", flush=True)
    assert pv > P_MIN
    assert abs(committed.mean() - want) < 4.0 * np.sqrt(var / N)
    # Given that position i is emitted (the i positions before it accepted),
    # its token follows p: an accepted draft or a residual draw for i < gamma,
    # the bonus draw at gamma.
    for i in range(gamma + 1):
        emitted = n >= i
        c = np.bincount(tok[emitted, i], minlength=V)
        pvi = chi2_pvalue(c, p)
        print(f"position {i}: emitted={int(emitted.sum())} chi2_p={pvi:.3g}", flush=True)
        assert pvi > P_MIN / (gamma + 1)
        assert np.all(tok[~emitted, i] == -1)
    _parity_sample(inp, n, tok, p_x, q_x)
