"""Pins of the round oracle (oracle/round.py): the draft loop, one target
verify call, the accept/residual draw and both cache truncations.

[P2] section 投機的デコーディングとは states the checks used here: at
temperature 0 speculative decoding reproduces the target's own greedy
decoding exactly; the truncated caches hold exactly the committed prefix's
K/V.  A draft identical to the target accepts every proposal, so the round
reduces to sampling from the target alone with the same uniforms.
"""

import numpy as np
import pytest

from oracle import model as M
from oracle import round as R
from oracle import sampler as S
from workloads import gen


def _params(cfg, seed):
    return gen.model_params(M.param_shapes(cfg), seed).astype(np.float64)


def _prompts(B, V, L, seed):
    return [list(np.random.default_rng([seed, b]).integers(0, V, size=L)) for b in range(B)]


def _run(flat_t, cfg_t, flat_d, cfg_d, prompts, gamma, T, rounds, seed, max_T=64):
    st = R.start(flat_t, cfg_t, flat_d, cfg_d, prompts, max_T, max_T)
    r = np.random.default_rng(seed)
    out = []
    for _ in range(rounds):
        ud = r.random((len(prompts), gamma))
        uv = r.random((len(prompts), gamma + 1))
        out.append(R.speculative_round(flat_t, cfg_t, flat_d, cfg_d, st, gamma, T, ud, uv))
    return st, out


def test_greedy_rounds_reproduce_target_greedy_decoding():
    t, d = _params(M.TARGET, 1), _params(M.DRAFT, 2)
    prompts = _prompts(3, 96, 5, 3)
    st, _ = _run(t, M.TARGET, d, M.DRAFT, prompts, 4, 0.0, 6, 4)
    for b, p in enumerate(prompts):
        seq = list(p)
        while len(seq) < len(st["seq"][b]):
            seq.append(int(np.argmax(M.forward_uncached(t, M.TARGET, np.array(seq))[-1])))
        assert st["seq"][b] == seq


def test_draft_equal_to_target_accepts_everything():
    """q = p: every test accepts, and the round is target sampling with the
    draft's uniforms for the proposals and u_verify[gamma] for the bonus."""
    cfg = M.DRAFT  # small and fast; the target role is played by the same model
    t = _params(cfg, 5)
    prompts = _prompts(2, 96, 4, 6)
    gamma, T = 3, 1.0
    st = R.start(t, cfg, t, cfg, prompts, 32, 32)
    r = np.random.default_rng(7)
    ud, uv = r.random((2, gamma)), r.random((2, gamma + 1))
    res = R.speculative_round(t, cfg, t, cfg, st, gamma, T, ud, uv)
    assert list(res["n_accepted"]) == [gamma, gamma]
    for b, p in enumerate(prompts):
        seq = list(p)
        for u in list(ud[b]) + [uv[b, gamma]]:
            z = M.forward_uncached(t, cfg, np.array(seq))[-1]
            seq.append(S.inverse_cdf(S.softmax_t(z, T), u))
        assert st["seq"][b] == seq
        # all accepted: the draft never ran the last proposal, so its cache
        # holds len - 2 tokens, exactly those of a fresh prefill
        dl = int(st["dlen"][b])
        assert dl == len(seq) - 2
        dk, _ = M.prefill(t, cfg, [seq[:dl]], 32)
        np.testing.assert_allclose(st["dkv"][:, :, b, :, :dl], dk[:, :, 0, :, :dl], rtol=0, atol=1e-12)


@pytest.mark.parametrize("T", [0.0, 1.0])
def test_truncated_caches_hold_the_committed_prefix(T):
    t, d = _params(M.TARGET, 8), _params(M.DRAFT, 9)
    prompts = _prompts(3, 96, 6, 10)
    st, _ = _run(t, M.TARGET, d, M.DRAFT, prompts, 4, T, 3, 11)
    for b in range(3):
        seq = st["seq"][b]
        tl, dl = int(st["tlen"][b]), int(st["dlen"][b])
        assert tl == len(seq) - 1 and len(seq) - 2 <= dl <= len(seq) - 1
        tk, _ = M.prefill(t, M.TARGET, [seq[:tl]], 64)
        dk, _ = M.prefill(d, M.DRAFT, [seq[:dl]], 64)
        np.testing.assert_allclose(st["tkv"][:, :, b, :, :tl], tk[:, :, 0, :, :tl], rtol=0, atol=1e-12)
        np.testing.assert_allclose(st["dkv"][:, :, b, :, :dl], dk[:, :, 0, :, :dl], rtol=0, atol=1e-12)


def test_round_stats_follow_the_pages_columns():
    s = R.round_stats([0, 2, 4], 4)
    assert s["alpha"] == pytest.approx(6 / 8)  # tested: 1, 3, 4
    assert s["accepted_per_proposed"] == pytest.approx(6 / 12)
    assert s["tokens_per_target_call"] == pytest.approx(3.0)
