"""Pins of the greedy (temperature 0) verification oracle.

  * [P2] section 投機的デコーディングとは reports that greedy speculative
    decoding reproduced target-only greedy decoding exactly.  Here a toy target
    and a toy draft (fixed next-token logit tables, so a model is a Markov
    chain) run many speculative rounds through the oracle; the committed text
    must equal plain greedy decoding of the target, token for token, for
    several draft lengths and both well-matched and poorly matched drafts.
  * The temperature-0 limit of the sampling oracle: with drafts that are the
    draft model's argmax and logits whose top two values are well apart, the
    modified rejection sampler at a tiny temperature makes the same decisions
    and emits the same tokens, whatever the uniforms.
  * The argmax conventions (first index among equal maxima; NaN is largest).
"""

import numpy as np
import pytest

from oracle import greedy as G
from oracle import sampler as S
from workloads.gen import bf16_bits


def _markov(V, seed, mix, noise, quantize):
    rng = np.random.default_rng(seed)
    zt = 3.0 * rng.standard_normal((V, V))
    zd = mix * zt + noise * rng.standard_normal((V, V))
    if quantize:  # bf16 logits: many exact ties near the top
        return bf16_bits(zt.astype(np.float32)), bf16_bits(zd.astype(np.float32))
    return zt, zd


def _greedy_decode(zt, start, n):
    out = [start]
    while len(out) < n + 1:
        out.append(G.argmax(zt[out[-1]]))
    return out[1:]


def _speculative_decode(zt, zd, start, n, gamma):
    seq = [start]
    rounds = 0
    while len(seq) < n + 1:
        xs = []
        ctx = seq[-1]
        for _ in range(gamma):  # greedy draft
            ctx = G.argmax(zd[ctx])
            xs.append(ctx)
        # target rows for [last committed] + drafts: row i predicts the token after context i
        rows = np.stack([zt[c] for c in [seq[-1]] + xs])
        n_acc, toks = G.verify_sequence(rows, np.array(xs))
        assert len(toks) == n_acc + 1 and toks[:n_acc] == xs[:n_acc]
        seq += toks
        rounds += 1
    return seq[1 : n + 1], rounds


@pytest.mark.parametrize("V,mix,noise,quantize", [(7, 1.0, 0.3, False), (50, 0.8, 1.0, False),
                                                  (200, 1.0, 0.0, True), (96, 0.5, 2.0, True)])
@pytest.mark.parametrize("gamma", [1, 2, 4, 8])
def test_speculative_equals_greedy_decoding(V, mix, noise, quantize, gamma):
    zt, zd = _markov(V, [V, gamma], mix, noise, quantize)
    for start in range(0, V, max(1, V // 5)):
        want = _greedy_decode(zt, start, 96)
        got, rounds = _speculative_decode(zt, zd, start, 96, gamma)
        assert got == want
        if noise == 0.0 and mix == 1.0:  # the draft is the target: everything is accepted
            assert rounds == -(-96 // (gamma + 1))


def test_zero_temperature_limit_of_the_sampler():
    rng = np.random.default_rng(11)
    V, gamma, T = 40, 4, 0.004
    checked = 0
    for trial in range(300):
        zt = rng.standard_normal((gamma + 1, V)) * 3
        zd = 0.7 * zt[:gamma] + rng.standard_normal((gamma, V))
        for z in (zt, zd):  # the limit needs a clear maximum in every row
            top = rng.integers(0, V, z.shape[0]) if trial % 2 else np.argmax(z, axis=1)
            z[np.arange(z.shape[0]), top] = z.max(axis=1) + 2.0
        x = np.argmax(zd, axis=1)  # a temperature-0 draft proposes its argmax
        if trial % 3 == 0:  # force agreement on a prefix to reach later positions
            k = trial % (gamma + 1)
            x[:k] = np.argmax(zt[:k], axis=1)
        u = rng.uniform(1e-3, 1 - 1e-3, gamma + 1)
        r = S.verify_sequence(zt, zd, x, u, T)
        n_g, toks_g = G.verify_sequence(zt, x)
        assert r["n_accepted"] == n_g
        assert r["tokens"] == toks_g
        checked += 1
    assert checked > 50


def test_argmax_conventions():
    assert G.argmax(np.array([1.0, 3.0, 3.0, 2.0])) == 1          # first of equal maxima
    assert G.argmax(np.array([-np.inf, -np.inf])) == 0
    assert G.argmax(np.array([1.0, np.nan, 5.0, np.nan])) == 1    # NaN counts as largest
    z = bf16_bits(np.array([0.5, 2.0, 2.0, -1.0], np.float32))     # bf16 bit patterns decode first
    assert G.argmax(z) == 1


def test_batch_form_matches_sequences():
    rng = np.random.default_rng(5)
    B, gamma, V = 20, 3, 9
    zt = rng.integers(-3, 3, (B, gamma + 1, V)).astype(np.float64)  # coarse values: ties
    x = rng.integers(0, V, (B, gamma)).astype(np.int32)
    x[::2] = np.argmax(zt[::2, :gamma], axis=2)                       # half the rows accept everything
    n, out, p = G.verify_batch(zt, x)
    for b in range(B):
        nb, tb = G.verify_sequence(zt[b], x[b])
        assert n[b] == nb and list(out[b, : nb + 1]) == tb and np.all(out[b, nb + 1 :] == -1)
        assert np.array_equal(p[b], (np.argmax(zt[b, :gamma], axis=1) == x[b]).astype(float))
    assert np.all(n[::2] == gamma)
