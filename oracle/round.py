"""Oracle: one speculative-decoding round of a draft and a target model (fp64).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

Follows [P2] section 投機的デコーディングとは (the round's listing and its
flowchart): the draft proposes gamma tokens, sampling each from its own
distribution q_j; the target is called once over [last committed token] +
the proposals; positions are tested in order with u < min(1, p(x)/q(x)) and
the scan stops at the first rejection; the final token comes from
normalize(max(0, p - q)) after a rejection, or from the target's next
distribution when every proposal was accepted; the sequence grows by the
accepted proposals and that token; the target cache is cut back to
base + 1 + n, the draft cache to min(its length, new length - 1).

Readings where the listing is silent:
  * The draft's proposal loop is not printed.  Here the draft first runs over
    every committed token it has not cached yet (``seq[dc.n:]``, one or two
    tokens: the draft cache is cut to min(dc.n, len - 1), and it lacks the
    last proposal's K/V when all were accepted), then over each proposal in
    turn; q_j = softmax(draft logits / T) of its last row, and x_j is the
    inverse-CDF draw of q_j at u_draft[j] (the same convention as the final
    draw, [P2]'s ``rng.choice``).
  * Temperature 0 is the greedy branch the listing omits: proposals are the
    draft's argmax and verification is the greedy rule (oracle.greedy).
State of one sequence: its committed tokens ``seq`` (length L >= 2), the
target cache holding the K/V of seq[:L-1] (``tlen`` = L - 1), and the draft
cache holding at least seq[:L-2] (``dlen`` in [L-2, L-1]).
"""

import numpy as np

from . import greedy as G
from . import model as M
from . import sampler as S


def _draw(z, temperature, u):
    """Token drawn from softmax(z / T) at u (argmax at T = 0), its margin and the
    probability that a uniform lands inside the band around its boundaries."""
    if temperature == 0.0:
        return G.argmax(z), float("inf"), 0.0
    w = S.softmax_t(z, temperature)
    t = S.inverse_cdf(w, u)
    return t, S.cdf_margin(w, t, float(u)), S.band_probability(w, S.BAND)


def propose(flat_d, cfg_d, seq, dkv, dlen, gamma, temperature, u_draft):
    """The draft's gamma proposals for one sequence.

    dkv: the draft cache of this sequence [L, 2, 1, H, max_T, D] (fp64, updated
    in place).  Returns (proposals, draft logits [gamma, V], new dlen, the
    smallest draw margin, the summed band probability of the draws).
    """
    pending = list(seq[dlen:])
    xs, zs, margin, band = [], [], float("inf"), 0.0
    for j in range(gamma):
        lg, new = M.forward_cached(flat_d, cfg_d, np.array([pending]), dkv, [dlen])
        dkv[...] = new
        dlen += len(pending)
        z = lg[0, -1]
        x, m, bp = _draw(z, temperature, u_draft[j])
        xs.append(x)
        zs.append(z)
        margin = min(margin, m)
        band += bp
        pending = [x]
    return xs, np.array(zs), dlen, margin, band


def speculative_round(flat_t, cfg_t, flat_d, cfg_d, state, gamma, temperature, u_draft, u_verify):
    """One round for every sequence of ``state`` (updated in place).

    state: dict with ``seq`` (list of token lists), ``tkv`` [L_t, 2, B, ...],
    ``tlen`` [B], ``dkv`` [L_d, 2, B, ...], ``dlen`` [B].
    u_draft [B, gamma], u_verify [B, gamma+1] fp64.
    Returns dict n_accepted [B], tokens (list of emitted lists), min_margin [B]
    (smallest decisive margin of the round: draft draws, accept tests and the
    final draw) and band_prob [B] (the summed chance of those decisions
    landing inside the band).
    """
    B = len(state["seq"])
    n_acc = np.zeros(B, dtype=np.int64)
    emitted, margins, bands = [], np.full(B, np.inf), np.zeros(B)
    for b in range(B):
        seq = state["seq"][b]
        L = len(seq)
        assert state["tlen"][b] == L - 1 and L - 2 <= state["dlen"][b] <= L - 1
        dkv = state["dkv"][:, :, b : b + 1]
        xs, zd, dlen, m_draft, b_draft = propose(flat_d, cfg_d, seq, dkv, int(state["dlen"][b]), gamma, temperature,
                                        u_draft[b])
        state["dkv"][:, :, b : b + 1] = dkv
        tkv = state["tkv"][:, :, b : b + 1]
        zt, tkv = M.forward_cached(flat_t, cfg_t, np.array([[seq[-1]] + xs]), tkv, [L - 1])
        state["tkv"][:, :, b : b + 1] = tkv
        if temperature == 0.0:
            n, toks = G.verify_sequence(zt[0], xs)
            m_ver, b_ver = float("inf"), 0.0
        else:
            r = S.verify_sequence(zt[0], zd, xs, u_verify[b], temperature)
            n, toks = r["n_accepted"], r["tokens"]
            m_ver = min(r["accept_margins"] + [r["draw_margin"]])
            b_ver = r["band_prob"]
        seq += toks
        # The target cache keeps the rows of the committed tokens before the
        # newest one: its old length, the verified last token and the n
        # accepted proposals.  The draft cache keeps what it holds, at most
        # up to that same point.
        state["tlen"][b] = L - 1 + 1 + n
        state["dlen"][b] = min(dlen, len(seq) - 1)
        n_acc[b] = n
        emitted.append(toks)
        margins[b] = min(m_draft, m_ver)
        bands[b] = b_draft + b_ver
    return {"n_accepted": n_acc, "tokens": emitted, "min_margin": margins, "band_prob": bands}


def start(flat_t, cfg_t, flat_d, cfg_d, prompts, max_T_t, max_T_d):
    """State after prefilling each prompt (length >= 2): the target caches its
    first L-1 tokens, the draft its first L-2."""
    tkv, tlen = M.prefill(flat_t, cfg_t, [p[:-1] for p in prompts], max_T_t)
    dkv, dlen = M.prefill(flat_d, cfg_d, [p[:-2] for p in prompts], max_T_d)
    return {"seq": [list(map(int, p)) for p in prompts], "tkv": tkv, "tlen": tlen, "dkv": dkv, "dlen": dlen}


def round_stats(n_accepted, gamma):
    """[P2] section 投機的デコーディングとは (the results table's columns): alpha
    counts accepts among the positions that were tested (a rejection ends the
    tests), accepted/proposed divides by every proposal, and tokens per target
    call is the mean of n + 1."""
    n = np.asarray(n_accepted, dtype=np.float64)
    tested = np.where(n < gamma, n + 1, gamma)
    return {
        "alpha": float(n.sum() / tested.sum()),
        "accepted_per_proposed": float(n.sum() / (gamma * len(n))),
        "tokens_per_target_call": float((n + 1).mean()),
    }
