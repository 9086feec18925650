"""Oracle: modified rejection sampling for one verification round (fp64, CPU).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

What is computed, per sequence, following
  [P1] section 受理判定の数理：修正版棄却サンプリング (the accept/reject rule and
       why the correction distribution is max(0, p - q)),
  [P2] section 投機的デコーディングとは (the verify listing: one target call over
       the last committed token plus the drafts, the accept loop that stops at the
       first rejection, the residual or bonus draw, the emitted tokens and the
       length reset),
  [P3] section 受理・棄却の規則と出力分布が変わらない理由 (the five-step round,
       including the bonus token from position gamma+1, and the V=5 toy):

  p_i = softmax(z_t[i] / T)   for the gamma+1 target rows i = 0..gamma
  q_i = softmax(z_d[i] / T)   for the gamma draft rows   i = 0..gamma-1
  n = number of leading positions i with u[i] < min(1, p_i(x_i) / q_i(x_i))
  if n < gamma: w = max(0, p_n - q_n)      (residual at the first rejection)
  else:         w = p_gamma                (bonus token)
  t = smallest j with C_j / C_{V-1} > u[gamma],  C = inclusive prefix sum of w
  emitted tokens = x_0 .. x_{n-1}, t;   n_accepted = n

Readings of points the pages leave open:
  * u[i] in [0, 1), one per judged position, drives the test at i; u[gamma]
    drives the final draw in either branch.
  * The test is the IEEE comparison u < min(1, p/q) with NaN propagating through
    the min: q = 0 < p gives p/q = inf and accepts; p = q = 0 gives NaN and
    rejects.
  * ``rng.choice(p=w)`` on the pages is read as inverse-CDF sampling in token
    order with numpy's convention (cumsum normalised by its last element,
    searchsorted side='right').  Zero-mass tokens are never chosen.
  * If the residual mass is exactly zero after a rejection (only reachable
    through rounding), the draw falls back to p_n.
  * softmax(z / T) applies to both target and draft logits, T > 0, computed with
    the maximum subtracted.  Sums are never assumed to be 1: every distribution
    is divided by its own computed mass.
"""

import numpy as np

from .bf16 import to_f64

# Decisions whose uniform lies closer than this to its threshold are counted,
# not compared, between the GPU and this oracle (fp32 versus fp64 rounding may
# flip them; [P3] section 受理・棄却の規則と出力分布が変わらない理由 notes that
# floating-point differences can change such outputs).
BAND = 1e-6


def softmax_t(z, temperature):
    """softmax(z / T) in fp64 with the maximum subtracted; T > 0."""
    z = to_f64(z) / float(temperature)
    e = np.exp(z - np.max(z))
    return e / np.sum(e)


def accept_threshold(p_x, q_x):
    """min(1, p(x)/q(x)) with IEEE semantics (NaN for 0/0 propagates)."""
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.float64(p_x) / np.float64(q_x)
    return np.minimum(np.float64(1.0), ratio)


def accepts(u, threshold):
    """The strict accept test u < threshold (a NaN threshold never accepts)."""
    return bool(np.float64(u) < threshold)


def residual(p, q):
    """Unnormalised correction distribution max(0, p - q)."""
    return np.maximum(p - q, 0.0)


def inverse_cdf(w, u):
    """Token index drawn from the unnormalised weights ``w`` by uniform ``u``.

    The smallest j with C_j / C_last > u, C the inclusive prefix sum of w.
    """
    c = np.cumsum(w)
    return int(np.searchsorted(c / c[-1], np.float64(u), side="right"))


def cdf_margin(w, t, u):
    """Distance of ``u`` from the two CDF boundaries of token ``t``.

    Returns min(|u - C_{t-1}/C_last|, |u - C_t/C_last|) with C_{-1} = 0.  The
    GPU parity rule exempts draws with a margin below 1e-6.  Since the draw
    puts u in [C_{t-1}/C_last, C_t/C_last), this is the distance from u to the
    nearest point of {0, C_0/C_last, ..., C_last/C_last}: the smallest shift of
    u that changes the drawn token or leaves [0, 1).
    """
    c = np.cumsum(w)
    c = c / c[-1]
    lo = c[t - 1] if t > 0 else 0.0
    hi = c[t]
    return float(min(abs(u - lo), abs(u - hi)))


def accept_margin(u, threshold):
    """Distance of ``u`` from the accept threshold min(1, p/q): the smallest
    shift of u that changes the strict test.  A NaN threshold rejects every u,
    so no shift changes it: the margin is infinite."""
    m = abs(np.float64(u) - np.float64(threshold))
    return float("inf") if np.isnan(m) else float(m)


def accept_band_probability(threshold, eps):
    """Probability that a uniform u on [0, 1) lands within ``eps`` of the accept
    threshold: the length of (thr - eps, thr + eps) inside [0, 1)."""
    thr = np.float64(threshold)
    if np.isnan(thr):
        return 0.0
    return float(max(0.0, min(1.0, thr + eps) - max(0.0, thr - eps)))


def band_probability(w, eps):
    """Probability that a uniform u on [0, 1) gives an inverse-CDF draw from the
    weights ``w`` whose ``cdf_margin`` is below ``eps``.

    That is the length of the set of u in [0, 1) within ``eps`` of a point of
    {0, C_0/C_last, ..., C_last/C_last} (the union of the intervals of
    half-width eps around the CDF boundaries, clipped to [0, 1)).  Used to
    bound how many sequences the 1e-6 band may take out of a comparison.
    """
    c = np.cumsum(np.asarray(w, dtype=np.float64))
    pts = np.concatenate(([0.0], c / c[-1]))
    lo = np.maximum(pts - eps, 0.0)
    hi = np.minimum(pts + eps, 1.0)
    # The points are sorted, so both ends of the intervals are too: interval i
    # adds what reaches past the end of interval i-1.
    new = np.maximum(hi[1:] - np.maximum(lo[1:], hi[:-1]), 0.0)
    return float(hi[0] - lo[0] + np.sum(new))


def verify_sequence(z_target, z_draft, draft_tokens, uniforms, temperature):
    """One verification round for one sequence.

    z_target      [gamma+1, V] target logits (any float width or bf16 bits)
    z_draft       [gamma, V]   draft logits
    draft_tokens  [gamma]      x_0..x_{gamma-1}, each in [0, V)
    uniforms      [gamma+1]    fp64 in [0, 1)
    Returns a dict with n_accepted, tokens (length n+1), p_x and q_x (the target
    and draft probabilities of every draft token), and margins: the distance of
    every decisive uniform from its threshold (accept tests that were evaluated,
    then the final draw), plus whether the zero-residual fallback fired.
    ``band_prob`` sums, over the same decisions, the probability that a uniform
    lands within BAND of the threshold (an upper bound on the chance that this
    sequence falls inside the band, given the decisions it took).
    """
    gamma = len(draft_tokens)
    z_target = to_f64(z_target)
    z_draft = to_f64(z_draft)
    assert z_target.shape[0] == gamma + 1 and z_draft.shape[0] == gamma
    p = [softmax_t(z_target[i], temperature) for i in range(gamma + 1)]
    q = [softmax_t(z_draft[i], temperature) for i in range(gamma)]
    x = [int(v) for v in draft_tokens]
    p_x = np.array([p[i][x[i]] for i in range(gamma)], dtype=np.float64)
    q_x = np.array([q[i][x[i]] for i in range(gamma)], dtype=np.float64)

    n = 0
    accept_margins, band_prob = [], 0.0
    for i in range(gamma):
        thr = accept_threshold(p_x[i], q_x[i])
        accept_margins.append(accept_margin(uniforms[i], thr))
        band_prob += accept_band_probability(thr, BAND)
        if not accepts(uniforms[i], thr):
            break
        n += 1

    fallback = False
    if n < gamma:
        w = residual(p[n], q[n])
        if np.sum(w) == 0.0:
            w = p[n]
            fallback = True
    else:
        w = p[gamma]
    t = inverse_cdf(w, uniforms[gamma])
    return {
        "n_accepted": n,
        "tokens": x[:n] + [t],
        "p_x": p_x,
        "q_x": q_x,
        "accept_margins": accept_margins,
        "draw_margin": cdf_margin(w, t, float(uniforms[gamma])),
        "band_prob": band_prob + band_probability(w, BAND),
        "fallback": fallback,
    }


def verify_batch(z_target, z_draft, draft_tokens, uniforms, temperature, seqs=None):
    """``verify_sequence`` for every sequence b (or those listed in ``seqs``).

    Shapes: z_target [B, gamma+1, V], z_draft [B, gamma, V], draft_tokens
    [B, gamma], uniforms [B, gamma+1].  Returns arrays n_accepted [S],
    out_tokens [S, gamma+1] (n+1 valid tokens then -1), p_x/q_x [S, gamma],
    min_margin [S] (smallest decisive margin of the sequence), band_prob [S]
    and fallback [S].
    """
    B, gamma = np.asarray(draft_tokens).shape
    seqs = range(B) if seqs is None else list(seqs)
    S = len(seqs)
    n_acc = np.zeros(S, dtype=np.int32)
    out = np.full((S, gamma + 1), -1, dtype=np.int32)
    p_x = np.zeros((S, gamma))
    q_x = np.zeros((S, gamma))
    margin = np.zeros(S)
    band_prob = np.zeros(S)
    fallback = np.zeros(S, dtype=bool)
    for k, b in enumerate(seqs):
        r = verify_sequence(z_target[b], z_draft[b], draft_tokens[b], uniforms[b], temperature)
        n_acc[k] = r["n_accepted"]
        out[k, : len(r["tokens"])] = r["tokens"]
        p_x[k] = r["p_x"]
        q_x[k] = r["q_x"]
        margin[k] = min(r["accept_margins"] + [r["draw_margin"]])
        band_prob[k] = r["band_prob"]
        fallback[k] = r["fallback"]
    return {
        "n_accepted": n_acc,
        "out_tokens": out,
        "p_x": p_x,
        "q_x": q_x,
        "min_margin": margin,
        "band_prob": band_prob,
        "fallback": fallback,
    }
