"""Exact outcome law of the oracle sampler, extracted by treating it as a black box.

For fixed logits and a fixed draft tuple, the oracle's decisions are threshold
functions of the uniforms: position i is accepted iff u[i] lies below some
theta_i, and the final token is a non-decreasing step function of u[gamma]
(inverse-CDF sampling).  The thresholds and the step boundaries are found by
bisection on the oracle itself, so the law below is the oracle's own law, not a
re-derivation of the pages' formulas.  Masses are exact to about 2^-50.
"""

import itertools

import numpy as np

from oracle import sampler as S

_ITERS = 60
_BELOW_ONE = float(np.nextafter(1.0, 0.0))


def _n_acc(zt, zd, x, u, T):
    return S.verify_sequence(zt, zd, x, u, T)["n_accepted"]


def _token(zt, zd, x, u, T):
    return S.verify_sequence(zt, zd, x, u, T)["tokens"][-1]


def _sup_true(pred):
    """sup{u in [0,1): pred(u)} for a predicate true on [0, a) and false after."""
    if not pred(0.0):
        return 0.0
    lo, hi = 0.0, 1.0
    for _ in range(_ITERS):
        mid = min(0.5 * (lo + hi), _BELOW_ONE)  # uniforms live in [0, 1)
        if mid <= lo:
            break
        if pred(mid):
            lo = mid
        else:
            hi = mid
    return hi  # 1.0 when the predicate never turned false


def _token_masses(fn, V):
    """Masses of a non-decreasing step function t(u) on [0, 1) -> {0..V-1}."""
    cuts = [0.0]
    for v in range(V - 1):
        cuts.append(_sup_true(lambda u, v=v: fn(u) <= v))
    cuts.append(1.0)
    cuts = np.maximum.accumulate(np.array(cuts))
    return np.diff(cuts)


def draft_tuple_law(zt, zd, x, T):
    """For one draft tuple: (P(n = k) for k = 0..gamma, token law per branch k)."""
    gamma = len(x)
    V = zt.shape[1]
    theta = []
    for i in range(gamma):
        base = [0.0] * i  # accept every earlier position (reachable only if theta_j > 0)
        th = _sup_true(lambda a: _n_acc(zt, zd, x, base + [a] + [0.0] * (gamma - i), T) > i)
        theta.append(th)
        if th == 0.0:
            break
    theta += [0.0] * (gamma - len(theta))
    p_branch = np.zeros(gamma + 1)
    tok = np.zeros((gamma + 1, V))
    reach = 1.0
    for k in range(gamma + 1):
        if k < gamma:
            p_branch[k] = reach * (1.0 - theta[k])
        else:
            p_branch[k] = reach
        if p_branch[k] > 0:
            # uniforms that realise branch k: accept below k, reject at k
            pre = [0.0] * k + ([np.nextafter(1.0, 0.0)] if k < gamma else [])
            pre = pre + [0.0] * (gamma - len(pre))
            tok[k] = _token_masses(lambda w: _token(zt, zd, x, pre + [w], T), V)
        if k < gamma:
            reach *= theta[k]
    return p_branch, tok


def full_law(zt, zd, q_rows, T):
    """Enumerate every draft tuple x (weight prod_i q_i(x_i)).

    Returns:
      first[v]              P(first emitted token = v)
      pos[k][v]             P(position k is emitted and equals v), k = 0..gamma
      reach[k]              P(n_accepted >= k)
      n_law[k]              P(n_accepted = k)
    """
    gamma = zd.shape[0]
    V = zt.shape[1]
    pos = np.zeros((gamma + 1, V))
    n_law = np.zeros(gamma + 1)
    for x in itertools.product(range(V), repeat=gamma):
        w = np.prod([q_rows[i][x[i]] for i in range(gamma)])
        if w == 0:
            continue
        pb, tok = draft_tuple_law(zt, zd, list(x), T)
        n_law += w * pb
        for k in range(gamma + 1):
            # n = k: positions 0..k-1 emit the drafts, position k emits the draw
            for j in range(k):
                pos[j, x[j]] += w * pb[k]
            pos[k] += w * pb[k] * tok[k]
    reach = np.array([n_law[k:].sum() for k in range(gamma + 1)])
    return {"first": pos[0], "pos": pos, "reach": reach, "n_law": n_law}
