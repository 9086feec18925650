"""Replay of the V=5 toy of [P3] section 受理・棄却の規則と出力分布が変わらない理由.

The page seeds numpy's ``default_rng(0)`` and, per trial, consumes one uniform
for the draft draw ``choice(V, p=q)``, one for the accept test, and one more
for ``choice(V, p=residual)`` only when the draft is rejected.  numpy's
``Generator.choice`` with ``p`` draws one ``random()`` and maps it by
``searchsorted(cumsum(p)/cumsum(p)[-1], u, side='right')``; the draft draw here
mirrors that library behaviour (it is the harness sampling the draft, not the
verifier).  The verifier's decisions come from the oracle, so the uniform
stream is consumed exactly as the page's program consumes it.

The toy has no bonus draw; when a trial is accepted the oracle still needs a
final uniform (position gamma+1), which is taken from ``default_rng(1)`` and
does not enter the page's statistics.
"""

import numpy as np

from oracle import sampler as S


def build(p, q, N, seed=0, bonus_seed=1):
    p = np.asarray(p, np.float64)
    q = np.asarray(q, np.float64)
    V = len(p)
    zt = np.log(np.stack([p, p]))  # target rows: position 1 and the bonus position
    zd = np.log(q)[None, :]
    rng = np.random.default_rng(seed)
    bonus = np.random.default_rng(bonus_seed)
    cdf_q = np.cumsum(q)
    cdf_q = cdf_q / cdf_q[-1]
    x = np.empty(N, np.int32)
    u = np.empty((N, 2), np.float64)
    first = np.empty(N, np.int64)
    accepted = np.empty(N, bool)
    for i in range(N):
        xi = int(np.searchsorted(cdf_q, rng.random(), side="right"))
        ua = rng.random()
        r = S.verify_sequence(zt, zd, [xi], [ua, 0.5], 1.0)
        if r["n_accepted"] == 0:
            ur = rng.random()
            r = S.verify_sequence(zt, zd, [xi], [ua, ur], 1.0)
        else:
            ur = bonus.random()
        x[i] = xi
        u[i] = (ua, ur)
        first[i] = r["tokens"][0]
        accepted[i] = r["n_accepted"] == 1
    return {"x": x, "u": u, "first_token": first, "accepted": accepted, "V": V}
