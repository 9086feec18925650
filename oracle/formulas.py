"""Oracle: closed forms the pages state for the verification step (CPU).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.
"""

import numpy as np


def acceptance_alpha(p, q):
    """Per-position acceptance probability sum_x min(p(x), q(x)).

    [P2] section 受理・棄却の式と出力の分布が変わらない理由 (alpha equals the sum
    of min(p, q), one minus the total-variation distance) and [P3] section
    受理・棄却の規則と出力分布が変わらない理由 (the toy's 0.78).
    """
    return float(np.sum(np.minimum(np.asarray(p, float), np.asarray(q, float))))


def tvd(p, q):
    """Total-variation distance 0.5 * sum |p - q|."""
    return float(0.5 * np.sum(np.abs(np.asarray(p, float) - np.asarray(q, float))))


def expected_committed(alpha, gamma):
    """Expected tokens committed per target call, (1 - alpha^(gamma+1)) / (1 - alpha).

    [P1] section 高速化はどこから来るか：受理長と期待値; [P3] section
    高速化倍率を見積もる式と早見表 (gamma + 1 when alpha = 1).  [P2] prints the
    exponent as "alpha^k+1"; it is read as alpha^(k+1), as the other two pages
    write it.
    """
    alpha = float(alpha)
    if alpha == 1.0:
        return float(gamma + 1)
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def n_accepted_law(alpha, gamma):
    """P(n_accepted = k), k = 0..gamma, when every position has the same alpha.

    The first rejection is geometric and truncated at gamma: alpha^k (1 - alpha)
    for k < gamma and alpha^gamma for k = gamma (the law behind the expected
    value above).
    """
    return np.array([alpha**k * (1 - alpha) for k in range(gamma)] + [alpha**gamma])


def speedup(alpha, gamma, c):
    """Estimated speed-up (1 - alpha^(gamma+1)) / ((1 - alpha)(gamma c + 1)).

    [P2] section 投機的デコーディングを実装して受理率と速度を実測 (the
    flat-verify column, Leviathan et al. Theorem 3.8) and [P3] section
    高速化倍率を見積もる式と早見表; c is the draft/target cost ratio.
    """
    return expected_committed(alpha, gamma) / (gamma * float(c) + 1.0)


def kv_cache_bytes(layers, kv_heads, head_dim, seq_len, elem_bytes, batch=1):
    """KV-cache bytes: layers x 2 x KV heads x head dim x length x bytes x batch.

    [P2] section KVキャッシュのメモリの式と主要モデルの試算.
    """
    return int(layers) * 2 * int(kv_heads) * int(head_dim) * int(seq_len) * int(elem_bytes) * int(batch)
