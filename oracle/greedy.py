"""Oracle: greedy (temperature 0) verification of one round (CPU).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

What is computed, per sequence, following
  [P2] section 投機的デコーディングとは: the verify listing leaves out its
       temperature-0 branch, and the results that follow it state what that
       branch does -- a draft is accepted when it equals the target's argmax,
       and the output is then identical to greedy decoding with the target alone;
  [P2] the same listing for the structure of the round (one target call over
       the last committed token plus the drafts, stop at the first rejection,
       one more token, length reset to base + 1 + n).

  a_i = (argmax_v z_t[i, v] == x_i)            for i = 0 .. gamma-1
  n   = number of leading true a_i
  t   = argmax_v z_t[n, v]                     (the correction at the first
                                                rejection, or the bonus token)
  emitted tokens = x_0 .. x_{n-1}, t;   n_accepted = n

Readings of points the pages leave open:
  * argmax is numpy's: the first index of the largest value; a NaN counts as
    the largest (the first NaN wins), as np.argmax does.
  * softmax(z / T) is monotone in z for T > 0, so the argmax of the logits is
    the argmax of p at any temperature; greedy verification reads no draft
    logits and no uniforms.
  * The greedy p_i(x_i) is the one-hot distribution's mass at x_i: 1.0 when
    x_i is the argmax, else 0.0.
"""

import numpy as np

from .bf16 import to_f64


def argmax(z):
    """First index of the largest value of a logit row (numpy's argmax, NaN largest)."""
    return int(np.argmax(to_f64(z)))


def verify_sequence(z_target, x):
    """One sequence: z_target [gamma+1, V] logits, x [gamma] drafts.

    Returns (n_accepted, tokens) with tokens = x_0 .. x_{n-1}, t.
    """
    g = len(x)
    n = 0
    for i in range(g):
        if argmax(z_target[i]) != int(x[i]):
            break
        n += 1
    t = argmax(z_target[n])
    return n, [int(v) for v in x[:n]] + [t]


def verify_batch(z_target, x):
    """Batch form: z_target [B, gamma+1, V], x [B, gamma].

    Returns n_accepted int32 [B], out_tokens int32 [B, gamma+1] (n+1 valid
    tokens, then -1) and p_x float64 [B, gamma] (1.0 where x_i is the target's
    argmax, else 0.0).
    """
    B, g = x.shape
    n_acc = np.zeros(B, np.int32)
    out = np.full((B, g + 1), -1, np.int32)
    p_x = np.zeros((B, g), np.float64)
    for b in range(B):
        n, toks = verify_sequence(z_target[b], x[b])
        n_acc[b] = n
        out[b, : n + 1] = toks
        for i in range(g):
            p_x[b, i] = 1.0 if argmax(z_target[b, i]) == int(x[b, i]) else 0.0
    return n_acc, out, p_x
