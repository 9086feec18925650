"""Helpers for GPU parity tests: host <-> device marshalling and the comparison rules.

Rules (from the verification step's statement of parity):
  * n_accepted and emitted tokens must be identical given the same uniforms,
    except sequences with a decisive draw within 1e-6 of its threshold (the
    accept test's min(1, p/q) or a CDF boundary of the drawn token, measured
    on the oracle's values); those are counted and reported, not compared;
  * p_i(x_i), q_i(x_i) within 1e-5 relative (fp32 outputs);
  * attention within 1e-4 absolute (fp32) or 2e-2 absolute (bf16), and for
    16-bit outputs every row within 2u of the oracle's row in the 2-norm
    (ROW_REL_TOL below).
"""

import numpy as np
import torch

from oracle import bf16 as obf16

BAND = 1e-6
P_RTOL = 1e-5
# fp16: the probabilities are rounded to fp16 for the PV product (2^-11
# relative, against |v| <= 5 for N(0,1) rows: <= 2.5e-3) and the output to
# fp16 (2^-11 relative on |o| <= 2: <= 1e-3), so 5e-3 absolute.
ATT_TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 5e-3}


# Per output row (one head at one verify position: D values), the error
# relative to the row's own size.  Two roundings of relative size at most u
# each reach the output: the probabilities fed to the PV product and the
# output itself (u = 2^-8 for bf16, 2^-11 for fp16), so rows must agree within
# 2u in the 2-norm.  An emulation of those roundings on the CPU stays below
# 0.0027 (bf16) and 0.0004 (fp16) at lengths 0 to 32,768, while one 32-key
# block left out of a 32,768-key cache moves every row of its KV head by more
# than 0.012 relative: the absolute bound alone (2e-2 against outputs of
# size 0.02-0.05 at those lengths) could not see it.
ROW_REL_TOL = {"bf16": 2.0**-7, "f16": 2.0**-10}


def row_rel_err(got, want):
    """Largest ||got - want||_2 / ||want||_2 over rows (the last axis)."""
    d = np.linalg.norm(np.asarray(got, np.float64) - want, axis=-1)
    w = np.linalg.norm(want, axis=-1)
    return float(np.max(np.where(d == 0, 0.0, d / np.maximum(w, 1e-300))))


def check_attention(got, want, dtype):
    """Element-wise absolute bound (ATT_TOL) and, for 16-bit outputs, the
    row-relative bound (ROW_REL_TOL).  Returns (max abs err, max row rel err)."""
    got = np.asarray(got, np.float64)
    assert np.all(np.isfinite(got)), "non-finite attention output"
    err = float(np.max(np.abs(got - want))) if got.size else 0.0
    rel = row_rel_err(got, want) if got.size else 0.0
    print(f"max abs err {err:.3g}, max row rel err {rel:.3g}", flush=True)
    assert err < ATT_TOL[dtype], ("absolute", err)
    if dtype in ROW_REL_TOL:
        assert rel < ROW_REL_TOL[dtype], ("row-relative", rel)
    return err, rel


from workloads.device import to_dev, to_host  # noqa: E402,F401


def as_f64(a):
    return obf16.to_f64(a)


def band_bound(expected):
    """Largest number of sequences the band may take out of one comparison.

    Whether a sequence falls in the band is a Bernoulli draw of probability at
    most its oracle ``band_prob`` (the length of the band around each decision
    it took), so the count has mean at most ``expected``; the bound adds five
    Poisson standard deviations and three.  A margin helper that returned 0
    would exclude every sequence and fail this.
    """
    return int(np.floor(expected + 5.0 * np.sqrt(expected) + 3.0))


def compare_sampler(orc, n_gpu, tok_gpu, p_gpu=None, q_gpu=None, seqs=None):
    """Compare GPU sampler outputs with the oracle's (``oracle.sampler.verify_batch``).

    Returns a dict of counts; asserts that the band holds no more sequences than
    ``band_bound`` allows, that no sequence outside the band differs, and that
    p/q agree within P_RTOL.
    """
    seqs = np.arange(len(n_gpu)) if seqs is None else np.asarray(seqs)
    n_g = np.asarray(n_gpu)[seqs]
    t_g = np.asarray(tok_gpu)[seqs]
    band = orc["min_margin"] < BAND
    same = (n_g == orc["n_accepted"]) & np.all(t_g == orc["out_tokens"], axis=1)
    bad = ~same & ~band
    expected = float(np.sum(orc["band_prob"]))
    stats = {
        "sequences": int(len(seqs)),
        "in_band": int(band.sum()),
        "band_expected": expected,
        "band_bound": band_bound(expected),
        "band_disagree": int((~same & band).sum()),
        "mismatch_outside_band": int(bad.sum()),
        "fallback": int(orc["fallback"].sum()),
    }
    print(f"[compare_sampler] {stats}", flush=True)
    assert stats["in_band"] <= stats["band_bound"], ("more sequences in the band than its bound", stats)
    assert not bad.any(), (stats, np.nonzero(bad)[0][:10], n_g[bad][:5], orc["n_accepted"][bad][:5])
    for got, want, name in ((p_gpu, orc["p_x"], "p"), (q_gpu, orc["q_x"], "q")):
        if got is None:
            continue
        g = np.asarray(got, np.float64)[seqs]
        ok = np.isclose(g, want, rtol=P_RTOL, atol=1e-37) | (np.isnan(g) & np.isnan(want))
        assert ok.all(), (name, np.nonzero(~ok)[:5], g[~ok][:5], want[~ok][:5])
    return stats
