"""Pins for oracle.formulas against values the pages print.

The k-sweep tables print alpha to 3 decimals and E / the flat-verify factor to
2, so each check is an interval check: the formula evaluated over the rounding
interval of its inputs must reach the printed value's rounding interval.  A
wrong exponent (alpha^k instead of alpha^(k+1)) or a dropped cost term fails
most rows.
"""

import json
import os

import numpy as np
import pytest

from oracle import formulas as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _interval(fn, lo, hi, n=41):
    vals = [fn(a) for a in np.linspace(lo, hi, n)]
    return min(vals), max(vals)


@pytest.mark.parametrize("row", _load("p2_ksweep.json")["rows"], ids=lambda r: f"T{r['T']}-k{r['k']}")
def test_expected_tokens_matches_printed_ksweep(row):
    a, k = row["alpha"], row["k"]
    lo, hi = _interval(lambda x: F.expected_committed(x, k), a - 5e-4, a + 5e-4)
    assert lo - 5e-3 - 1e-12 <= row["E"] <= hi + 5e-3 + 1e-12, (lo, hi, row)


@pytest.mark.parametrize("row", _load("p2_ksweep.json")["rows"], ids=lambda r: f"T{r['T']}-k{r['k']}")
def test_flat_verify_factor_matches_printed_ksweep(row):
    a, k = row["alpha"], row["k"]
    vals = [
        F.speedup(x, k, c)
        for x in np.linspace(a - 5e-4, a + 5e-4, 21)
        for c in np.linspace(0.215, 0.225, 21)
    ]
    assert min(vals) - 5e-3 <= row["factor"] <= max(vals) + 5e-3, (min(vals), max(vals), row)


def test_expected_tokens_worked_value_alpha_half():
    # [P2] section 投機的デコーディングが効く場面・効かない場面: alpha = 0.5 and
    # k = 4 give about 1.94 tokens per target call.
    assert round(F.expected_committed(0.5, 4), 2) == 1.94
    assert F.expected_committed(0.5, 4) == 1.9375


def test_expected_tokens_alpha_one_is_gamma_plus_one():
    # [P3] section 高速化倍率を見積もる式と早見表: gamma + 1 when alpha = 1.
    for g in range(1, 10):
        assert F.expected_committed(1.0, g) == g + 1
        assert abs(F.expected_committed(1 - 1e-9, g) - (g + 1)) < 1e-6


def test_quick_reference_speedups():
    # [P3] section 高速化倍率を見積もる式と早見表: alpha = 0.6, c = 0.05 gives
    # 1.91 at gamma = 5 and 1.77 at gamma = 8; with c = 0.3, gamma = 5 is below 1.
    assert round(F.speedup(0.6, 5, 0.05), 2) == 1.91
    assert round(F.speedup(0.6, 8, 0.05), 2) == 1.77
    assert F.speedup(0.6, 5, 0.3) < 1.0


def test_n_accepted_law_sums_to_one_and_gives_expectation():
    for alpha in (0.0, 0.3, 0.78, 0.99):
        for g in (1, 2, 4, 8):
            law = F.n_accepted_law(alpha, g)
            assert abs(law.sum() - 1) < 1e-14
            # E[n_accepted + 1] equals the expected committed tokens.
            assert abs(np.dot(np.arange(g + 1) + 1, law) - F.expected_committed(alpha, g)) < 1e-12


def test_alpha_is_one_minus_tvd_for_toy():
    # [P3]: the toy's acceptance rate and 1 - TVD(p, q) both print as 0.78.
    g = _load("p3_toy_v5.json")
    a = F.acceptance_alpha(g["p"], g["q"])
    assert abs(a - (1 - F.tvd(g["p"], g["q"]))) < 1e-15
    assert round(a, 3) == g["printed_one_minus_tvd_round3"]


def test_kv_cache_bytes_printed_values():
    gold = _load("kv_bytes.json")
    for c in gold["cases"]:
        nbytes = F.kv_cache_bytes(c["layers"], c["kv_heads"], c["head_dim"], c["T"], c["elem_bytes"], c["batch"])
        if "bytes" in c:
            assert nbytes == c["bytes"]
        if "mib" in c:
            assert round(nbytes / 2**20, 1) == c["mib"]
        if "kib" in c:
            assert nbytes / 2**10 == c["kib"]
        if "gib" in c:
            assert nbytes / 2**30 == c["gib"]
    # int8 cache: one byte per element plus one fp16 scale per (layer, K/V, head, position).
    i8 = gold["int8_case"]
    body = F.kv_cache_bytes(i8["layers"], i8["kv_heads"], i8["head_dim"], i8["T"], 1)
    scales = F.kv_cache_bytes(i8["layers"], i8["kv_heads"], 1, i8["T"], 2)
    assert body + scales == i8["bytes"]
