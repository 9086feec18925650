"""Pins of the int8 KV-cache oracle.

  * [P2] section PagedAttentionとKVキャッシュの量子化 prints the bytes at 112
    positions of its 4-layer, 4-head, head-dim-24 model: 344,064 in float32,
    93,184 in int8 with a float16 scale per head and position -- 27% of the
    float32 size.  The byte helper must give exactly those numbers.
  * The rounding itself: rows that are integers times a power of two round
    trip exactly; halves round to even; every element is within half a step
    (plus the float16 rounding of the scale) of its converted-back value; the
    largest element of a row codes to +-127; each row's scale depends on that
    row alone; a zero row stays zero.
  * Attention over the converted-back cache stays close to the unquantised
    oracle, and the append stores the quantised new rows at [L, L + n).
"""

import json
import os

import numpy as np
import pytest

from oracle import attention as A
from oracle import formulas as F
from oracle import quant as Q

GOLD = os.path.join(os.path.dirname(__file__), "golden", "kv_bytes.json")


def test_int8_bytes_match_the_page():
    i8 = json.load(open(GOLD))["int8_case"]
    n = Q.kv_cache_bytes_int8(i8["layers"], i8["kv_heads"], i8["head_dim"], i8["T"])
    assert n == i8["bytes"] == 93184
    f32 = F.kv_cache_bytes(i8["layers"], i8["kv_heads"], i8["head_dim"], i8["T"], 4)
    assert f32 == 344064 and round(100 * n / f32) == 27


def test_power_of_two_rows_round_trip_exactly():
    rng = np.random.default_rng(0)
    for e in (-6, -1, 0, 3):
        k = rng.integers(-127, 128, (5, 24))
        k[:, 0] = 127
        x = (k * 2.0**e).astype(np.float32)
        q, s = Q.quantize_rows(x)
        assert np.array_equal(q, k) and np.all(s == np.float16(2.0**e))
        assert np.array_equal(Q.dequantize(q, s), x.astype(np.float64))


def test_halves_round_to_even():
    s = 2.0**-3
    x = np.array([[127 * s, 2.5 * s, 3.5 * s, -2.5 * s, -0.5 * s, 0.5 * s]], np.float32)
    q, _ = Q.quantize_rows(x)
    assert q.tolist() == [[127, 2, 4, -2, 0, 0]]


def test_error_bound_and_granularity():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 4, 17, 128)).astype(np.float32)
    x[1, 2, 5] *= 1000.0  # one loud row
    q, s = Q.quantize_rows(x)
    s32 = np.max(np.abs(x), axis=-1) / np.float32(127)
    back = Q.dequantize(q, s)
    bound = 0.5 * s32 * (1 + 1e-6) + 127 * np.abs(s32 - s.astype(np.float64))
    assert np.all(np.abs(back - x) <= bound[..., None])
    assert np.all(np.max(np.abs(q.astype(int)), axis=-1) == 127)
    q2, s2 = Q.quantize_rows(np.where(np.arange(3)[:, None, None, None] == 1, x / 1000.0, x))
    keep = np.ones((3, 4, 17), bool)
    keep[1] = False
    assert np.array_equal(q2[keep], q[keep]) and np.array_equal(s2[keep], s[keep])


def test_zero_row():
    q, s = Q.quantize_rows(np.zeros((2, 8), np.float32))
    assert np.all(q == 0) and np.all(s == 0)
    assert np.all(Q.dequantize(q, s) == 0)


@pytest.mark.parametrize("lens", [[0, 9, 40], [33, 1, 64]])
def test_attention_over_int8_cache(lens):
    rng = np.random.default_rng(len(lens) + sum(lens))
    B, Hq, Hkv, n, D, T = 3, 8, 2, 5, 64, 80
    q = rng.standard_normal((B, Hq, n, D))
    kn, vn = rng.standard_normal((2, B, Hkv, n, D))
    kc, vc = rng.standard_normal((2, B, Hkv, T, D)).astype(np.float32)
    kq, ks = Q.quantize_rows(kc)
    vq, vs = Q.quantize_rows(vc)
    lens = np.array(lens)
    got = Q.verify_attention_int8(q, kn, vn, kq, ks, vq, vs, lens)
    want = A.verify_attention(q, kn, vn, kc, vc, lens)
    assert np.max(np.abs(got - want)) < 2e-2
    kq2, ks2, vq2, vs2 = Q.kv_append_int8(kq, ks, vq, vs, kn, vn, lens)
    qk, sk = Q.quantize_rows(kn)
    for b, L in enumerate(lens):
        assert np.array_equal(kq2[b, :, L : L + n], qk[b]) and np.array_equal(ks2[b, :, L : L + n], sk[b])
        assert np.array_equal(kq2[b, :, :L], kq[b, :, :L]) and np.array_equal(kq2[b, :, L + n :], kq[b, :, L + n :])
