"""Oracle: verify attention over an int8-quantised KV cache (CPU).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

Follows [P2] section PagedAttentionとKVキャッシュの量子化 (quantisation): every
cached row -- one KV head at one position -- is rounded to int8 with a scale
from that row's largest absolute value, and the scale is kept in float16; the
page reproduces the error by rounding and converting back, and counts the
bytes as the int8 values plus the float16 scales.  The attention is then that
of ``oracle.attention`` (the ``forward_cached`` listing of [P2] section
numpyで小さなTransformerを自作する) on the converted-back cache.

Readings where the pages leave the point open:
  * s = max|x| / 127, q = round-half-even(x / s) clipped to [-127, 127], both
    in float32 (the precision the codes are decided in on both sides, so the
    codes are exact integers to compare); a row of zeros has s = 0, q = 0.
  * The stored scale is float16(s); a row converts back as q * float16(s).
  * The n new rows of a verify call are quantised when they are appended, and
    the call attends to their converted-back values, as to every cached row.
"""

import numpy as np

from . import attention as A
from .bf16 import to_f64


def quantize_rows(x):
    """Rows over the last axis -> (q int8, s float16)."""
    x32 = np.asarray(to_f64(x), np.float32)
    a = np.max(np.abs(x32), axis=-1, keepdims=True)
    s32 = a / np.float32(127.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(s32 > 0, np.rint(x32 / s32), np.float32(0.0))
    q = np.clip(q, -127, 127).astype(np.int8)
    return q, s32[..., 0].astype(np.float16)


def dequantize(q, s):
    """q * s in fp64 (s broadcast over the last axis of q)."""
    return np.asarray(q, np.float64) * np.asarray(s, np.float64)[..., None]


def kv_append_int8(kq, ks, vq, vs, k_new, v_new, lens):
    """Copies of the int8 caches and scales with the quantised new rows at [L_b, L_b + n)."""
    kq, ks, vq, vs = kq.copy(), ks.copy(), vq.copy(), vs.copy()
    n = k_new.shape[2]
    qk, sk = quantize_rows(k_new)
    qv, sv = quantize_rows(v_new)
    for b, L in enumerate(lens):
        L = int(L)
        kq[b, :, L : L + n], ks[b, :, L : L + n] = qk[b], sk[b]
        vq[b, :, L : L + n], vs[b, :, L : L + n] = qv[b], sv[b]
    return kq, ks, vq, vs


def verify_attention_int8(q, k_new, v_new, kq, ks, vq, vs, lens, scale=None, seqs=None):
    """Verify attention over the converted-back int8 cache, the new rows quantised too."""
    k_cache = dequantize(kq, ks)
    v_cache = dequantize(vq, vs)
    qk, sk = quantize_rows(k_new)
    qv, sv = quantize_rows(v_new)
    return A.verify_attention(q, dequantize(qk, sk), dequantize(qv, sv), k_cache, v_cache, lens, scale=scale,
                              seqs=seqs)


def kv_cache_bytes_int8(layers, kv_heads, head_dim, seq_len, batch=1):
    """int8 values plus one float16 scale per (layer, K/V, head, position)."""
    return int(layers) * 2 * int(kv_heads) * int(seq_len) * (int(head_dim) + 2) * int(batch)
