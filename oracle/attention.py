"""Oracle: KV append and causal multi-query verify attention (fp64, CPU).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

Follows [P2] section numpyで小さなTransformerを自作する (the ``KVCache`` class
and the ``forward_cached`` listing): the n new tokens' K and V are written at
rows [p0, p0+n) of the cache, where p0 is the cache length before the call;
the i-th new query attends to cache rows [0, p0+i] (the causal offset of the
upper-triangular mask); scores are scaled by 1/sqrt(D) and soft-maxed per row.
Grouped-query sharing ([P2] section GQA・MQAでKVキャッシュを減らす): several
query heads read one KV head; head h uses KV head h // (Hq / Hkv).

Layouts (all fp64 here; inputs of any float width or bf16 bits):
  q                 [B, Hq,  n, D]
  k_new, v_new      [B, Hkv, n, D]
  k_cache, v_cache  [B, Hkv, max_T, D]   rows >= lens[b] are never read
  lens              [B]  committed length L_b before the call
"""

import numpy as np

from .bf16 import to_f64


def visible_keys(L, i):
    """Number of keys query row i (0-based among the new rows) may see: L+i+1."""
    return L + i + 1


def softmax_rows(s):
    """Row-wise softmax with the row maximum subtracted."""
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def kv_append(k_cache, v_cache, k_new, v_new, lens):
    """Return copies of the caches with the new rows written at [L_b, L_b+n).

    The pages' cache keeps the stored dtype; the oracle returns the caches in
    their input dtype with the new rows copied bit for bit.
    """
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    n = np.asarray(k_new).shape[2]
    for b, L in enumerate(np.asarray(lens)):
        L = int(L)
        k_out[b, :, L : L + n] = k_new[b]
        v_out[b, :, L : L + n] = v_new[b]
    return k_out, v_out


def verify_attention(q, k_new, v_new, k_cache, v_cache, lens, scale=None, seqs=None):
    """Attention output [S, Hq, n, D] (fp64) for the sequences in ``seqs``.

    For each b, KV head g and query head h in g's group, row i:
      K_full = k_cache[b, g, :L_b] followed by k_new[b, g]   (the append)
      s      = q[b, h, i] . K_full[: L_b+i+1]^T * scale
      out    = softmax(s) . V_full[: L_b+i+1]
    """
    B, Hq, n, D = np.asarray(q).shape
    Hkv = np.asarray(k_new).shape[1]
    assert Hq % Hkv == 0
    group = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    seqs = range(B) if seqs is None else list(seqs)
    out = np.zeros((len(seqs), Hq, n, D))
    for k, b in enumerate(seqs):
        L = int(lens[b])
        for g in range(Hkv):
            K = np.concatenate([to_f64(k_cache[b, g, :L]), to_f64(k_new[b, g])], axis=0)
            V = np.concatenate([to_f64(v_cache[b, g, :L]), to_f64(v_new[b, g])], axis=0)
            for h in range(g * group, (g + 1) * group):
                Q = to_f64(q[b, h])
                for i in range(n):
                    m = visible_keys(L, i)
                    s = (K[:m] @ Q[i]) * scale
                    w = softmax_rows(s[None, :])[0]
                    out[k, h, i] = w @ V[:m]
    return out


def attention_uncached(q_all, k_all, v_all, n_last, scale=None):
    """Full causal attention over a whole sequence; keep the last ``n_last`` rows.

    This is the recompute without a cache that the cached path must equal
    ([P2] section numpyで小さなTransformerを自作する: the uncached version runs
    the same computation over every token of the sequence).  It uses the pages'
    additive mask: -1e9 strictly above the diagonal of the square score matrix.

    q_all [H, T, D], k_all / v_all [Hkv, T, D]; returns [H, n_last, D].
    """
    H, T, D = q_all.shape
    Hkv = k_all.shape[0]
    group = H // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    mask = np.triu(np.full((T, T), -1e9), 1)
    out = np.zeros((H, n_last, D))
    for h in range(H):
        g = h // group
        s = (to_f64(q_all[h]) @ to_f64(k_all[g]).T) * scale + mask
        out[h] = (softmax_rows(s) @ to_f64(v_all[g]))[T - n_last :]
    return out
