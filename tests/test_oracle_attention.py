"""Pins for oracle.attention and oracle.truncate.

* torch's CPU scaled_dot_product_attention (fp64, explicit causal-offset mask,
  KV heads expanded per query-head group) -- an independent library routine;
* cached = uncached: the cached verify rows equal the last rows of a full
  causal recompute over the whole sequence with the pages' additive mask
  ([P2] section numpyで小さなTransformerを自作する and its cached-vs-uncached
  check);
* closed forms: identical keys give the mean of the visible values; a row that
  sees one key returns that key's value; contiguous GQA grouping;
* the cache tail past L_b is never read (it is NaN-poisoned here);
* truncate gives L_b + 1 + n_accepted.
"""

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import truncate as Tr


def _inputs(rng, B, Hq, Hkv, n, D, lens, max_T, poison=True):
    q = rng.normal(size=(B, Hq, n, D))
    kn = rng.normal(size=(B, Hkv, n, D))
    vn = rng.normal(size=(B, Hkv, n, D))
    kc = rng.normal(size=(B, Hkv, max_T, D))
    vc = rng.normal(size=(B, Hkv, max_T, D))
    if poison:
        for b, L in enumerate(lens):
            kc[b, :, L:] = np.nan
            vc[b, :, L:] = np.nan
    return q, kn, vn, kc, vc


def _sdpa(q, kn, vn, kc, vc, lens):
    B, Hq, n, D = q.shape
    Hkv = kn.shape[1]
    out = np.zeros_like(q)
    for b in range(B):
        L = int(lens[b])
        K = torch.from_numpy(np.concatenate([kc[b, :, :L], kn[b]], axis=1))  # [Hkv, L+n, D]
        V = torch.from_numpy(np.concatenate([vc[b, :, :L], vn[b]], axis=1))
        K = K.repeat_interleave(Hq // Hkv, dim=0)
        V = V.repeat_interleave(Hq // Hkv, dim=0)
        keys = torch.arange(L + n)[None, :]
        rows = torch.arange(n)[:, None]
        mask = keys <= (L + rows)  # True = may attend
        o = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q[b]), K, V, attn_mask=mask
        )
        out[b] = o.numpy()
    return out


@pytest.mark.parametrize(
    "B,Hq,Hkv,n,D,lens",
    [
        (3, 4, 2, 5, 16, [0, 7, 33]),
        (2, 8, 1, 9, 8, [1, 64]),
        (2, 4, 4, 5, 24, [384, 100]),
        (1, 6, 3, 1, 32, [17]),
    ],
)
def test_matches_torch_sdpa(B, Hq, Hkv, n, D, lens):
    rng = np.random.default_rng(sum(lens) + D)
    max_T = max(lens) + n + 3
    q, kn, vn, kc, vc = _inputs(rng, B, Hq, Hkv, n, D, lens, max_T)
    got = A.verify_attention(q, kn, vn, kc, vc, np.array(lens))
    want = _sdpa(q, kn, vn, kc, vc, lens)
    assert np.all(np.isfinite(got))  # the poisoned tail was never read
    assert np.max(np.abs(got - want)) < 1e-12


@pytest.mark.parametrize("L,n,H,Hkv", [(384, 5, 4, 4), (0, 3, 2, 1), (50, 9, 8, 2)])
def test_cached_equals_uncached_recompute(L, n, H, Hkv):
    rng = np.random.default_rng(L + n)
    D = 24
    Tt = L + n
    q_all = rng.normal(size=(H, Tt, D))
    k_all = rng.normal(size=(Hkv, Tt, D))
    v_all = rng.normal(size=(Hkv, Tt, D))
    max_T = Tt + 4
    kc = np.full((1, Hkv, max_T, D), np.nan)
    vc = np.full((1, Hkv, max_T, D), np.nan)
    kc[0, :, :L] = k_all[:, :L]
    vc[0, :, :L] = v_all[:, :L]
    cached = A.verify_attention(
        q_all[None, :, L:], k_all[None, :, L:], v_all[None, :, L:], kc, vc, np.array([L])
    )[0]
    uncached = A.attention_uncached(q_all, k_all, v_all, n)
    assert np.max(np.abs(cached - uncached)) < 1e-12


def test_identical_keys_give_mean_of_visible_values():
    rng = np.random.default_rng(1)
    B, Hq, Hkv, n, D, L = 1, 2, 1, 4, 8, 10
    q, kn, vn, kc, vc = _inputs(rng, B, Hq, Hkv, n, D, [L], L + n, poison=False)
    key = rng.normal(size=D)
    kc[:] = key
    kn[:] = key
    got = A.verify_attention(q, kn, vn, kc, vc, np.array([L]))
    Vfull = np.concatenate([vc[0, 0, :L], vn[0, 0]], axis=0)
    for i in range(n):
        want = Vfull[: L + i + 1].mean(axis=0)
        assert np.max(np.abs(got[0, :, i] - want)) < 1e-12


def test_row_with_one_visible_key_returns_its_value():
    rng = np.random.default_rng(2)
    q, kn, vn, kc, vc = _inputs(rng, 1, 3, 1, 5, 16, [0], 8)
    got = A.verify_attention(q, kn, vn, kc, vc, np.array([0]))
    for h in range(3):
        assert np.array_equal(got[0, h, 0], vn[0, 0, 0])


def test_gqa_grouping_is_contiguous():
    rng = np.random.default_rng(3)
    B, Hq, Hkv, n, D, L = 1, 8, 2, 3, 8, 6
    q, kn, vn, kc, vc = _inputs(rng, B, Hq, Hkv, n, D, [L], L + n, poison=False)
    vc[0, 0], vn[0, 0] = 1.0, 1.0
    vc[0, 1], vn[0, 1] = -2.0, -2.0
    got = A.verify_attention(q, kn, vn, kc, vc, np.array([L]))
    assert np.allclose(got[0, :4], 1.0) and np.allclose(got[0, 4:], -2.0)


def test_kv_append_writes_only_new_rows():
    rng = np.random.default_rng(4)
    lens = [3, 0, 9]
    q, kn, vn, kc, vc = _inputs(rng, 3, 2, 2, 4, 8, lens, 16, poison=False)
    k2, v2 = A.kv_append(kc, vc, kn, vn, np.array(lens))
    for b, L in enumerate(lens):
        assert np.array_equal(k2[b, :, L : L + 4], kn[b]) and np.array_equal(v2[b, :, L : L + 4], vn[b])
        keep = np.ones(16, bool)
        keep[L : L + 4] = False
        assert np.array_equal(k2[b, :, keep], kc[b, :, keep])
        assert np.array_equal(v2[b, :, keep], vc[b, :, keep])


def test_truncate_is_base_plus_one_plus_accepted():
    lens = np.array([0, 5, 384, 32768])
    n = np.array([0, 4, 2, 8])
    assert list(Tr.truncate(lens, n)) == [1, 10, 387, 32777]
