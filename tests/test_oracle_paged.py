"""Pins of the paged-cache oracle.

  * [P2] section PagedAttentionとKVキャッシュの量子化 counts the allocation
    waste of 1,000 requests with lengths uniform in [50, 2047]: 47.2% when
    every request reserves 2,048 positions, 0.7% with 16-position blocks and
    1.4% with 32-position blocks.  The page's draw is not reproducible, so
    the waste helper is checked against those figures over many seeded draws
    of the same recipe (the printed value must lie inside the spread), and
    against exact counts on constructed lengths.
  * Paging does not change attention: a cache split into pages through any
    block table (identity, permuted, with shared prefix pages) gives the
    contiguous oracle's output; the append lands in the pages the table
    names; unused page slots are never read.
"""

import numpy as np
import pytest

from oracle import attention as A
from oracle import paged as P


def _draws(seeds=200):
    return [np.random.default_rng(s).integers(50, 2048, 1000) for s in range(seeds)]


@pytest.mark.parametrize("kind,printed", [("prealloc", 0.472), (16, 0.007), (32, 0.014)])
def test_allocation_waste_matches_the_page(kind, printed):
    w = np.array([P.allocation_waste(L, prealloc=2048) if kind == "prealloc" else P.allocation_waste(L, page=kind)
                  for L in _draws()])
    half_step = 0.0005  # printed to 0.1%
    assert w.min() - half_step <= printed <= w.max() + half_step, (w.min(), w.mean(), w.max())


def test_allocation_waste_exact_counts():
    assert P.blocks_needed(0, 16) == 0 and P.blocks_needed(1, 16) == 1 and P.blocks_needed(16, 16) == 1
    assert P.blocks_needed(17, 16) == 2
    # lengths 1..32 in 16-blocks: 48 blocks = 768 slots for 528 positions
    L = np.arange(1, 33)
    assert np.isclose(P.allocation_waste(L, page=16), 1 - 528 / ((16 * 1 + 16 * 2) * 16))
    assert np.isclose(P.allocation_waste([2048, 1024], prealloc=2048), 0.25)


def _contiguous_case(B=3, Hq=4, Hkv=2, n=3, D=8, page=4, lens=(0, 5, 13), seed=0):
    rng = np.random.default_rng(seed)
    max_T = max(lens) + n + page
    q = rng.standard_normal((B, Hq, n, D))
    kn = rng.standard_normal((B, Hkv, n, D))
    vn = rng.standard_normal((B, Hkv, n, D))
    kc = rng.standard_normal((B, Hkv, max_T, D))
    vc = rng.standard_normal((B, Hkv, max_T, D))
    return q, kn, vn, kc, vc, np.array(lens), page


def _paginate(cache, page, perm):
    """Pages [Hkv, num_pages, page, D] and block table holding `cache` [B, Hkv, T, D];
    block (b, i) goes to page perm[b * nb + i]."""
    B, Hkv, T, D = cache.shape
    nb = T // page
    pages = np.full((Hkv, B * nb, page, D), np.nan)
    table = np.zeros((B, nb), np.int32)
    for b in range(B):
        for i in range(nb):
            p = perm[b * nb + i]
            pages[:, p] = cache[b, :, i * page : (i + 1) * page]
            table[b, i] = p
    return pages, table


@pytest.mark.parametrize("permute", [False, True])
def test_paging_does_not_change_attention(permute):
    q, kn, vn, kc, vc, lens, page = _contiguous_case()
    T = kc.shape[2] // page * page
    kc, vc = kc[:, :, :T], vc[:, :, :T]
    nb = T // page
    perm = np.random.default_rng(1).permutation(3 * nb) if permute else np.arange(3 * nb)
    kp, table = _paginate(kc, page, perm)
    vp, _ = _paginate(vc, page, perm)
    want = A.verify_attention(q, kn, vn, kc, vc, lens)
    got = P.verify_attention_paged(q, kn, vn, kp, vp, table, lens)
    assert np.array_equal(got, want)


def test_shared_prefix_pages_and_unused_slots():
    q, kn, vn, kc, vc, lens, page = _contiguous_case(lens=(9, 9, 9))
    kc[1, :, :8] = kc[0, :, :8]  # requests 0 and 1 share their first two blocks
    vc[1, :, :8] = vc[0, :, :8]
    T = kc.shape[2] // page * page
    nb = T // page
    kp, table = _paginate(kc[:, :, :T], page, np.arange(3 * nb))
    vp, _ = _paginate(vc[:, :, :T], page, np.arange(3 * nb))
    table[1, :2] = table[0, :2]  # point request 1 at request 0's pages
    kp[:, nb : nb + 2] = np.nan  # its own copies are now unused: poisoned
    vp[:, nb : nb + 2] = np.nan
    for b in range(3):           # positions at or past L are unused too
        for pos in range(9, T):
            kp[:, table[b, pos // page], pos % page] = np.nan
            vp[:, table[b, pos // page], pos % page] = np.nan
    got = P.verify_attention_paged(q, kn, vn, kp, vp, table, lens)
    assert np.all(np.isfinite(got))
    assert np.allclose(got, A.verify_attention(q, kn, vn, kc, vc, lens), rtol=0, atol=0)


def test_append_lands_in_the_tabled_pages():
    q, kn, vn, kc, vc, lens, page = _contiguous_case(lens=(3, 4, 7))
    T = kc.shape[2] // page * page
    nb = T // page
    perm = np.random.default_rng(2).permutation(3 * nb)
    kp, table = _paginate(kc[:, :, :T], page, perm)
    vp, _ = _paginate(vc[:, :, :T], page, perm)
    kp2, vp2 = P.kv_append_paged(kp, vp, kn, vn, table, lens)
    kc2, vc2 = A.kv_append(kc[:, :, :T], vc[:, :, :T], kn, vn, lens)
    for b, L in enumerate(lens):
        assert np.array_equal(P.gather(kp2, table[b], L + 3), kc2[b, :, : L + 3])
        assert np.array_equal(P.gather(vp2, table[b], L + 3), vc2[b, :, : L + 3])
