"""Oracle: verify attention over a paged KV cache (CPU).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

Follows [P2] section PagedAttentionとKVキャッシュの量子化 (paging): the cache of
a request is held in fixed blocks ("pages") of 16 or 32 token positions,
allocated as the request grows, so that only the last block of a request can
have unused room.  A block table lists, for each request, the physical page of
each of its logical blocks.  The attention itself is unchanged: gathering a
request's pages in table order gives back its contiguous cache, and the
verify step is then exactly ``oracle.attention`` (the ``forward_cached``
listing of [P2] section numpyで小さなTransformerを自作する).

Layouts:
  k_pages, v_pages  [Hkv, num_pages, page, D]   page p holds positions
                    [i*page, (i+1)*page) of the request whose table maps its
                    logical block i to p (for every KV head)
  block_table       [B, max_blocks] int      physical page of logical block i
  lens              [B]                      committed length L_b before the call

Reading where the pages are silent: the KV head is the outermost index, then the
page, then the position in the page: one head's part of a page is
contiguous, and so is a run of consecutive pages; the pages fix only that a
request's positions are grouped into fixed-size blocks.
"""

import numpy as np

from . import attention as A


def blocks_needed(length, page):
    """Blocks of `page` positions that hold `length` positions: ceil(length / page)."""
    return -(-int(length) // int(page))


def allocation_waste(lengths, page=None, prealloc=None):
    """Fraction of allocated positions left unused.

    page: blocks of `page` positions per request (ceil(L / page) * page each);
    prealloc: every request reserves `prealloc` positions up front.
    """
    lengths = np.asarray(lengths, np.int64)
    used = lengths.sum()
    if prealloc is not None:
        alloc = prealloc * len(lengths)
    else:
        alloc = sum(blocks_needed(L, page) * page for L in lengths)
    return 1.0 - used / alloc


def gather(pages, table_row, length):
    """The first `length` positions of one request, [Hkv, length, D], from its pages."""
    page = pages.shape[2]
    nb = blocks_needed(length, page)
    blocks = [pages[:, int(table_row[i])] for i in range(nb)]  # each [Hkv, page, D]
    full = np.concatenate(blocks, axis=1) if blocks else pages[:, :0].reshape(pages.shape[0], 0, pages.shape[3])
    return full[:, :length]


def kv_append_paged(k_pages, v_pages, k_new, v_new, block_table, lens):
    """Copies of the pages with the n new rows of request b written at positions [L_b, L_b + n)."""
    kp, vp = k_pages.copy(), v_pages.copy()
    page = kp.shape[2]
    n = k_new.shape[2]
    for b, L in enumerate(lens):
        for r in range(n):
            pos = int(L) + r
            p = int(block_table[b][pos // page])
            kp[:, p, pos % page] = k_new[b, :, r]
            vp[:, p, pos % page] = v_new[b, :, r]
    return kp, vp


def verify_attention_paged(q, k_new, v_new, k_pages, v_pages, block_table, lens, scale=None, seqs=None):
    """Verify attention where request b's committed K/V live in the pages its table lists."""
    B = q.shape[0]
    seqs = range(B) if seqs is None else seqs
    out = []
    for b in seqs:
        L = int(lens[b])
        kc = gather(k_pages, block_table[b], L)[None]
        vc = gather(v_pages, block_table[b], L)[None]
        out.append(A.verify_attention(q[b : b + 1], k_new[b : b + 1], v_new[b : b + 1], kc, vc, np.array([L]),
                                      scale=scale)[0])
    return np.stack(out)
