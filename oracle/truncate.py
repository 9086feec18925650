"""Oracle: the KV length reset after verification (CPU).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py``.

[P2] section numpyで小さなTransformerを自作する (``KVCache.truncate``: dropping
rejected K/V is only a length reset) and section 投機的デコーディングとは (after
the round the target cache is cut back to base + 1 + n_accepted): the last
committed token plus the n accepted drafts stay; the rejected drafts' rows are
dead.  The corrected or bonus token has no K/V yet -- it is the first input of
the next round.
"""

import numpy as np


def truncate(lens, n_accepted):
    """New cache lengths L_b + 1 + n_accepted[b] (int32)."""
    return (np.asarray(lens, dtype=np.int64) + 1 + np.asarray(n_accepted, dtype=np.int64)).astype(np.int32)
