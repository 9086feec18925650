"""The attention comparison can see a lost key block at long lengths.

At 32K-key caches of N(0, 1) rows the outputs are of size 0.02-0.05, so the
absolute bound of 2e-2 alone passes an output that misses a 32-key block
(one block moves a row by about 1e-4 to 1e-3).  The row-relative bound of
tests/_gpu.check_attention must refuse it while accepting the bf16 rounding a
correct kernel makes.  Everything here runs on the CPU: the "kernel outputs"
are the oracle's own outputs, rounded to bf16, with or without a block of the
cache removed from the oracle's inputs.
"""

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as A
from tests import _gpu


def _bf16(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).float().numpy().astype(np.float64)


@pytest.fixture(scope="module")
def long_case():
    # one sequence of config 5's shape at its longest length: one KV head with
    # its 8 query heads, 9 verify rows, D = 128
    L, n = 32768, 9
    cfg = W.Config(93, "long", B=1, gamma=n - 1, V=1, dtype="bf16", Hq=8, Hkv=1, D=128, L=(L, L), max_T=L + n)
    inp = W.attention_inputs(cfg, B=1, max_T=L + n, lens=[L])
    inp["k_cache"] = inp["k_cache"][:, :, :L]
    inp["v_cache"] = inp["v_cache"][:, :, :L]
    want = A.verify_attention(inp["q"], inp["k_new"], inp["v_new"], inp["k_cache"], inp["v_cache"], inp["lens"])
    return inp, want


def _drop_block(inp, j0):
    """The oracle's inputs with cache rows [j0, j0 + 32) left out."""
    keep = np.r_[0:j0, j0 + 32 : inp["k_cache"].shape[2]]
    out = dict(inp)
    out["k_cache"] = inp["k_cache"][:, :, keep]
    out["v_cache"] = inp["v_cache"][:, :, keep]
    out["lens"] = np.array([len(keep)], np.int32)
    return out


def test_rounded_oracle_passes(long_case):
    inp, want = long_case
    _gpu.check_attention(_bf16(want), want, "bf16")


@pytest.mark.parametrize("j0", [0, 16384, 32736])
def test_missing_block_fails_the_row_bound_not_the_absolute_one(long_case, j0):
    inp, want = long_case
    lost = A.verify_attention(**{k: v for k, v in _drop_block(inp, j0).items()})
    got = _bf16(lost)
    assert np.max(np.abs(got - want)) < _gpu.ATT_TOL["bf16"]  # the absolute bound alone is blind to it
    with pytest.raises(AssertionError, match="row-relative"):
        _gpu.check_attention(got, want, "bf16")


def test_missing_block_fails_at_fp16_too(long_case):
    inp, want = long_case
    lost = A.verify_attention(**{k: v for k, v in _drop_block(inp, 4096).items()})
    got = np.asarray(lost, np.float32).astype(np.float16).astype(np.float64)
    with pytest.raises(AssertionError, match="row-relative"):
        _gpu.check_attention(got, want, "f16")
    _gpu.check_attention(np.asarray(want, np.float32).astype(np.float16).astype(np.float64), want, "f16")
