"""The pins must catch plausible mistakes.

Each test plants one mistake in the oracle on the CPU (monkeypatch, undone after
the test) and checks that a pin of the other test files fails under it.  This
is evidence that the pins constrain the oracle, not a test of the GPU path.
"""

import numpy as np
import pytest

from oracle import attention as A
from oracle import formulas as F
from oracle import sampler as S
from tests import _law
from tests import test_oracle_attention as TA
from tests import test_oracle_sampler as TS


def _small_law_pin():
    """Brute-force pin on V=3, gamma=2 (fast version of the full pin)."""
    TS.test_bruteforce_law_preserves_target_distribution(3, 2, 1, 0.0)


def _assert_pin_fails(fn):
    with pytest.raises(AssertionError):
        fn()


def test_pins_hold_unmutated():
    _small_law_pin()
    TA.test_matches_torch_sdpa(2, 4, 2, 5, 16, [0, 9])


def test_swapped_ratio_is_caught(monkeypatch):
    monkeypatch.setattr(S, "accept_threshold", lambda p, q: np.minimum(1.0, np.float64(q) / np.float64(p)))
    _assert_pin_fails(_small_law_pin)


def test_swapped_residual_is_caught(monkeypatch):
    monkeypatch.setattr(S, "residual", lambda p, q: np.maximum(q - p, 0.0))
    _assert_pin_fails(_small_law_pin)


def test_unclipped_residual_is_caught(monkeypatch):
    monkeypatch.setattr(S, "residual", lambda p, q: np.abs(p - q))
    _assert_pin_fails(_small_law_pin)


def test_non_strict_accept_is_caught(monkeypatch):
    monkeypatch.setattr(S, "accepts", lambda u, thr: bool(np.float64(u) <= thr))
    _assert_pin_fails(TS.test_accept_test_is_strict)


def test_left_searchsorted_is_caught(monkeypatch):
    def left(w, u):
        c = np.cumsum(w)
        return int(np.searchsorted(c / c[-1], u, side="left"))

    monkeypatch.setattr(S, "inverse_cdf", left)
    _assert_pin_fails(TS.test_zero_mass_tokens_never_drawn)


def test_reversed_token_order_is_caught(monkeypatch):
    def reversed_cdf(w, u):
        c = np.cumsum(w[::-1])
        return len(w) - 1 - int(np.searchsorted(c / c[-1], u, side="right"))

    monkeypatch.setattr(S, "inverse_cdf", reversed_cdf)
    _assert_pin_fails(TS.test_q_equal_p_accepts_all_and_bonus_is_numpy_choice)


def test_temperature_as_multiplier_is_caught(monkeypatch):
    orig = S.softmax_t
    monkeypatch.setattr(S, "softmax_t", lambda z, T: orig(z, 1.0 / T))
    # case (V=3, gamma=2, seed=1) runs at T = 0.7
    _assert_pin_fails(lambda: TS.test_bruteforce_law_preserves_target_distribution(3, 2, 1, 0.0))


def test_missing_causal_mask_is_caught(monkeypatch):
    # every new row sees all n new keys
    monkeypatch.setattr(A, "visible_keys", lambda L, i: L + 10**9)
    _assert_pin_fails(lambda: TA.test_matches_torch_sdpa(2, 4, 2, 5, 16, [0, 9]))


def test_off_by_one_mask_is_caught(monkeypatch):
    monkeypatch.setattr(A, "visible_keys", lambda L, i: L + i)  # drops the row's own key
    _assert_pin_fails(lambda: TA.test_matches_torch_sdpa(2, 4, 2, 5, 16, [3, 9]))


def test_wrong_exponent_is_caught(monkeypatch):
    from tests import test_oracle_formulas as TF

    orig = F.expected_committed
    monkeypatch.setattr(F, "expected_committed", lambda a, g: orig(a, g - 1) if g > 1 else orig(a, g) * 0.9)
    row = {"T": 0.7, "k": 4, "alpha": 0.901, "E": 4.10, "factor": 2.19}
    _assert_pin_fails(lambda: TF.test_expected_tokens_matches_printed_ksweep(row))


# ---- greedy verification ----------------------------------------------------

from oracle import greedy as G  # noqa: E402
from tests import test_oracle_greedy as TG  # noqa: E402


def _greedy_pin():
    TG.test_speculative_equals_greedy_decoding(50, 0.8, 1.0, False, 4)


def _mutant(row_of_t=0, accept_on_mismatch=False):
    def verify_sequence(z_target, x):
        n = 0
        for i in range(len(x)):
            same = G.argmax(z_target[i]) == int(x[i])
            if same == accept_on_mismatch:
                break
            n += 1
        t = G.argmax(z_target[min(n + row_of_t, len(x))])
        return n, [int(v) for v in x[:n]] + [t]

    return verify_sequence


def test_greedy_pins_hold_unmutated():
    _greedy_pin()
    TG.test_zero_temperature_limit_of_the_sampler()


def test_greedy_correction_from_the_next_row_is_caught(monkeypatch):
    monkeypatch.setattr(G, "verify_sequence", _mutant(row_of_t=1))
    _assert_pin_fails(_greedy_pin)


def test_greedy_inverted_accept_is_caught(monkeypatch):
    monkeypatch.setattr(G, "verify_sequence", _mutant(accept_on_mismatch=True))
    _assert_pin_fails(_greedy_pin)
    _assert_pin_fails(TG.test_zero_temperature_limit_of_the_sampler)


def test_greedy_last_index_ties_are_caught(monkeypatch):
    monkeypatch.setattr(G, "argmax", lambda z: int(len(z) - 1 - np.argmax(np.asarray(G.to_f64(z))[::-1])))
    _assert_pin_fails(TG.test_argmax_conventions)


# ---- paged cache --------------------------------------------------------------

from oracle import paged as Pg  # noqa: E402
from tests import test_oracle_paged as TP  # noqa: E402


def test_paged_pins_hold_unmutated():
    TP.test_allocation_waste_matches_the_page(16, 0.007)
    TP.test_paging_does_not_change_attention(True)


def test_floor_block_count_is_caught(monkeypatch):
    monkeypatch.setattr(Pg, "blocks_needed", lambda length, page: int(length) // int(page))
    _assert_pin_fails(lambda: TP.test_allocation_waste_matches_the_page(16, 0.007))


def test_ignoring_the_block_table_is_caught(monkeypatch):
    real = Pg.gather
    monkeypatch.setattr(Pg, "gather", lambda pages, row, length: real(pages, np.arange(len(row)), length))
    _assert_pin_fails(lambda: TP.test_paging_does_not_change_attention(True))


# ---- int8 cache -----------------------------------------------------------------

from oracle import quant as Qn  # noqa: E402
from tests import test_oracle_quant as TQ  # noqa: E402


def test_quant_pins_hold_unmutated():
    TQ.test_halves_round_to_even()
    TQ.test_error_bound_and_granularity()


def test_floor_rounding_is_caught(monkeypatch):
    def floor_q(x):
        x32 = np.asarray(x, np.float32)
        s32 = np.max(np.abs(x32), axis=-1, keepdims=True) / np.float32(127)
        with np.errstate(divide="ignore", invalid="ignore"):
            q = np.where(s32 > 0, np.floor(x32 / s32), 0)
        return np.clip(q, -127, 127).astype(np.int8), s32[..., 0].astype(np.float16)

    monkeypatch.setattr(Qn, "quantize_rows", floor_q)
    _assert_pin_fails(TQ.test_halves_round_to_even)


def test_scale_shared_over_heads_is_caught(monkeypatch):
    def per_position(x):
        x32 = np.asarray(x, np.float32)
        a = np.max(np.abs(x32), axis=(-3, -1), keepdims=True) if x32.ndim >= 3 else np.max(np.abs(x32), axis=-1,
                                                                                             keepdims=True)
        s32 = np.broadcast_to(a / np.float32(127), x32.shape[:-1] + (1,))
        with np.errstate(divide="ignore", invalid="ignore"):
            q = np.where(s32 > 0, np.rint(x32 / s32), 0)
        return np.clip(q, -127, 127).astype(np.int8), s32[..., 0].astype(np.float16)

    monkeypatch.setattr(Qn, "quantize_rows", per_position)
    _assert_pin_fails(TQ.test_error_bound_and_granularity)


# ---- the model oracle ------------------------------------------------------

from oracle import model as MO  # noqa: E402
from tests import test_oracle_model as TM  # noqa: E402


def test_model_pins_hold_unmutated():
    TM.test_layer_norm_matches_torch()
    TM.test_gelu_matches_torch_tanh_form()
    TM.test_model_attention_matches_attention_oracle()
    TM.test_value_path_and_head_layout_closed_form()


def test_wrong_layer_norm_eps_is_caught(monkeypatch):
    monkeypatch.setattr(MO, "LN_EPS", 1e-3)
    _assert_pin_fails(TM.test_layer_norm_matches_torch)


def test_erf_gelu_is_caught(monkeypatch):
    from math import erf

    monkeypatch.setattr(MO, "gelu", lambda x: 0.5 * x * (1 + np.vectorize(erf)(x / np.sqrt(2.0))))
    _assert_pin_fails(TM.test_gelu_matches_torch_tanh_form)


def test_unscaled_model_attention_is_caught(monkeypatch):
    def unscaled(q, K, V, p0):
        out = np.zeros_like(q)
        for i in range(q.shape[1]):
            m = p0 + i + 1
            s = np.einsum("hd,hkd->hk", q[:, i], K[:, :m])
            out[:, i] = np.einsum("hk,hkd->hd", MO.softmax(s), V[:, :m])
        return out

    monkeypatch.setattr(MO, "_causal_attention", unscaled)
    _assert_pin_fails(TM.test_model_attention_matches_attention_oracle)


def test_model_attention_seeing_the_next_key_is_caught(monkeypatch):
    def peeks(q, K, V, p0):
        out = np.zeros_like(q)
        for i in range(q.shape[1]):
            m = min(p0 + i + 2, K.shape[1])
            s = np.einsum("hd,hkd->hk", q[:, i], K[:, :m]) / np.sqrt(q.shape[2])
            out[:, i] = np.einsum("hk,hkd->hd", MO.softmax(s), V[:, :m])
        return out

    monkeypatch.setattr(MO, "_causal_attention", peeks)
    _assert_pin_fails(TM.test_model_attention_matches_attention_oracle)


# ---- the round oracle ------------------------------------------------------

from oracle import round as RO  # noqa: E402
from tests import test_oracle_round as TR  # noqa: E402


def test_round_pins_hold_unmutated():
    TR.test_draft_equal_to_target_accepts_everything()
    TR.test_truncated_caches_hold_the_committed_prefix(1.0)


def test_draft_cache_kept_at_full_length_is_caught(monkeypatch):
    """Cutting the draft cache to len - 1 even when it lacks the last proposal."""
    real = RO.propose

    def lying(*a, **k):
        xs, zs, dlen, m, band = real(*a, **k)
        return xs, zs, dlen + 1, m, band

    monkeypatch.setattr(RO, "propose", lying)
    _assert_pin_fails(TR.test_draft_equal_to_target_accepts_everything)


def test_target_cache_cut_one_short_is_caught(monkeypatch):
    real = RO.speculative_round

    def short(flat_t, cfg_t, flat_d, cfg_d, state, *a):
        res = real(flat_t, cfg_t, flat_d, cfg_d, state, *a)
        state["tlen"] -= 1
        return res

    monkeypatch.setattr(RO, "speculative_round", short)
    _assert_pin_fails(lambda: TR.test_truncated_caches_hold_the_committed_prefix(1.0))
