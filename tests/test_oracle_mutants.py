"""Planted mistakes in the oracle (on the CPU): each must make at least one pin fail.

This shows the pins in test_oracle.py are sensitive to the plausible errors they are meant to
catch: a missing max-subtraction, a sign error, a wrong index, a dropped term, an ignored
target in the block filter, a forgotten ignore mask, a target test that also claims the next
block, an entry floor that drops targets or compares the wrong quantity."""
import numpy as np
import pytest

import test_oracle as T
from oracle import cce_oracle as co

_orig_lse = co._rows_lse_and_target
_orig_neg = co.block_negligible


def test_mutant_lse_without_max_shift_overflows(monkeypatch):
    def bad(E_rows, C, t_rows, vchunk):
        z = co.logits(E_rows, C)
        with np.errstate(over="ignore"):
            lse = np.log(np.exp(z).sum(axis=1))
        zt = np.where(t_rows >= 0, z[np.arange(len(t_rows)), np.maximum(t_rows, 0)], 0.0)
        return lse, zt
    monkeypatch.setattr(co, "_rows_lse_and_target", bad)
    with pytest.raises(AssertionError):
        T.test_dominant_logit_no_overflow()


def test_mutant_gradient_sign_flip(monkeypatch):
    orig = co._dloss_vector
    monkeypatch.setattr(co, "_dloss_vector", lambda d, N: -orig(d, N))
    with pytest.raises(AssertionError):
        T.test_gradients_match_central_differences(0)


def test_mutant_wrong_feature_index(monkeypatch):
    monkeypatch.setattr(co, "logits",
                        lambda E_rows, C, v0=0, v1=None: np.asarray(E_rows, np.float64)
                        @ np.asarray(C[v0:v1], np.float64)[:, ::-1].T)
    with pytest.raises(AssertionError):
        T.test_forward_matches_mpmath(0, 6, 11, 5)


def test_mutant_dropped_last_vocab_chunk(monkeypatch):
    def bad(E_rows, C, t_rows, vchunk):
        V = C.shape[0]
        keep = max(vchunk, V - vchunk) if V > vchunk else V
        return _orig_lse(E_rows, C[:keep], np.where(t_rows < keep, t_rows, -1), vchunk)
    monkeypatch.setattr(co, "_rows_lse_and_target", bad)
    with pytest.raises(AssertionError):
        T.test_chunking_does_not_change_results()


def test_mutant_filter_ignores_targets(monkeypatch):
    def bad(P, t_rows, valid_rows, eps, n0, v0, bn, bv):
        return _orig_neg(P, np.full_like(t_rows, -1), valid_rows, eps, n0, v0, bn, bv)
    monkeypatch.setattr(co, "block_negligible", bad)
    with pytest.raises(AssertionError):
        T.test_far_vocabulary_blocks_are_skipped_exactly()


def test_mutant_filter_counts_ignored_rows(monkeypatch):
    def bad(P, t_rows, valid_rows, eps, n0, v0, bn, bv):
        return _orig_neg(P, np.where(t_rows == T.II, 200, t_rows), np.ones_like(valid_rows),
                         eps, n0, v0, bn, bv)
    monkeypatch.setattr(co, "block_negligible", bad)
    with pytest.raises(AssertionError):
        T.test_far_vocabulary_blocks_are_skipped_exactly()


def test_mutant_entry_floor_drops_targets(monkeypatch):
    def bad(P, t_rows, valid_rows, floor, v0):
        return (P < floor) & valid_rows[:, None]
    monkeypatch.setattr(co, "entry_negligible", bad)
    with pytest.raises(AssertionError):
        T.test_entry_floor_closed_form_equal_rows(0.0)
    with pytest.raises(AssertionError):
        T.test_entry_floor_matches_brute_force()


def test_mutant_entry_floor_compares_the_gradient(monkeypatch):
    """The floor applied to dloss * p rather than p (a plausible mix-up of the softmax value
    with the gradient entry): the equal-rows closed form, whose dloss weights straddle 1, fails."""
    orig = co.entry_negligible

    def bad(P, t_rows, valid_rows, floor, v0):
        return orig(P * 1.3, t_rows, valid_rows, floor, v0)
    monkeypatch.setattr(co, "entry_negligible", bad)
    with pytest.raises(AssertionError):
        T.test_entry_floor_closed_form_equal_rows(0.0)


def test_mutant_target_claims_the_next_block(monkeypatch):
    """A target on the first row of a vocabulary block also keeps the block before it (an
    inclusive upper bound in the target test)."""
    def bad(P, t_rows, valid_rows, eps, n0, v0, bn, bv):
        out = _orig_neg(P, t_rows, valid_rows, eps, n0, v0, bn, bv)
        for i in range(out.shape[0]):
            r = slice(i * bn, (i + 1) * bn)
            tv = t_rows[r][valid_rows[r]] - v0
            for j in range(out.shape[1]):
                if np.any(tv == (j + 1) * bv):
                    out[i, j] = False
        return out
    monkeypatch.setattr(co, "block_negligible", bad)
    with pytest.raises(AssertionError):
        T.test_block_filter_closed_form_flat_softmax()
