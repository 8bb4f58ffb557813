"""Planted mistakes in the Gram-selection oracle (on the CPU) must fail at
least one pin of ``test_oracle_gram.py``.

Each mutant replaces one function of ``oracle.gram`` with a plausible wrong
version: an absolute cosine, a mask that includes the token itself or looks
forward, a non-strict or unsquared threshold, an unnormalised product, a
missing zero-token guard, and cascade checks over the wrong set or without
the causal order.
"""
import numpy as np
import pytest

from oracle import gram
import test_oracle_gram as pins

PIN_SET = [
    ("brute0", lambda: pins.test_brute_force_loops(0)),
    ("brute1", lambda: pins.test_brute_force_loops(1)),
    ("duplicates", pins.test_duplicates_are_redundant),
    ("orthogonal", pins.test_orthogonal_tokens_are_all_representatives),
    ("circle_rep", lambda: pins.test_tokens_on_a_circle(36.8699, True)),
    ("circle_dup", lambda: pins.test_tokens_on_a_circle(20.0, False)),
    ("anti_parallel", pins.test_anti_parallel_token_is_not_a_duplicate),
    ("strict", pins.test_strict_threshold_at_tau_zero),
    ("invariances", pins.test_invariances),
    ("cascade_all", pins.test_cascade_inheriting_everything_is_the_selection),
    ("cascade_none", pins.test_cascade_inheriting_nothing_selects_everything),
    ("conservative", lambda: pins.test_cascade_is_conservative(0)),
    ("cross_valid", pins.test_cascade_cross_check_uses_valid_members_only),
    ("member_check", pins.test_cascade_member_check_uses_members_only),
    ("cross_causal", pins.test_cascade_cross_check_is_causal),
    ("cascade_brute", lambda: pins.test_cascade_brute_force(0)),
]

_orig_cosines = gram.cosines
_orig_max_cosine = gram.max_cosine


def _mut_abs_cosine(x):
    return np.abs(_orig_cosines(x))


def _mut_unnormalised(x):
    x = np.asarray(x, dtype=np.float64)
    return x @ np.swapaxes(x, -1, -2)


def _mut_no_zero_guard(x):
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(invalid="ignore", divide="ignore"):
        return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def _mut_max_includes_self(x):
    c = gram.cosines(x)
    T = c.shape[-1]
    return np.max(np.where(np.tril(np.ones((T, T), dtype=bool)), c, -np.inf), axis=-1)


def _mut_max_over_following(x):
    c = gram.cosines(x)
    T = c.shape[-1]
    return np.max(np.where(np.triu(np.ones((T, T), dtype=bool), k=1), c, -np.inf), axis=-1)


def _mut_select_non_strict(x, tau):
    m = gram.max_cosine(x)
    return m, m <= gram.threshold(tau)


def _mut_threshold_unsquared(tau):
    return 1.0 - float(tau)


def _cascade_variant(cross_over_R=False, members_over_all=False, cross_acausal=False):
    def cascade(x, tau, prev):
        x = np.asarray(x, dtype=np.float64)
        T = x.shape[0]
        inR = np.asarray(prev).astype(bool).reshape(T)
        thr = gram.threshold(tau)
        c = gram.cosines(x)
        R, N = np.flatnonzero(inR), np.flatnonzero(~inR)
        m = np.empty(T)
        m[R] = gram._masked_max(c, R, np.arange(T) if members_over_all else R)
        valid = np.zeros(T, dtype=bool)
        valid[R] = m[R] < thr
        cols = R if cross_over_R else np.flatnonzero(valid)
        if cross_acausal:
            m[N] = np.array([np.max(c[i, cols]) if cols.size else -np.inf for i in N])
        else:
            m[N] = gram._masked_max(c, N, cols)
        rep = valid.copy()
        rep[N] = m[N] < thr
        return m, rep, valid
    return cascade


MUTANTS = {
    "abs_cosine": ("cosines", _mut_abs_cosine),
    "unnormalised": ("cosines", _mut_unnormalised),
    "no_zero_guard": ("normalise", _mut_no_zero_guard),
    "includes_self": ("max_cosine", _mut_max_includes_self),
    "looks_forward": ("max_cosine", _mut_max_over_following),
    "non_strict": ("select", _mut_select_non_strict),
    "unsquared_tau": ("threshold", _mut_threshold_unsquared),
    "cross_over_R": ("cascade", _cascade_variant(cross_over_R=True)),
    "members_over_all": ("cascade", _cascade_variant(members_over_all=True)),
    "cross_acausal": ("cascade", _cascade_variant(cross_acausal=True)),
}


def _run_pins():
    failed = []
    for name, fn in PIN_SET:
        try:
            with np.errstate(all="ignore"):
                fn()
        except Exception:  # an assertion, or a crash on a mutant's output
            failed.append(name)
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(gram, attr, fn)
    failed = _run_pins()
    assert failed, f"mutant {name} passed every pin"


def test_unmutated_oracle_passes_pin_set():
    assert _run_pins() == []
