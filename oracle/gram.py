"""Float64 CPU oracle of Gram-threshold token selection and its cascade.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import this module.  It shares no code with
the HIP path and imports nothing from it.

What it computes, from "Cascade token selection for transformer attention
acceleration":

  selection   (Problem statement, the ADA rule) token i of a sequence is a
              representative when its largest cosine correlation with the
              tokens before it is below 1 - tau^2.  Written out: with
              c(i, j) = <x_i, x_j> / (|x_i| |x_j|),
                  m_i = max_{j < i} c(i, j)      (m_0 = -inf: nothing before),
                  rep_i = m_i < 1 - tau^2.
              The full T x T Gram matrix of the normalised tokens gives every
              c(i, j); only its strict lower triangle is used.
  cascade     (Methodology, steps 1-3) given the set R inherited from the
              layer before:
                1. inherit R;
                2. validate it with two smaller Gram products:
                   the r x r product among R: a member i stays valid when
                       max_{j in R, j < i} c(i, j) < 1 - tau^2;
                   the (T - r) x r cross product between the tokens outside
                   R and the valid members V: such a token i becomes a new
                   representative when
                       max_{j in V, j < i} c(i, j) < 1 - tau^2;
                3. the updated set is V plus the new representatives.
              Every true representative (of the selection rule on the same
              tokens) is in the result, for any inherited R, because each of
              the two maxima runs over a subset of the tokens before i
              (Contributions, Proposition 4: the cascade is conservative).

Readings where the page leaves a step open (each also listed in the design
notes): the cosine is signed (an anti-parallel token is not a duplicate);
"below" is strict; "preceding" means earlier in the sequence (j < i); a
zero token has cosine 0 with every token; the per-token maxima returned by
the cascade are the ones its decisions used (over R for members of R, over V
for the others).

Inputs are arrays [T, d] (one sequence) or [B, T, d] of any float type,
upcast exactly to float64.
"""
from __future__ import annotations

import numpy as np


def threshold(tau: float) -> float:
    """1 - tau^2, the Gram threshold of the ADA rule."""
    return 1.0 - float(tau) ** 2


def normalise(x: np.ndarray) -> np.ndarray:
    """Rows scaled to unit length; zero rows stay zero (cosine 0)."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return np.where(n > 0, x / np.where(n > 0, n, 1.0), 0.0)


def cosines(x: np.ndarray) -> np.ndarray:
    """The full Gram matrix of the normalised tokens, c(i, j)."""
    u = normalise(x)
    return u @ np.swapaxes(u, -1, -2)


def max_cosine(x: np.ndarray) -> np.ndarray:
    """m_i = max_{j < i} c(i, j), -inf for the first token ([..., T])."""
    c = cosines(x)
    T = c.shape[-1]
    below = np.tril(np.ones((T, T), dtype=bool), k=-1)
    return np.max(np.where(below, c, -np.inf), axis=-1)


def select(x: np.ndarray, tau: float):
    """(m, rep): the per-token maxima and the representative flags."""
    m = max_cosine(x)
    return m, m < threshold(tau)


def _masked_max(c: np.ndarray, rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
    """For each token in ``rows``: max of c(i, j) over j in ``cols`` with
    j < i (-inf when there is none)."""
    out = np.full(rows.size, -np.inf)
    for a, i in enumerate(rows):
        js = cols[cols < i]
        if js.size:
            out[a] = np.max(c[i, js])
    return out


def max_cosine_rows(x: np.ndarray, rows, cols=None) -> np.ndarray:
    """m_i for the tokens ``rows`` of one sequence [T, d]: max of c(i, j)
    over j < i, with j restricted to the tokens ``cols`` when given (the
    same definition, evaluated at sampled rows for long sequences)."""
    u = normalise(x)
    rows = np.asarray(rows)
    T = u.shape[0]
    allowed = np.ones(T, dtype=bool) if cols is None else np.zeros(T, dtype=bool)
    if cols is not None:
        allowed[np.asarray(cols, dtype=np.int64)] = True
    c = u[rows] @ u.T
    keep = (np.arange(T)[None, :] < rows[:, None]) & allowed[None, :]
    return np.max(np.where(keep, c, -np.inf), axis=1)


def cascade(x: np.ndarray, tau: float, prev, valid_given=None):
    """One cascade step on one sequence [T, d] with the inherited set given
    as flags ``prev`` [T] (nonzero = in R).  Returns (m, rep, valid): the
    maxima the decisions used, the updated representative flags, and which
    members of R stayed valid (False outside R).

    ``valid_given`` (flags [T]) replaces the validity decisions of step 2 by
    decisions taken elsewhere; the tests use it to follow an implementation
    whose decisions on members within rounding of the threshold differ."""
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    inR = np.asarray(prev).astype(bool).reshape(T)
    thr = threshold(tau)
    c = cosines(x)
    R = np.flatnonzero(inR)
    N = np.flatnonzero(~inR)
    m = np.empty(T)
    m[R] = _masked_max(c, R, R)                # the r x r product
    valid = np.zeros(T, dtype=bool)
    valid[R] = m[R] < thr
    if valid_given is not None:
        valid = np.asarray(valid_given).astype(bool).reshape(T) & inR
    V = np.flatnonzero(valid)
    m[N] = _masked_max(c, N, V)                # the (T - r) x r product
    rep = valid.copy()
    rep[N] = m[N] < thr
    return m, rep, valid


def jaccard(a, b) -> float:
    """|a and b| / |a or b| of two flag vectors (1.0 for two empty sets)."""
    a, b = np.asarray(a, dtype=bool), np.asarray(b, dtype=bool)
    u = np.count_nonzero(a | b)
    return 1.0 if u == 0 else np.count_nonzero(a & b) / u
