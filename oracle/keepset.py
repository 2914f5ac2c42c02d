"""Keep-set construction, the offline step before the hot path (test infrastructure only).

[VT] §3 builds the trimmed vocabulary from a token-frequency counter c over a calibration
corpus (Algorithm 1), keeps Top-K(c, k) (Eq. 1), and slices the matching rows of the LM head.
The same section names Top-P and a minimum frequency as other admissible selection rules.

READINGS (the pages leave these open):
  * ids outside [0, V) are not tokens of the vocabulary and are not counted;
  * Top-K ranks ids by count, larger first, and breaks ties by the lower id;
  * Top-P keeps the shortest prefix of that ranking whose summed count reaches ceil(P * N),
    N the total count, P * N evaluated in float64; at least one id is always kept;
  * minimum frequency f keeps every id whose count is at least f (possibly none);
  * the kept set is stored in ascending id order (a set has no order of its own), with the
    inverse map full_to_trim (-1 off the set).
"""
from __future__ import annotations

import math

import numpy as np


def count_tokens(tokens, V: int, counts=None) -> np.ndarray:
    """[VT] §3 Algorithm 1: a zero-initialised counter over the vocabulary, incremented once per
    token occurrence.  counts, if given, is the counter to continue (several corpus parts);
    returns uint64 [V]."""
    t = np.asarray(tokens, dtype=np.int64).ravel()
    t = t[(t >= 0) & (t < V)]
    c = np.bincount(t, minlength=V).astype(np.uint64)
    if counts is not None:
        c = c + np.asarray(counts, dtype=np.uint64)
    return c


def ranking(counts) -> np.ndarray:
    """All ids ordered by count descending, ties by ascending id."""
    c = np.asarray(counts, dtype=np.int64)
    ids = np.arange(len(c))
    return np.lexsort((ids, -c))


def _as_kept_set(chosen, V: int):
    keep = np.sort(np.asarray(chosen, dtype=np.int64)).astype(np.int32)
    f2t = np.full(V, -1, dtype=np.int32)
    f2t[keep] = np.arange(len(keep), dtype=np.int32)
    return keep, f2t


def top_k(counts, k: int):
    """[VT] §3 Eq. 1: the k most frequent ids -> (keep_ids ascending int32 [k], full_to_trim)."""
    V = len(counts)
    if not 1 <= k <= V:
        raise ValueError("k must lie in [1, V]")
    return _as_kept_set(ranking(counts)[:k], V)


def top_p_size(counts, p: float) -> int:
    """Number of ids Top-P keeps: the shortest ranked prefix whose summed count reaches
    ceil(p * N) (at least one id)."""
    if not 0.0 < p <= 1.0:
        raise ValueError("p must lie in (0, 1]")
    c = np.asarray(counts, dtype=np.uint64)
    total = int(c.sum())
    target = math.ceil(p * float(total))
    prefix = np.cumsum(c[ranking(c)].astype(np.int64))  # exact: totals stay far below 2**63
    k = int(np.searchsorted(prefix, target, side="left")) + 1
    return max(1, min(k, len(c)))


def top_p(counts, p: float):
    """[VT] §3 (Top-P selection): the most frequent ids up to cumulative share p."""
    return top_k(counts, top_p_size(counts, p))


def min_frequency(counts, f: int):
    """[VT] §3 (minimum-frequency selection): every id seen at least f times."""
    c = np.asarray(counts, dtype=np.uint64)
    return _as_kept_set(np.nonzero(c >= np.uint64(f))[0], len(c))


def trim_head(weight_bits, keep_ids) -> np.ndarray:
    """[VT] §3 Eq. 1, second line: W^Trim = the rows of W at the kept ids, in keep_ids order."""
    return np.ascontiguousarray(np.asarray(weight_bits)[np.asarray(keep_ids, dtype=np.int64)])
