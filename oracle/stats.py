"""Acceptance statistics of speculative decoding in closed form (test infrastructure only).

[RR] "What draft accuracy buys, measured in tokens per call": beta(ctx) = sum_x min(p, q) is the
probability that a draft token survives at context ctx, alpha = E[beta] over the target chain's
long-run (stationary) distribution of contexts, and a block of gamma drafts emits
(1 - alpha^(gamma+1)) / (1 - alpha) tokens in expectation (Leviathan et al., Eq. 1, as the page
states it).  [RR] "Acceptance rate has to beat cost": the expected walltime improvement is
E[#tokens] / (gamma c + 1) for a draft/target cost ratio c; [VT] §4 names the same ratio with the
measured block efficiency tau the memory-bound speed-up MBSU = tau / (c gamma + 1).
"""
from __future__ import annotations

import numpy as np

from .ref import softmax_temp


def transition_matrix(target_table, T: float) -> np.ndarray:
    """Order-1 toy: P[a, b] = p(next = b | previous = a), from table rows 1..V (row 0 is the
    start context, which the long-run chain never revisits)."""
    _, p = softmax_temp(np.asarray(target_table, dtype=np.float64)[1:], T)
    return p


def stationary(P, tol: float = 1e-15, max_iter: int = 1_000_000) -> np.ndarray:
    """Long-run distribution of a row-stochastic matrix by power iteration (as the page finds its
    context distribution): pi <- pi P from the uniform start until the change is below tol."""
    P = np.asarray(P, dtype=np.float64)
    pi = np.full(P.shape[0], 1.0 / P.shape[0])
    for _ in range(max_iter):
        nxt = pi @ P
        if np.abs(nxt - pi).sum() < tol:
            return nxt
        pi = nxt
    raise RuntimeError("power iteration did not converge")


def beta(p_row, q_row) -> float:
    """Overlap of two next-token distributions: sum_x min(p(x), q(x))."""
    return float(np.minimum(np.asarray(p_row, np.float64), np.asarray(q_row, np.float64)).sum())


def alpha_toy(target_table, draft_table, target_T: float, draft_T: float) -> float:
    """alpha = sum over previous tokens a of pi(a) * beta(p(.|a), q(.|a))."""
    _, p = softmax_temp(np.asarray(target_table, dtype=np.float64)[1:], target_T)
    _, q = softmax_temp(np.asarray(draft_table, dtype=np.float64)[1:], draft_T)
    pi = stationary(p)
    return float(sum(pi[a] * beta(p[a], q[a]) for a in range(len(pi))))


def expected_tokens(alpha: float, gamma: int) -> float:
    """Leviathan et al. Eq. 1: tokens per block when each draft survives with probability alpha."""
    if alpha >= 1.0:
        return float(gamma + 1)
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def walltime_improvement(tokens_per_block: float, gamma: int, c: float) -> float:
    """Expected walltime improvement E[#tokens] / (gamma c + 1) (equivalently [VT]'s MBSU with
    the measured tau and c the draft/target size ratio)."""
    return tokens_per_block / (gamma * c + 1.0)
