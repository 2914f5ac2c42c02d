"""Exact-rational form of the verification rule for tiny vocabularies (test infrastructure only).

Where `ref` runs the rule with given uniforms, this module enumerates every branch of it in
fractions.Fraction arithmetic and returns the exact distribution of what a block emits.  It
pins `ref` (grid frequencies converge to it) and is itself pinned by the pages' worked
example, the exactness identity and the closed forms in tests/test_oracle_exact.py.

Distributions are tuples of Fractions indexed by full token id; a draft distribution is zero
off the kept set ([VT] §3: the trimmed head cannot propose those tokens).
Pages: [VT] VocabTrim; [GL] glossary "Speculative decoding"; [RR] "A rejection rule keeps
speculative decoding's output exact".
"""
from __future__ import annotations

from fractions import Fraction
from typing import Callable, Dict, Sequence, Tuple

Dist = Sequence[Fraction]
Cond = Callable[[Tuple[int, ...]], Dist]


def residual(p: Dist, q: Dist) -> Tuple[Fraction, ...]:
    """[GL] "Why a rejection needs a special draw": r = max(p - q, 0) normalised by its sum."""
    raw = [max(pi - qi, Fraction(0)) for pi, qi in zip(p, q)]
    z = sum(raw, Fraction(0))
    return tuple(r / z for r in raw)


def accept_prob(p_x: Fraction, q_x: Fraction) -> Fraction:
    """[GL]: a proposal x drawn from q is kept with probability min(1, p(x)/q(x))."""
    return min(Fraction(1), p_x / q_x)


def beta(p: Dist, q: Dist) -> Fraction:
    """[RR] "What draft accuracy buys": the overlap sum_x min(p(x), q(x)) = P(one draft survives)."""
    return sum((min(a, b) for a, b in zip(p, q)), Fraction(0))


def block_distribution(p_at: Cond, q_at: Cond, gamma: int, prefix: Tuple[int, ...] = (),
                       correction: str = "residual") -> Dict[Tuple[int, ...], Fraction]:
    """Exact distribution of the tokens one block emits, starting after `prefix`.

    p_at(ctx) / q_at(ctx): target / draft next-token distributions after the token tuple ctx.
    Branches ([RR] "Extending the rule from one token to a drafted run"; [GL]):
      draft x ~ q(.|ctx); keep it with probability min(1, p/q) and go on; otherwise emit one
      token from the residual at ctx (or, correction="naive", from p(.|ctx) itself) and stop;
      after gamma kept drafts emit one bonus token from p(.|ctx).
    Returns {emitted token tuple (length 1..gamma+1): probability}.
    """
    out: Dict[Tuple[int, ...], Fraction] = {}

    def emit(seq, mass):
        out[seq] = out.get(seq, Fraction(0)) + mass

    def walk(ctx, accepted, mass, i):
        p = p_at(ctx)
        if i == gamma:
            for y, py in enumerate(p):
                if py:
                    emit(accepted + (y,), mass * py)
            return
        q = q_at(ctx)
        rej = Fraction(0)
        for x, qx in enumerate(q):
            if not qx:
                continue
            a = accept_prob(p[x], qx)
            if a:
                walk(ctx + (x,), accepted + (x,), mass * qx * a, i + 1)
            rej += qx * (1 - a)
        if rej:
            fix = p if correction == "naive" else residual(p, q)
            for y, ry in enumerate(fix):
                if ry:
                    emit(accepted + (y,), mass * rej * ry)

    walk(tuple(prefix), (), Fraction(1), 0)
    return out


def generation_distribution(p_at: Cond, q_at: Cond, gamma: int, K: int,
                            correction: str = "residual") -> Dict[Tuple[int, ...], Fraction]:
    """Exact distribution of the first K tokens when blocks are chained, each block starting
    after everything emitted so far ([RR] "Extending the rule...", the generation loop)."""
    out: Dict[Tuple[int, ...], Fraction] = {}

    def run(seq, mass):
        if len(seq) >= K:
            key = seq[:K]
            out[key] = out.get(key, Fraction(0)) + mass
            return
        for emitted, pr in block_distribution(p_at, q_at, gamma, seq, correction).items():
            run(seq + emitted, mass * pr)

    run((), Fraction(1))
    return out


def target_joint(p_at: Cond, seq: Tuple[int, ...]) -> Fraction:
    """Probability the target alone generates seq token by token: prod_j p(y_j | y_<j)."""
    pr = Fraction(1)
    for j, y in enumerate(seq):
        pr *= p_at(tuple(seq[:j]))[y]
    return pr


def expected_emitted(dist: Dict[Tuple[int, ...], Fraction]) -> Fraction:
    """E[number of tokens one block emits] under an exact block distribution."""
    return sum((len(k) * v for k, v in dist.items()), Fraction(0))


def first_token_marginal(dist: Dict[Tuple[int, ...], Fraction], V: int) -> Tuple[Fraction, ...]:
    m = [Fraction(0)] * V
    for k, v in dist.items():
        m[k[0]] += v
    return tuple(m)
