"""Pins for the exact-rational enumerator: the glossary page's two-token worked example, the
naive-redraw negative control, the exactness identity, chained-block joints against the target
chain, and the closed forms for the overlap beta and the expected tokens per block."""
import itertools
import json
import os
import random
from fractions import Fraction as F

import pytest

from oracle import exact


def _golden(golden_dir):
    with open(os.path.join(golden_dir, "two_token.json")) as f:
        g = json.load(f)
    return {k: ([F(x) for x in v] if isinstance(v, list) and k != "tokens" else
                (F(v) if isinstance(v, str) and k not in ("source",) else v)) for k, v in g.items()}


def test_worked_example_table(golden_dir):
    g = _golden(golden_dir)
    p, q = g["target"], g["draft"]
    acc = [exact.accept_prob(p[x], q[x]) for x in range(2)]
    assert acc == g["acceptance_given_proposal"]
    assert [q[x] * acc[x] for x in range(2)] == g["accepted_mass"]
    assert sum(q[x] * acc[x] for x in range(2)) == g["total_accepted"]
    assert exact.beta(p, q) == g["total_accepted"]
    assert list(exact.residual(p, q)) == g["residual"]
    dist = exact.block_distribution(lambda c: p, lambda c: q, gamma=1)
    assert list(exact.first_token_marginal(dist, 2)) == g["final"]
    # the rejection mass: sequences of length 1 are exactly the rejected blocks
    assert sum(v for k, v in dist.items() if len(k) == 1) == g["rejection"]


def test_worked_example_naive_redraw_is_biased(golden_dir):
    g = _golden(golden_dir)
    p, q = g["target"], g["draft"]
    dist = exact.block_distribution(lambda c: p, lambda c: q, gamma=1, correction="naive")
    assert list(exact.first_token_marginal(dist, 2)) == g["naive_redraw_final"]
    assert list(exact.first_token_marginal(dist, 2)) != g["final"]


def _rand_dist(rng, V, zeros=0):
    w = [rng.randint(1, 9) for _ in range(V)]
    for i in rng.sample(range(V), zeros):
        w[i] = 0
    s = sum(w)
    return tuple(F(x, s) for x in w)


@pytest.mark.parametrize("seed", range(20))
def test_exactness_identity_per_token(seed):
    # direct acceptance min(p, q) plus (1 - beta) times the residual equals p at every token
    rng = random.Random(seed)
    V = rng.randint(2, 4)
    p = _rand_dist(rng, V, zeros=rng.randint(0, 1))
    q = _rand_dist(rng, V, zeros=rng.randint(0, 1))
    b = exact.beta(p, q)
    if b == 1:
        return
    r = exact.residual(p, q)
    for x in range(V):
        assert min(p[x], q[x]) + (1 - b) * r[x] == p[x]


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("gamma", [1, 2, 3])
def test_first_emitted_token_is_target_iid(seed, gamma):
    rng = random.Random(100 * gamma + seed)
    V = rng.randint(2, 4)
    ps = [_rand_dist(rng, V) for _ in range(gamma + 1)]
    qs = [_rand_dist(rng, V, zeros=rng.randint(0, V - 1)) for _ in range(gamma)]
    dist = exact.block_distribution(lambda c: ps[len(c)], lambda c: qs[len(c)], gamma)
    assert sum(dist.values()) == 1
    assert exact.first_token_marginal(dist, V) == ps[0]


def _bigram(rng, V, zeros_max=0):
    tab = {c: _rand_dist(rng, V, zeros=rng.randint(0, zeros_max)) for c in range(-1, V)}
    return lambda ctx: tab[ctx[-1] if ctx else -1]


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("gamma,K", [(1, 3), (2, 3), (3, 3), (2, 4)])
def test_chained_blocks_reproduce_target_chain(seed, gamma, K):
    # blocks chained from whatever was emitted reproduce the target chain's exact joint
    rng = random.Random(7 * seed + gamma)
    V = 3 if K <= 3 else 2
    p_at = _bigram(rng, V)
    q_at = _bigram(rng, V, zeros_max=1)
    dist = exact.generation_distribution(p_at, q_at, gamma, K)
    for seq in itertools.product(range(V), repeat=K):
        assert dist.get(seq, 0) == exact.target_joint(p_at, seq)


def test_chained_naive_redraw_breaks_target_chain():
    rng = random.Random(5)
    p_at = _bigram(rng, 3)
    q_at = _bigram(rng, 3)
    dist = exact.generation_distribution(p_at, q_at, 2, 3, correction="naive")
    assert any(dist.get(s, 0) != exact.target_joint(p_at, s) for s in itertools.product(range(3), repeat=3))


@pytest.mark.parametrize("seed", range(8))
@pytest.mark.parametrize("gamma", [1, 2, 4])
def test_expected_tokens_closed_form(seed, gamma):
    # context-independent rows: beta = alpha at every position and the count of emitted tokens
    # is truncated-geometric: E = (1 - alpha^(gamma+1)) / (1 - alpha)
    rng = random.Random(seed)
    V = rng.randint(2, 4)
    p = _rand_dist(rng, V)
    q = _rand_dist(rng, V)
    alpha = exact.beta(p, q)
    dist = exact.block_distribution(lambda c: p, lambda c: q, gamma)
    want = (1 - alpha ** (gamma + 1)) / (1 - alpha) if alpha != 1 else F(gamma + 1)
    assert exact.expected_emitted(dist) == want
    # P(first draft accepted) = beta
    assert sum(v for k, v in dist.items() if len(k) >= 2) == (alpha if gamma >= 1 else 0)


def test_identical_distributions_accept_everything():
    p = (F(1, 2), F(1, 3), F(1, 6))
    dist = exact.block_distribution(lambda c: p, lambda c: p, gamma=3)
    assert all(len(k) == 4 for k in dist)
    assert exact.expected_emitted(dist) == 4


def test_disjoint_supports_reject_first_and_draw_target():
    p = (F(0), F(1, 4), F(3, 4))
    q = (F(1), F(0), F(0))
    dist = exact.block_distribution(lambda c: p, lambda c: q, gamma=2)
    assert all(len(k) == 1 for k in dist)
    assert exact.first_token_marginal(dist, 3) == p


def test_trimmed_aligned_draft_accepts_kept_mass():
    # draft = target restricted to a kept set and renormalised: beta = p(kept) and every
    # residual token lies off the kept set, distributed as p restricted there
    p = (F(1, 10), F(2, 10), F(3, 10), F(4, 10))
    kept = [3, 1]
    pk = sum(p[i] for i in kept)
    q = tuple(p[i] / pk if i in kept else F(0) for i in range(4))
    assert exact.beta(p, q) == pk
    r = exact.residual(p, q)
    off = sum(p[i] for i in range(4) if i not in kept)
    assert r == tuple(F(0) if i in kept else p[i] / off for i in range(4))
