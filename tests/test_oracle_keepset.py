"""Pins of the keep-set oracle (token counting and the selection rules of [VT] §3) against
literal restatements on tiny inputs, hand-worked examples and invariants."""
import numpy as np
import pytest

from oracle import keepset, ref
from workloads import token_stream, zipf_ranking


def alg1_counts(tokens, V):
    """[VT] §3 Algorithm 1 written out: zero counter, one increment per in-vocabulary token."""
    c = [0] * V
    for t in tokens:
        if 0 <= int(t) < V:
            c[int(t)] += 1
    return c


@pytest.mark.parametrize("seed", range(5))
def test_count_tokens_matches_algorithm_1(seed):
    rng = np.random.default_rng(seed)
    V = int(rng.integers(1, 40))
    toks = rng.integers(-3, V + 3, size=int(rng.integers(0, 300)))
    got = keepset.count_tokens(toks, V)
    assert got.dtype == np.uint64 and got.shape == (V,)
    assert got.tolist() == alg1_counts(toks, V)
    valid = int(((toks >= 0) & (toks < V)).sum())
    assert int(got.sum()) == valid
    # continuing a counter equals counting the concatenation
    more = rng.integers(0, V, size=50)
    assert keepset.count_tokens(more, V, got).tolist() == alg1_counts(np.concatenate([toks, more]), V)


def brute_rank(c):
    return sorted(range(len(c)), key=lambda v: (-int(c[v]), v))


@pytest.mark.parametrize("seed", range(6))
def test_top_k_against_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    V = int(rng.integers(1, 30))
    c = rng.integers(0, 4, size=V).astype(np.uint64)  # many ties
    order = brute_rank(c)
    for k in range(1, V + 1):
        keep, f2t = keepset.top_k(c, k)
        assert keep.tolist() == sorted(order[:k])
        assert np.all(np.diff(keep) > 0)
        dropped = np.setdiff1d(np.arange(V), keep)
        if len(dropped):
            assert c[keep].min() >= c[dropped].max()
            # at the boundary count, kept ties have lower ids than dropped ties
            b = c[keep].min()
            kt, dt = keep[c[keep] == b], dropped[c[dropped] == b]
            if len(kt) and len(dt):
                assert kt.max() < dt.min()
        assert np.array_equal(f2t[keep], np.arange(k))
        assert np.all(f2t[dropped] == -1)
    with pytest.raises(ValueError):
        keepset.top_k(c, 0)


def test_top_p_worked_example():
    c = np.array([3, 5, 0, 2], dtype=np.uint64)  # ranking 1, 0, 3, 2; N = 10
    assert keepset.top_p(c, 0.5)[0].tolist() == [1]          # ceil(5.0) = 5 <= 5
    assert keepset.top_p(c, 0.51)[0].tolist() == [0, 1]      # ceil(5.1) = 6 > 5
    assert keepset.top_p(c, 0.8)[0].tolist() == [0, 1]       # 8 <= 5 + 3
    assert keepset.top_p(c, 0.81)[0].tolist() == [0, 1, 3]  # ceil(8.1) = 9
    assert keepset.top_p(c, 1.0)[0].tolist() == [0, 1, 3]   # the support, not the zero-count id
    assert keepset.top_p(np.zeros(4, np.uint64), 0.3)[0].tolist() == [0]  # nothing counted: one id
    with pytest.raises(ValueError):
        keepset.top_p(c, 0.0)


@pytest.mark.parametrize("seed", range(5))
def test_top_p_is_the_shortest_ranked_prefix(seed):
    rng = np.random.default_rng(200 + seed)
    V = int(rng.integers(2, 50))
    c = rng.integers(0, 6, size=V).astype(np.uint64)
    order = brute_rank(c)
    N = int(c.sum())
    for p in (0.05, 0.3, 0.5, 0.77, 0.999, 1.0):
        keep, _ = keepset.top_p(c, p)
        k = len(keep)
        assert keep.tolist() == sorted(order[:k])
        target = int(np.ceil(p * N))
        mass = lambda j: sum(int(c[v]) for v in order[:j])
        assert mass(k) >= target
        if k > 1:
            assert mass(k - 1) < target


def test_min_frequency():
    c = np.array([3, 5, 0, 2, 3], dtype=np.uint64)
    assert keepset.min_frequency(c, 3)[0].tolist() == [0, 1, 4]  # count >= f, ties included
    assert keepset.min_frequency(c, 1)[0].tolist() == [0, 1, 3, 4]
    assert keepset.min_frequency(c, 0)[0].tolist() == [0, 1, 2, 3, 4]
    keep, f2t = keepset.min_frequency(c, 6)
    assert keep.tolist() == [] and np.all(f2t == -1)


def test_trimmed_head_gives_the_gathered_logits():
    rng = np.random.default_rng(7)
    V, H, M = 40, 16, 3
    W = rng.integers(0, 1 << 16, size=(V, H), dtype=np.uint16) & np.uint16(0x3FFF)  # finite bf16
    h = rng.integers(0, 1 << 16, size=(M, H), dtype=np.uint16) & np.uint16(0x3FFF)
    keep, _ = keepset.top_k(rng.integers(0, 9, size=V).astype(np.uint64), 11)
    Wt = keepset.trim_head(W, keep)
    assert Wt.shape == (11, H)
    for j, v in enumerate(keep):
        assert np.array_equal(Wt[j], W[v])
    assert np.array_equal(ref.lm_head(h, Wt, None), ref.lm_head(h, W, keep))


def test_zipf_stream_ranks_like_the_target():
    # input recipe check: the stream's most frequent ids are the permutation's best-ranked ids
    V = 5000
    toks = token_stream(V, 1 << 20, seed=3)
    perm, _ = zipf_ranking(V)
    c = keepset.count_tokens(toks, V)
    top = set(keepset.top_k(c, 50)[0].tolist())
    assert len(top & set(perm[:50].tolist())) >= 47
    assert int(c.sum()) == 1 << 20
